// Host side of the backward pass: workspace size and the launch entry that
// picks the translation unit compiled for the dtype and head dimension.
#include "internal.hpp"

namespace flexmi {

// Rows of the per-row workspace arrays: L padded to a multiple of 128 (the
// largest Q block), so every Q tile a block mask can name has its rows there.
static int64_t padded_rows(int L) { return ((int64_t)L + 127) / 128 * 128; }

size_t attn_bwd_workspace_bytes(int B, int Hq, int L) {
    return (size_t)2 * B * Hq * padded_rows(L) * sizeof(float);
}

hipError_t launch_attn_bwd(int dtype, int D, const BwdArgs& a, hipStream_t stream) {
    if (a.Lp != padded_rows(a.L)) return hipErrorInvalidValue;
    if (dtype == 1 && D == 64) return launch_attn_bwd_bf16_d64(a, stream);
    if (dtype == 1 && D == 128) return launch_attn_bwd_bf16_d128(a, stream);
    if (dtype == 0 && D == 64) return launch_attn_bwd_f32_d64(a, stream);
    if (dtype == 0 && D == 128) return launch_attn_bwd_f32_d128(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace flexmi
