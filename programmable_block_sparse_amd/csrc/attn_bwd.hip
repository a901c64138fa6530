// Host side of the backward pass: workspace size and the launch entry that
// picks the translation unit compiled for the dtype and head dimension.
#include <algorithm>

#include "internal.hpp"

namespace flexmi {

// Rows of the per-row workspace arrays: L padded to a multiple of 128 (the
// largest Q block), so every Q tile a block mask can name has its rows there.
static int64_t padded_rows(int L) { return ((int64_t)L + 127) / 128 * 128; }

int bwd_kv_splits(int group, int nQB, int q_block) {
    const int64_t max_tiles = (int64_t)group * nQB * (q_block / 64);
    return (int)std::min<int64_t>(4, std::max<int64_t>(1, (max_tiles + kBwdChunkTiles - 1) / kBwdChunkTiles));
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int L, int S, int D, int q_block, int kv_block, int nQB,
                                int nKB) {
    (void)S;
    size_t bytes = (size_t)2 * B * Hq * padded_rows(L) * sizeof(float);
    const int splits = bwd_kv_splits(Hq / Hkv, nQB, q_block);
    if (splits > 1) {
        const size_t cols = (size_t)B * Hkv * nKB * (kv_block / 64);
        bytes += (size_t)splits * cols * 2 * 64 * D * sizeof(float);
    }
    return bytes;
}

hipError_t launch_attn_bwd(int dtype, int D, const BwdArgs& a, hipStream_t stream) {
    if (a.Lp != padded_rows(a.L) || a.kv_splits != bwd_kv_splits(a.group, a.nQB, a.q_block) ||
        (a.kv_splits > 1 && a.ws_part == nullptr))
        return hipErrorInvalidValue;
    if (dtype == 1 && D == 64) return launch_attn_bwd_bf16_d64(a, stream);
    if (dtype == 1 && D == 128) return launch_attn_bwd_bf16_d128(a, stream);
    if (dtype == 0 && D == 64) return launch_attn_bwd_f32_d64(a, stream);
    if (dtype == 0 && D == 128) return launch_attn_bwd_f32_d128(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace flexmi
