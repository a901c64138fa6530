// Forward kernels instantiated for bf16 inputs at head dimension 64 (one
// translation unit per dtype and head dimension so they compile in parallel).
#include "attn_fwd_impl.hpp"

namespace flexmi {

hipError_t launch_attn_fwd_bf16_d64(const FwdArgs& a, hipStream_t stream) {
    if (a.splits > 0) return dispatch<__bf16, 64, true>(a, stream);
    return dispatch<__bf16, 64, false>(a, stream);
}

}  // namespace flexmi
