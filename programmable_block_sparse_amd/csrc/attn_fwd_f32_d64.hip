// Forward kernels instantiated for fp32 inputs at head dimension 64 (one
// translation unit per dtype and head dimension so they compile in parallel).
#include "attn_fwd_impl.hpp"

namespace flexmi {

hipError_t launch_attn_fwd_f32_d64(const FwdArgs& a, hipStream_t stream) {
    return dispatch<float, 64, false>(a, stream);
}

}  // namespace flexmi
