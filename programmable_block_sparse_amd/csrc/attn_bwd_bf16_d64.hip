// Backward kernels instantiated for bf16 inputs at head dimension 64 (one
// translation unit per dtype and head dimension so they compile in parallel).
#include "attn_bwd_impl.hpp"

namespace flexmi {

hipError_t launch_attn_bwd_bf16_d64(const BwdArgs& a, hipStream_t stream) { return bwd_dispatch<__bf16, 64>(a, stream); }

}  // namespace flexmi
