// bf16 instantiations of the FlashAttention-2 forward kernel (fa2_fwd_kernel.h):
// every head dimension, mask and split setting.
#include "fa2_fwd_kernel.h"

namespace fa2 {

hipError_t launch_fwd_bf16(const FwdArgs& a) { return dispatch_fwd_mfma<__bf16>(a); }

}  // namespace fa2
