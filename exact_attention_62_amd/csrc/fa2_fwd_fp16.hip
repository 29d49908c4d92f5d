// fp16 instantiations of the FlashAttention-2 forward kernel (fa2_fwd_kernel.h):
// every head dimension, mask and split setting.
#include "fa2_fwd_kernel.h"

namespace fa2 {

hipError_t launch_fwd_fp16(const FwdArgs& a) { return dispatch_fwd_mfma<_Float16>(a); }

}  // namespace fa2
