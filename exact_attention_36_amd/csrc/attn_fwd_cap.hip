// attn_fwd_cap.hip -- the forward kernels of score variant EXT_CAP.
#include "attn_fwd_kernels.h"

namespace attn {
template hipError_t launch_fwd_variant<EXT_CAP>(const FwdArgs&, int, bool, hipStream_t);
}  // namespace attn
