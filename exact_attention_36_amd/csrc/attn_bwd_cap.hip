// attn_bwd_cap.hip -- the backward kernels of score variant EXT_CAP.
#include "attn_bwd_kernels.h"

namespace attn {
template hipError_t launch_bwd_variant<EXT_CAP>(const BwdArgs&, int, bool, hipStream_t);
}  // namespace attn
