// attn_fwd_alibi.hip -- the forward kernels of score variant EXT_ALIBI.
#include "attn_fwd_kernels.h"

namespace attn {
template hipError_t launch_fwd_variant<EXT_ALIBI>(const FwdArgs&, int, bool, hipStream_t);
}  // namespace attn
