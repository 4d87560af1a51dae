// attn_bwd_alibi.hip -- the backward kernels of score variant EXT_ALIBI.
#include "attn_bwd_kernels.h"

namespace attn {
template hipError_t launch_bwd_variant<EXT_ALIBI>(const BwdArgs&, int, bool, hipStream_t);
}  // namespace attn
