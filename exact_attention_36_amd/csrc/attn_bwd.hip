// attn_bwd.hip -- backward launchers: clearing dsinks, then the dQ and dK/dV
// kernels of the call's score variant (soft cap / ALiBi instances compile in
// their own translation units).
#include "attn_bwd_kernels.h"

namespace attn {

__global__ void bwd_zero_kernel(float* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

extern template hipError_t launch_bwd_variant<EXT_CAP>(const BwdArgs&, int, bool, hipStream_t);
extern template hipError_t launch_bwd_variant<EXT_ALIBI>(const BwdArgs&, int, bool, hipStream_t);
extern template hipError_t launch_bwd_variant<EXT_CAP | EXT_ALIBI>(const BwdArgs&, int, bool, hipStream_t);

hipError_t launch_bwd(const BwdArgs& a, int tile_d, bool f16, hipStream_t st) {
  if (a.sinks && a.dsinks) {
    timing_begin(K_BWD_ZERO, st);
    hipLaunchKernelGGL(bwd_zero_kernel, dim3((a.dsink_count + 255) / 256), dim3(256), 0, st, a.dsinks,
                       a.dsink_count);
    timing_end(K_BWD_ZERO, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  switch (a.x.ext) {
    case EXT_CAP: return launch_bwd_variant<EXT_CAP>(a, tile_d, f16, st);
    case EXT_ALIBI: return launch_bwd_variant<EXT_ALIBI>(a, tile_d, f16, st);
    case EXT_CAP | EXT_ALIBI: return launch_bwd_variant<EXT_CAP | EXT_ALIBI>(a, tile_d, f16, st);
    default: return launch_bwd_variant<0>(a, tile_d, f16, st);
  }
}

}  // namespace attn
