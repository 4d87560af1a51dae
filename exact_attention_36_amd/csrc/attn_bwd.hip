// attn_bwd.hip -- backward launchers: the dQ and dK/dV kernels of the call's
// score variant (soft cap / ALiBi instances compile in their own translation
// units), then the sum of the sink gradient.
#include "attn_bwd_kernels.h"

namespace attn {

// d(sink): each q head's gradient is the sum of the dQ workgroups' partial
// sums, taken in workgroup order so that it is the same on every run; sink k
// of a head gets the share 2^(s_hk log2 e - s2) of it (s2 = the head's sinks
// as one logit), and a row of sinks shared by the heads sums the heads' in
// head order.  One thread per output.
__global__ void bwd_dsink_kernel(const BwdArgs a) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= a.dsink_count) return;
  const int G = a.s.group, n = a.x.nsinks;
  auto head_sum = [&](int h) {
    const int g = h / G;
    const float* src = a.dsink_part + (int64_t)g * a.nbq * G + (h - g * G);
    float v = 0.f;
    for (int b = 0; b < a.nbq; b++) v += src[(int64_t)b * G];
    return v;
  };
  auto share = [&](int h, int k) {
    if (n == 1) return 1.f;
    return exp2_fast(fmaf(a.sinks[h * a.x.sink_hstride + k], LOG2E, -sink_log2(a.sinks, a.x, h)));
  };
  if (a.x.sink_hstride == 0) {
    float v = 0.f;
    for (int h = 0; h < a.s.hq; h++) v += head_sum(h) * share(h, e);
    a.dsinks[e] = v;
  } else {
    const int h = e / n;
    a.dsinks[e] = head_sum(h) * share(h, e - h * n);
  }
}

extern template hipError_t launch_bwd_variant<EXT_CAP>(const BwdArgs&, int, bool, hipStream_t);
extern template hipError_t launch_bwd_variant<EXT_ALIBI>(const BwdArgs&, int, bool, hipStream_t);
extern template hipError_t launch_bwd_variant<EXT_CAP | EXT_ALIBI>(const BwdArgs&, int, bool, hipStream_t);

hipError_t launch_bwd(const BwdArgs& a, int tile_d, bool f16, hipStream_t st) {
  hipError_t e;
  switch (a.x.ext) {
    case EXT_CAP: e = launch_bwd_variant<EXT_CAP>(a, tile_d, f16, st); break;
    case EXT_ALIBI: e = launch_bwd_variant<EXT_ALIBI>(a, tile_d, f16, st); break;
    case EXT_CAP | EXT_ALIBI: e = launch_bwd_variant<EXT_CAP | EXT_ALIBI>(a, tile_d, f16, st); break;
    default: e = launch_bwd_variant<0>(a, tile_d, f16, st); break;
  }
  if (e != hipSuccess || !a.dsinks || !a.dsink_part) return e;
  BwdArgs r = a;
  if (a.total_ctas_q == 0) r.nbq = 0;  // no dQ workgroup ran: every sum is 0
  timing_begin(K_BWD_DSINK, st);
  hipLaunchKernelGGL(bwd_dsink_kernel, dim3((a.dsink_count + 255) / 256), dim3(256), 0, st, r);
  timing_end(K_BWD_DSINK, st);
  return hipGetLastError();
}

}  // namespace attn
