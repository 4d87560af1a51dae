// attn_bwd.hip -- backward launchers: the dQ and dK/dV kernels of the call's
// score variant (soft cap / ALiBi instances compile in their own translation
// units), then the sum of the sink gradient.
#include "attn_bwd_kernels.h"

namespace attn {

// d(sink): each q head's gradient is the sum of the dQ workgroups' partial
// sums, and sink k of a head gets the share 2^(s_hk log2 e - s2) of it (s2 =
// the head's sinks as one logit); a row of sinks shared by the heads gets the
// sum over the heads.  One workgroup per output: thread t adds the partials
// t, t + 256, ... of the head (heads in order for a shared row), then a tree
// of fixed shape in LDS adds the threads' sums -- the same order on every run.
constexpr int DSINK_THREADS = 256;
__global__ __launch_bounds__(DSINK_THREADS) void bwd_dsink_kernel(const BwdArgs a) {
  const int e = blockIdx.x, t = threadIdx.x;
  const int G = a.s.group, n = a.x.nsinks;
  const bool shared = a.x.sink_hstride == 0;
  const int h0 = shared ? 0 : e / n, h1 = shared ? a.s.hq : h0 + 1, k = shared ? e : e - h0 * n;
  float acc = 0.f;
  for (int h = h0; h < h1; h++) {
    const int g = h / G;
    const float* src = a.dsink_part + (int64_t)g * a.nbq * G + (h - g * G);
    for (int b = t; b < a.nbq; b += DSINK_THREADS) acc += src[(int64_t)b * G];
  }
  __shared__ float red[DSINK_THREADS];
  red[t] = acc;
  __syncthreads();
#pragma unroll
  for (int w = DSINK_THREADS / 2; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  if (t == 0) {
    float share = 1.f;  // the same for every head of a shared row
    if (n > 1) share = exp2_fast(fmaf(a.sinks[h0 * a.x.sink_hstride + k], LOG2E, -sink_log2(a.sinks, a.x, h0)));
    a.dsinks[e] = red[0] * share;
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
  hipLaunchKernelGGL(bwd_dsink_kernel, dim3(a.dsink_count), dim3(DSINK_THREADS), 0, st, r);
  timing_end(K_BWD_DSINK, st);
  return hipGetLastError();
}

}  // namespace attn
