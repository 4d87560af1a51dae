// attn_fwd.hip -- forward launchers: the kernel of the call's score variant
// (soft cap / ALiBi instances compile in their own translation units) and the
// split-KV combine kernel.
#include "attn_fwd_kernels.h"

namespace attn {

extern template hipError_t launch_fwd_variant<EXT_CAP>(const FwdArgs&, int, bool, hipStream_t);
extern template hipError_t launch_fwd_variant<EXT_ALIBI>(const FwdArgs&, int, bool, hipStream_t);
extern template hipError_t launch_fwd_variant<EXT_CAP | EXT_ALIBI>(const FwdArgs&, int, bool, hipStream_t);

hipError_t launch_fwd(const FwdArgs& a, int tile_d, bool f16, hipStream_t st) {
  timing_begin(K_FWD, st);
  hipError_t e;
  switch (a.x.ext) {
    case EXT_CAP: e = launch_fwd_variant<EXT_CAP>(a, tile_d, f16, st); break;
    case EXT_ALIBI: e = launch_fwd_variant<EXT_ALIBI>(a, tile_d, f16, st); break;
    case EXT_CAP | EXT_ALIBI: e = launch_fwd_variant<EXT_CAP | EXT_ALIBI>(a, tile_d, f16, st); break;
    default: e = launch_fwd_variant<0>(a, tile_d, f16, st); break;
  }
  timing_end(K_FWD, st);
  return e;
}

template <int D, bool F16>
static hipError_t launch_combine_t(const FwdArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.s.nseq * a.s.hkv * a.nmb * a.bm;
  timing_begin(K_FWD_COMBINE, st);
  const int64_t per_block = 4 * (64 / (D / 4));  // rows per workgroup: 4 waves
  hipLaunchKernelGGL((fwd_combine_kernel<D, F16>), dim3((unsigned)((rows + per_block - 1) / per_block)), dim3(THREADS),
                     0, st, a);
  timing_end(K_FWD_COMBINE, st);
  return hipGetLastError();
}

hipError_t launch_fwd_combine(const FwdArgs& a, int tile_d, bool f16, hipStream_t st) {
  if (tile_d == 256) return f16 ? launch_combine_t<256, true>(a, st) : launch_combine_t<256, false>(a, st);
  if (tile_d == 128) return f16 ? launch_combine_t<128, true>(a, st) : launch_combine_t<128, false>(a, st);
  return f16 ? launch_combine_t<64, true>(a, st) : launch_combine_t<64, false>(a, st);
}

}  // namespace attn
