// attn_common.h -- sequence geometry and the causal / sliding-window band,
// shared by the forward and backward kernels.
#pragma once
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// n / group for 0 <= n < 2^32 / G (packed rows of one sequence; the host
// rejects sequences with queries * G^2 >= 2^32): with M = ceil(2^32 / G),
// n*M/2^32 = n/G + n*(M - 2^32/G)/2^32 exceeds n/G by less than n/2^32 < 1/G,
// which cannot carry past the next multiple of 1/G, so the high word is the
// quotient.
__device__ __forceinline__ int div_group(int n, const SeqArgs& s) {
  return s.group == 1 ? n : (int)__umulhi((uint32_t)n, s.group_magic);
}

struct SeqInfo {
  int q0, lq, k0, lk;  // first token and used length of the sequence in q and in k/v
  int lk_slot;         // key rows the slot holds (>= lk; dK/dV rows past lk are zero)
};

__device__ __forceinline__ SeqInfo seq_info(const SeqArgs& s, int seq) {
  SeqInfo r;
  int lq_slot;
  if (s.cu_q) {
    r.q0 = s.cu_q[seq];
    lq_slot = s.cu_q[seq + 1] - r.q0;
    r.k0 = s.cu_k[seq];
    r.lk_slot = s.cu_k[seq + 1] - r.k0;
  } else {
    r.q0 = seq * s.sq;
    lq_slot = s.sq;
    r.k0 = seq * s.sk;
    r.lk_slot = s.sk;
  }
  // used lengths, read as given but kept inside the slot
  r.lq = s.seqused_q ? min(max(s.seqused_q[seq], 0), lq_slot) : lq_slot;
  r.lk = s.seqused_k ? min(max(s.seqused_k[seq], 0), r.lk_slot) : r.lk_slot;
  return r;
}

// Keys visible to query i: [kmin(i), kmax(i)] (empty when kmax < kmin).
// Causal and window bounds are aligned bottom-right: query i lines up with
// key i + lk - lq (fa4-jax page, bottom-right alignment paragraph; window
// interval of the flash_attn_func docstring, vllm-project/flash-attention
// README on the GitHub search page).  Both bounds are nondecreasing in i.
struct Band {
  int wl, wr, causal, delta, lk;
  __device__ __forceinline__ Band(const SeqArgs& s, const SeqInfo& si)
      : wl(s.wl), wr(s.wr), causal(s.causal), delta(si.lk - si.lq), lk(si.lk) {}
  __device__ __forceinline__ int kmin(int i) const { return wl >= 0 ? max(0, i + delta - wl) : 0; }
  __device__ __forceinline__ int kmax(int i) const {
    int hi = lk - 1;
    if (causal) hi = min(hi, i + delta + (wr >= 0 ? min(0, wr) : 0));
    else if (wr >= 0) hi = min(hi, i + delta + wr);
    return hi;
  }
};

// No causal mask and no window: every block of a batched grid's group does
// the same work.
__device__ __forceinline__ bool unmasked(const SeqArgs& s) { return !s.causal && s.wl < 0 && s.wr < 0; }

// Queries that see key j: [qmin(j), qmax(j)], the inverse of the band.
// Used by the key-major backward to visit only the query blocks that see a
// key block.
struct QBand {
  int wl, wr, causal, delta, lq;
  __device__ __forceinline__ QBand(const SeqArgs& s, const SeqInfo& si)
      : wl(s.wl), wr(s.wr), causal(s.causal), delta(si.lk - si.lq), lq(si.lq) {}
  // j <= i + delta + r  <=>  i >= j - delta - r   (r = effective right offset)
  __device__ __forceinline__ int qmin(int j) const {
    int r = causal ? (wr >= 0 ? min(0, wr) : 0) : wr;
    if (!causal && wr < 0) return 0;
    return max(0, j - delta - r);
  }
  // j >= i + delta - wl  <=>  i <= j - delta + wl
  __device__ __forceinline__ int qmax(int j) const { return wl >= 0 ? min(lq - 1, j - delta + wl) : lq - 1; }
};

// Packed-batch block start of sequence i: floor(cu[i] * G / BM) + i, so a
// sequence's blocks start right after the previous sequence's and a batch of
// empty or short sequences costs what its tokens do (dew-flash-attn page, the
// packed-backward paragraph).
__device__ __forceinline__ int packed_block_start(const int32_t* cu, int i, int G, int BM) {
  return (int)(((int64_t)cu[i] * G) / BM) + i;
}

// Largest i in [0, n) with packed_block_start(i) <= t (block starts are
// strictly increasing, and start(0) = 0).
__device__ __forceinline__ int find_sequence(const int32_t* cu, int n, int t, int G, int BM) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (packed_block_start(cu, mid, G, BM) <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------- sinks
// The sinks of q head h act as one logit, log sum_k exp(s_hk) (each is a
// value-less logit of the row's softmax: dew-flash-attn page, sinks
// paragraph; several per head: ejkernel flash_attention API page,
// softmax_aux).  Returned in log2 units; -inf when every sink is -inf.
__device__ __forceinline__ float sink_log2(const float* sinks, const ScoreArgs& x, int h) {
  const float* s = sinks + h * x.sink_hstride;
  if (x.nsinks == 1) return s[0] * LOG2E;
  float mx = -INFINITY;
  for (int k = 0; k < x.nsinks; k++) mx = fmaxf(mx, s[k]);
  if (mx == -INFINITY) return -INFINITY;
  float sum = 0.f;
  for (int k = 0; k < x.nsinks; k++) sum += exp2_fast((s[k] - mx) * LOG2E);
  return mx * LOG2E + log2_fast(sum);
}

// ---------------------------------------------------------------- score variants
// Raw score x of a (row, key) pair -> x' (see ScoreArgs): soft cap
// (vllm-project/flash-attention README on the GitHub search page, "2.6:
// Softcapping"; ejkernel page, logits_soft_cap), then the ALiBi bias
// -slope |i + Lk - Lq - j| (alibi_slopes, flash_attn_func docstring of the
// same README).  kb = slope / scale of the row's q head, dist = i + Lk - Lq - j.
// t receives tanh(x scale / cap) (dx'/dx = 1 - t^2) under the cap.
template <int EXT>
__device__ __forceinline__ float ext_score(float x, const ScoreArgs& a, float kb, float dist, float& t) {
  if constexpr ((EXT & EXT_CAP) != 0) {
    // tanh(u) = 1 - 2 / (1 + e^(2u)); e^(2u) = 2^(x k2) overflows to inf for
    // large u (t = 1) and underflows to 0 for very negative u (t = -1)
    t = fmaf(-2.f, __builtin_amdgcn_rcpf(1.f + exp2_fast(x * a.cap_k2)), 1.f);
    x = a.cap_k3 * t;
  }
  if constexpr ((EXT & EXT_ALIBI) != 0) x = fmaf(-kb, fabsf(dist), x);
  return x;
}

// slope / scale of q head h in sequence seq (0 without ALiBi)
__device__ __forceinline__ float alibi_kb(const ScoreArgs& x, int seq, int h) {
  return x.alibi ? x.alibi[(int64_t)seq * x.alibi_bstride + h] * x.inv_scale : 0.f;
}

}  // namespace attn
