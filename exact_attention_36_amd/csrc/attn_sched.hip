// attn_sched.hip -- dispatch order of the packed grids.
//
// A packed batch lays its blocks out sequence after sequence (block start
// floor(cu[i] G / BM) + i, dew-flash-attn page, the packed-backward
// paragraph).  Under a causal mask the work of a block grows with the
// length of its sequence and with its position in it, so in layout order
// the longest blocks of a batch whose long sequences sit together start
// late and finish last, and the XCDs that drew those sequences end long
// after the others.  Before such a grid is launched, one workgroup estimates
// every block's work from the same band the kernels use (visible K/V tiles
// of a query block, visible 32-row query steps of a key block), sorts the
// blocks by it, largest first, and writes the permutation the kernels then
// read their block from: the longest-processing-time-first order, dealt to
// the XCDs round robin by the hardware.  The sort is a stable counting sort
// over 128 logarithmic work classes, so the table is the same on every run
// and a permutation of the block ids whatever cu_seqlens holds.
#include "attn_common.h"

namespace attn {

constexpr int ORDER_THREADS = 1024;
constexpr int ORDER_CLASSES = 128;   // work classes, 4 per doubling
constexpr int ORDER_COUNTERS = 256;  // threads that count and scatter, each a contiguous run of blocks

struct OrderGrids {
  OrderArgs g[2];
};

// Estimated cost of block b of a sequence, in steps of its kernel's loop
// plus a fixed cost per workgroup (its loads before the loop and its stores
// after it); 0 for an idle slot of the packed grid.
__device__ int block_work(const OrderArgs& a, const SeqInfo& si, int b) {
  const int G = a.s.group;
  const int prows = si.lq * G;
  if (a.key_major) {
    const int j0 = b * BWD_BN;
    if (j0 >= si.lk_slot) return 0;
    if (j0 >= si.lk || prows <= 0) return 2;  // writes zero gradients
    const QBand qb(a.s, si);
    const int q_lo = qb.qmin(j0), q_hi = qb.qmax(min(j0 + BWD_BN, si.lk) - 1);
    const int steps = q_hi >= q_lo ? ((q_hi + 1) * G - 1) / BWD_BM - (q_lo * G) / BWD_BM + 1 : 0;
    return steps + 3;
  }
  const int p0 = b * a.bm;
  if (p0 >= prows) return 0;
  const Band band(a.s, si);
  const int i_lo = div_group(p0, a.s), i_hi = div_group(min(p0 + a.bm, prows) - 1, a.s);
  const int kv_lo = band.kmin(i_lo), kv_hi = band.kmax(i_hi);
  const int tiles = kv_hi >= kv_lo ? kv_hi / FWD_BN - kv_lo / FWD_BN + 1 : 0;
  return tiles + 2;
}

// Work class, larger for more work: 0 for idle slots, else 1 + 4 log2(work).
// Blocks within about a fifth of each other's work share a class and keep
// their layout order, so runs of neighbouring blocks of one sequence (which
// read mostly the same rows) are still dispatched together.
__device__ __forceinline__ int work_class(int w) {
  if (w <= 0) return 0;
  return min(ORDER_CLASSES - 1, 1 + (int)(4.f * __builtin_amdgcn_logf((float)w)));
}

__global__ __launch_bounds__(ORDER_THREADS) void packed_order_kernel(const OrderGrids grids) {
  const OrderArgs a = blockIdx.x == 0 ? grids.g[0] : grids.g[1];
  __shared__ uint8_t cls[ORDER_MAX_BLOCKS];
  // [class][counter]: counts, then offsets; before that, per sequence: its
  // first block and its lengths (the sequence table of step 1)
  __shared__ uint32_t cnt[ORDER_CLASSES * ORDER_COUNTERS];
  __shared__ uint32_t part[ORDER_THREADS / 64];  // the waves' running totals
  const int t = threadIdx.x, n = a.nblk, nseq = a.s.nseq;
  // 1. every block's work class: the sequences' first blocks and lengths
  // into LDS (one thread per sequence), then every block finds its sequence
  // there by binary search
  int* const start = (int*)cnt;  // [nseq + 1]
  int* const len = start + nseq + 1;  // [nseq][3]: lq, lk, lk_slot
  const int G = a.key_major ? 1 : a.s.group, BM = a.key_major ? BWD_BN : a.bm;
  const int32_t* cu = a.key_major ? a.s.cu_k : a.s.cu_q;
  for (int seq = t; seq <= nseq; seq += ORDER_THREADS) {
    start[seq] = packed_block_start(cu, seq, G, BM);
    if (seq < nseq) {
      const SeqInfo si = seq_info(a.s, seq);
      len[3 * seq] = si.lq;
      len[3 * seq + 1] = si.lk;
      len[3 * seq + 2] = si.lk_slot;
    }
  }
  __syncthreads();
  for (int i = t; i < n; i += ORDER_THREADS) {
    int w = 0;  // a block no sequence claims stays idle
    if (i >= start[0]) {
      int lo = 0, hi = nseq - 1;  // last sequence starting at or before i
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      if (i < start[lo + 1]) {
        SeqInfo si{};
        si.lq = len[3 * lo];
        si.lk = len[3 * lo + 1];
        si.lk_slot = len[3 * lo + 2];
        w = block_work(a, si, i - start[lo]);
      }
    }
    cls[i] = (uint8_t)work_class(w);
  }
  __syncthreads();
  for (int i = t; i < ORDER_CLASSES * ORDER_COUNTERS; i += ORDER_THREADS) cnt[i] = 0;
  __syncthreads();
  // 2. counter c owns blocks [c * per, (c + 1) * per): its count per class
  const int per = (n + ORDER_COUNTERS - 1) / ORDER_COUNTERS;
  if (t < ORDER_COUNTERS)
    for (int i = t * per; i < min(n, (t + 1) * per); i++) cnt[cls[i] * ORDER_COUNTERS + t]++;
  __syncthreads();
  // 3. exclusive prefix over (class descending, counter ascending): thread t
  // owns the 32 consecutive entries of that order starting at 32 t
  constexpr int SPAN = ORDER_CLASSES * ORDER_COUNTERS / ORDER_THREADS;
  auto entry = [&](int l) -> uint32_t& {
    const int c = ORDER_CLASSES - 1 - l / ORDER_COUNTERS;
    return cnt[c * ORDER_COUNTERS + l % ORDER_COUNTERS];
  };
  uint32_t sum = 0;
  for (int l = t * SPAN; l < (t + 1) * SPAN; l++) sum += entry(l);
  // inclusive scan of the threads' sums: within each wave by shuffles, then
  // over the waves' totals
  const int lane = t & 63, wv = t >> 6;
  uint32_t inc = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t v = __shfl_up(inc, d);
    if (lane >= d) inc += v;
  }
  if (lane == 63) part[wv] = inc;
  __syncthreads();
  if (t == 0)
    for (int w = 1; w < ORDER_THREADS / 64; w++) part[w] += part[w - 1];
  __syncthreads();
  uint32_t run = inc - sum + (wv > 0 ? part[wv - 1] : 0u);
  for (int l = t * SPAN; l < (t + 1) * SPAN; l++) {
    const uint32_t c = entry(l);
    entry(l) = run;
    run += c;
  }
  __syncthreads();
  // 4. each counter places its blocks in order: a stable sort, so equal
  // classes keep the layout order
  const int hkv = a.s.hkv;
  if (t < ORDER_COUNTERS)
    for (int i = t * per; i < min(n, (t + 1) * per); i++) {
      const uint32_t pos = cnt[cls[i] * ORDER_COUNTERS + t]++;
      for (int g = 0; g < hkv; g++) a.order[(int64_t)pos * hkv + g] = g * n + i;
    }
}

hipError_t launch_order(const OrderArgs* grids, int n, hipStream_t st) {
  OrderGrids o{};
  for (int i = 0; i < n; i++) o.g[i] = grids[i];
  timing_begin(K_ORDER, st);
  hipLaunchKernelGGL(packed_order_kernel, dim3(n), dim3(ORDER_THREADS), 0, st, o);
  timing_end(K_ORDER, st);
  return hipGetLastError();
}

}  // namespace attn
