// attn_api.cpp -- the C ABI: host-side argument checks, work decomposition
// and kernel launches.  Nothing here reads device memory or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/attn.h"
#include "attn_kernels.h"
#include "attn_device.h"

using namespace attn;

namespace {

thread_local char g_err[512] = "no error";

attn_status fail(attn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

constexpr int64_t OFF_LIMIT = (int64_t)1 << 31;  // byte offsets inside one sequence are 32-bit
constexpr size_t ALIGN = 256;
constexpr int MAX_SINKS = 64;  // sinks per q head

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Head dim of the kernel tiles that serve head_dim: the next of 64, 128, 256
// (the tile columns past head_dim are zero).
int tile_dim(int head_dim) { return head_dim <= 64 ? 64 : head_dim <= 128 ? 128 : 256; }

float resolve_scale(const attn_params* p) {
  const float s = p->softmax_scale;
  if (!(s > 0.f) || std::isnan(s)) return 1.0f / std::sqrt((float)p->head_dim);
  return s;
}

attn_status check_params(const attn_params* p) {
  if (!p) return fail(ATTN_EINVAL, "params is NULL");
  if (p->dtype != ATTN_BF16 && p->dtype != ATTN_FP16)
    return fail(ATTN_EINVAL, "dtype must be ATTN_BF16 or ATTN_FP16 (got %d)", p->dtype);
  if (p->head_dim < 8 || p->head_dim > 256 || p->head_dim % 8)
    return fail(ATTN_EINVAL, "head_dim must be a multiple of 8 in [8, 256] (got %d)", p->head_dim);
  if (p->heads_q < 1 || p->heads_kv < 1)
    return fail(ATTN_EINVAL, "heads_q and heads_kv must be >= 1 (got %d, %d)", p->heads_q, p->heads_kv);
  if (p->heads_q % p->heads_kv)
    return fail(ATTN_EINVAL, "heads_kv (%d) must divide heads_q (%d)", p->heads_kv, p->heads_q);
  if (p->heads_q > FWD_BM && p->heads_q / p->heads_kv > FWD_BM)
    return fail(ATTN_ENOTSUP, "more than %d q heads per kv head", FWD_BM);
  if (p->window_left < -1 || p->window_right < -1)
    return fail(ATTN_EINVAL, "window bounds must be >= -1 (got %d, %d)", p->window_left, p->window_right);
  if (p->causal != 0 && p->causal != 1) return fail(ATTN_EINVAL, "causal must be 0 or 1");
  if (p->num_sinks < 0 || p->num_sinks > MAX_SINKS)
    return fail(ATTN_EINVAL, "num_sinks must be in [0, %d] (got %d)", MAX_SINKS, p->num_sinks);
  if (p->sinks_shared != 0 && p->sinks_shared != 1) return fail(ATTN_EINVAL, "sinks_shared must be 0 or 1");
  if (!(p->softcap >= 0.f) || std::isinf(p->softcap))
    return fail(ATTN_EINVAL, "softcap must be finite and >= 0 (got %g)", (double)p->softcap);
  if (p->alibi_per_batch != 0 && p->alibi_per_batch != 1) return fail(ATTN_EINVAL, "alibi_per_batch must be 0 or 1");
  return ATTN_OK;
}

// Score variants and the sinks' layout, from the params.
ScoreArgs score_args(const attn_params* p, float scale) {
  ScoreArgs x{};
  x.inv_scale = 1.f / scale;
  if (p->softcap > 0.f) {
    x.ext |= EXT_CAP;
    x.cap_k2 = 2.f * scale * 1.4426950408889634f / p->softcap;
    x.cap_k3 = p->softcap / scale;
  }
  if (p->alibi_slopes) {
    x.ext |= EXT_ALIBI;
    x.alibi = p->alibi_slopes;
    x.alibi_bstride = p->alibi_per_batch ? p->heads_q : 0;
  }
  x.nsinks = p->num_sinks < 1 ? 1 : p->num_sinks;
  x.sink_hstride = p->sinks_shared ? 0 : x.nsinks;
  return x;
}

attn_status check_extent(int64_t max_q, int64_t max_k, const attn_params* p) {
  const int64_t D = p->head_dim;
  const int64_t G = p->heads_q / p->heads_kv;
  // The kernels divide a sequence's packed row index n < max_q * G by G with a
  // multiply-high by ceil(2^32 / G), exact for n < 2^32 / G.
  if (G >= 2 && max_q * G * G >= ((int64_t)1 << 32))
    return fail(ATTN_ENOTSUP, "a sequence of %lld queries with %lld q heads per kv head exceeds the exact range "
                "of the kernels' group division (queries * G^2 < 2^32)", (long long)max_q, (long long)G);
  if ((max_q + 256) * p->heads_q * D * 4 >= OFF_LIMIT)
    return fail(ATTN_ENOTSUP, "a sequence of %lld queries exceeds the 32-bit offset range", (long long)max_q);
  if ((max_k + BWD_BN) * p->heads_kv * D * 4 >= OFF_LIMIT)
    return fail(ATTN_ENOTSUP, "a sequence of %lld keys exceeds the 32-bit offset range", (long long)max_k);
  return ATTN_OK;
}

SeqArgs seq_args(const attn_params* p, const int32_t* cu_q, const int32_t* cu_k, int32_t nseq, int64_t sq,
                 int64_t sk, int64_t total_q) {
  SeqArgs s{};
  s.cu_q = cu_q;
  s.cu_k = cu_k;
  s.nseq = nseq;
  s.sq = (int32_t)sq;
  s.sk = (int32_t)sk;
  s.total_q = (int32_t)total_q;
  s.hq = p->heads_q;
  s.hkv = p->heads_kv;
  s.group = p->heads_q / p->heads_kv;
  s.dg = p->head_dim;
  s.seqused_q = p->seqused_q;
  s.seqused_k = p->seqused_k;
  s.group_magic = s.group >= 2 ? (uint32_t)((((uint64_t)1 << 32) + s.group - 1) / s.group) : 0u;
  s.causal = p->causal;
  s.wl = p->window_left;
  s.wr = p->window_right;
  return s;
}

// Split-KV when the grid would not fill the chip and each split keeps >= 8
// tiles: about 512 workgroups, one per slot of the chip (two per CU).  On the
// decode shape (256 base workgroups) targets of 1024, 2048 and 4096 measured
// 1.5 %, 6 % and 15 % slower: the splits' merge grows and the split kernel
// does not speed up.
int choose_split(int64_t base_ctas, int64_t sk) {
  const int64_t tiles = cdiv(sk, FWD_BN);
  if (base_ctas >= 512 || tiles < 16) return 1;
  int64_t n = cdiv(512, base_ctas);
  n = std::min<int64_t>(n, tiles / 8);
  n = std::min<int64_t>(n, 64);
  return (int)std::max<int64_t>(n, 1);
}

size_t fwd_ws(const attn_params* p, int64_t B, int64_t sq, int64_t sk, int* n_split_out, int* bm_out) {
  const int G = p->heads_q / p->heads_kv;
  const int bm = FWD_BM;
  const int64_t nmb = cdiv(sq * G, bm);
  const int ns = choose_split(nmb * p->heads_kv * B, sk);
  if (n_split_out) *n_split_out = ns;
  if (bm_out) *bm_out = bm;
  if (ns <= 1) return 0;
  const int64_t rows = (int64_t)ns * B * p->heads_kv * nmb * bm;
  return align_up(rows * tile_dim(p->head_dim) * 4) + align_up(rows * 4);
}

// dQ workgroups per kv head: batched, nseq * ceil(sq G / 128); packed, the
// linear grid's floor(total_q G / 128) + nseq.
int64_t dq_blocks(const attn_params* p, bool packed, int64_t nseq, int64_t sq, int64_t total_q) {
  const int64_t G = p->heads_q / p->heads_kv;
  return packed ? (total_q * G) / BWD_QBM + nseq : nseq * cdiv(sq * G, BWD_QBM);
}

// The packed backward's grids run in the order of schedule tables built on
// the device before them (attn_sched.hip, one extra launch) when the dK/dV
// grid has at least ORDER_MIN_CTAS workgroups (four rounds of two per CU) and
// some sequence may be ORDER_MIN_LEN queries long or more: then the work of
// its key blocks ranges widely and the layout order can leave whole XCDs
// running a few long blocks at the end.  Smaller grids finish in a round or
// two anyway, and batches of short sequences have no long blocks.
constexpr int64_t ORDER_MIN_CTAS = 2048;
constexpr int64_t ORDER_MIN_LEN = 1024;
bool use_order(const attn_params* p, int64_t nblk_k, int64_t nblk_q, int64_t nseq, int64_t max_q) {
  return nblk_k * p->heads_kv >= ORDER_MIN_CTAS && max_q >= ORDER_MIN_LEN && nblk_k <= ORDER_MAX_BLOCKS &&
         nblk_q <= ORDER_MAX_BLOCKS && nseq <= ORDER_MAX_SEQS;
}

// Backward workspace: D_i and the sink-adjusted log-sum-exp, laid out like
// lse; each dQ workgroup's largest row norm of dO and largest |D_i|
// ([Hkv][blocks][2]), from which the dK/dV kernel scales dS into fp16's
// range; with sinks, each dQ workgroup's sums of the sink gradient per q head
// of its group ([Hkv][blocks][G]), which a last kernel adds up in a fixed
// order; for packed calls, the schedule tables of the dQ and dK/dV grids
// (nblk_k: key blocks per kv head, 0 when batched; nseq: the sequences;
// max_q: the bound on their query counts).
struct BwdWs {
  size_t delta, lse2, dscale_part, dsink_part, order_q, order_k, total;
};
BwdWs bwd_ws(const attn_params* p, int64_t tq, int64_t nbq, int64_t nblk_k, int64_t nseq, int64_t max_q,
             int32_t grad_dtype) {
  (void)grad_dtype;
  BwdWs w{};
  const int64_t rows = tq * p->heads_q;
  w.delta = align_up(rows * 4);
  w.lse2 = align_up(rows * 4);
  w.dscale_part = align_up(nbq * p->heads_kv * 2 * 4);
  w.dsink_part = p->sinks ? align_up(nbq * p->heads_q * 4) : 0;  // Hkv * nbq * G = nbq * Hq
  if (nblk_k > 0 && use_order(p, nblk_k, nbq, nseq, max_q)) {
    w.order_q = align_up(nbq * p->heads_kv * 4);
    w.order_k = align_up(nblk_k * p->heads_kv * 4);
  }
  w.total = w.delta + w.lse2 + w.dscale_part + w.dsink_part + w.order_q + w.order_k;
  return w;
}

attn_status launched(hipError_t e) {
  if (e != hipSuccess) return fail(ATTN_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

attn_status check_ws(const void* ws, size_t have, size_t need) {
  if (have < need) return fail(ATTN_EINVAL, "workspace too small: %zu bytes given, %zu needed", have, need);
  if (need && !ws) return fail(ATTN_EINVAL, "workspace is NULL but %zu bytes are needed", need);
  if (need && ((uintptr_t)ws % 16)) return fail(ATTN_EINVAL, "workspace must be 16-byte aligned");
  return ATTN_OK;
}

// KV-cache addressing of a batched forward (all null / 0: plain K, V).
struct KvCache {
  const int32_t* seqused_k = nullptr;
  const int32_t* block_table = nullptr;
  int32_t page_rows = 0, pages_per_seq = 0;
};

attn_status run_fwd(const attn_params* p, const int32_t* cu_q, const int32_t* cu_k, int32_t nseq, int64_t sq,
                    int64_t sk, int64_t total_q, int64_t max_q, const void* q, const void* k, const void* v, void* o,
                    float* lse, void* ws, size_t ws_bytes, void* stream, const KvCache& kvc = KvCache{}) {
  const bool packed = cu_q != nullptr;
  FwdArgs a{};
  a.s = seq_args(p, cu_q, cu_k, nseq, sq, sk, total_q);
  if (kvc.seqused_k) a.s.seqused_k = kvc.seqused_k;  // the cache's used lengths
  a.s.block_table = kvc.block_table;
  a.s.page_rows = kvc.page_rows;
  a.s.pages_per_seq = kvc.pages_per_seq;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.sinks = p->sinks;
  a.scale_log2 = resolve_scale(p) * 1.4426950408889634f;
  a.x = score_args(p, resolve_scale(p));
  const int G = a.s.group;
  a.n_split = 1;
  if (packed) {
    a.bm = FWD_BM;
    a.nblk = (int32_t)((total_q * G) / a.bm + nseq);
    const int64_t ctas = (int64_t)a.nblk * p->heads_kv;
    if (ctas >= INT32_MAX) return fail(ATTN_ENOTSUP, "grid too large");
    a.total_ctas = (int32_t)ctas;
    // every sequence's packed rows fit one work tile: each K/V tile is read
    // once (max_q only selects the cache policy; a wrong value costs speed,
    // not correctness)
    a.kv_once = (int64_t)max_q * G <= a.bm;
  } else {
    int ns = 1, bm = 128;
    const size_t need = fwd_ws(p, nseq, sq, sk, &ns, &bm);
    attn_status st = check_ws(ws, ws_bytes, need);
    if (st != ATTN_OK) return st;
    a.bm = bm;
    a.nmb = (int32_t)cdiv(sq * G, bm);
    a.n_split = ns;
    if (ns > 1) {
      const int64_t rows = (int64_t)ns * nseq * p->heads_kv * a.nmb * bm;
      a.o_part = (float*)ws;
      a.lse_part = (float*)((char*)ws + align_up(rows * tile_dim(p->head_dim) * 4));
    }
    const int64_t ctas = GroupGrid{(int)(ns * p->heads_kv * (int64_t)nseq), a.nmb}.grid_size();
    if (ctas >= INT32_MAX || (int64_t)ns * p->heads_kv * nseq >= INT32_MAX) return fail(ATTN_ENOTSUP, "grid too large");
    a.total_ctas = (int32_t)ctas;
    a.kv_once = a.nmb == 1;  // one work tile per (sequence, kv head)
  }
  if (a.total_ctas == 0) return ATTN_OK;
  hipStream_t s = (hipStream_t)stream;
  attn_status st = launched(launch_fwd(a, tile_dim(p->head_dim), p->dtype == ATTN_FP16, s));
  if (st != ATTN_OK || a.n_split <= 1) return st;
  return launched(launch_fwd_combine(a, tile_dim(p->head_dim), p->dtype == ATTN_FP16, s));
}

attn_status run_bwd(const attn_params* p, const int32_t* cu_q, const int32_t* cu_k, int32_t nseq, int64_t sq,
                    int64_t sk, int64_t total_q, int64_t total_k, int64_t max_q, const void* q, const void* k, const void* v,
                    const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv, float* dsinks,
                    int32_t grad_dtype, void* ws, size_t ws_bytes, void* stream) {
  const bool packed = cu_q != nullptr;
  const int64_t tq = packed ? total_q : nseq * sq;
  const int64_t nbq = dq_blocks(p, packed, nseq, sq, total_q);
  // the row statistics (fp32 per query row and q head) are read through one
  // buffer descriptor whose byte size must stay below 2^31
  if (tq * p->heads_q >= ((int64_t)1 << 29))
    return fail(ATTN_ENOTSUP, "%lld query rows x %d q heads exceed the backward's 2^29 row-statistics limit",
                (long long)tq, p->heads_q);
  const BwdWs w = bwd_ws(p, tq, nbq, packed ? total_k / BWD_BN + nseq : 0, nseq, max_q, grad_dtype);
  attn_status st = check_ws(ws, ws_bytes, w.total);
  if (st != ATTN_OK) return st;
  BwdArgs a{};
  a.s = seq_args(p, cu_q, cu_k, nseq, sq, sk, total_q);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.sinks = p->sinks;
  a.dsinks = dsinks;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.grad_f32 = grad_dtype == ATTN_FP32;
  char* wp = (char*)ws;
  a.delta = (float*)wp;
  wp += w.delta;
  a.lse2 = (float*)wp;
  wp += w.lse2;
  a.dscale_part = (float*)wp;
  wp += w.dscale_part;
  a.dsink_part = w.dsink_part ? (float*)wp : nullptr;
  wp += w.dsink_part;
  int32_t* const order_q = w.order_q ? (int32_t*)wp : nullptr;
  wp += w.order_q;
  int32_t* const order_k = w.order_k ? (int32_t*)wp : nullptr;
  a.nbq = (int32_t)nbq;
  const float scale = resolve_scale(p);
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.x = score_args(p, scale);
  a.dsink_count = p->sinks ? (p->sinks_shared ? 1 : p->heads_q) * a.x.nsinks : 0;
  const int64_t G = p->heads_q / p->heads_kv;
  if (packed) {
    a.nblk = (int32_t)(total_k / BWD_BN + nseq);
    a.nblk_q = (int32_t)((total_q * G) / BWD_QBM + nseq);
    const int64_t ctas = (int64_t)a.nblk * p->heads_kv, ctas_q = (int64_t)a.nblk_q * p->heads_kv;
    if (ctas >= INT32_MAX || ctas_q >= INT32_MAX) return fail(ATTN_ENOTSUP, "grid too large");
    a.total_ctas = total_k > 0 ? (int32_t)ctas : 0;
    a.total_ctas_q = total_q > 0 ? (int32_t)ctas_q : 0;
    // schedule tables (nblk_q == nbq, so the workspace sized them for these grids)
    OrderArgs og[2];
    int no = 0;
    if (order_q && a.total_ctas_q > 0) {
      og[no++] = OrderArgs{a.s, a.nblk_q, 0, BWD_QBM, order_q};
      a.order_q = order_q;
    }
    if (order_k && a.total_ctas > 0) {
      og[no++] = OrderArgs{a.s, a.nblk, 1, BWD_BN, order_k};
      a.order_k = order_k;
    }
    if (no > 0 && (st = launched(launch_order(og, no, (hipStream_t)stream))) != ATTN_OK) return st;
  } else {
    if ((int64_t)p->heads_kv * nseq >= INT32_MAX) return fail(ATTN_ENOTSUP, "grid too large");
    a.nkb = (int32_t)cdiv(sk, BWD_BN);
    a.nmb = (int32_t)cdiv(sq * G, BWD_QBM);
    const int64_t ctas = GroupGrid{(int)((int64_t)p->heads_kv * nseq), a.nkb}.grid_size();
    const int64_t ctas_q = GroupGrid{(int)((int64_t)p->heads_kv * nseq), a.nmb}.grid_size();
    if (ctas >= INT32_MAX || ctas_q >= INT32_MAX) return fail(ATTN_ENOTSUP, "grid too large");
    a.total_ctas = (int32_t)ctas;
    a.total_ctas_q = (int32_t)ctas_q;
  }
  return launched(launch_bwd(a, tile_dim(p->head_dim), p->dtype == ATTN_FP16, (hipStream_t)stream));
}

attn_status check_grad_dtype(const attn_params* p, int32_t grad_dtype) {
  if (grad_dtype != p->dtype && grad_dtype != ATTN_FP32)
    return fail(ATTN_EINVAL, "grad_dtype must be the input dtype or ATTN_FP32 (got %d)", grad_dtype);
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_last_error(void) { return g_err; }

int32_t attn_version(void) { return 100; }

size_t attn_fwd_workspace_size(const attn_params* p, int64_t batch, int64_t seqlen_q, int64_t seqlen_k) {
  if (check_params(p) != ATTN_OK || batch < 1 || seqlen_q < 1 || seqlen_k < 1) return 0;
  return fwd_ws(p, batch, seqlen_q, seqlen_k, nullptr, nullptr);
}

size_t attn_bwd_workspace_size(const attn_params* p, int64_t batch, int64_t seqlen_q, int64_t seqlen_k,
                               int32_t grad_dtype) {
  (void)seqlen_k;
  if (check_params(p) != ATTN_OK || batch < 1 || seqlen_q < 1) return 0;
  return bwd_ws(p, batch * seqlen_q, dq_blocks(p, false, batch, seqlen_q, 0), 0, batch, seqlen_q, grad_dtype).total;
}

// Bound on a KV-cache call's keys per slot: the slot capacity, or the pages
// of one block-table row.
static int64_t kvcache_max_keys(const int32_t* block_table, int32_t max_blocks_per_seq, int32_t page_block_size,
                         int64_t cache_capacity) {
  return block_table ? (int64_t)max_blocks_per_seq * page_block_size : cache_capacity;
}

size_t attn_fwd_kvcache_workspace_size(const attn_params* p, int64_t batch, int64_t seqlen_q,
                                       const int32_t* block_table, int32_t max_blocks_per_seq,
                                       int32_t page_block_size, int64_t cache_capacity) {
  const int64_t max_k = kvcache_max_keys(block_table, max_blocks_per_seq, page_block_size, cache_capacity);
  if (check_params(p) != ATTN_OK || batch < 1 || seqlen_q < 1 || max_k < 1) return 0;
  return fwd_ws(p, batch, seqlen_q, max_k, nullptr, nullptr);
}

attn_status attn_fwd_kvcache(const attn_params* p, int64_t batch, int64_t seqlen_q, const void* q,
                             const void* k_cache, const void* v_cache, const int32_t* cache_seqlens,
                             const int32_t* block_table, int32_t max_blocks_per_seq, int32_t page_block_size,
                             int64_t cache_capacity, void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  attn_status st = check_params(p);
  if (st != ATTN_OK) return st;
  if (batch < 1 || seqlen_q < 1)
    return fail(ATTN_EINVAL, "batch and seqlen_q must be >= 1 (got %lld, %lld)", (long long)batch,
                (long long)seqlen_q);
  if (!q || !k_cache || !v_cache || !o || !lse || !cache_seqlens)
    return fail(ATTN_EINVAL, "q, k_cache, v_cache, cache_seqlens, o and lse must be non-NULL");
  if (block_table) {
    if (max_blocks_per_seq < 1) return fail(ATTN_EINVAL, "max_blocks_per_seq must be >= 1 (got %d)", max_blocks_per_seq);
    if (page_block_size < FWD_BN || page_block_size % FWD_BN != 0)
      return fail(ATTN_EINVAL, "page_block_size must be a positive multiple of %d (got %d)", FWD_BN, page_block_size);
  } else if (cache_capacity < 1) {
    return fail(ATTN_EINVAL, "cache_capacity must be >= 1 without a block table (got %lld)", (long long)cache_capacity);
  }
  const int64_t max_k = kvcache_max_keys(block_table, max_blocks_per_seq, page_block_size, cache_capacity);
  if ((st = check_extent(seqlen_q, max_k, p)) != ATTN_OK) return st;
  if (batch * seqlen_q * (p->heads_q / p->heads_kv) >= INT32_MAX || batch >= INT32_MAX ||
      batch * max_blocks_per_seq >= INT32_MAX)
    return fail(ATTN_ENOTSUP, "problem too large");
  KvCache kvc;
  kvc.seqused_k = cache_seqlens;
  kvc.block_table = block_table;
  kvc.page_rows = block_table ? page_block_size : 0;
  kvc.pages_per_seq = block_table ? max_blocks_per_seq : 0;
  // without a block table, slot b's keys start at row b * cache_capacity
  return run_fwd(p, nullptr, nullptr, (int32_t)batch, seqlen_q, max_k, batch * seqlen_q, seqlen_q, q, k_cache,
                 v_cache, o, lse, ws, ws_bytes, stream, kvc);
}

// Rotary tables: a rotary_dim that is a positive multiple of 16 no larger
// than the head dim, tables of at least one row.
static attn_status check_rotary(const attn_params* p, const float* cos, const float* sin, int32_t rotary_dim,
                                int32_t interleaved, int64_t seqlen_ro) {
  if (!cos || !sin) return fail(ATTN_EINVAL, "rotary_cos and rotary_sin must be non-NULL");
  if (rotary_dim < 16 || rotary_dim % 16 || rotary_dim > p->head_dim)
    return fail(ATTN_EINVAL, "rotary_dim must be a multiple of 16 in [16, head_dim] (got %d)", rotary_dim);
  if (interleaved != 0 && interleaved != 1) return fail(ATTN_EINVAL, "rotary_interleaved must be 0 or 1");
  if (seqlen_ro < 1 || seqlen_ro >= INT32_MAX) return fail(ATTN_EINVAL, "seqlen_ro must be >= 1");
  return ATTN_OK;
}

attn_status attn_kvcache_append(const attn_params* p, int64_t batch, int64_t seqlen_new, const void* k_new,
                                const void* v_new, void* k_cache, void* v_cache, const int32_t* cache_seqlens,
                                int32_t* seqlens_out, const int32_t* block_table, int32_t max_blocks_per_seq,
                                int32_t page_block_size, int64_t cache_capacity, const float* rotary_cos,
                                const float* rotary_sin, int32_t rotary_dim, int32_t rotary_interleaved,
                                int64_t seqlen_ro, void* stream) {
  attn_status st = check_params(p);
  if (st != ATTN_OK) return st;
  if (batch < 1 || seqlen_new < 1 || batch >= INT32_MAX || seqlen_new >= INT32_MAX)
    return fail(ATTN_EINVAL, "batch and seqlen_new must be >= 1 (got %lld, %lld)", (long long)batch,
                (long long)seqlen_new);
  if (!k_new || !v_new || !k_cache || !v_cache || !cache_seqlens)
    return fail(ATTN_EINVAL, "k_new, v_new, k_cache, v_cache and cache_seqlens must be non-NULL");
  if (block_table) {
    if (max_blocks_per_seq < 1) return fail(ATTN_EINVAL, "max_blocks_per_seq must be >= 1 (got %d)", max_blocks_per_seq);
    if (page_block_size < 1) return fail(ATTN_EINVAL, "page_block_size must be >= 1 (got %d)", page_block_size);
  } else if (cache_capacity < 1) {
    return fail(ATTN_EINVAL, "cache_capacity must be >= 1 without a block table (got %lld)", (long long)cache_capacity);
  }
  RotaryArgs r{};
  if (rotary_dim != 0 || rotary_cos || rotary_sin) {
    if ((st = check_rotary(p, rotary_cos, rotary_sin, rotary_dim, rotary_interleaved, seqlen_ro)) != ATTN_OK)
      return st;
    r = RotaryArgs{rotary_cos, rotary_sin, rotary_dim, rotary_interleaved, (int32_t)seqlen_ro};
  }
  AppendArgs a{};
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.k_cache = (uint16_t*)k_cache;
  a.v_cache = (uint16_t*)v_cache;
  a.seqlens = cache_seqlens;
  a.block_table = block_table;
  a.page_rows = block_table ? page_block_size : 0;
  a.pages_per_seq = block_table ? max_blocks_per_seq : 0;
  a.capacity = cache_capacity;
  a.rows = batch * seqlen_new * p->heads_kv;
  a.batch = (int32_t)batch;
  a.seqlen_new = (int32_t)seqlen_new;
  a.hkv = p->heads_kv;
  a.D = p->head_dim;
  a.rot = r;
  return launched(launch_append(a, seqlens_out, p->dtype == ATTN_FP16, (hipStream_t)stream));
}

attn_status attn_rotary(const attn_params* p, int64_t batch, int64_t seqlen, int32_t heads, const void* x, void* out,
                        const int32_t* positions, int32_t per_token, const float* rotary_cos, const float* rotary_sin,
                        int32_t rotary_dim, int32_t rotary_interleaved, int64_t seqlen_ro, void* stream) {
  attn_status st = check_params(p);
  if (st != ATTN_OK) return st;
  if (batch < 1 || seqlen < 1 || heads < 1 || batch >= INT32_MAX || seqlen >= INT32_MAX)
    return fail(ATTN_EINVAL, "batch, seqlen and heads must be >= 1");
  if (!x || !out || !positions) return fail(ATTN_EINVAL, "x, out and positions must be non-NULL");
  if (per_token != 0 && per_token != 1) return fail(ATTN_EINVAL, "per_token must be 0 or 1");
  if ((st = check_rotary(p, rotary_cos, rotary_sin, rotary_dim, rotary_interleaved, seqlen_ro)) != ATTN_OK)
    return st;
  const RotaryArgs r{rotary_cos, rotary_sin, rotary_dim, rotary_interleaved, (int32_t)seqlen_ro};
  return launched(launch_rotary(x, out, batch * seqlen * heads, (int)seqlen, heads, p->head_dim, positions, per_token,
                                r, p->dtype == ATTN_FP16, (hipStream_t)stream));
}

size_t attn_fwd_varlen_workspace_size(const attn_params* p, int32_t num_seqs, int64_t total_q, int64_t total_k,
                                      int32_t max_seqlen_q, int32_t max_seqlen_k) {
  (void)p;
  (void)num_seqs;
  (void)total_q;
  (void)total_k;
  (void)max_seqlen_q;
  (void)max_seqlen_k;
  return 0;
}

size_t attn_bwd_varlen_workspace_size(const attn_params* p, int32_t num_seqs, int64_t total_q, int64_t total_k,
                                      int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t grad_dtype) {
  (void)max_seqlen_k;
  if (check_params(p) != ATTN_OK || total_q < 0 || num_seqs < 0) return 0;
  if (total_k < 0) return 0;
  return bwd_ws(p, total_q, dq_blocks(p, true, num_seqs, 0, total_q), total_k / BWD_BN + num_seqs, num_seqs,
                max_seqlen_q, grad_dtype).total;
}

attn_status attn_fwd(const attn_params* p, int64_t batch, int64_t seqlen_q, int64_t seqlen_k, const void* q,
                     const void* k, const void* v, void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  attn_status st = check_params(p);
  if (st != ATTN_OK) return st;
  if (batch < 1 || seqlen_q < 1 || seqlen_k < 1)
    return fail(ATTN_EINVAL, "batch, seqlen_q, seqlen_k must be >= 1 (got %lld, %lld, %lld)", (long long)batch,
                (long long)seqlen_q, (long long)seqlen_k);
  if (!q || !k || !v || !o || !lse) return fail(ATTN_EINVAL, "q, k, v, o and lse must be non-NULL");
  if ((st = check_extent(seqlen_q, seqlen_k, p)) != ATTN_OK) return st;
  if (batch * seqlen_q * (p->heads_q / p->heads_kv) >= INT32_MAX || batch >= INT32_MAX)
    return fail(ATTN_ENOTSUP, "problem too large");
  return run_fwd(p, nullptr, nullptr, (int32_t)batch, seqlen_q, seqlen_k, batch * seqlen_q, seqlen_q, q, k, v, o,
                 lse, ws, ws_bytes, stream);
}

static attn_status check_bwd(const attn_params* p, int64_t batch, int64_t seqlen_q, int64_t seqlen_k, const void* q,
                             const void* k, const void* v, const void* o, const float* lse, const void* dout,
                             void* dq, void* dk, void* dv, float* dsinks, int32_t grad_dtype) {
  attn_status st = check_params(p);
  if (st != ATTN_OK) return st;
  if ((st = check_grad_dtype(p, grad_dtype)) != ATTN_OK) return st;
  if (batch < 1 || seqlen_q < 1 || seqlen_k < 1)
    return fail(ATTN_EINVAL, "batch, seqlen_q, seqlen_k must be >= 1 (got %lld, %lld, %lld)", (long long)batch,
                (long long)seqlen_q, (long long)seqlen_k);
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return fail(ATTN_EINVAL, "q, k, v, o, lse, dout, dq, dk and dv must be non-NULL");
  if (p->sinks && !dsinks) return fail(ATTN_EINVAL, "dsinks must be non-NULL when sinks are given");
  if ((st = check_extent(seqlen_q, seqlen_k, p)) != ATTN_OK) return st;
  if (batch * seqlen_q * (p->heads_q / p->heads_kv) >= INT32_MAX || batch >= INT32_MAX)
    return fail(ATTN_ENOTSUP, "problem too large");
  return ATTN_OK;
}

attn_status attn_bwd_noalloc(const attn_params* p, int64_t batch, int64_t seqlen_q, int64_t seqlen_k,
                             const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, float* dsinks, int32_t grad_dtype,
                             void* stream) {
  attn_status st = check_bwd(p, batch, seqlen_q, seqlen_k, q, k, v, o, lse, dout, dq, dk, dv, dsinks, grad_dtype);
  if (st != ATTN_OK) return st;
  const size_t need =
      bwd_ws(p, batch * seqlen_q, dq_blocks(p, false, batch, seqlen_q, 0), 0, batch, seqlen_q, grad_dtype).total;
  if (need > ATTN_NOALLOC_SCRATCH_BYTES)
    return fail(ATTN_ENOTSUP, "attn_bwd_noalloc: this call needs %zu bytes of workspace, more than the %zu bytes "
                "of fixed scratch (use attn_bwd with a workspace)", need, (size_t)ATTN_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return fail(ATTN_EHIP, "attn_bwd_noalloc: scratch lookup failed: %s", hipGetErrorString(e));
  return run_bwd(p, nullptr, nullptr, (int32_t)batch, seqlen_q, seqlen_k, batch * seqlen_q, batch * seqlen_k,
                 seqlen_q, q, k, v, o, lse, dout, dq, dk, dv, dsinks, grad_dtype, ws, ATTN_NOALLOC_SCRATCH_BYTES,
                 stream);
}

attn_status attn_bwd(const attn_params* p, int64_t batch, int64_t seqlen_q, int64_t seqlen_k, const void* q,
                     const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
                     void* dk, void* dv, float* dsinks, int32_t grad_dtype, void* ws, size_t ws_bytes,
                     void* stream) {
  const attn_status st =
      check_bwd(p, batch, seqlen_q, seqlen_k, q, k, v, o, lse, dout, dq, dk, dv, dsinks, grad_dtype);
  if (st != ATTN_OK) return st;
  return run_bwd(p, nullptr, nullptr, (int32_t)batch, seqlen_q, seqlen_k, batch * seqlen_q, batch * seqlen_k,
                 seqlen_q, q, k, v, o, lse, dout, dq, dk, dv, dsinks, grad_dtype, ws, ws_bytes, stream);
}

static attn_status check_varlen(const attn_params* p, int32_t num_seqs, int64_t total_q, int64_t total_k,
                                const int32_t* cu_q, const int32_t* cu_k, int32_t max_q, int32_t max_k) {
  attn_status st = check_params(p);
  if (st != ATTN_OK) return st;
  if (num_seqs < 1) return fail(ATTN_EINVAL, "num_seqs must be >= 1 (got %d)", num_seqs);
  if (total_q < 0 || total_k < 0) return fail(ATTN_EINVAL, "total_q and total_k must be >= 0");
  if (!cu_q || !cu_k) return fail(ATTN_EINVAL, "cu_seqlens_q and cu_seqlens_k must be non-NULL");
  if (max_q < 0 || max_k < 0) return fail(ATTN_EINVAL, "max_seqlen_q and max_seqlen_k must be >= 0");
  if ((st = check_extent(max_q, max_k, p)) != ATTN_OK) return st;
  const int64_t G = p->heads_q / p->heads_kv;
  if ((total_q * G) / 128 + num_seqs >= INT32_MAX / p->heads_kv || total_q >= INT32_MAX ||
      total_k >= INT32_MAX)
    return fail(ATTN_ENOTSUP, "problem too large");
  return ATTN_OK;
}

attn_status attn_fwd_varlen(const attn_params* p, int32_t num_seqs, int64_t total_q, int64_t total_k,
                            const int32_t* cu_q, const int32_t* cu_k, int32_t max_q, int32_t max_k, const void* q,
                            const void* k, const void* v, void* o, float* lse, void* ws, size_t ws_bytes,
                            void* stream) {
  attn_status st = check_varlen(p, num_seqs, total_q, total_k, cu_q, cu_k, max_q, max_k);
  if (st != ATTN_OK) return st;
  if ((total_q > 0 && (!q || !o || !lse)) || (total_k > 0 && (!k || !v)))
    return fail(ATTN_EINVAL, "q, k, v, o and lse must be non-NULL");
  (void)ws;
  (void)ws_bytes;
  if (total_q == 0) return ATTN_OK;
  return run_fwd(p, cu_q, cu_k, num_seqs, 0, 0, total_q, max_q, q, k, v, o, lse, nullptr, 0, stream);
}

attn_status attn_bwd_varlen(const attn_params* p, int32_t num_seqs, int64_t total_q, int64_t total_k,
                            const int32_t* cu_q, const int32_t* cu_k, int32_t max_q, int32_t max_k, const void* q,
                            const void* k, const void* v, const void* o, const float* lse, const void* dout,
                            void* dq, void* dk, void* dv, float* dsinks, int32_t grad_dtype, void* ws,
                            size_t ws_bytes, void* stream) {
  attn_status st = check_varlen(p, num_seqs, total_q, total_k, cu_q, cu_k, max_q, max_k);
  if (st != ATTN_OK) return st;
  if ((st = check_grad_dtype(p, grad_dtype)) != ATTN_OK) return st;
  if ((total_q > 0 && (!q || !o || !lse || !dout || !dq)) || (total_k > 0 && (!k || !v || !dk || !dv)))
    return fail(ATTN_EINVAL, "q, k, v, o, lse, dout, dq, dk and dv must be non-NULL");
  if (p->sinks && !dsinks) return fail(ATTN_EINVAL, "dsinks must be non-NULL when sinks are given");
  return run_bwd(p, cu_q, cu_k, num_seqs, 0, 0, total_q, total_k, max_q, q, k, v, o, lse, dout, dq, dk, dv, dsinks,
                 grad_dtype, ws, ws_bytes, stream);
}

}  // extern "C"
