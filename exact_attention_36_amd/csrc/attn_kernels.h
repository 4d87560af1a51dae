// attn_kernels.h -- kernel argument blocks and launchers (host <-> device
// contract inside the library; not part of the public C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Rows of one work tile.  Query rows of the kv group g are packed
// query-major: packed row p is query p / G of q head g*G + p % G, so a tile
// of FWD_BM packed rows reads each K/V byte once for all G heads.
constexpr int FWD_BM = 128;     // packed query rows per forward workgroup
constexpr int FWD_BN = 64;      // keys per K/V tile
constexpr int BWD_BN = 128;     // keys per backward workgroup
constexpr int BWD_BM = 32;      // packed query rows per backward step
constexpr int THREADS = 256;    // 4 wave64s
// Waves per SIMD the kernels of tile width D are built for: two up to 128
// (256 registers per lane each), one at 256, whose Q, O and K fragments need
// up to 512 (the MFMA accumulators then sit in AGPRs) and whose K/V tiles
// take 128 KB of LDS, one workgroup per CU.
constexpr int waves_per_simd(int D) { return D > 128 ? 1 : 2; }
// The forward and the dK/dV kernel at the 64 width without score variants
// (EXT = 0): three (168 registers, 32-33 KB of LDS per workgroup).  Their
// D <= 64 work leaves the softmax-side VALU a larger share than at 128, which
// a third wave overlaps: causal B=4, H=16, S=2048 at D = 64 forward 51 vs
// 54-58 us and dK/dV 85 vs 95-103 us.  The dQ kernel measured 8 % slower
// there and stays at two, as do the variant instances (they would spill).
constexpr int waves_per_simd_fwd_dkdv(int D, int EXT) { return D > 128 ? 1 : (D > 64 || EXT != 0) ? 2 : 3; }

// Sequence geometry shared by all kernels.  Batched problems have
// cu_q == nullptr: sequence b starts at token b*sq (queries) and b*sk (keys).
struct SeqArgs {
  const int32_t* cu_q;   // [nseq+1] or nullptr
  const int32_t* cu_k;   // [nseq+1] or nullptr
  int32_t nseq;
  int32_t sq, sk;        // per-sequence lengths in batched mode
  int32_t total_q;       // tokens of q (lse row stride in packed mode)
  int32_t hq, hkv, group;
  int32_t dg;            // head dim of the tensors in memory, a multiple of 8 no larger than the
                         // kernel's tile D; tile columns past it are zero and never stored
  uint32_t group_magic;  // ceil(2^32 / group) for group >= 2 (fast division, see div_group)
  int32_t causal, wl, wr;  // window bounds, -1 = unbounded
  // Used lengths: slot seq (a batch entry, or a packed sequence whose tokens
  // cu_seqlens allot) uses its first seqused_q[seq] queries and
  // seqused_k[seq] keys (fa4-jax page, varlen semantics paragraph; the KV
  // cache's cache_seqlens).  With a block table (KV-cache forward), key j of
  // slot seq is row j % page_rows of page
  // block_table[seq * pages_per_seq + j / page_rows] ([page][row][hkv][D]).
  const int32_t* seqused_q;    // [nseq] or nullptr
  const int32_t* seqused_k;    // [nseq] or nullptr
  const int32_t* block_table;  // [nseq][pages_per_seq] or nullptr
  int32_t page_rows, pages_per_seq;
};

// Score variants and sinks.  The kernels work on raw scores x = <q, k> and
// P = 2^(x c - m), c = scale log2(e); a variant replaces x by x' such that
// x' c is the variant's logit in log2 units:
//   soft cap: x' = (cap / scale) tanh(x scale / cap), tanh(u) = 1 - 2 / (1 + 2^(2 u log2 e));
//   ALiBi:    x' -= (slope_h / scale) |i + Lk - Lq - j|.
// Variants are compile-time (EXT_CAP, EXT_ALIBI bits); sinks are not.
constexpr int EXT_CAP = 1, EXT_ALIBI = 2;
struct ScoreArgs {
  float cap_k2;           // 2 scale log2(e) / cap
  float cap_k3;           // cap / scale
  const float* alibi;     // slopes [nseq or 1][hq], or nullptr
  int32_t alibi_bstride;  // hq (per sequence) or 0 (one row for all)
  float inv_scale;        // 1 / scale
  int32_t nsinks;         // sinks per q head (>= 1 when sinks are given)
  int32_t sink_hstride;   // nsinks ([hq][nsinks]) or 0 (one row shared by the heads)
  int32_t ext;            // the EXT_* bits this call needs
};

struct FwdArgs {
  SeqArgs s;
  ScoreArgs x;
  const void* q; const void* k; const void* v;
  void* o; float* lse;
  const float* sinks;     // sink logits (layout in x), or nullptr
  float* o_part;          // split-KV partial outputs (fp32) or nullptr
  float* lse_part;        // split-KV partial log-sum-exps
  float scale_log2;       // softmax scale * log2(e)
  int32_t bm;             // packed query rows per workgroup (FWD_BM)
  int32_t nmb;            // m-blocks per (sequence, kv head) in batched mode
  int32_t nblk;           // linear blocks per kv head in packed mode
  int32_t n_split;
  int32_t total_ctas;
  int32_t kv_once;        // every K/V tile is read by one work tile only (see FwdPath)
};

// Forward instances: K/V tiles shared between work tiles (default cache
// policy), K/V read once by a single work tile (streamed with the
// non-temporal hint), or split-KV (read once, fp32 partials + combine).
enum FwdPath : int { FWD_SHARED = 0, FWD_STREAM = 1, FWD_SPLIT = 2 };

struct BwdArgs {
  SeqArgs s;
  ScoreArgs x;
  const void* q; const void* k; const void* v; const void* o; const void* dout;
  const float* lse;       // sink-free log-sum-exp from the forward
  const float* sinks;     // sink logits (layout in x), or nullptr
  float* dsinks;          // gradient, laid out like sinks, or nullptr
  int32_t dsink_count;    // floats in dsinks
  float* dsink_part;      // [hkv][nbq][G]: each dQ workgroup's per-head sums (workspace)
  float* dscale_part;     // [hkv][nbq][2]: each dQ workgroup's max |dO_i|_2 and max |D_i| (workspace)
  int32_t nbq;            // dQ workgroups per kv head (batched: nseq * nmb; packed: nblk_q)
  float* delta;           // fp32, laid out like lse: D_i = <dO_i, O_i>
  float* lse2;            // fp32, laid out like lse: log-sum-exp with the sink, in log2 units
  void* dq; void* dk; void* dv;
  int32_t grad_f32;       // gradients written as fp32 (else the input dtype)
  float scale;            // softmax scale
  float scale_log2;       // scale * log2(e)
  // key-major dK/dV kernel
  int32_t nkb;            // key blocks per (sequence, kv head) in batched mode
  int32_t nblk;           // linear key blocks per kv head in packed mode
  int32_t total_ctas;
  // query-major dQ kernel
  int32_t nmb;            // query blocks per (sequence, kv head) in batched mode
  int32_t nblk_q;         // linear query blocks per kv head in packed mode
  int32_t total_ctas_q;
  // packed mode: dispatch slot -> block id of the dQ and dK/dV grids
  // (schedule tables), or nullptr
  const int32_t* order_q;
  const int32_t* order_k;
};
constexpr int BWD_QBM = 128;    // packed query rows per dQ workgroup

// Dispatch order of a packed grid (attn_sched.hip).  Block t of kv head g is
// logical id g * nblk + t; order[slot] is the id that dispatch slot `slot`
// runs.  The table lists the blocks by their estimated work, largest first
// (the heads of one block next to each other), so that the longest blocks
// of the batch start first wherever their sequences sit in it.
struct OrderArgs {
  SeqArgs s;
  int32_t nblk;       // linear blocks per kv head
  int32_t key_major;  // blocks of BWD_BN keys (dK/dV grid) instead of bm packed query rows
  int32_t bm;         // packed query rows per block (query-major grids)
  int32_t* order;     // [hkv * nblk]
};
// Grids that get a schedule table: up to ORDER_MAX_BLOCKS blocks per kv head
// and ORDER_MAX_SEQS sequences (the one workgroup that builds it keeps a byte
// per block and four words per sequence in LDS).
constexpr int ORDER_MAX_BLOCKS = 16384;
constexpr int ORDER_MAX_SEQS = 8191;

// Optional per-launch timing (attn_timing_enable): the launchers call these
// around every kernel launch; they record HIP events only while enabled.
enum KernelId { K_FWD = 0, K_FWD_COMBINE, K_BWD_DSINK, K_BWD_DQ, K_BWD_DKDV, K_ORDER, K_COUNT };
void timing_begin(int kid, hipStream_t st);
void timing_end(int kid, hipStream_t st);

// Rotary tables and layout: cos, sin [seqlen_ro][dim / 2] fp32; dim = 0: none.
struct RotaryArgs {
  const float* cos; const float* sin;
  int32_t dim, interleaved, seqlen_ro;
};
// The in-place KV-cache append: new rows [batch][seqlen_new][hkv][D] into a
// cache [batch][capacity][hkv][D], or pages [num_blocks][page_rows][hkv][D]
// through block_table [batch][pages_per_seq], at positions seqlens[b] + i.
struct AppendArgs {
  const uint16_t* k_new; const uint16_t* v_new;
  uint16_t* k_cache; uint16_t* v_cache;
  const int32_t* seqlens;
  const int32_t* block_table;
  int32_t page_rows, pages_per_seq;
  int64_t capacity;
  int64_t rows;  // batch * seqlen_new * hkv
  int32_t batch, seqlen_new, hkv, D;
  RotaryArgs rot;
};

// Launchers (defined in the .hip files).  Return hipGetLastError().
hipError_t launch_fwd(const FwdArgs& a, int tile_d, bool f16, hipStream_t st);
hipError_t launch_fwd_combine(const FwdArgs& a, int tile_d, bool f16, hipStream_t st);
hipError_t launch_bwd(const BwdArgs& a, int tile_d, bool f16, hipStream_t st);
// Builds the schedule tables of n (1 or 2) packed grids, one workgroup each.
hipError_t launch_order(const OrderArgs* grids, int n, hipStream_t st);
hipError_t launch_rotary(const void* x, void* out, int64_t rows, int S, int H, int D, const int32_t* pos0,
                         int per_token, const RotaryArgs& r, bool f16, hipStream_t st);
hipError_t launch_append(const AppendArgs& a, int32_t* seqlens_out, bool f16, hipStream_t st);
// Device address of the fixed scratch behind attn_bwd_noalloc on the current
// device (attn_noalloc.hip).
hipError_t noalloc_scratch(void** out);

}  // namespace attn
