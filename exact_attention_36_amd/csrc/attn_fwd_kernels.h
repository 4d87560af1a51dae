// attn_fwd_kernels.h -- fused exact-attention forward for gfx950 (kernel templates).
//
// One pass over the visible K/V tiles with an online softmax: the running
// row max m and row sum l are rescaled by exp(m_old - m_new) as each tile is
// merged, so the output and the per-row log-sum-exp are written once
// (GitHub search page, gitctrlx/flash-attention-tutorial README, sections 3
// "Online Softmax", 4 and 5 "Flash Attention (With Tiling)").  Keys outside
// the causal / sliding-window band are skipped a whole tile at a time
// (fa4-jax page, the two-sided sliding window item).  Attention sinks add
// one value-less logit per q head to each row's denominator, which scales
// the output by sigmoid(lse - sink) (dew-flash-attn page, sinks paragraph;
// several sinks of a head act as their log-sum-exp).  The score variants --
// soft cap and ALiBi bias -- are applied to each tile's scores before the
// mask, in instances compiled for them (EXT).
//
// Work tile: 128 packed query rows (the G q heads of one kv head, query
// major) x one kv head x one sequence, 4 waves of 32 rows, two workgroups per
// CU.  Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16 so that a lane
// owns a query row: the row max needs one cross-half exchange and the row sum
// none until the end, and the output O^T = V^T P^T keeps the same lane
// ownership, so the rescale is lane-local.  P never leaves registers.  K/V
// tiles of 64 keys are streamed global -> LDS directly (buffer_load ... lds)
// in an XOR-swizzled layout that the 16-byte K reads and the transposing V
// reads (ds_read_b64_tr_b16) both hit without bank conflicts; K runs one tile
// ahead of V so that S of tile t+1 is computed on the MFMA pipe while the
// softmax of tile t runs on the VALU.  Each wave computes only the tiles its
// 32 rows can see (on the others it just takes part in the loads and
// barriers).  O leaves through LDS so that the stores write whole rows.
//
// Split-KV (decode shapes): the visible tiles of a work tile are divided
// among n_split workgroups, each writing a normalised fp32 partial output
// and its log-sum-exp; a combine kernel merges them with weights
// exp(lse_s - lse) (vllm-project/flash-attention README on the GitHub search
// page, "2.2: Optimize for inference").
#pragma once
#include <type_traits>

#include "attn_common.h"

namespace attn {

// PATH (FwdPath): FWD_SPLIT is the split-KV instance (a.n_split > 1), whose
// epilogue writes fp32 partials for the combine kernel.  In it and in
// FWD_STREAM each K/V tile is read by one workgroup only, so the tiles stream
// with the non-temporal hint; FWD_SHARED keeps the default cache policy for
// tiles that several workgroups of a head read.
template <int D, bool F16, bool PAD, int EXT, int PATH>
__global__ __launch_bounds__(THREADS)
__attribute__((amdgpu_waves_per_eu(waves_per_simd_fwd_dkdv(D, EXT), waves_per_simd_fwd_dkdv(D, EXT))))
void fwd_kernel(const FwdArgs a) {
  constexpr bool SPLIT = PATH == FWD_SPLIT;
  constexpr bool KV_NT = PATH != FWD_SHARED;
  // Two workgroups per CU, each with two K and two V buffers (64 KB of LDS
  // for D = 128).  The waits and loads below are written for NST buffers.
  constexpr int NW = THREADS / 64;         // waves per workgroup
  constexpr int NST = 2;                   // K buffers = V buffers
  constexpr int BM = 32 * NW;              // packed query rows per workgroup
  static_assert(BM == FWD_BM, "work tile");
  constexpr int KS = D / 16;               // MFMA k-steps over the head dim
  constexpr int DB = D / 32;               // 32-wide blocks of the head dim
  constexpr int ROWB = D * 2;              // bytes per K/V row
  constexpr int TILE = FWD_BN * ROWB;      // bytes per K (or V) tile
  constexpr int SLABS = TILE / 1024 / NW;  // 1 KB wave-loads per tile per wave
  constexpr int KB = FWD_BN / 32;          // 32-key blocks per tile
  constexpr int PT = FWD_BN / 16;          // 16-key MFMA steps per tile
  static_assert(SLABS >= 1 && (NST & (NST - 1)) == 0, "tile split");
  __shared__ __attribute__((aligned(1024))) char smem[2 * NST * TILE];  // K slots, then V slots

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int G = a.s.group;
  // ---- which work tile
  int seq, g, mb, sp = 0;
  if (a.s.cu_q) {
    const int id = xcd_remap(blockIdx.x, a.total_ctas);
    g = id / a.nblk;
    const int t = id - g * a.nblk;
    seq = find_sequence(a.s.cu_q, a.s.nseq, t, G, BM);
    mb = t - packed_block_start(a.s.cu_q, seq, G, BM);
  } else {
    // groups are (sequence, kv head, split); rank 0 is the last m-block, the
    // longest one under a causal mask
    int grp, rank;
    if (!GroupGrid{a.s.nseq * a.s.hkv * a.n_split, a.nmb, unmasked(a.s)}.decode(blockIdx.x, grp, rank)) return;
    sp = grp % a.n_split;
    const int r = grp / a.n_split;
    g = r % a.s.hkv;
    seq = r / a.s.hkv;
    mb = a.nmb - 1 - rank;
  }
  const SeqInfo si = seq_info(a.s, seq);
  const int prows = si.lq * G;
  const int p0 = mb * BM;
  if (p0 >= prows) return;  // idle slot of the packed grid (whole workgroup)

  const Band band(a.s, si);
  const int i_lo = div_group(p0, a.s), i_hi = div_group(min(p0 + BM, prows) - 1, a.s);
  const int kv_lo = band.kmin(i_lo), kv_hi = band.kmax(i_hi);
  int t_begin = 0, t_end = 0;
  if (kv_hi >= kv_lo) {
    t_begin = kv_lo / FWD_BN;
    t_end = kv_hi / FWD_BN + 1;
  }
  if constexpr (SPLIT) {
    const int per = (t_end - t_begin + a.n_split - 1) / a.n_split;
    const int b0 = t_begin + sp * per;
    t_end = min(t_end, b0 + per);
    t_begin = min(b0, t_end);
  }
  // Tiles inside [full_lo, full_hi] are visible to every row of the work tile.
  const int full_lo = band.kmin(i_hi), full_hi = band.kmax(i_lo);
  // Tiles this wave's 32 rows can see at all: [w_begin, w_end).  Outside it
  // the wave only takes part in the loads and barriers of the workgroup.
  int w_begin = t_end, w_end = t_end;
  {
    const int wp0 = p0 + 32 * wave, wp1 = min(wp0 + 32, prows) - 1;
    if (wp0 < prows) {
      const int klo = band.kmin(div_group(wp0, a.s)), khi = band.kmax(div_group(wp1, a.s));
      if (khi >= klo) {
        w_begin = min(t_end, max(t_begin, klo / FWD_BN));
        w_end = max(w_begin, min(t_end, khi / FWD_BN + 1));
      }
    }
  }

  // In memory a head holds dg <= D values (PAD: a run-time dg < D); the tile
  // columns past dg are zero (their loads read zero, their stores are dropped).
  const int dg = PAD ? a.s.dg : D;
  const int64_t qrow = (int64_t)a.s.hq * dg;   // elements per q/o token
  const int64_t krow = (int64_t)a.s.hkv * dg;  // elements per k/v token
  const int64_t qbase_e = ((int64_t)si.q0 * a.s.hq + (int64_t)g * G) * dg;
  const uint32_t qbytes = si.lq > 0 ? (uint32_t)(((int64_t)(si.lq - 1) * qrow + (int64_t)G * dg) * 2) : 0u;
  const int64_t kbase_e = ((int64_t)si.k0 * a.s.hkv + g) * dg;
  const uint32_t kbytes = si.lk > 0 ? (uint32_t)(((int64_t)(si.lk - 1) * krow + dg) * 2) : 0u;
  const auto rq = make_rsrc((const uint16_t*)a.q + qbase_e, qbytes);

  // ---- this lane's query row: p0 + 32 wave + l32
  const int my_p = p0 + 32 * wave + l32;
  const int my_i = div_group(my_p, a.s);
  const int my_hl = my_p - my_i * G;
  const uint32_t qoff = (uint32_t)(((int64_t)my_i * qrow + (int64_t)my_hl * dg) * 2);
  u32x4 qf[KS];  // Q^T as the B operand: 8 consecutive dims of the row per k-step
#pragma unroll
  for (int s = 0; s < KS; s++) qf[s] = buf_load16(rq, chunk_off(qoff, 2 * s + hh, dg));
  // Visibility of key j0 + o for this lane's row, o = the key's offset in the
  // tile minus 4 hh:  0 <= o - lo_base + j0 <= span  (unsigned compare).
  // score variants: this row's ALiBi slope / scale and its diagonal, less 4 hh
  // (key j of tile t is t*BN + o + 4 hh for the element at tile offset o)
  const float ext_kb = (EXT & EXT_ALIBI) ? alibi_kb(a.x, seq, g * G + my_hl) : 0.f;
  const float ext_diag = (float)(my_i + si.lk - si.lq - 4 * hh);
  int lo_base = band.kmin(my_i) - 4 * hh, span = band.kmax(my_i) - band.kmin(my_i);
  if (span < 0) {  // no visible key: nothing passes
    lo_base = -1 - 4 * hh;
    span = 0;
  }

  // ---- loop-invariant addressing
  // K/V tile t is read through descriptors rebased to its first row, so the
  // per-lane DMA offsets below do not change from tile to tile.
  uint32_t dma_off[SLABS];
#pragma unroll
  for (int n = 0; n < SLABS; n++) {
    const int byte = (wave * SLABS + n) * 1024 + lane * 16;
    const int r = byte / ROWB, pos = (byte % ROWB) >> 4;
    dma_off[n] = chunk_off((uint32_t)(r * krow * 2), pos ^ swz<D>(r), dg);
  }
  // K as the A operand: lane reads row (32 kb + l32), chunk (2 s + hh); the
  // swizzle of row 32 kb + l32 equals that of l32, so kb is a constant offset.
  int k_off[KS];
#pragma unroll
  for (int s = 0; s < KS; s++) k_off[s] = tile_off<D>(l32, 2 * s + hh);
  // V^T as the A operand through transposing reads: rows 16 t2 + 4 hh + esrc
  // (+8 for the second half of the k-step), 4 columns starting at col.
  const int gq = lane >> 4, li = lane & 15, esrc = li >> 2, jsrc = li & 3;
  int v_off[DB][2];
#pragma unroll
  for (int d = 0; d < DB; d++) {
    const int col = d * 32 + 16 * (gq & 1) + 4 * jsrc;
#pragma unroll
    for (int w = 0; w < 2; w++) v_off[d][w] = tile_off<D>(4 * hh + esrc + 8 * w, col >> 3) + (jsrc & 1) * 8;
  }

  // Tile t lives in K slot and V slot (t - t_begin) mod NST.
  // (byte offsets inside one sequence's K/V fit in 31 bits)
  const uint32_t tile_stride = (uint32_t)(FWD_BN * krow * 2);
  // Paged KV cache: the block-table entries of 64 consecutive pages of this
  // slot, one per lane, [tbl_base, tbl_base + 64); a tile's page is then a
  // readlane, and the window moves (one global load) only every 64 pages.
  // Requested pages never fall more than one below the latest request.
  int tbl_base = -(1 << 30), tbl = 0;
  auto page_phys = [&](int page) __attribute__((always_inline)) {
    if (page >= tbl_base + 64) {
      tbl_base = max(page - 1, 0);
      const int idx = tbl_base + lane;
      tbl = idx < a.s.pages_per_seq ? a.s.block_table[(int64_t)seq * a.s.pages_per_seq + idx] : 0;
      wait_vmcnt<0>();  // the entries land before use (and no table load stays in the DMA counts)
    }
    return (int64_t)__builtin_amdgcn_readlane(tbl, page - tbl_base);
  };
  auto load_rows = [&](const void* src, int t, char* dst) __attribute__((always_inline)) {
    i32x4 r;
    if (a.s.block_table) {
      // paged KV cache: the tile's page, and the bytes up to its last valid key
      // (a tile never crosses a page: page_rows is a multiple of the tile)
      const int key0 = t * FWD_BN, page = key0 / a.s.page_rows;
      const int64_t phys = page_phys(page);
      const int64_t row0 = phys * a.s.page_rows + (key0 - page * a.s.page_rows);
      r = make_rsrc_words((const uint16_t*)src + (row0 * a.s.hkv + g) * dg,
                          (uint32_t)(((int64_t)(min(FWD_BN, si.lk - key0) - 1) * krow + dg) * 2));
    } else {
      const uint32_t skip = (uint32_t)t * tile_stride;  // bytes before tile t
      r = make_rsrc_words((const char*)((const uint16_t*)src + kbase_e) + skip, kbytes - skip);
    }
#pragma unroll
    for (int n = 0; n < SLABS; n++) dma_lds16<KV_NT>(r, dst + (wave * SLABS + n) * 1024, dma_off[n]);
  };
  auto kslot = [&](int t) { return smem + ((t - t_begin) & (NST - 1)) * TILE; };
  auto vslot = [&](int t) { return smem + (NST + ((t - t_begin) & (NST - 1))) * TILE; };

  f32x16 acc[DB];
#pragma unroll
  for (int d = 0; d < DB; d++) acc[d] = f32x16{};
  // m_run: the reference max (raw score units) the accumulators are scaled to.
  // It is raised only when a tile's max exceeds it by more than 8 in log2
  // units, so p = 2^(s*c - m_run*c) stays below 2^8 and most tiles skip the
  // rescale of the accumulators; O = acc / l is the same for any reference.
  float m_run = -INFINITY, l_part = 0.f;
  const float c = a.scale_log2;
  constexpr float RESCALE_LOG2 = 8.f;

  // S^T = K Q^T for one tile (raw scores; the scale is folded into the exponent)
  auto s_tile = [&](const char* kt, f32x16 (&st)[KB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < KB; kb++)
#pragma unroll
      for (int s = 0; s < KS; s++)
        st[kb] = mfma32<F16>(lds_read16(kt + kb * 32 * ROWB + k_off[s]), qf[s], s == 0 ? f32x16{} : st[kb]);
  };

  // Loads issued at the top of step t (after its barrier): K(t+NST) into the
  // slot of K(t), which step t-1 used, and V(t+NST-1) into the slot of V(t-1).
  auto refill = [&](int t) __attribute__((always_inline)) {
    if (t + NST < t_end) load_rows(a.k, t + NST, kslot(t + NST));
    if (t + NST - 1 < t_end) load_rows(a.v, t + NST - 1, vslot(t + NST - 1));
  };
  // A step of a tile this wave does not compute: its share of the loads and
  // the barrier, and with NEXT the scores of tile t+1.
  auto idle_step = [&](int t, f32x16 (&sn)[KB], auto NEXT) __attribute__((always_inline)) {
    if (t + NST - 1 < t_end) wait_vmcnt<2 * (NST - 2) * SLABS>();
    else wait_vmcnt<0>();
    barrier_reads_done();
    refill(t);
    if constexpr (decltype(NEXT)::value) {
      s_tile(kslot(t + 1), sn);
      sched_reads_ahead<KB * KS, 1, 1, 4>();
    }
  };

  // One step: softmax and PV of tile t (scores in st), overlapped with S of
  // tile t+1 (into sn).  At its top the step needs V(t) and K(t+1); the loads
  // issued after them are those of the NST-2 steps before (2 tiles each).
  auto step = [&](int t, f32x16 (&st)[KB], f32x16 (&sn)[KB], auto MASK, auto LAST) __attribute__((always_inline)) {
    constexpr bool masked = decltype(MASK)::value;
    constexpr bool last = decltype(LAST)::value;
    if (t + NST - 1 < t_end) wait_vmcnt<2 * (NST - 2) * SLABS>();
    else wait_vmcnt<0>();
    barrier_reads_done();  // everyone's part is in; everyone is done with step t-1
    refill(t);
    if constexpr (EXT != 0) {  // variant logits, before the mask sets invisible keys to -inf
      const float base = ext_diag - (float)(t * FWD_BN);
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
          float th;
          st[kb][i] = ext_score<EXT>(st[kb][i], a.x, ext_kb, base - (float)(kb * 32 + 8 * (i >> 2) + (i & 3)), th);
        }
    }
    if constexpr (masked) {
      const int lo = lo_base - t * FWD_BN;
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const int o = kb * 32 + 8 * (i >> 2) + (i & 3);
          if ((unsigned)(o - lo) > (unsigned)span) st[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; kb++)
#pragma unroll
      for (int i = 0; i < 16; i++) mx = fmaxf(mx, st[kb][i]);
    mx = half_max(mx);
    const bool raise = mx * c > m_run * c + RESCALE_LOG2;  // false while both are -inf
    if (__builtin_amdgcn_ballot_w64(raise)) {
      // lanes that do not raise keep their reference (alpha = 1; their m_run
      // may still be -inf); a first finite max gives alpha = 2^-inf = 0
      const float alpha = raise ? exp2_fast((m_run - mx) * c) : 1.f;
      m_run = raise ? mx : m_run;
      l_part *= alpha;
#pragma unroll
      for (int d = 0; d < DB; d++) acc[d] *= alpha;
    }
    if constexpr (!last) s_tile(kslot(t + 1), sn);
    u32x4 pf[PT];
    {
      const float mc = m_run == -INFINITY ? 0.f : m_run * c;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const float p = exp2_fast(fmaf(st[kb][i], c, -mc));
          st[kb][i] = p;
          rs += p;
        }
      l_part += rs;
      // P^T as the B operand: k-step t2 = 2 kb + u covers keys
      // 32 kb + 16 u + {4hh..4hh+3, 8+4hh..8+4hh+3}: accumulator registers
      // 8u..8u+7 of this lane.
#pragma unroll
      for (int t2 = 0; t2 < PT; t2++) {
        const int kb = t2 >> 1, u = t2 & 1;
        pf[t2] = u32x4{pack2<F16>(st[kb][8 * u + 0], st[kb][8 * u + 1]), pack2<F16>(st[kb][8 * u + 2], st[kb][8 * u + 3]),
                       pack2<F16>(st[kb][8 * u + 4], st[kb][8 * u + 5]), pack2<F16>(st[kb][8 * u + 6], st[kb][8 * u + 7])};
      }
    }
    // O^T += V^T P^T, V^T read with the same key order as P.
    const char* vt = vslot(t);
#pragma unroll
    for (int d = 0; d < DB; d++)
#pragma unroll
      for (int t2 = 0; t2 < PT; t2++) {
        const u32x2 a1 = lds_read_tr(vt + t2 * 16 * ROWB + v_off[d][0]);
        const u32x2 a2 = lds_read_tr(vt + t2 * 16 * ROWB + v_off[d][1]);
        acc[d] = mfma32<F16>(u32x4{a1[0], a1[1], a2[0], a2[1]}, pf[t2], acc[d]);
      }
    // S of the next tile: 1 K read per MFMA, 4 MFMAs ahead; PV: 2 transposing
    // reads per MFMA, 4 MFMAs ahead
    if constexpr (!last) sched_reads_ahead<KB * KS, 1, 1, 4>();
    sched_reads_ahead<DB * PT, 1, 2, 4>();
  };

  // Masked head, unmasked interior and masked tail loops; each runs two steps
  // per iteration so that the current and next score tiles swap registers
  // instead of being copied.  The last tile is peeled off (no next tile).
  int ti0 = t_begin, ti1 = t_begin;  // interior tiles [ti0, ti1)
  if (full_hi >= full_lo) {
    ti0 = max(t_begin, (full_lo + FWD_BN - 1) / FWD_BN);
    ti1 = min(t_end, (full_hi + 1) / FWD_BN);
    if (ti1 <= ti0) ti0 = ti1 = t_begin;
  }
  if (t_begin < t_end) {
    // prologue: K(b), V(b), K(b+1), V(b+1), ..., K(b+NST-1), then S(b)
#pragma unroll
    for (int j = 0; j < NST; j++) {
      if (t_begin + j < t_end) load_rows(a.k, t_begin + j, kslot(t_begin + j));
      if (j < NST - 1 && t_begin + j < t_end) load_rows(a.v, t_begin + j, vslot(t_begin + j));
    }
    if (t_begin + NST - 1 < t_end) wait_vmcnt<(2 * NST - 2) * SLABS>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    f32x16 sa[KB], sb[KB];
    // steps before this wave's first tile; the last of them computes S of it
    int t = t_begin;
    for (; t + 1 < w_begin; t++) idle_step(t, sa, std::false_type{});
    if (w_begin < w_end) {
      if (w_begin == t_begin) s_tile(kslot(t_begin), sa);
      else idle_step(t++, sa, std::true_type{});
      const int tl = w_end - 1;
      auto run = [&](int t0, int t1, auto MASK) __attribute__((always_inline)) {
        int u = t0;
        for (; u + 1 < t1; u += 2) {
          step(u, sa, sb, MASK, std::false_type{});
          step(u + 1, sb, sa, MASK, std::false_type{});
        }
        if (u < t1) {
          step(u, sa, sb, MASK, std::false_type{});
#pragma unroll
          for (int kb = 0; kb < KB; kb++) sa[kb] = sb[kb];
        }
      };
      run(w_begin, min(ti0, tl), std::true_type{});
      run(max(ti0, w_begin), min(ti1, tl), std::false_type{});
      run(max(ti1, w_begin), tl, std::true_type{});
      step(tl, sa, sb, std::true_type{}, std::true_type{});
      t = w_end;
    }
    // steps after this wave's last tile
    for (; t < t_end; t++) idle_step(t, sa, std::false_type{});
  }

  // ---- epilogue
  const float l_tot = half_sum(l_part);
  const float lse_v = l_tot > 0.f ? (m_run * c + log2_fast(l_tot)) * LN2 : -INFINITY;
  if constexpr (SPLIT) {
    const int64_t pidx = ((int64_t)(sp * a.s.nseq + seq) * a.s.hkv + g) * ((int64_t)a.nmb * BM) + my_p;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* op = a.o_part + pidx * D;
#pragma unroll
    for (int d = 0; d < DB; d++)
#pragma unroll
      for (int j4 = 0; j4 < 4; j4++) {
        const int dd = d * 32 + 8 * j4 + 4 * hh;
        *(f32x4*)(op + dd) = f32x4{acc[d][4 * j4] * inv, acc[d][4 * j4 + 1] * inv, acc[d][4 * j4 + 2] * inv,
                                   acc[d][4 * j4 + 3] * inv};
      }
    if (hh == 0) a.lse_part[pidx] = lse_v;
    return;
  }
  const int my_h = g * G + my_hl;
  float denom = l_tot;
  if (a.sinks && l_tot > 0.f) denom += exp2_fast(sink_log2(a.sinks, a.x, my_h) - m_run * c);
  const float inv = l_tot > 0.f ? 1.f / denom : 0.f;
  if (hh == 0 && my_p < prows) {
    const int64_t li_ = a.s.cu_q ? (int64_t)my_h * a.s.total_q + si.q0 + my_i
                                 : ((int64_t)seq * a.s.hq + my_h) * a.s.sq + my_i;
    a.lse[li_] = lse_v;
  }
  // O goes out through LDS so that every store writes whole rows: the wave
  // puts its 32 rows (swizzled like the K/V tiles) in its own 32-row region,
  // then each store instruction writes 1 KB of consecutive 16-byte chunks.
  barrier_reads_done();  // all waves are done reading the K/V slots
  char* const ost = smem + wave * 32 * ROWB;
#pragma unroll
  for (int d = 0; d < DB; d++)
#pragma unroll
    for (int j4 = 0; j4 < 4; j4++)
      *LDS_PTR(u32x2, ost + tile_off<D>(l32, 4 * d + j4) + 8 * hh) =
          u32x2{pack2<F16>(acc[d][4 * j4] * inv, acc[d][4 * j4 + 1] * inv),
                pack2<F16>(acc[d][4 * j4 + 2] * inv, acc[d][4 * j4 + 3] * inv)};
  const auto ro = make_rsrc((uint16_t*)a.o + qbase_e, qbytes);
  constexpr int CPR = ROWB / 16;  // 16-byte chunks per row
#pragma unroll
  for (int it = 0; it < 32 / (64 / CPR); it++) {
    const int r = it * (64 / CPR) + lane / CPR, ch = lane % CPR;
    const u32x4 v = *LDS_PTR(const u32x4, ost + tile_off<D>(r, ch));
    const int p = p0 + 32 * wave + r;
    const int i = div_group(p, a.s), hl = p - i * G;
    // rows past the work tile fall outside the descriptor (dropped)
    const uint32_t off = p < prows ? chunk_off((uint32_t)(((int64_t)i * qrow + (int64_t)hl * dg) * 2), ch, dg) : DROP_ROW;
    buf_store16(v, ro, off);
  }
}

// Merge split-KV partials: lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s,
// then the sink gate sigmoid(lse - sink).  D/4 lanes per packed row, each
// reading 16 bytes (4 dims) of every split's partial; 64/(D/4) rows per wave.
template <int D, bool F16>
__global__ __launch_bounds__(THREADS) void fwd_combine_kernel(const FwdArgs a) {
  constexpr int LPR = D / 4;     // lanes per row
  constexpr int RPW = 64 / LPR;  // rows per wave
  const int lane = threadIdx.x & 63, sub = lane % LPR;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int rows_bg = a.nmb * a.bm;
  const int64_t total = (int64_t)a.s.nseq * a.s.hkv * rows_bg;
  if (row >= total) return;
  const int p = (int)(row % rows_bg);
  const int r = (int)(row / rows_bg);
  const int g = r % a.s.hkv, seq = r / a.s.hkv;
  const int G = a.s.group;
  const SeqInfo si = seq_info(a.s, seq);
  if (p >= si.lq * G) return;
  const int i = div_group(p, a.s), hl = p - i * G, h = g * G + hl;
  const int64_t split_stride = (int64_t)a.s.nseq * a.s.hkv * rows_bg;
  const int ns = a.n_split;
  // The first NST splits' partials (lse and this lane's 4 dims) are loaded
  // together, before any is used, so that they are in flight at once; splits
  // past them, if any, are read in the loops below.  A split with no visible
  // key wrote O_s = 0 and lse_s = -inf, and so adds 0.
  constexpr int NST = 4;
  const float* op = a.o_part + row * D + sub * 4;
  float lv[NST];
  f32x4 ov[NST];
#pragma unroll
  for (int s = 0; s < NST; s++) {
    lv[s] = s < ns ? a.lse_part[row + s * split_stride] : -INFINITY;
    ov[s] = s < ns ? *(const f32x4*)(op + s * split_stride * D) : f32x4{};
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < NST; s++) mx = fmaxf(mx, lv[s]);
  for (int s = NST; s < ns; s++) mx = fmaxf(mx, a.lse_part[row + s * split_stride]);
  float sum = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int s = 0; s < NST; s++) sum += exp2_fast((lv[s] - mx) * LOG2E);
    for (int s = NST; s < ns; s++) sum += exp2_fast((a.lse_part[row + s * split_stride] - mx) * LOG2E);
  }
  const float lse = mx == -INFINITY ? -INFINITY : mx + log2_fast(sum) * LN2;
  f32x4 o{};
  if (mx != -INFINITY) {
#pragma unroll
    for (int s = 0; s < NST; s++) o += exp2_fast((lv[s] - lse) * LOG2E) * ov[s];
    for (int s = NST; s < ns; s++) {
      const float w = exp2_fast((a.lse_part[row + s * split_stride] - lse) * LOG2E);
      o += w * *(const f32x4*)(op + s * split_stride * D);
    }
  }
  float gate = mx == -INFINITY ? 0.f : 1.f;
  if (a.sinks && mx != -INFINITY) gate = 1.f / (1.f + exp2_fast(sink_log2(a.sinks, a.x, h) - lse * LOG2E));
  uint16_t* ob = (uint16_t*)a.o + ((int64_t)(si.q0 + i) * a.s.hq + h) * a.s.dg + sub * 4;
  if (sub * 4 < a.s.dg)  // the head's dg values (tile columns past them are zero)
    *(u32x2*)ob = u32x2{pack2<F16>(o[0] * gate, o[1] * gate), pack2<F16>(o[2] * gate, o[3] * gate)};
  if (sub == 0) a.lse[((int64_t)seq * a.s.hq + h) * a.s.sq + i] = lse;
}

// The forward kernel of score variant EXT for every tile width and dtype.
// Each variant is instantiated in a translation unit of its own (explicit
// instantiation there, `extern template` in the dispatcher), so that the
// variants compile in parallel.
template <int EXT, int D, bool F16>
hipError_t launch_fwd_dt(const FwdArgs& a, hipStream_t st) {
  const bool pad = a.s.dg != D;
  const dim3 grid(a.total_ctas), block(THREADS);
  if (a.n_split > 1) {
    if (pad) hipLaunchKernelGGL((fwd_kernel<D, F16, true, EXT, FWD_SPLIT>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd_kernel<D, F16, false, EXT, FWD_SPLIT>), grid, block, 0, st, a);
  } else if (a.kv_once) {
    if (pad) hipLaunchKernelGGL((fwd_kernel<D, F16, true, EXT, FWD_STREAM>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd_kernel<D, F16, false, EXT, FWD_STREAM>), grid, block, 0, st, a);
  } else {
    if (pad) hipLaunchKernelGGL((fwd_kernel<D, F16, true, EXT, FWD_SHARED>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd_kernel<D, F16, false, EXT, FWD_SHARED>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <int EXT>
hipError_t launch_fwd_variant(const FwdArgs& a, int tile_d, bool f16, hipStream_t st) {
  if (tile_d == 256) return f16 ? launch_fwd_dt<EXT, 256, true>(a, st) : launch_fwd_dt<EXT, 256, false>(a, st);
  if (tile_d == 128) return f16 ? launch_fwd_dt<EXT, 128, true>(a, st) : launch_fwd_dt<EXT, 128, false>(a, st);
  return f16 ? launch_fwd_dt<EXT, 64, true>(a, st) : launch_fwd_dt<EXT, 64, false>(a, st);
}

}  // namespace attn
