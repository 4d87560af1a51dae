// attn_bwd_kernels.h -- exact-attention backward for gfx950 (kernel templates).
//
// The probabilities are recomputed tile by tile from the saved log-sum-exp
// instead of being stored (GitHub search page, gitctrlx/flash-attention-
// tutorial README, section 6 "Flash Attention Backward Pass"):
//     P   = exp(scale * Q K^T - lse')        lse' = logaddexp(lse, sink)
//     dV  = P^T dO
//     dP  = dO V^T
//     D_i = <dO_i, O_i>
//     dS  = P o (dP - D)
//     dQ  = scale * dS K,    dK = scale * dS^T Q
// (the scale factor on dQ and dK is the chain rule through the scaled
// logits).  With sinks, P already carries the sink's share of the
// denominator (lse' includes the sink), and d(loss)/d(sink_h) is
// -sum_i (1 - g_i) D_i with g_i = sigmoid(lse_i - sink_h)
// (dew-flash-attn page, sinks paragraph: the sinks get their gradient from
// the backward).
//
// Kernels, in stream order:
//   bwd_dq_kernel     query-major: one workgroup per 128 packed query rows
//                     computes the rows' D_i and lse' (log2 units, with
//                     the sink), streams the visible K/V tiles (like the
//                     forward), recomputes S, P, dP, dS and accumulates dQ
//                     in registers; after its loop it forms the block's
//                     per-head dsink sums and its largest |dO_i|_2 and
//                     |D_i| (the dK/dV kernel's dS scale); dQ is written
//                     once, no atomics
//   bwd_dkdv_kernel   key-major: one workgroup per 128-key block of one kv
//                     head streams the visible query blocks of all the
//                     group's q heads, recomputes S, P, dP, dS and
//                     accumulates dK and dV in registers (fp32 across the
//                     GQA group: fa4-jax page, restrictions paragraph)
//   bwd_dsink_kernel  (with sinks) adds the dQ workgroups' dsink sums in a
//                     fixed order
// No output is accumulated with atomics, so every result of the backward is
// the same bit for bit on every run (the deterministic backward of the
// vllm-project/flash-attention README's flash_attn_func docstring, here the
// only backward).
// The two main kernels recompute S and dP each (7 products per visible
// block instead of 5) in exchange for no fp32 atomics, no dS exchange
// through LDS and two waves per SIMD in both.  The packed (varlen) grids
// cover only the real blocks: sequence i's blocks start at
// floor(cu[i] * rows / block) + i and a workgroup finds its sequence by
// binary search (dew-flash-attn page, packed-backward paragraph).
#pragma once
#include <type_traits>

#include "attn_common.h"

namespace attn {

// ------------------------------------------------------------------ dQ
// Work tile as in the forward: 128 packed query rows of one kv group, 4 waves
// of 32 rows; a lane owns one query row (S^T = K Q^T orientation).  Per K/V
// tile of 64 keys:  S^T = K Q^T,  dP^T = V dO^T  (K, V natural 16-byte LDS
// reads), P and dS lane-locally from the row's lse' and D, then
// dQ^T += K^T dS^T with K^T through transposing LDS reads.
template <int D, bool F16, bool PAD, int EXT>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(waves_per_simd(D), waves_per_simd(D))))
void bwd_dq_kernel(const BwdArgs a) {
  constexpr int BM = BWD_QBM;
  constexpr int KS = D / 16, DB = D / 32, ROWB = D * 2;
  constexpr int TILE = FWD_BN * ROWB;
  constexpr int SLABS = TILE / 1024 / 4;
  constexpr int KB = FWD_BN / 32, PT = FWD_BN / 16;
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];  // K0 K1 V0 V1

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int G = a.s.group;
  int seq, g, mb, blk;  // blk: this workgroup's index among its kv head's dQ workgroups
  if (a.s.cu_q) {
    const int id = a.order_q ? a.order_q[blockIdx.x] : xcd_remap(blockIdx.x, a.total_ctas_q);
    g = id / a.nblk_q;
    blk = id - g * a.nblk_q;
    seq = find_sequence(a.s.cu_q, a.s.nseq, blk, G, BM);
    mb = blk - packed_block_start(a.s.cu_q, seq, G, BM);
  } else {
    int grp, rank;
    if (!GroupGrid{a.s.nseq * a.s.hkv, a.nmb, unmasked(a.s)}.decode(blockIdx.x, grp, rank)) return;
    g = grp % a.s.hkv;
    seq = grp / a.s.hkv;
    mb = a.nmb - 1 - rank;  // causal: the longest tiles start first
    blk = seq * a.nmb + mb;
  }
  // this workgroup's per-head sums of the sink gradient (every slot written)
  float* const dsink_out = a.dsink_part ? a.dsink_part + ((int64_t)g * a.nbq + blk) * G : nullptr;
  const SeqInfo si = seq_info(a.s, seq);
  const int prows = si.lq * G;
  const int p0 = mb * BM;
  float* const dscale_out = a.dscale_part + ((int64_t)g * a.nbq + blk) * 2;
  if (p0 >= prows) {  // idle slot of the packed grid (whole workgroup)
    if (dsink_out && (int)threadIdx.x < G) dsink_out[threadIdx.x] = 0.f;
    if (threadIdx.x < 2) dscale_out[threadIdx.x] = 0.f;
    return;
  }

  const Band band(a.s, si);
  const int i_lo = div_group(p0, a.s), i_hi = div_group(min(p0 + BM, prows) - 1, a.s);
  const int kv_lo = band.kmin(i_lo), kv_hi = band.kmax(i_hi);
  int t_begin = 0, t_end = 0;
  if (kv_hi >= kv_lo) {
    t_begin = kv_lo / FWD_BN;
    t_end = kv_hi / FWD_BN + 1;
  }
  const int full_lo = band.kmin(i_hi), full_hi = band.kmax(i_lo);

  const int my_p = p0 + wave * 32 + l32;
  const int my_i = div_group(my_p, a.s);
  const int my_hl = my_p - my_i * G;
  const int my_h = g * G + my_hl;
  // this row's keys [kmin, kmin + span] as one unsigned compare (none for a
  // row that sees no key)
  int my_kmin = band.kmin(my_i);
  uint32_t my_kspan = (uint32_t)(band.kmax(my_i) - my_kmin);
  if (band.kmax(my_i) < my_kmin) {
    my_kmin = 1 << 30;
    my_kspan = 0;
  }

  // In memory a head holds dg <= D values (PAD: a run-time dg < D); the tile
  // columns past dg are zero.
  const int dg = PAD ? a.s.dg : D;
  const int64_t qrow = (int64_t)a.s.hq * dg, krow = (int64_t)a.s.hkv * dg;
  const int64_t qbase_e = ((int64_t)si.q0 * a.s.hq + (int64_t)g * G) * dg;
  const uint32_t qbytes = si.lq > 0 ? (uint32_t)(((int64_t)(si.lq - 1) * qrow + (int64_t)G * dg) * 2) : 0u;
  const uint32_t qoff = (uint32_t)(((int64_t)my_i * qrow + (int64_t)my_hl * dg) * 2);
  const int64_t kbase_e = ((int64_t)si.k0 * a.s.hkv + g) * dg;
  const uint32_t kbytes = si.lk > 0 ? (uint32_t)(((int64_t)(si.lk - 1) * krow + dg) * 2) : 0u;
  const auto rq = make_rsrc((const uint16_t*)a.q + qbase_e, qbytes);
  const auto rdo = make_rsrc((const uint16_t*)a.dout + qbase_e, qbytes);

  // K/V tiles stream through LDS like the forward's (two K and two V slots).
  uint32_t dma_off[SLABS];
#pragma unroll
  for (int n = 0; n < SLABS; n++) {
    const int byte = (wave * SLABS + n) * 1024 + lane * 16;
    const int r = byte / ROWB, pos = (byte % ROWB) >> 4;
    dma_off[n] = chunk_off((uint32_t)(r * krow * 2), pos ^ swz<D>(r), dg);
  }
  // (byte offsets inside one sequence's K/V fit in 31 bits)
  const uint32_t tile_stride = (uint32_t)(FWD_BN * krow * 2);
  auto load_tile = [&](int t) {
    const int buf = (t - t_begin) & 1;
    const uint32_t skip = (uint32_t)t * tile_stride;  // bytes before tile t
    const uint32_t left = kbytes - skip;
    const i32x4 rk = make_rsrc_words((const char*)((const uint16_t*)a.k + kbase_e) + skip, left);
    const i32x4 rv = make_rsrc_words((const char*)((const uint16_t*)a.v + kbase_e) + skip, left);
#pragma unroll
    for (int n = 0; n < SLABS; n++) {
      dma_lds16(rk, smem + buf * TILE + (wave * SLABS + n) * 1024, dma_off[n]);
      dma_lds16(rv, smem + (2 + buf) * TILE + (wave * SLABS + n) * 1024, dma_off[n]);
    }
  };

  // Every load the prologue needs is issued before any of them is waited on
  // (each dependent round trip to HBM costs microseconds at full load): the
  // row's Q, dO and O chunks, its lse and sink logit, and the first K/V tile.
  const auto ro = make_rsrc((const uint16_t*)a.o + qbase_e, qbytes);
  u32x4 qf[KS], df[KS], ov[KS];
#pragma unroll
  for (int s = 0; s < KS; s++) {
    qf[s] = buf_load16(rq, chunk_off(qoff, 2 * s + hh, dg));
    df[s] = buf_load16(rdo, chunk_off(qoff, 2 * s + hh, dg));
    ov[s] = buf_load16(ro, chunk_off(qoff, 2 * s + hh, dg));
  }
  const int64_t row_idx = a.s.cu_q ? (int64_t)my_h * a.s.total_q + si.q0 + my_i
                                   : ((int64_t)seq * a.s.hq + my_h) * a.s.sq + my_i;
  const float lse = my_p < prows ? a.lse[row_idx] : -INFINITY;
  const float sink2 = a.sinks ? sink_log2(a.sinks, a.x, my_h) : 0.f;
  if (t_begin < t_end) load_tile(t_begin);

  // Row statistics, computed here once per (query row, q head) and left in
  // the workspace for the dK/dV kernel that runs after this one:
  //   D = rowsum(dO * O), O being the stored (sink-gated) output;
  //   lse' = log2(2^lse + 2^sink) in log2 units (+inf for an empty row, so
  //   that P = 0 there);  dsink = -sum_rows (1 - gate) D, gate = sigmoid(lse - sink)
  //   (dew-flash-attn page, sinks paragraph).
  float row_d, row_dn;  // D_i and |dO_i|_2
  {
    float part = 0.f, sq = 0.f;
#pragma unroll
    for (int s = 0; s < KS; s++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float d0 = to_f32<F16>((uint16_t)(df[s][e] & 0xFFFF)), d1 = to_f32<F16>((uint16_t)(df[s][e] >> 16));
        part = fmaf(to_f32<F16>((uint16_t)(ov[s][e] & 0xFFFF)), d0, part);
        part = fmaf(to_f32<F16>((uint16_t)(ov[s][e] >> 16)), d1, part);
        sq = fmaf(d0, d0, fmaf(d1, d1, sq));
      }
    row_d = half_sum(part);  // the two lanes holding one row's halves
    row_dn = my_p < prows ? __builtin_sqrtf(half_sum(sq)) : 0.f;
  }
  float row_lse2 = INFINITY, dsink_part = 0.f;
  if (my_p < prows) {
    if (lse != -INFINITY) {
      row_lse2 = lse * LOG2E;
      if (a.sinks) {
        const float mx = fmaxf(row_lse2, sink2), mn = fminf(row_lse2, sink2);
        dsink_part = -row_d / (1.f + exp2_fast(row_lse2 - sink2));
        row_lse2 = mx + log2_fast(1.f + exp2_fast(mn - mx));
      }
    } else {
      dsink_part = -row_d;  // no visible key: the sink takes the whole denominator
    }
    if (hh == 0) {
      a.delta[row_idx] = row_d;
      a.lse2[row_idx] = row_lse2;
    }
  }
  // Per-row inputs of the workgroup's reductions, parked in LDS until after
  // the loop: |dO_i|_2, |D_i| and the row's d(sink) term (rows past the
  // sequence contribute 0).
  __shared__ float red_rows[3][BM];
  if (hh == 0) {
    const bool in = my_p < prows;
    red_rows[0][my_p - p0] = row_dn;
    red_rows[1][my_p - p0] = in ? fabsf(row_d) : 0.f;
    red_rows[2][my_p - p0] = dsink_part;
  }
  const float c = a.scale_log2;
  const float mlse = row_lse2 == INFINITY ? 0.f : row_lse2;  // empty rows are fully masked
  // score variants: this row's ALiBi slope / scale and its diagonal, less 4 hh
  const float ext_kb = (EXT & EXT_ALIBI) ? alibi_kb(a.x, seq, my_h) : 0.f;
  const float ext_diag = (float)(my_i + si.lk - si.lq - 4 * hh);

  int k_off[KS];
#pragma unroll
  for (int s = 0; s < KS; s++) k_off[s] = tile_off<D>(l32, 2 * s + hh);
  const int gq = lane >> 4, li = lane & 15, esrc = li >> 2, jsrc = li & 3;
  int t_off[DB][2];
#pragma unroll
  for (int d = 0; d < DB; d++) {
    const int col = d * 32 + 16 * (gq & 1) + 4 * jsrc;
#pragma unroll
    for (int w = 0; w < 2; w++) t_off[d][w] = tile_off<D>(4 * hh + esrc + 8 * w, col >> 3) + (jsrc & 1) * 8;
  }

  f32x16 acc[DB];
#pragma unroll
  for (int d = 0; d < DB; d++) acc[d] = f32x16{};

  auto tile = [&](int t, auto MASK) {
    constexpr bool masked = decltype(MASK)::value;
    const int buf = (t - t_begin) & 1;
    const char* kt = smem + buf * TILE;
    const char* vt = smem + (2 + buf) * TILE;
    f32x16 st[KB], dp[KB];
#pragma unroll
    for (int kb = 0; kb < KB; kb++)
#pragma unroll
      for (int s = 0; s < KS; s++) {
        st[kb] = mfma32<F16>(lds_read16(kt + kb * 32 * ROWB + k_off[s]), qf[s], s == 0 ? f32x16{} : st[kb]);
        dp[kb] = mfma32<F16>(lds_read16(vt + kb * 32 * ROWB + k_off[s]), df[s], s == 0 ? f32x16{} : dp[kb]);
      }
    if constexpr ((EXT & EXT_CAP) == 0) {
      if constexpr (EXT != 0) {
        // ALiBi alone: the variant logit in place of the raw score, before the
        // mask, which then treats it as a plain score
        const float base = ext_diag - (float)(t * FWD_BN);
#pragma unroll
        for (int kb = 0; kb < KB; kb++)
#pragma unroll
          for (int i = 0; i < 16; i++) {
            float th;
            st[kb][i] = ext_score<EXT>(st[kb][i], a.x, ext_kb, base - (float)(kb * 32 + 8 * (i >> 2) + (i & 3)), th);
          }
      }
      if constexpr (masked) {  // scores of invisible keys -> -inf, so that P = 0 there
        const int lo = my_kmin - t * FWD_BN - 4 * hh;
#pragma unroll
        for (int kb = 0; kb < KB; kb++)
#pragma unroll
          for (int i = 0; i < 16; i++) {
            const int o = kb * 32 + 8 * (i >> 2) + (i & 3);
            if ((uint32_t)(o - lo) > my_kspan) st[kb][i] = -INFINITY;
          }
      }
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const float p = exp2_fast(fmaf(st[kb][i], c, -mlse));
          st[kb][i] = p * (dp[kb][i] - row_d);  // dS
        }
    } else {
      // soft cap (and ALiBi): variant logit, P, and dS with 1 - tanh^2 in one
      // pass (the tanh stays a temporary); invisible keys are zeroed after
      // (their logits may be anything)
      const float base = ext_diag - (float)(t * FWD_BN);
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
          float th = 0.f;
          const float x = ext_score<EXT>(st[kb][i], a.x, ext_kb, base - (float)(kb * 32 + 8 * (i >> 2) + (i & 3)), th);
          float ds = exp2_fast(fmaf(x, c, -mlse)) * (dp[kb][i] - row_d);
          if constexpr ((EXT & EXT_CAP) != 0) ds *= fmaf(-th, th, 1.f);
          st[kb][i] = ds;
        }
      if constexpr (masked) {
        const int lo = my_kmin - t * FWD_BN - 4 * hh;
#pragma unroll
        for (int kb = 0; kb < KB; kb++)
#pragma unroll
          for (int i = 0; i < 16; i++) {
            const int o = kb * 32 + 8 * (i >> 2) + (i & 3);
            if ((uint32_t)(o - lo) > my_kspan) st[kb][i] = 0.f;
          }
      }
    }
    u32x4 sf[PT];
#pragma unroll
    for (int t2 = 0; t2 < PT; t2++) {
      const int kb = t2 >> 1, u = t2 & 1;
      sf[t2] = u32x4{pack2<F16>(st[kb][8 * u + 0], st[kb][8 * u + 1]), pack2<F16>(st[kb][8 * u + 2], st[kb][8 * u + 3]),
                     pack2<F16>(st[kb][8 * u + 4], st[kb][8 * u + 5]), pack2<F16>(st[kb][8 * u + 6], st[kb][8 * u + 7])};
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int d = 0; d < DB; d++)
#pragma unroll
      for (int t2 = 0; t2 < PT; t2++) {
        const u32x2 a1 = lds_read_tr(kt + t2 * 16 * ROWB + t_off[d][0]);
        const u32x2 a2 = lds_read_tr(kt + t2 * 16 * ROWB + t_off[d][1]);
        acc[d] = mfma32<F16>(u32x4{a1[0], a1[1], a2[0], a2[1]}, sf[t2], acc[d]);
      }
    // S/dP: 2 reads feed 2 MFMAs per step, reads 3 steps ahead; dQ: 2
    // transposing reads per MFMA, 4 MFMAs ahead
    sched_reads_ahead<KB * KS, 2, 2, 3>();
    sched_reads_ahead<DB * PT, 1, 2, 4>();
  };
  auto run = [&](int t0, int t1, auto MASK) {
    for (int t = t0; t < t1; t++) {
      wait_vmcnt<0>();
      barrier_reads_done();  // tile t is in; everyone is done with tile t - 1, whose buffers load_tile refills
      if (t + 1 < t_end) load_tile(t + 1);
      tile(t, MASK);
    }
  };
  int ti0 = t_begin, ti1 = t_begin;
  if (full_hi >= full_lo) {
    ti0 = max(t_begin, (full_lo + FWD_BN - 1) / FWD_BN);
    ti1 = min(t_end, (full_hi + 1) / FWD_BN);
    if (ti1 <= ti0) ti0 = ti1 = t_begin;
  }
  run(t_begin, ti0, std::true_type{});
  run(ti0, ti1, std::false_type{});
  run(ti1, t_end, std::true_type{});

  // The workgroup's maxima and sums for the later kernels, formed after the
  // loop so that they do not delay its first tile: the largest |dO_i|_2 and
  // |D_i| of the block (the dK/dV kernel takes their maxima over the blocks of
  // a sequence and kv head for its bound on |dS|), and with sinks the block's
  // rows summed per q head in a fixed order (no atomics).  Row r of the block (packed row
  // p0 + r) belongs to head slot r mod G; slot s is q head (p0 + s) mod G of
  // the group.  The sum of slot s takes chunk c = 0..7 of its rows (rows
  // s + G (c + 8 j)) in one thread each (fewer chunks when G > 32), then
  // adds the chunk sums in order.
  {
    constexpr int NC = 8;
    __shared__ float chunk_sum[NC][BM];
    __syncthreads();
    if (wave == 0) {
      float m0 = fmaxf(red_rows[0][lane], red_rows[0][lane + 64]);
      float m1 = fmaxf(red_rows[1][lane], red_rows[1][lane + 64]);
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        m0 = fmaxf(m0, __shfl_xor(m0, o));
        m1 = fmaxf(m1, __shfl_xor(m1, o));
      }
      if (lane == 0) {
        dscale_out[0] = m0;
        dscale_out[1] = m1;
      }
    }
    if (dsink_out) {
      const int t = threadIdx.x;
      const int nc = G <= THREADS / NC ? NC : THREADS / G;  // G <= 128 q heads per kv head
      if (t < G * nc) {
        const int sl = t % G, ch = t / G;
        float v = 0.f;
        for (int r = sl + G * ch; r < BM; r += G * nc) v += red_rows[2][r];
        chunk_sum[ch][sl] = v;
      }
      __syncthreads();
      if (t < G) {
        float v = 0.f;
        for (int ch = 0; ch < nc; ch++) v += chunk_sum[ch][t];
        dsink_out[(p0 + t) % G] = v;
      }
    }
  }

  // dQ = scale * acc; lane = query row, registers = dims 8(i/4) + 4hh + i%4 of each 32-block
  if (a.grad_f32) {
    const auto rw = make_rsrc((float*)a.dq + qbase_e, qbytes * 2);
#pragma unroll
    for (int d = 0; d < DB; d++)
#pragma unroll
      for (int j4 = 0; j4 < 4; j4++) {
        const int dd = d * 32 + 8 * j4 + 4 * hh;
        const u32x4 w{__builtin_bit_cast(uint32_t, acc[d][4 * j4] * a.scale),
                      __builtin_bit_cast(uint32_t, acc[d][4 * j4 + 1] * a.scale),
                      __builtin_bit_cast(uint32_t, acc[d][4 * j4 + 2] * a.scale),
                      __builtin_bit_cast(uint32_t, acc[d][4 * j4 + 3] * a.scale)};
        buf_store16(w, rw, dd < dg ? qoff * 2 + (uint32_t)(dd * 4) : DROP_ROW);
      }
  } else {
    static_assert(4 * 32 * ROWB <= 4 * TILE, "dQ staging fits in the tile space");
    __syncthreads();  // all waves are done reading the K/V tiles
    const auto rw = make_rsrc((uint16_t*)a.dq + qbase_e, qbytes);
    store_rows16<D, F16>(acc, a.scale, smem + wave * 32 * ROWB, rw, [&](int r) {
      const int p = p0 + wave * 32 + r;
      const int i = div_group(p, a.s), hl = p - i * G;
      return p < prows ? (uint32_t)(((int64_t)i * qrow + (int64_t)hl * dg) * 2) : DROP_ROW;
    }, dg);
  }
}

// ------------------------------------------------------------------ dK, dV
// One workgroup per 128-key block of one kv head; wave w owns keys
// 32w .. 32w+31 and keeps dK^T, dV^T (dims x its keys) in registers.  Per
// block of 32 packed query rows: S = Q K^T and dP = dO V^T (lane = key
// column, registers = query rows), P and dS with the rows' lse' and D from
// LDS, dV^T += dO^T P and dK^T += Q^T dS (dO, Q through transposing LDS
// reads).  dS is kept in fp16 (10 fraction bits) for dK; the Q tiles are
// therefore fp16 and K, used for S, is converted likewise (exact for inputs
// inside fp16's range, |x| <= 65504).  dO and the row statistics reach LDS by
// DMA, double buffered; bf16 Q is loaded into registers one step ahead,
// converted and written to LDS by the waves (fp16 Q goes by DMA as it is).
// WSKIP (windows with a left bound; bf16 up to 128 wide): each wave skips the
// compute of the query blocks that see none of its keys; the plain instance
// has no such branch in its loop (it measured a few per cent slower on
// causal-only problems).
template <int D, bool F16, bool PAD, int EXT, bool WSKIP>
__global__ __launch_bounds__(THREADS)
__attribute__((amdgpu_waves_per_eu(waves_per_simd_fwd_dkdv(D, EXT), waves_per_simd_fwd_dkdv(D, EXT))))
void bwd_dkdv_kernel(const BwdArgs a) {
  constexpr int KS = D / 16, DB = D / 32, ROWB = D * 2;
  constexpr int BN = BWD_BN, BM = BWD_BM;
  constexpr int VBLK = BN * ROWB;           // V block in LDS (B operand of dP)
  constexpr int QTILE = BM * ROWB;          // one Q (or dO) tile
  constexpr bool ALIBI = (EXT & EXT_ALIBI) != 0;
  constexpr int EXT_LDS = ALIBI ? 2 * 256 + 512 : 0;  // per-row ALiBi terms, the group's slopes
  __shared__ __attribute__((aligned(1024))) char smem[VBLK + 4 * QTILE + 2 * 256 + EXT_LDS];
  char* const v_lds = smem;
  char* const q_lds = smem + VBLK;              // [buf] fp16 Q tile
  char* const do_lds = q_lds + 2 * QTILE;       // [buf] dO tile, input dtype
  float* const st_lds = (float*)(do_lds + 2 * QTILE);  // [buf][lse2 32 | delta 32]
  float* const ext_lds = st_lds + 128;          // ALiBi: [buf][diagonal 32 | slope/scale 32]
  float* const slope_lds = ext_lds + 128;       // ALiBi: slope/scale of the group's G q heads

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int gq = lane >> 4, li = lane & 15, esrc = li >> 2, jsrc = li & 3;
  const int G = a.s.group;

  int seq, g, nb;
  if (a.s.cu_q) {
    const int id = a.order_k ? a.order_k[blockIdx.x] : xcd_remap(blockIdx.x, a.total_ctas);
    g = id / a.nblk;
    const int t = id - g * a.nblk;
    seq = find_sequence(a.s.cu_k, a.s.nseq, t, 1, BN);
    nb = t - packed_block_start(a.s.cu_k, seq, 1, BN);
  } else {
    // groups are (sequence, kv head); rank 0 is key block 0, the one most
    // query rows see under a causal mask
    int grp;
    if (!GroupGrid{a.s.nseq * a.s.hkv, a.nkb, unmasked(a.s)}.decode(blockIdx.x, grp, nb)) return;
    g = grp % a.s.hkv;
    seq = grp / a.s.hkv;
  }
  const SeqInfo si = seq_info(a.s, seq);
  const int j0 = nb * BN;
  if (j0 >= si.lk_slot) return;  // idle slot of the packed grid
  // (a block past the used keys but inside the slot visits no query block and
  // writes the zero gradients of its keys)
  const int prows = si.lq * G;
  const Band band(a.s, si);
  const QBand qband(a.s, si);
  const int j_last = min(j0 + BN, si.lk) - 1;
  const int q_lo = qband.qmin(j0), q_hi = qband.qmax(j_last);
  int pb_begin = 0, pb_end = 0;  // packed q-blocks of BM rows
  if (j0 < si.lk && q_hi >= q_lo && prows > 0) {
    pb_begin = (q_lo * G) / BM;
    pb_end = ((q_hi + 1) * G - 1) / BM + 1;
  }

  // In memory a head holds dg <= D values (PAD: a run-time dg < D); the tile
  // columns past dg are zero.
  const int dg = PAD ? a.s.dg : D;
  const int64_t qrow = (int64_t)a.s.hq * dg, krow = (int64_t)a.s.hkv * dg;
  const int64_t qbase_e = ((int64_t)si.q0 * a.s.hq + (int64_t)g * G) * dg;
  const uint32_t qbytes = si.lq > 0 ? (uint32_t)(((int64_t)(si.lq - 1) * qrow + (int64_t)G * dg) * 2) : 0u;
  const int64_t kbase_e = ((int64_t)si.k0 * a.s.hkv + g) * dg;
  const uint32_t kbytes = si.lk > 0 ? (uint32_t)(((int64_t)(si.lk - 1) * krow + dg) * 2) : 0u;
  // dK, dV are stored for every key row of the slot (zero past the used keys)
  const uint32_t kbytes_slot = (uint32_t)(((int64_t)(si.lk_slot - 1) * krow + dg) * 2);
  const i32x4 rq16 = make_rsrc_words((const uint16_t*)a.q + qbase_e, qbytes);  // DMA of fp16 Q
  const auto rq = make_rsrc((const uint16_t*)a.q + qbase_e, qbytes);            // register loads of bf16 Q
  const i32x4 rdo = make_rsrc_words((const uint16_t*)a.dout + qbase_e, qbytes);
  const auto rk = make_rsrc((const uint16_t*)a.k + kbase_e, kbytes);
  const int64_t st_base = a.s.cu_q ? si.q0 : (int64_t)seq * a.s.hq * a.s.sq;
  const int64_t st_hs = a.s.cu_q ? a.s.total_q : a.s.sq;
  const int64_t st_total = a.s.cu_q ? (int64_t)a.s.hq * a.s.total_q : (int64_t)a.s.nseq * a.s.hq * a.s.sq;
  const i32x4 rl = make_rsrc_words(a.lse2, (uint32_t)(st_total * 4));
  const i32x4 rd = make_rsrc_words(a.delta, (uint32_t)(st_total * 4));

  // V block -> LDS (swizzled) once
  {
    const i32x4 rv = make_rsrc_words((const uint16_t*)a.v + kbase_e, kbytes);
    constexpr int SLABS = VBLK / 1024 / 4;
#pragma unroll
    for (int n = 0; n < SLABS; n++) {
      const int slab = wave * SLABS + n;
      const int byte = slab * 1024 + lane * 16;
      const int r = byte / ROWB, pos = (byte % ROWB) >> 4;
      dma_lds16(rv, v_lds + slab * 1024, chunk_off((uint32_t)((int64_t)(j0 + r) * krow * 2), pos ^ swz<D>(r), dg));
    }
  }
  // this wave's 32 keys as the B operand of S (lane: key, 8 dims per k-step), fp16
  const int my_key = j0 + wave * 32 + l32;
  u32x4 kf[KS];
  {
    const uint32_t ko = (uint32_t)((int64_t)my_key * krow * 2);
#pragma unroll
    for (int s = 0; s < KS; s++) {
      const u32x4 k = buf_load16(rk, chunk_off(ko, 2 * s + hh, dg));
      kf[s] = F16 ? k : bf16x8_to_f16x8(k);
    }
  }
  // dS reaches dK through fp16 (11 significant bits, normal from 2^-14, at
  // most 65504).  For every row i that sees this key j,
  //   |dS_ij| = P_ij |<dO_i, v_j> - D_i| <= max_i |dO_i|_2 |v_j|_2 + max_i |D_i|
  // (P <= 1, Cauchy-Schwarz; the maxima over the sequence's rows come from
  // the dQ kernel's workgroups), so dS * 2^ds_e with 2^ds_e bringing that
  // bound to 2^14 stays in fp16's normal range whatever the scale of dO and
  // V; the epilogue divides the factor out of dK.
  int ds_e = 0;
  {
    int b0, b1;  // this sequence's dQ workgroups
    if (a.s.cu_q) {
      b0 = packed_block_start(a.s.cu_q, seq, G, BWD_QBM);
      b1 = packed_block_start(a.s.cu_q, seq + 1, G, BWD_QBM);
    } else {
      b0 = seq * a.nmb;
      b1 = b0 + a.nmb;
    }
    float mdo = 0.f, md = 0.f;
    for (int b = b0 + lane; b < b1; b += 64) {
      const float* sl = a.dscale_part + ((int64_t)g * a.nbq + b) * 2;
      mdo = fmaxf(mdo, sl[0]);
      md = fmaxf(md, sl[1]);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      mdo = fmaxf(mdo, __shfl_xor(mdo, o));
      md = fmaxf(md, __shfl_xor(md, o));
    }
    const auto rv = make_rsrc((const uint16_t*)a.v + kbase_e, kbytes);
    const uint32_t vo = (uint32_t)((int64_t)my_key * krow * 2);
    float sq = 0.f;
#pragma unroll
    for (int s = 0; s < KS; s++) {
      const u32x4 vv = buf_load16(rv, chunk_off(vo, 2 * s + hh, dg));
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float v0 = to_f32<F16>((uint16_t)(vv[e] & 0xFFFF)), v1 = to_f32<F16>((uint16_t)(vv[e] >> 16));
        sq = fmaf(v0, v0, fmaf(v1, v1, sq));
      }
    }
    const float bound = fmaf(mdo, __builtin_sqrtf(half_sum(sq)), md);
    if (bound > 0.f && bound < INFINITY) ds_e = min(max(14 - __builtin_amdgcn_frexp_expf(bound), -100), 100);
  }
  const float ds_sc = __builtin_amdgcn_ldexpf(1.f, ds_e);

  // Q and dO tiles of one block of BM packed rows -> LDS, and the rows' lse'
  // and D; rows past the sequence read as 0 (and are masked).  Each wave
  // moves SL 1 KB slabs of a tile: lane l's 16 bytes of slab n are global
  // chunk pos ^ swz(r) of tile row r, stored at LDS byte slab * 1024 + 16 l.
  constexpr int SL = QTILE / 1024 / 4;  // 1 KB slabs per wave
  auto slab_src = [&](int pb, int n) __attribute__((always_inline)) {
    const int slab = wave * SL + n;
    const int byte = slab * 1024 + lane * 16;
    const int r = byte / ROWB, pos = (byte % ROWB) >> 4;
    const int p = pb * BM + r;
    const int i = div_group(p, a.s), hl = p - i * G;
    return chunk_off((uint32_t)(((int64_t)i * qrow + (int64_t)hl * dg) * 2), pos ^ swz<D>(r), dg);
  };
  auto tile_dma = [&](const i32x4& rs, char* dst, int pb) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < SL; n++) dma_lds16(rs, dst + (wave * SL + n) * 1024, slab_src(pb, n));
  };
  // bf16 Q: this wave's slabs into registers (q_load), then as fp16 into LDS
  // (q_store) once they have landed
  u32x4 q_stage[F16 ? 1 : SL];
  auto q_load = [&](int pb) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < SL; n++) q_stage[n] = buf_load16(rq, slab_src(pb, n));
  };
  auto q_store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < SL; n++)
      *LDS_PTR(u32x4, q_lds + buf * QTILE + (wave * SL + n) * 1024 + lane * 16) = bf16x8_to_f16x8(q_stage[n]);
  };
  auto do_fetch = [&](int pb, int buf) __attribute__((always_inline)) {
    if constexpr (F16) tile_dma(rq16, q_lds + buf * QTILE, pb);
    else q_load(pb);
    tile_dma(rdo, do_lds + buf * QTILE, pb);
    if constexpr (ALIBI) {
      // each row's diagonal i + Lk - Lq and slope/scale, for the variant logits
      if (wave == 1) {
        const int p = pb * BM + l32;
        const int i = div_group(p, a.s), hl = p - i * G;
        ext_lds[buf * 64 + 32 * hh + l32] = hh == 0 ? (float)(i + si.lk - si.lq) : slope_lds[hl];
      }
    }
    if (wave == 0) {
      const int p = pb * BM + l32;
      const int i = div_group(p, a.s), hl = p - i * G;
      const int64_t idx = st_base + (int64_t)(g * G + hl) * st_hs + i;
      // rows past the sequence fall outside the descriptor and read as 0
      // (lse' = 0, D = 0): their scores are masked to -inf, so P = 0 and
      // dS = 0 * (dP - 0) = 0 whatever the workspace holds there
      const uint32_t off = p < prows ? (uint32_t)(idx * 4) : DROP_ROW;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(st_lds + buf * 64));
      // lanes 0-31 fetch lse', lanes 32-63 fetch D: lane l's dword lands at m0 + 4 l
      if (hh == 0)
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(off), "s"(rl)
                     : "memory", "m0");
      else
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(off), "s"(rd)
                     : "memory", "m0");
    }
  };

  // loop-invariant LDS offsets
  int q_off[KS];  // Q / dO as the A operand: row l32, chunk 2 s + hh
#pragma unroll
  for (int s = 0; s < KS; s++) q_off[s] = tile_off<D>(l32, 2 * s + hh);
  int t_off[DB][2];  // transposing reads of Q / dO: rows 16 u + 4 hh + esrc (+8)
#pragma unroll
  for (int d = 0; d < DB; d++) {
    const int col = d * 32 + 16 * (gq & 1) + 4 * jsrc;
#pragma unroll
    for (int w = 0; w < 2; w++) t_off[d][w] = tile_off<D>(4 * hh + esrc + 8 * w, col >> 3) + (jsrc & 1) * 8;
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int d = 0; d < DB; d++) {
    dk[d] = f32x16{};
    dv[d] = f32x16{};
  }
  const float c = a.scale_log2;
  const char* vrow = v_lds + wave * 32 * ROWB;  // this wave's 32 V rows
  // The packed rows that see this lane's key form one range,
  // [pr_lo, pr_lo + pr_span] (the queries [qmin, qmax] of the key times the
  // group); the mask of a row is then one unsigned compare.  A key past the
  // sequence is seen by no row.
  int pr_lo = 1 << 30;
  uint32_t pr_span = 0;
  {
    const int qlo = qband.qmin(my_key), qhi = qband.qmax(my_key);
    if (my_key < si.lk && qhi >= qlo) {
      pr_lo = qlo * G;
      pr_span = (uint32_t)((qhi + 1) * G - 1 - pr_lo);
    }
  }

  if constexpr (ALIBI) {  // the group's slopes (G <= 128 q heads per kv head)
    if ((int)threadIdx.x < G) slope_lds[threadIdx.x] = alibi_kb(a.x, seq, g * G + (int)threadIdx.x);
    __syncthreads();
  }
  const float keyf = (float)my_key;
  // Query blocks that see any of this wave's 32 keys: [ws_lo, ws_hi] (the
  // inverse band's bounds are nondecreasing in the key).  On the other steps
  // the wave only takes part in the loads and barriers.
  int ws_lo = 0, ws_hi = 1 << 30;
  if constexpr (WSKIP) {
    ws_lo = 1;
    ws_hi = 0;
    const int kw0 = j0 + 32 * wave, kw1 = min(kw0 + 31, si.lk - 1);
    if (kw0 < si.lk && prows > 0) {
      const int qlo = qband.qmin(kw0), qhi = qband.qmax(kw1);
      if (qhi >= qlo) {
        ws_lo = (qlo * G) / BM;
        ws_hi = ((qhi + 1) * G - 1) / BM;
      }
    }
  }
  // The query blocks are visited last to first: under a causal mask every key
  // block of a sequence sees its last query block, so the workgroups of one
  // sequence (dispatched together, on one XCD) start at the same Q / dO tiles
  // and walk them in step, sharing them in L2.
  const int nsteps = pb_end - pb_begin;
  if (nsteps > 0) {
    do_fetch(pb_end - 1, 0);
    if constexpr (!F16) {
      wait_vmcnt<0>();
      q_store(0);
    }
  }
  for (int it = 0; it < nsteps; it++) {
    const int pb = pb_end - 1 - it;
    const int buf = it & 1;
    wait_vmcnt<0>();               // dO tile, row statistics (and V block) are in LDS
    // the Q tile's LDS writes (and with ALiBi the per-row terms) are done, and
    // everyone's reads of the buffers do_fetch refills have returned
    barrier_reads_done();  // everyone's writes visible; everyone is done with the previous step
    if (it + 1 < nsteps) do_fetch(pb - 1, buf ^ 1);  // buffers of the previous step, which everyone has left
    const char* qt = q_lds + buf * QTILE;
    const char* dot = do_lds + buf * QTILE;
    const float* stt = st_lds + buf * 64;

    if (!WSKIP || (pb >= ws_lo && pb <= ws_hi)) {
      // S and dP, [32 queries x 32 keys]: lane = key column, registers = query rows
      f32x16 s_acc, dp;
#pragma unroll
      for (int s = 0; s < KS; s++) {
        s_acc = mfma32<true>(lds_read16(qt + q_off[s]), kf[s], s == 0 ? f32x16{} : s_acc);
        dp = mfma32<F16>(lds_read16(dot + q_off[s]), lds_read16(vrow + q_off[s]), s == 0 ? f32x16{} : dp);
      }
      const int p0 = pb * BM;
      const int qi_lo = div_group(p0, a.s), qi_hi = div_group(min(p0 + BM, prows) - 1, a.s);
      const bool interior = (p0 + BM <= prows) && j0 + wave * 32 >= band.kmin(qi_hi) &&
                            j0 + wave * 32 + 31 <= band.kmax(qi_lo);
      // P and dS from the row statistics of this lane's 16 rows (rows
      // 8a + 4hh + 0..3); only steps that straddle the band, the last query
      // rows or the last keys mask
      if constexpr ((EXT & EXT_CAP) == 0) {
        if constexpr (EXT != 0) {
          // ALiBi alone: the variant logit in place of the raw score, with the
          // rows' terms from LDS, before the mask
          const float* ext = ext_lds + buf * 64;
#pragma unroll
          for (int a4 = 0; a4 < 4; a4++) {
            const f32x4 dg4 = *(const f32x4*)(ext + 8 * a4 + 4 * hh);
            const f32x4 kb4 = *(const f32x4*)(ext + 32 + 8 * a4 + 4 * hh);
#pragma unroll
            for (int e = 0; e < 4; e++) {
              float th;
              s_acc[4 * a4 + e] = ext_score<EXT>(s_acc[4 * a4 + e], a.x, kb4[e], dg4[e] - keyf, th);
            }
          }
        }
        if (!interior) {
          // scores of invisible (row, key) pairs -> -inf, so that P = 0 there
#pragma unroll
          for (int i = 0; i < 16; i++) {
            const int pr = p0 + 8 * (i >> 2) + 4 * hh + (i & 3);
            if ((uint32_t)(pr - pr_lo) > pr_span) s_acc[i] = -INFINITY;
          }
        }
#pragma unroll
        for (int a4 = 0; a4 < 4; a4++) {
          const f32x4 l2 = *(const f32x4*)(stt + 8 * a4 + 4 * hh);
          const f32x4 dl = *(const f32x4*)(stt + 32 + 8 * a4 + 4 * hh);
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const int i = 4 * a4 + e;
            const float p = exp2_fast(fmaf(s_acc[i], c, -l2[e]));
            s_acc[i] = p;
            dp[i] = (p * ds_sc) * (dp[i] - dl[e]);  // dS * 2^ds_e
          }
        }
      } else {
        // soft cap (and ALiBi, rows' terms from LDS): variant logits, P, and dS
        // with 1 - tanh^2 in one pass; invisible pairs are zeroed after
        const float* ext = ext_lds + buf * 64;
#pragma unroll
        for (int a4 = 0; a4 < 4; a4++) {
          const f32x4 l2 = *(const f32x4*)(stt + 8 * a4 + 4 * hh);
          const f32x4 dl = *(const f32x4*)(stt + 32 + 8 * a4 + 4 * hh);
          f32x4 dg4{}, kb4{};
          if constexpr (ALIBI) {
            dg4 = *(const f32x4*)(ext + 8 * a4 + 4 * hh);
            kb4 = *(const f32x4*)(ext + 32 + 8 * a4 + 4 * hh);
          }
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const int i = 4 * a4 + e;
            float th = 0.f;
            const float x = ext_score<EXT>(s_acc[i], a.x, kb4[e], dg4[e] - keyf, th);
            const float p = exp2_fast(fmaf(x, c, -l2[e]));
            float ds = (p * ds_sc) * (dp[i] - dl[e]);  // dS * 2^ds_e
            if constexpr ((EXT & EXT_CAP) != 0) ds *= fmaf(-th, th, 1.f);
            s_acc[i] = p;
            dp[i] = ds;
          }
        }
        if (!interior) {
#pragma unroll
          for (int i = 0; i < 16; i++) {
            const int pr = p0 + 8 * (i >> 2) + 4 * hh + (i & 3);
            if ((uint32_t)(pr - pr_lo) > pr_span) {
              s_acc[i] = 0.f;
              dp[i] = 0.f;
            }
          }
        }
      }
      // P^T / dS^T as B operands: k-step u covers queries 16u + {4hh..4hh+3, 8+4hh..8+4hh+3}
      u32x4 pf[2], sf[2];
#pragma unroll
      for (int u = 0; u < 2; u++) {
        pf[u] = u32x4{pack2<F16>(s_acc[8 * u + 0], s_acc[8 * u + 1]), pack2<F16>(s_acc[8 * u + 2], s_acc[8 * u + 3]),
                      pack2<F16>(s_acc[8 * u + 4], s_acc[8 * u + 5]), pack2<F16>(s_acc[8 * u + 6], s_acc[8 * u + 7])};
        sf[u] = u32x4{pack2<true>(dp[8 * u + 0], dp[8 * u + 1]), pack2<true>(dp[8 * u + 2], dp[8 * u + 3]),
                      pack2<true>(dp[8 * u + 4], dp[8 * u + 5]), pack2<true>(dp[8 * u + 6], dp[8 * u + 7])};
      }
      // dV^T += dO^T P,  dK^T += Q^T dS   (M = dims, N = this wave's keys, K = queries)
#pragma unroll
      for (int d = 0; d < DB; d++)
#pragma unroll
        for (int u = 0; u < 2; u++) {
          const int rb = u * 16 * ROWB;
          const u32x2 o1 = lds_read_tr(dot + rb + t_off[d][0]), o2 = lds_read_tr(dot + rb + t_off[d][1]);
          dv[d] = mfma32<F16>(u32x4{o1[0], o1[1], o2[0], o2[1]}, pf[u], dv[d]);
          const u32x2 q1 = lds_read_tr(qt + rb + t_off[d][0]), q2 = lds_read_tr(qt + rb + t_off[d][1]);
          dk[d] = mfma32<true>(u32x4{q1[0], q1[1], q2[0], q2[1]}, sf[u], dk[d]);
        }
      // S/dP: 3 reads (Q, dO, V) feed 2 MFMAs per step, 2 steps ahead;
      // dV/dK: 4 transposing reads feed 2 MFMAs per step, 2 steps ahead
      sched_reads_ahead<KS, 2, 3, 2>();
      sched_reads_ahead<2 * DB, 2, 4, 2>();
    }  // this wave's step
    if constexpr (!F16) {
      // the next step's Q into the other buffer, which every wave left before
      // this step's barrier
      if (it + 1 < nsteps) {
        wait_vmcnt<0>();
        q_store(buf ^ 1);
      }
    }
  }

  // ---- epilogue: dK = scale * dK_acc, dV; lane = key, registers = dims
  if (!a.grad_f32) {
    __syncthreads();  // all waves are done reading the V block and the Q/dO tiles
    static_assert(4 * 2 * 32 * ROWB <= VBLK + 4 * QTILE, "dK/dV staging fits in the tile space");
    char* const stg = smem + wave * 2 * 32 * ROWB;  // this wave's dK and dV rows
    auto row_off = [&](int r) {
      const int kk = j0 + wave * 32 + r;
      return kk < si.lk_slot ? (uint32_t)((int64_t)kk * krow * 2) : DROP_ROW;
    };
    store_rows16<D, F16>(dk, a.scale * __builtin_amdgcn_ldexpf(1.f, -ds_e), stg,
                         make_rsrc((uint16_t*)a.dk + kbase_e, kbytes_slot), row_off, dg);
    store_rows16<D, F16>(dv, 1.f, stg + 32 * ROWB, make_rsrc((uint16_t*)a.dv + kbase_e, kbytes_slot), row_off, dg);
  } else if (my_key < si.lk_slot) {
    const int64_t ob = ((int64_t)(si.k0 + my_key) * a.s.hkv + g) * dg;
    const float ksc = a.scale * __builtin_amdgcn_ldexpf(1.f, -ds_e);
#pragma unroll
    for (int d = 0; d < DB; d++)
#pragma unroll
      for (int j4 = 0; j4 < 4; j4++) {
        const int dd = d * 32 + 8 * j4 + 4 * hh;
        if (dd >= dg) continue;  // zero tile columns past the head dim
        *(f32x4*)((float*)a.dk + ob + dd) = f32x4{dk[d][4 * j4] * ksc, dk[d][4 * j4 + 1] * ksc,
                                                  dk[d][4 * j4 + 2] * ksc, dk[d][4 * j4 + 3] * ksc};
        *(f32x4*)((float*)a.dv + ob + dd) = f32x4{dv[d][4 * j4], dv[d][4 * j4 + 1], dv[d][4 * j4 + 2], dv[d][4 * j4 + 3]};
      }
  }
}

// The dQ and dK/dV kernels of score variant EXT for every tile width and
// dtype; one translation unit per variant, as for the forward.
template <int EXT, int D, bool F16>
hipError_t launch_bwd_dt(const BwdArgs& a, hipStream_t st) {
  const bool pad = a.s.dg != D;
  // the skipping instance only where it fits in registers without spills
  constexpr bool WSKIP_OK = D <= 128 && !F16;
  if (a.total_ctas_q > 0) {
    timing_begin(K_BWD_DQ, st);
    if (!pad)
      hipLaunchKernelGGL((bwd_dq_kernel<D, F16, false, EXT>), dim3(a.total_ctas_q), dim3(THREADS), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, F16, true, EXT>), dim3(a.total_ctas_q), dim3(THREADS), 0, st, a);
    timing_end(K_BWD_DQ, st);
  }
  if (a.total_ctas > 0) {
    timing_begin(K_BWD_DKDV, st);
    if (pad)
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, F16, true, EXT, false>), dim3(a.total_ctas), dim3(THREADS), 0, st, a);
    else if (WSKIP_OK && a.s.wl >= 0)
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, F16, false, EXT, WSKIP_OK>), dim3(a.total_ctas), dim3(THREADS), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, F16, false, EXT, false>), dim3(a.total_ctas), dim3(THREADS), 0, st, a);
    timing_end(K_BWD_DKDV, st);
  }
  return hipGetLastError();
}

template <int EXT>
hipError_t launch_bwd_variant(const BwdArgs& a, int tile_d, bool f16, hipStream_t st) {
  if (tile_d == 256) return f16 ? launch_bwd_dt<EXT, 256, true>(a, st) : launch_bwd_dt<EXT, 256, false>(a, st);
  if (tile_d == 128) return f16 ? launch_bwd_dt<EXT, 128, true>(a, st) : launch_bwd_dt<EXT, 128, false>(a, st);
  return f16 ? launch_bwd_dt<EXT, 64, true>(a, st) : launch_bwd_dt<EXT, 64, false>(a, st);
}

}  // namespace attn
