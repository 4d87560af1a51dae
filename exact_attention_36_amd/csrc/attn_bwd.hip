// attn_bwd.hip -- exact-attention backward for gfx950.
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
//   bwd_zero_kernel   clears dsinks
//   bwd_pre_kernel    D_i, lse' (log2 units), dsink partials, clears dQ_acc
//   bwd_dkdv_kernel   key-major main loop: one workgroup per 128-key block of
//                     one kv head; dK and dV accumulate in registers over the
//                     visible query rows of all the group's q heads (fp32
//                     across the GQA group: fa4-jax page, restrictions
//                     paragraph); dQ is accumulated with fp32 atomics
//   bwd_dq_kernel     dQ_acc -> the gradient dtype
// The packed (varlen) grid covers only the real key blocks: sequence i's
// blocks start at floor(cu_k[i] / 128) + i and a workgroup finds its
// sequence by binary search (dew-flash-attn page, packed-backward paragraph).
#include "attn_common.h"

namespace attn {

__global__ void bwd_zero_kernel(float* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// One group of D/8 lanes per (token, q head) row: each lane owns 8 dims.
template <int D, bool F16>
__global__ __launch_bounds__(THREADS) void bwd_pre_kernel(const BwdArgs a) {
  constexpr int LPR = D / 8;            // lanes per row
  constexpr int RPB = THREADS / LPR;    // rows per block
  const int64_t rows = (int64_t)(a.s.cu_q ? a.s.total_q : a.s.nseq * a.s.sq) * a.s.hq;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float part = 0.f;
  int h = 0;
  const bool ok = row < rows;
  if (ok) {
    const int64_t t = row / a.s.hq;  // token
    h = (int)(row - t * a.s.hq);
    const uint16_t* o = (const uint16_t*)a.o + row * D + sub * 8;
    const uint16_t* g = (const uint16_t*)a.dout + row * D + sub * 8;
    const u32x4 ov = *(const u32x4*)o, gv = *(const u32x4*)g;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      part = fmaf(to_f32<F16>((uint16_t)(ov[e] & 0xFFFF)), to_f32<F16>((uint16_t)(gv[e] & 0xFFFF)), part);
      part = fmaf(to_f32<F16>((uint16_t)(ov[e] >> 16)), to_f32<F16>((uint16_t)(gv[e] >> 16)), part);
    }
    float* dq = a.dq_acc + row * D + sub * 8;
    *(f32x4*)dq = f32x4{};
    *(f32x4*)(dq + 4) = f32x4{};
  }
  // reduce over the LPR lanes of the row
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off, LPR);
  float dsink_part = 0.f;
  if (ok && sub == 0) {
    const int64_t t = row / a.s.hq;
    int64_t li;
    if (a.s.cu_q) li = (int64_t)h * a.s.total_q + t;
    else {
      const int64_t b = t / a.s.sq, i = t - b * a.s.sq;
      li = (b * a.s.hq + h) * a.s.sq + i;
    }
    const float lse = a.lse[li];
    float lse2 = lse * LOG2E;
    if (a.sinks) {
      const float s2 = a.sinks[h] * LOG2E;
      const float mx = fmaxf(lse2, s2), mn = fminf(lse2, s2);
      lse2 = mx + log2_fast(1.f + exp2_fast(mn - mx));  // log2(2^lse2 + 2^s2)
      // 1 - g = sigmoid(sink - lse): the sink's share of the denominator
      const float one_minus_g = lse == -INFINITY ? 1.f : 1.f / (1.f + exp2_fast(lse * LOG2E - s2));
      dsink_part = -one_minus_g * part;
    }
    a.delta[li] = part;
    a.lse2[li] = lse == -INFINITY ? INFINITY : lse2;  // empty rows: P = 0
  }
  if (a.sinks && a.dsinks) {
    // rows of one block may span several heads: add per row-leader lane
    if (ok && sub == 0 && dsink_part != 0.f) atomicAdd(a.dsinks + h, dsink_part);
  }
}

template <int D, bool F16>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(const BwdArgs a) {
  constexpr int KS = D / 16, DB = D / 32, ROWB = D * 2;
  constexpr int BN = BWD_BN, BM = BWD_BM;
  constexpr int KTILE = BN * ROWB;          // K block in LDS (for dQ)
  constexpr int QTILE = BM * ROWB;          // one Q (or dO) tile
  constexpr int QSLABS = QTILE / 1024;      // 1 KB slabs per Q tile
  constexpr int DST_ROWB = BM * 2;          // dS^T row: BM queries
  __shared__ __attribute__((aligned(1024))) char smem[KTILE + 5 * QTILE + BN * DST_ROWB + 2 * 256];
  char* const k_lds = smem;                              // K block (fp16 for the dQ product)
  char* const q_lds = smem + KTILE;                      // [buf][Q, dO], input dtype
  char* const qh_lds = q_lds + 4 * QTILE;                // Q tile as fp16 (bf16 inputs)
  char* const ds_lds = qh_lds + QTILE;                   // dS^T [BN keys][BM queries], fp16
  float* const st_lds = (float*)(ds_lds + BN * DST_ROWB);  // [buf][lse2 32 | delta 32]

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int gq = lane >> 4, li = lane & 15, esrc = li >> 2, jsrc = li & 3;
  const int G = a.s.group;
  int seq, g, nb;
  if (a.s.cu_q) {
    const int id = xcd_remap(blockIdx.x, a.total_ctas);
    g = id / a.nblk;
    const int t = id - g * a.nblk;
    seq = find_sequence(a.s.cu_k, a.s.nseq, t, 1, BN);
    nb = t - packed_block_start(a.s.cu_k, seq, 1, BN);
  } else {
    // groups are (sequence, kv head); rank 0 is key block 0, the one most
    // query rows see under a causal mask
    int grp;
    if (!GroupGrid{a.s.nseq * a.s.hkv, a.nkb}.decode(blockIdx.x, grp, nb)) return;
    g = grp % a.s.hkv;
    seq = grp / a.s.hkv;
  }
  const SeqInfo si = seq_info(a.s, seq);
  const int j0 = nb * BN;
  if (j0 >= si.lk) return;  // idle slot of the packed grid
  const int prows = si.lq * G;
  const Band band(a.s, si);
  const QBand qband(a.s, si);
  const int j_last = min(j0 + BN, si.lk) - 1;
  const int q_lo = qband.qmin(j0), q_hi = qband.qmax(j_last);
  int pb_begin = 0, pb_end = 0;  // packed q-blocks of BM rows
  if (q_hi >= q_lo && prows > 0) {
    pb_begin = (q_lo * G) / BM;
    pb_end = ((q_hi + 1) * G - 1) / BM + 1;
  }

  const int64_t qrow = (int64_t)a.s.hq * D, krow = (int64_t)a.s.hkv * D;
  const int64_t qbase_e = ((int64_t)si.q0 * a.s.hq + (int64_t)g * G) * D;
  const uint32_t qbytes = si.lq > 0 ? (uint32_t)(((int64_t)(si.lq - 1) * qrow + (int64_t)G * D) * 2) : 0u;
  const int64_t kbase_e = ((int64_t)si.k0 * a.s.hkv + g) * D;
  const uint32_t kbytes = (uint32_t)(((int64_t)(si.lk - 1) * krow + D) * 2);
  const auto rq = make_rsrc((const uint16_t*)a.q + qbase_e, qbytes);
  const auto rdo = make_rsrc((const uint16_t*)a.dout + qbase_e, qbytes);
  const auto rk = make_rsrc((const uint16_t*)a.k + kbase_e, kbytes);
  const auto rv = make_rsrc((const uint16_t*)a.v + kbase_e, kbytes);
  // lse2 / delta of the group: index of packed row p is base + h*hstride + i
  const int64_t st_base = a.s.cu_q ? si.q0 : (int64_t)seq * a.s.hq * a.s.sq;
  const int64_t st_hs = a.s.cu_q ? a.s.total_q : a.s.sq;
  const int64_t st_total = a.s.cu_q ? (int64_t)a.s.hq * a.s.total_q : (int64_t)a.s.nseq * a.s.hq * a.s.sq;
  const auto rl = make_rsrc(a.lse2, (uint32_t)(st_total * 4));
  // dQ accumulator rows of this (sequence, kv group), fp32
  const auto rdq = make_rsrc(a.dq_acc + qbase_e, si.lq > 0 ? (uint32_t)(((int64_t)(si.lq - 1) * qrow + (int64_t)G * D) * 4) : 0u);
  const auto rd = make_rsrc(a.delta, (uint32_t)(st_total * 4));

  // K block -> LDS (swizzled), for the transposing reads of dQ = dS K
  {
    constexpr int SLABS = KTILE / 1024 / 4;
#pragma unroll
    for (int n = 0; n < SLABS; n++) {
      const int slab = wave * SLABS + n;
      const int byte = slab * 1024 + lane * 16;
      const int r = byte / ROWB, pos = (byte % ROWB) >> 4;
      const int c = pos ^ swz<D>(r);
      buf_load_lds16(rk, k_lds + slab * 1024, (uint32_t)((((int64_t)(j0 + r)) * krow + c * 8) * 2));
    }
  }
  // this wave's 32 keys as B operands (lane: key, 8 dims per k-step)
  const int my_key = j0 + wave * 32 + l32;
  u32x4 kf[KS], vf[KS];
  {
    const uint32_t ko = (uint32_t)((int64_t)(my_key)*krow * 2);
#pragma unroll
    for (int s = 0; s < KS; s++) {
      kf[s] = buf_load16(rk, ko + (uint32_t)((16 * s + 8 * hh) * 2));
      vf[s] = buf_load16(rv, ko + (uint32_t)((16 * s + 8 * hh) * 2));
    }
  }

  auto load_q = [&](int pb, int buf) {
    char* qd = q_lds + buf * 2 * QTILE;
    char* dd = qd + QTILE;
    constexpr int SL = QSLABS / 4;  // slabs per wave
#pragma unroll
    for (int n = 0; n < SL; n++) {
      const int slab = wave * SL + n;
      const int byte = slab * 1024 + lane * 16;
      const int r = byte / ROWB, pos = (byte % ROWB) >> 4;
      const int c = pos ^ swz<D>(r);
      const int p = pb * BM + r;
      const int i = div_group(p, a.s), hl = p - i * G;
      const uint32_t off = (uint32_t)(((int64_t)i * qrow + (int64_t)hl * D + c * 8) * 2);
      buf_load_lds16(rq, qd + slab * 1024, off);
      buf_load_lds16(rdo, dd + slab * 1024, off);
    }
    if (wave == 0) {
      const int p = pb * BM + l32;
      const int i = div_group(p, a.s), hl = p - i * G;
      const int64_t idx = st_base + (int64_t)(g * G + hl) * st_hs + i;
      // rows past the sequence read index 0 (valid memory); they are masked
      const uint32_t off = p < prows ? (uint32_t)(idx * 4) : 0u;
      void* dst = st_lds + buf * 64;
      if (hh == 0) __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, LDS_PTR(void, dst), 4, off, 0, 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, LDS_PTR(void, dst), 4, off, 0, 0, 0);
    }
  };

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int d = 0; d < DB; d++) {
    dk[d] = f32x16{};
    dv[d] = f32x16{};
  }
  const float c = a.scale_log2;
  // key range fully visible to every row of q-block pb?  (checked per block)
  const int my_kj = my_key;
  // dQ step: wave -> (d block, key range)
  constexpr int WPD = 4 / DB;                 // waves sharing one d block
  const int dq_dblk = wave % DB, dq_kpart = wave / DB;
  constexpr int DQ_KEYS = BN / WPD;           // keys summed by this wave

  if (pb_begin < pb_end) load_q(pb_begin, 0);
  for (int pb = pb_begin; pb < pb_end; pb++) {
    const int buf = (pb - pb_begin) & 1;
    // tile pb was issued before the previous step's 16 dQ atomics
    if (pb == pb_begin) wait_vmcnt<0>();
    else wait_vmcnt<16>();
    __builtin_amdgcn_s_barrier();
    if (pb + 1 < pb_end) load_q(pb + 1, buf ^ 1);
    const char* qt = q_lds + buf * 2 * QTILE;
    const char* dot = qt + QTILE;
    const float* stt = st_lds + buf * 64;
    // dS is kept in fp16 (10 fraction bits instead of bf16's 7), so the dK and
    // dQ products take fp16 copies of the Q tile and of the K block.
    if constexpr (!F16) {
      if (pb == pb_begin) {
#pragma unroll
        for (int n = 0; n < KTILE / 16 / THREADS; n++) {
          char* p16 = k_lds + (threadIdx.x + n * THREADS) * 16;
          *LDS_PTR(u32x4, p16) = bf16x8_to_f16x8(lds_read16(p16));
        }
      }
#pragma unroll
      for (int n = 0; n < QTILE / 16 / THREADS; n++) {
        const int off = (threadIdx.x + n * THREADS) * 16;
        *LDS_PTR(u32x4, qh_lds + off) = bf16x8_to_f16x8(lds_read16(qt + off));
      }
    }
    const char* qh = F16 ? qt : qh_lds;

    // S and dP, [32 queries x 32 keys]: lane = key column, registers = query rows
    f32x16 s_acc = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int s = 0; s < KS; s++) {
      s_acc = mfma32<F16>(lds_read16(qt + tile_off<D>(l32, 2 * s + hh)), kf[s], s_acc);
      dp = mfma32<F16>(lds_read16(dot + tile_off<D>(l32, 2 * s + hh)), vf[s], dp);
    }
    // row statistics of this lane's 16 rows: rows 8a + 4hh + 0..3
    f32x4 l2[4], dl[4];
#pragma unroll
    for (int a4 = 0; a4 < 4; a4++) {
      l2[a4] = *(const f32x4*)(stt + 8 * a4 + 4 * hh);
      dl[a4] = *(const f32x4*)(stt + 32 + 8 * a4 + 4 * hh);
    }
    const int p0 = pb * BM;
    const int qi_lo = div_group(p0, a.s), qi_hi = div_group(min(p0 + BM, prows) - 1, a.s);
    const bool interior = (p0 + BM <= prows) && j0 + wave * 32 >= band.kmin(qi_hi) &&
                          j0 + wave * 32 + 31 <= band.kmax(qi_lo);
    f32x16 pm, dsm;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int r = 8 * (i >> 2) + 4 * hh + (i & 3);
      const float lse2 = l2[i >> 2][i & 3];
      float p = exp2_fast(fmaf(s_acc[i], c, -lse2));
      if (!interior) {
        const int pr = p0 + r;
        const int qi = div_group(pr, a.s);
        const bool vis = pr < prows && my_kj < si.lk && my_kj >= band.kmin(qi) && my_kj <= band.kmax(qi);
        if (!vis) p = 0.f;
      }
      pm[i] = p;
      dsm[i] = p * (dp[i] - dl[i >> 2][i & 3]);
    }
    // dV^T += dO^T P  (M = dims, N = this wave's keys, K = queries)
    u32x4 pf[2], sf[2];
#pragma unroll
    for (int u = 0; u < 2; u++) {
      pf[u] = u32x4{pack2<F16>(pm[8 * u + 0], pm[8 * u + 1]), pack2<F16>(pm[8 * u + 2], pm[8 * u + 3]),
                    pack2<F16>(pm[8 * u + 4], pm[8 * u + 5]), pack2<F16>(pm[8 * u + 6], pm[8 * u + 7])};
      sf[u] = u32x4{pack2<true>(dsm[8 * u + 0], dsm[8 * u + 1]), pack2<true>(dsm[8 * u + 2], dsm[8 * u + 3]),
                    pack2<true>(dsm[8 * u + 4], dsm[8 * u + 5]), pack2<true>(dsm[8 * u + 6], dsm[8 * u + 7])};
    }
#pragma unroll
    for (int d = 0; d < DB; d++) {
      const int col = d * 32 + 16 * (gq & 1) + 4 * jsrc;
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int rb = u * 16 + 4 * hh + esrc;
        const int off1 = tile_off<D>(rb, col >> 3) + (jsrc & 1) * 8;
        const int off2 = tile_off<D>(rb + 8, col >> 3) + (jsrc & 1) * 8;
        const u32x2 o1 = lds_read_tr(dot + off1), o2 = lds_read_tr(dot + off2);
        dv[d] = mfma32<F16>(u32x4{o1[0], o1[1], o2[0], o2[1]}, pf[u], dv[d]);
      }
    }
    // dS^T -> LDS: row = key, 4 consecutive queries per 8-byte write
    {
      char* drow = ds_lds + (wave * 32 + l32) * DST_ROWB;
#pragma unroll
      for (int a4 = 0; a4 < 4; a4++) {
        const int q4 = 8 * a4 + 4 * hh;  // first of 4 consecutive queries
        *(u32x2*)(drow + q4 * 2) = u32x2{sf[a4 >> 1][2 * (a4 & 1)], sf[a4 >> 1][2 * (a4 & 1) + 1]};
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_s_barrier();
    // dK^T += Q^T dS  (fp16)
#pragma unroll
    for (int d = 0; d < DB; d++) {
      const int col = d * 32 + 16 * (gq & 1) + 4 * jsrc;
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int rb = u * 16 + 4 * hh + esrc;
        const u32x2 q1 = lds_read_tr(qh + tile_off<D>(rb, col >> 3) + (jsrc & 1) * 8);
        const u32x2 q2 = lds_read_tr(qh + tile_off<D>(rb + 8, col >> 3) + (jsrc & 1) * 8);
        dk[d] = mfma32<true>(u32x4{q1[0], q1[1], q2[0], q2[1]}, sf[u], dk[d]);
      }
    }
    // dQ[32 q x 32 dims] += dS K over this wave's key range:
    // A = dS (lane: query, 8 keys) via transposing reads of dS^T;
    // B = K  (lane: dim, 8 keys) via transposing reads of the K block.
    {
      f32x16 dqa = f32x16{};
#pragma unroll
      for (int ks = 0; ks < DQ_KEYS / 16; ks++) {
        const int kb = dq_kpart * DQ_KEYS + ks * 16 + 8 * hh + esrc;  // key row for this lane's source
        const int qcol = 16 * (gq & 1) + 4 * jsrc;
        const u32x2 s1 = lds_read_tr(ds_lds + kb * DST_ROWB + qcol * 2);
        const u32x2 s2 = lds_read_tr(ds_lds + (kb + 4) * DST_ROWB + qcol * 2);
        const int dcol = dq_dblk * 32 + 16 * (gq & 1) + 4 * jsrc;
        const u32x2 k1 = lds_read_tr(k_lds + tile_off<D>(kb, dcol >> 3) + (jsrc & 1) * 8);
        const u32x2 k2 = lds_read_tr(k_lds + tile_off<D>(kb + 4, dcol >> 3) + (jsrc & 1) * 8);
        dqa = mfma32<true>(u32x4{s1[0], s1[1], s2[0], s2[1]}, u32x4{k1[0], k1[1], k2[0], k2[1]}, dqa);
      }
      // C: lane = dim column, registers = query rows.  Exactly 16 atomics per
      // lane per step (rows past the sequence fall outside the buffer and are
      // dropped by the hardware), so the next step can wait for its tile
      // loads with vmcnt(16) without waiting for these atomics.
      const int dcol = dq_dblk * 32 + l32;
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int pr = p0 + 8 * (i >> 2) + 4 * hh + (i & 3);
        const int qi = div_group(pr, a.s), hl = pr - qi * G;
        const uint32_t off = (uint32_t)((((int64_t)qi * a.s.hq + hl) * D + dcol) * 4);
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(dqa[i] * a.scale, rdq, off, 0, 0);
      }
    }
  }

  // ---- epilogue: dK = scale * dK_acc, dV; lane = key, registers = dims
  if (my_key < si.lk) {
    const int64_t ob = ((int64_t)(si.k0 + my_key) * a.s.hkv + g) * D;
#pragma unroll
    for (int d = 0; d < DB; d++)
#pragma unroll
      for (int j4 = 0; j4 < 4; j4++) {
        const int dd = d * 32 + 8 * j4 + 4 * hh;
        const float k0v = dk[d][4 * j4] * a.scale, k1v = dk[d][4 * j4 + 1] * a.scale;
        const float k2v = dk[d][4 * j4 + 2] * a.scale, k3v = dk[d][4 * j4 + 3] * a.scale;
        if (a.grad_f32) {
          *(f32x4*)((float*)a.dk + ob + dd) = f32x4{k0v, k1v, k2v, k3v};
          *(f32x4*)((float*)a.dv + ob + dd) = f32x4{dv[d][4 * j4], dv[d][4 * j4 + 1], dv[d][4 * j4 + 2], dv[d][4 * j4 + 3]};
        } else {
          *(u32x2*)((uint16_t*)a.dk + ob + dd) = u32x2{pack2<F16>(k0v, k1v), pack2<F16>(k2v, k3v)};
          *(u32x2*)((uint16_t*)a.dv + ob + dd) =
              u32x2{pack2<F16>(dv[d][4 * j4], dv[d][4 * j4 + 1]), pack2<F16>(dv[d][4 * j4 + 2], dv[d][4 * j4 + 3])};
        }
      }
  }
}

template <bool F16>
__global__ __launch_bounds__(THREADS) void bwd_dq_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                                         int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * THREADS + threadIdx.x;
  if (i < n4) {
    const f32x4 v = ((const f32x4*)src)[i];
    ((u32x2*)dst)[i] = u32x2{pack2<F16>(v[0], v[1]), pack2<F16>(v[2], v[3])};
  }
}

template <int D, bool F16>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  if (a.sinks && a.dsinks) {
    timing_begin(K_BWD_ZERO, st);
    hipLaunchKernelGGL(bwd_zero_kernel, dim3((a.s.hq + 255) / 256), dim3(256), 0, st, a.dsinks, a.s.hq);
    timing_end(K_BWD_ZERO, st);
  }
  const int64_t tq = a.s.cu_q ? a.s.total_q : (int64_t)a.s.nseq * a.s.sq;
  const int64_t rows = tq * a.s.hq;
  constexpr int RPB = THREADS / (D / 8);
  if (rows > 0) {
    timing_begin(K_BWD_PRE, st);
    hipLaunchKernelGGL((bwd_pre_kernel<D, F16>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(THREADS), 0, st, a);
    timing_end(K_BWD_PRE, st);
  }
  if (a.total_ctas > 0) {
    timing_begin(K_BWD_DKDV, st);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, F16>), dim3(a.total_ctas), dim3(THREADS), 0, st, a);
    timing_end(K_BWD_DKDV, st);
  }
  if (!a.grad_f32 && rows > 0) {
    const int64_t n4 = rows * D / 4;
    timing_begin(K_BWD_DQ, st);
    hipLaunchKernelGGL((bwd_dq_kernel<F16>), dim3((unsigned)((n4 + THREADS - 1) / THREADS)), dim3(THREADS), 0, st,
                       (const float*)a.dq_acc, (uint16_t*)a.dq, n4);
    timing_end(K_BWD_DQ, st);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int head_dim, bool f16, hipStream_t st) {
  if (head_dim == 128) return f16 ? launch_bwd_t<128, true>(a, st) : launch_bwd_t<128, false>(a, st);
  return f16 ? launch_bwd_t<64, true>(a, st) : launch_bwd_t<64, false>(a, st);
}

}  // namespace attn
