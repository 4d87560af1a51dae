/*
 * attn_oracle.c -- plain fp64 CPU oracle for exact scaled-dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent reference that the
 * GPU library is checked against.  Only the test suite, the package smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or constant with the HIP library and includes none of its
 * files.
 *
 * What it computes is the plain definition of attention, written out one
 * query row at a time with the whole score row materialised, masked, and
 * soft-maxed in double precision:
 *
 *   - logits x_ij = scale * <q_i, k_j>, O = softmax(x) V  (GitHub search
 *     page, gitctrlx/flash-attention-tutorial README, section 1 "Standard
 *     Self-Attention"; default scale 1/sqrt(D) from the flash_attn_func
 *     docstring in the vllm-project/flash-attention README on the same page);
 *   - the softmax is the max-subtracted ("safe") form of section 2 of that
 *     tutorial;
 *   - causal and window masks are bottom-right aligned: query i of a
 *     sequence with Lq queries and Lk keys sees key j iff
 *       (!causal || j <= i + Lk - Lq) &&
 *       (left  < 0 || j >= i + Lk - Lq - left) &&
 *       (right < 0 || j <= i + Lk - Lq + right)
 *     (fa4-jax page, the paragraph on bottom-right alignment; the window
 *     interval and the causal examples in the flash_attn_func /
 *     flash_attn_with_kvcache docstrings and the "2.1: Change behavior of
 *     causal flag" note of the vllm-project/flash-attention README on the
 *     GitHub search page; dew-flash-attn page, window_size paragraph);
 *   - a row that sees no key has output 0 (same docstring: an all-zero mask
 *     row gives zero output) and log-sum-exp -inf;
 *   - grouped-query attention: q head h reads kv head h / (Hq/Hkv)
 *     (flash_attn_func docstring, the 6-head / 2-head example);
 *   - attention sinks: one logit s_h per q head that joins the softmax
 *     denominator with no value, so the output is scaled by
 *     sigmoid(lse - s_h) (dew-flash-attn page, sinks paragraph); the
 *     returned lse is the sink-free one;
 *   - several sinks per q head (ejkernel flash_attention API page, the
 *     softmax_aux parameter, one row of sink logits per head): each is one
 *     more value-less logit in the denominator, so the gate becomes
 *     1 / (1 + sum_k exp(s_hk - lse));
 *   - score variants, applied to the scaled logit x = scale <q_i, k_j> in
 *     this order: the soft cap x -> cap * tanh(x / cap) (the softcapping of
 *     the vllm-project/flash-attention README, "2.6: Softcapping", and the
 *     logits_soft_cap parameter of the ejkernel page; the pages name it
 *     without a formula, and the tanh form is the plain reading), then the
 *     ALiBi bias -slope_h * |i + Lk - Lq - j| (alibi_slopes in the
 *     flash_attn_func docstring of the same README), one slope per q head,
 *     optionally per sequence;
 *   - gradients by the chain rule of the above (tutorial section 6
 *     "Flash Attention Backward Pass": dV = P^T dO, D_i = dO_i . O_i,
 *     dS = P o (dP - D), dQ = dS K, dK = dS^T Q), with the derivative of
 *     the logit with respect to <q_i, k_j> (scale, times 1 - tanh^2 under
 *     the soft cap; the bias does not depend on q or k) restored on dQ and
 *     dK, and the sink's gradient -(1 - g_i) D_i summed over rows.
 *
 * Inputs are the raw 16-bit encodings of bf16 or fp16 tensors (or plain
 * doubles, for finite-difference checks), token-major [token][head][dim];
 * each element is decoded exactly to double here.
 * A batched [B,S,H,D] problem is the packed problem whose sequence b starts
 * at token b*S.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int32_t dtype;          /* 0 = bf16 bits, 1 = fp16 bits, 2 = float64 values */
    int32_t causal;         /* nonzero: causal, bottom-right aligned */
    int64_t window_left;    /* -1 = unbounded */
    int64_t window_right;   /* -1 = unbounded */
    int64_t nseq;           /* number of sequences (batch size) */
    int64_t hq, hkv, d;     /* heads of Q, heads of K/V, head dim */
    double scale;           /* softmax scale applied to <q,k> */
    const int64_t *q_start; /* [nseq] first token of each sequence in q */
    const int64_t *q_len;   /* [nseq] */
    const int64_t *k_start; /* [nseq] first token of each sequence in k, v */
    const int64_t *k_len;   /* [nseq] */
    const void *q;          /* [tokens_q][hq][d] */
    const void *k;          /* [tokens_k][hkv][d] */
    const void *v;          /* [tokens_k][hkv][d] */
    const void *dout;       /* [tokens_q][hq][d], may be NULL */
    const double *sinks;    /* [hq][num_sinks] or NULL */
    double softcap;         /* > 0: soft cap of the logits; 0: none */
    const double *alibi;    /* [nseq][hq] ALiBi slopes or NULL */
    int64_t num_sinks;      /* sinks per q head (values < 1 count as 1) */
} oracle_problem;

/* ---- exact decoding of the 16-bit input formats ---- */

static double decode_bf16(uint16_t h)
{
    /* bf16 is the top half of an IEEE binary32 */
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double decode_fp16(uint16_t h)
{
    /* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits */
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24);                 /* subnormal: f * 2^-14 / 2^10 */
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(f + 1024), e - 25);     /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -mag : mag;
}

static double elem(const oracle_problem *p, const void *base, int64_t idx)
{
    if (p->dtype == 2) return ((const double *)base)[idx];
    const uint16_t h = ((const uint16_t *)base)[idx];
    return p->dtype == 0 ? decode_bf16(h) : decode_fp16(h);
}

double oracle_decode(int32_t dtype, uint16_t h)
{
    return dtype == 0 ? decode_bf16(h) : decode_fp16(h);
}

/* ---- the mask ---- */

int oracle_visible(int32_t causal, int64_t left, int64_t right,
                   int64_t lq, int64_t lk, int64_t i, int64_t j)
{
    int64_t diag = i + lk - lq; /* the key that lines up with query i */
    if (causal && j > diag) return 0;
    if (left >= 0 && j < diag - left) return 0;
    if (right >= 0 && j > diag + right) return 0;
    return 1;
}

/* ---- the logit of one (query, key) pair ---- */

/*
 * Logit of query i and key j of sequence s (Lq queries, Lk keys), q head h,
 * from qk = <q_i, k_j>; *dx receives d(logit)/d(qk).
 */
static double logit(const oracle_problem *p, int64_t s, int64_t h, int64_t lq, int64_t lk,
                    int64_t i, int64_t j, double qk, double *dx)
{
    double x = p->scale * qk, d = p->scale;
    if (p->softcap > 0.0) {
        const double t = tanh(x / p->softcap);
        x = p->softcap * t;
        d *= 1.0 - t * t;
    }
    if (p->alibi) x -= p->alibi[s * p->hq + h] * fabs((double)(i + lk - lq - j));
    if (dx) *dx = d;
    return x;
}

/* sum_k exp(s_hk - l): the sinks' share of the denominator relative to exp(l) */
static double sink_terms(const oracle_problem *p, int64_t h, double l)
{
    const int64_t n = p->num_sinks < 1 ? 1 : p->num_sinks;
    double acc = 0.0;
    for (int64_t k = 0; k < n; k++) acc += exp(p->sinks[h * n + k] - l);
    return acc;
}

/* ---- one query row: forward, and optionally dQ ---- */

/*
 * Computes, for query `row` of sequence `s`, q head `h`:
 *   o[d]      output row (already multiplied by the sink gate)
 *   *lse      log-sum-exp over visible keys (no sink), -inf if none
 *   *gate     sigmoid(lse - sink) with sinks, 1 without, 0 for an empty row
 *   *delta    D = <dO_row, O_row>            (needs dout)
 *   dq[d]     gradient of <dO, O> w.r.t. q_row (needs dout)
 * `x` is caller scratch of length Lk.  Any output pointer may be NULL.
 */
static void one_row(const oracle_problem *p, int64_t s, int64_t h, int64_t row,
                    double *x, double *o, double *lse, double *gate,
                    double *delta, double *dq)
{
    const int64_t D = p->d;
    const int64_t G = p->hq / p->hkv;
    const int64_t g = h / G;
    const int64_t lq = p->q_len[s], lk = p->k_len[s];
    const int64_t qtok = p->q_start[s] + row;
    const int64_t qoff = (qtok * p->hq + h) * D;
    double o_loc[512], q_loc[512], do_loc[512];
    int64_t nvis = 0;
    double m = -INFINITY;

    for (int64_t c = 0; c < D; c++) q_loc[c] = elem(p, p->q, qoff + c);

    /* 1. materialise the score row, masked entries as -inf */
    for (int64_t j = 0; j < lk; j++) {
        if (!oracle_visible(p->causal, p->window_left, p->window_right, lq, lk, row, j)) {
            x[j] = -INFINITY;
            continue;
        }
        const int64_t koff = ((p->k_start[s] + j) * p->hkv + g) * D;
        double acc = 0.0;
        for (int64_t c = 0; c < D; c++) acc += q_loc[c] * elem(p, p->k, koff + c);
        x[j] = logit(p, s, h, lq, lk, row, j, acc, NULL);
        if (x[j] > m) m = x[j];
        nvis++;
    }

    for (int64_t c = 0; c < D; c++) o_loc[c] = 0.0;
    double l = -INFINITY, gt = 0.0;
    if (nvis > 0) {
        /* 2. safe softmax: subtract the row max */
        double sum = 0.0;
        for (int64_t j = 0; j < lk; j++)
            if (x[j] != -INFINITY) sum += exp(x[j] - m);
        l = m + log(sum);
        /* 3. sink gate: each sink is one more logit in the denominator */
        gt = p->sinks ? 1.0 / (1.0 + sink_terms(p, h, l)) : 1.0;
        /* 4. O = gate * sum_j P_ij v_j */
        for (int64_t j = 0; j < lk; j++) {
            if (x[j] == -INFINITY) continue;
            const double pij = exp(x[j] - l);
            const int64_t voff = ((p->k_start[s] + j) * p->hkv + g) * D;
            for (int64_t c = 0; c < D; c++) o_loc[c] += pij * elem(p, p->v, voff + c);
        }
        for (int64_t c = 0; c < D; c++) o_loc[c] *= gt;
    }
    if (o) for (int64_t c = 0; c < D; c++) o[c] = o_loc[c];
    if (lse) *lse = l;
    if (gate) *gate = gt;

    if (!p->dout || (!delta && !dq)) return;
    for (int64_t c = 0; c < D; c++) do_loc[c] = elem(p, p->dout, qoff + c);
    double dl = 0.0;
    for (int64_t c = 0; c < D; c++) dl += do_loc[c] * o_loc[c];
    if (delta) *delta = dl;
    if (!dq) return;
    for (int64_t c = 0; c < D; c++) dq[c] = 0.0;
    if (nvis == 0) return;
    /* dS_ij = gate * P_ij * (dP_ij - D_i),  dQ_i = sum_j dS_ij x'_ij k_j
       with x'_ij = d(logit)/d(qk) */
    for (int64_t j = 0; j < lk; j++) {
        if (x[j] == -INFINITY) continue;
        const int64_t kvoff = ((p->k_start[s] + j) * p->hkv + g) * D;
        double dp = 0.0, qk = 0.0, dx;
        for (int64_t c = 0; c < D; c++) {
            dp += do_loc[c] * elem(p, p->v, kvoff + c);
            qk += q_loc[c] * elem(p, p->k, kvoff + c);
        }
        logit(p, s, h, lq, lk, row, j, qk, &dx);
        const double ds = gt * exp(x[j] - l) * (dp - dl);
        for (int64_t c = 0; c < D; c++) dq[c] += dx * ds * elem(p, p->k, kvoff + c);
    }
}

static int check_problem(const oracle_problem *p)
{
    if (!p || p->d <= 0 || p->d > 512 || p->hq <= 0 || p->hkv <= 0 || p->hq % p->hkv) return -1;
    if (p->dtype < 0 || p->dtype > 2) return -1;
    if (!p->q || !p->k || !p->v || !p->q_start || !p->q_len || !p->k_start || !p->k_len) return -1;
    return 0;
}

static int64_t max_k_len(const oracle_problem *p)
{
    int64_t mx = 1;
    for (int64_t s = 0; s < p->nseq; s++) if (p->k_len[s] > mx) mx = p->k_len[s];
    return mx;
}

/*
 * Rows: for each request r, query row[r] of sequence seq[r], q head head[r].
 * Outputs (each may be NULL): o [n][d], lse [n], gate [n], delta [n], dq [n][d].
 */
int oracle_rows(const oracle_problem *p, int64_t n, const int64_t *seq,
                const int64_t *head, const int64_t *row, double *o, double *lse,
                double *gate, double *delta, double *dq)
{
    if (check_problem(p)) return -1;
    for (int64_t r = 0; r < n; r++)
        if (seq[r] < 0 || seq[r] >= p->nseq || head[r] < 0 || head[r] >= p->hq ||
            row[r] < 0 || row[r] >= p->q_len[seq[r]]) return -2;
    const int64_t lkmax = max_k_len(p);
    int err = 0;
#pragma omp parallel
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)lkmax);
        if (!x) {
#pragma omp atomic write
            err = -3;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n; r++) {
            if (!x) continue;
            one_row(p, seq[r], head[r], row[r], x,
                    o ? o + r * p->d : NULL, lse ? lse + r : NULL,
                    gate ? gate + r : NULL, delta ? delta + r : NULL,
                    dq ? dq + r * p->d : NULL);
        }
        free(x);
    }
    return err;
}

/*
 * Columns: dK and dV of keys col[0..ncol) of sequence s, kv head g.
 *   dV_j = sum over the group's q heads h and rows i of  gate_i P_ij dO_i
 *   dK_j = sum over h, i of  x'_ij gate_i P_ij (dP_ij - D_i) q_i
 * with x'_ij = d(logit)/d(qk).
 * The per-row statistics lse, gate and delta of every row of the group's q
 * heads are inputs ([G][Lq] each, from oracle_rows), so that a column is the
 * plain sum over rows.
 */
int oracle_cols(const oracle_problem *p, int64_t s, int64_t g, int64_t ncol,
                const int64_t *col, const double *lse_rows, const double *gate_rows,
                const double *delta_rows, double *dk, double *dv)
{
    if (check_problem(p) || !p->dout) return -1;
    if (s < 0 || s >= p->nseq || g < 0 || g >= p->hkv) return -2;
    const int64_t D = p->d, G = p->hq / p->hkv;
    const int64_t lq = p->q_len[s], lk = p->k_len[s];
    for (int64_t c = 0; c < ncol; c++) if (col[c] < 0 || col[c] >= lk) return -2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t c = 0; c < ncol; c++) {
        const int64_t j = col[c];
        const int64_t kvoff = ((p->k_start[s] + j) * p->hkv + g) * D;
        double kj[512], vj[512], dkj[512], dvj[512];
        for (int64_t e = 0; e < D; e++) {
            kj[e] = elem(p, p->k, kvoff + e);
            vj[e] = elem(p, p->v, kvoff + e);
            dkj[e] = 0.0;
            dvj[e] = 0.0;
        }
        for (int64_t hh = 0; hh < G; hh++) {
            const int64_t h = g * G + hh;
            for (int64_t i = 0; i < lq; i++) {
                if (!oracle_visible(p->causal, p->window_left, p->window_right, lq, lk, i, j)) continue;
                const double l = lse_rows[hh * lq + i];
                if (l == -INFINITY) continue;
                const int64_t qoff = ((p->q_start[s] + i) * p->hq + h) * D;
                double qk = 0.0, dp = 0.0;
                for (int64_t e = 0; e < D; e++) {
                    qk += elem(p, p->q, qoff + e) * kj[e];
                    dp += elem(p, p->dout, qoff + e) * vj[e];
                }
                double dx;
                const double pg = gate_rows[hh * lq + i] * exp(logit(p, s, h, lq, lk, i, j, qk, &dx) - l);
                const double ds = pg * (dp - delta_rows[hh * lq + i]);
                for (int64_t e = 0; e < D; e++) {
                    dvj[e] += pg * elem(p, p->dout, qoff + e);
                    dkj[e] += dx * ds * elem(p, p->q, qoff + e);
                }
            }
        }
        for (int64_t e = 0; e < D; e++) {
            if (dk) dk[c * D + e] = dkj[e];
            if (dv) dv[c * D + e] = dvj[e];
        }
    }
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
