/*
 * attn.h -- C ABI of the gfx950 fused exact-attention library (libattn36.so).
 *
 * The library computes exact scaled-dot-product attention,
 *     O = softmax(scale * Q K^T + mask) V,
 * in one tiled pass with an online softmax, and its backward pass by
 * recomputing the probabilities from the saved per-row log-sum-exp
 * (GitHub search page, gitctrlx/flash-attention-tutorial README: sections
 * 1 "Standard Self-Attention", 3 "Online Softmax", 5 "Flash Attention (With
 * Tiling)" and 6 "Flash Attention Backward Pass").
 *
 * Semantics (all four entry points):
 *  - Inputs are bf16 or fp16, head dim a multiple of 8 up to 256 (fa4-jax
 *    page, restrictions paragraph).
 *  - Grouped-query attention: heads_q % heads_kv == 0 and q head h reads kv
 *    head h / (heads_q / heads_kv) (flash_attn_func docstring, 6/2-head
 *    example, vllm-project/flash-attention README on the GitHub search page;
 *    dew-flash-attn page, grouped-query sentence).
 *  - Causal masking and the two-sided sliding window (left, right) are
 *    aligned bottom-right: query i of a sequence with Lq queries and Lk keys
 *    sees key j iff  (!causal || j <= i + Lk - Lq)
 *                 && (left  == -1 || j >= i + Lk - Lq - left)
 *                 && (right == -1 || j <= i + Lk - Lq + right)
 *    (fa4-jax page, bottom-right alignment paragraph; window interval of the
 *    flash_attn_func docstring; dew-flash-attn page, window_size paragraph).
 *    A row that sees no key gets output 0 and log-sum-exp -inf (same
 *    docstring: an all-zero mask row gives zero output).
 *  - Attention sinks: one fp32 logit per q head joins each row's softmax
 *    denominator with no value, which multiplies the row's output by
 *    sigmoid(lse - sink); the returned lse is the sink-free one, and the
 *    backward returns d(loss)/d(sink) (dew-flash-attn page, sinks paragraph).
 *    Several sinks per q head (ejkernel flash_attention API page,
 *    softmax_aux [num_heads, num_sinks] or [num_sinks]) each join the
 *    denominator; together they act as one sink at log sum_k exp(sink_k).
 *  - Score variants: a soft cap, softcap * tanh(x / softcap) of each logit
 *    x = scale * q.k (vllm-project/flash-attention README on the GitHub
 *    search page, "2.6: Softcapping"; ejkernel page, logits_soft_cap; the
 *    pages give no formula and the tanh form is the plain reading), then the
 *    ALiBi bias -slope_h * |i + Lk - Lq - j| (alibi_slopes in the
 *    flash_attn_func docstring of the same README).  Gradients follow the
 *    chain rule through both.
 *  - Used lengths (fa4-jax page, varlen semantics paragraph: seqused_q,
 *    seqused_k): a batch entry or packed sequence may use only the first
 *    tokens of its slot; see attn_params.
 *  - Packed variable-length batches: [T, H, D] tensors with int32 offsets
 *    cu_seqlens [N+1] from 0 to T; attention never crosses sequences; the
 *    mask applies per sequence with that sequence's own Lq, Lk; zero-length
 *    sequences are allowed; the lse of a packed call is laid out [Hq, T_q]
 *    (fa4-jax page, varlen semantics paragraph).  cu_seqlens contents are NOT
 *    checked: they must be nondecreasing, start at 0 and end at the token
 *    count.  The grid covers only the batch's real blocks: sequence i's blocks
 *    start at floor(cu_seqlens[i] * G / 128) + i and a workgroup finds its
 *    sequence by binary search (dew-flash-attn page, packed-backward
 *    paragraph).
 *
 * Layouts (all contiguous, last dim stride 1):
 *   batched:  q, o, dout, dq   [B, Sq, Hq, D];  k, v, dk, dv  [B, Sk, Hkv, D]
 *             lse              fp32 [B, Hq, Sq]
 *   packed:   q, o, dout, dq   [Tq, Hq, D];     k, v, dk, dv  [Tk, Hkv, D]
 *             lse              fp32 [Hq, Tq]
 *   sinks, dsinks              fp32 [Hq][num_sinks], or [num_sinks] shared
 *   alibi_slopes               fp32 [Hq], or [B or num_seqs][Hq]
 *
 * Ownership: every pointer except `params` is device memory owned by the
 * caller; the library allocates nothing and keeps no device state.  Scratch
 * memory is the caller's `workspace` of at least the size the matching
 * *_workspace_size function returns (0 is allowed when that size is 0).
 * Work is enqueued on `stream` (a hipStream_t, NULL = the default stream);
 * calls return without synchronising.  Concurrent calls are safe if they
 * use distinct workspaces and outputs.
 *
 * Errors: a status code is returned and a message is kept per thread
 * (attn_last_error).  Argument checks run on the host before anything is
 * launched and never read device memory.  Nothing aborts or prints.
 */
#ifndef ATTN36_H
#define ATTN36_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_EINVAL = 1,   /* bad argument: null pointer, bad shape, Hq % Hkv != 0,
                          window < -1, workspace too small, bad dtype */
    ATTN_ENOTSUP = 2,  /* valid request the kernels do not support: byte
                          offsets exceed 2^31, more than 128 q heads per kv head */
    ATTN_EHIP = 3      /* the HIP runtime reported an error at launch */
} attn_status;

typedef enum { ATTN_BF16 = 0, ATTN_FP16 = 1, ATTN_FP32 = 2 } attn_dtype;

typedef struct {
    int32_t dtype;          /* ATTN_BF16 or ATTN_FP16: q, k, v, o, dout */
    int32_t head_dim;       /* D: a multiple of 8 in [8, 256].  Kernels are built
                               64, 128 and 256 wide; a smaller head dim runs on
                               the next width up with zero columns, so it costs
                               what that width costs */
    int32_t heads_q;        /* Hq */
    int32_t heads_kv;       /* Hkv, divides Hq */
    float softmax_scale;    /* <= 0 or NaN selects 1/sqrt(D) */
    int32_t causal;         /* 0 or 1 */
    int32_t window_left;    /* >= -1; -1 = unbounded */
    int32_t window_right;   /* >= -1; -1 = unbounded */
    const float *sinks;     /* device fp32 sink logits or NULL: num_sinks per q
                               head, [Hq][num_sinks], or one row [num_sinks]
                               for all heads when sinks_shared = 1 */
    int32_t num_sinks;      /* sinks per q head, 0..64 (0 counts as 1) */
    int32_t sinks_shared;   /* 0 or 1, see sinks */
    float softcap;          /* >= 0; > 0 replaces each logit x (scale * q.k)
                               by softcap * tanh(x / softcap) */
    const float *alibi_slopes; /* device fp32 ALiBi slopes or NULL: [Hq], or
                               [batch][Hq] (packed: [num_seqs][Hq]) when
                               alibi_per_batch = 1; adds
                               -slope * |i + Lk - Lq - j| to the logit of
                               query i and key j, after the soft cap */
    int32_t alibi_per_batch; /* 0 or 1, see alibi_slopes */
    const int32_t *seqused_q; /* device int32 [B or num_seqs] or NULL: slot b uses its
                               first seqused_q[b] queries; the other rows' outputs,
                               lse and dq are unspecified (not written) */
    const int32_t *seqused_k; /* device int32 [B or num_seqs] or NULL: slot b uses its
                               first seqused_k[b] keys; the others are invisible and
                               their dk, dv are written as 0.  The causal/window band
                               aligns to the used lengths.  Contents are not checked
                               (like cu_seqlens); values outside [0, slot length] act
                               as the nearest bound.  attn_fwd_kvcache's
                               cache_seqlens replaces seqused_k */
} attn_params;

/*
 * Forward, batched [B,S,H,D].  Writes o (input dtype) and lse (fp32).
 * seqlen_q, seqlen_k >= 1, batch >= 1.  Decode-shaped calls (few query rows
 * per kv head, long seqlen_k) split the keys among workgroups and need
 * workspace; see attn_fwd_workspace_size.
 */
attn_status attn_fwd(const attn_params *params, int64_t batch, int64_t seqlen_q, int64_t seqlen_k,
                     const void *q, const void *k, const void *v, void *o, float *lse,
                     void *workspace, size_t workspace_bytes, void *stream);
size_t attn_fwd_workspace_size(const attn_params *params, int64_t batch, int64_t seqlen_q,
                               int64_t seqlen_k);

/*
 * Backward, batched.  Inputs are the forward's q, k, v, o and lse plus the
 * output gradient dout.  Writes dq [B,Sq,Hq,D], dk, dv [B,Sk,Hkv,D] as
 * grad_dtype (the input dtype, or ATTN_FP32 for fp32 gradients) and, when
 * params->sinks is set, dsinks (fp32, laid out like the sinks; must then be
 * non-NULL; heads that share a row of sinks add into it).
 * dK/dV of a kv head sum over the q heads that share it (fa4-jax page,
 * restrictions paragraph: fp32 accumulation across the q heads).
 * Numeric range: products accumulate in fp32.  The dK/dV pass holds Q, K and
 * dS in fp16 for bf16 inputs too (10 fraction bits, which dK's long sums
 * need): bf16 values of q and k are exact there up to |x| <= 65504 (beyond,
 * the results are not finite) and keep fewer bits below 6.1e-5 (fp16
 * subnormals); dS is scaled per key by a power of two chosen from
 * max |dO_i|_2 |v_j|_2 + max |D_i| and divided out again, so the magnitudes of
 * dout and v do not limit it.  dS for dQ is in the input dtype.
 */
attn_status attn_bwd(const attn_params *params, int64_t batch, int64_t seqlen_q, int64_t seqlen_k,
                     const void *q, const void *k, const void *v, const void *o, const float *lse,
                     const void *dout, void *dq, void *dk, void *dv, float *dsinks,
                     int32_t grad_dtype, void *workspace, size_t workspace_bytes, void *stream);
size_t attn_bwd_workspace_size(const attn_params *params, int64_t batch, int64_t seqlen_q,
                               int64_t seqlen_k, int32_t grad_dtype);

/*
 * Backward that allocates nothing: attn_bwd with the library's own fixed
 * device scratch in place of a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving or
 * training loops, harnesses that forbid hipMalloc).  Arguments, outputs and
 * results are attn_bwd's.  The scratch is a static device array of
 * ATTN_NOALLOC_SCRATCH_BYTES per GPU, held from the library's load on that
 * GPU until the process ends; its address is looked up on the first call on
 * each device (so make that first call before capturing a graph).  A call
 * needing more than ATTN_NOALLOC_SCRATCH_BYTES of workspace (what
 * attn_bwd_workspace_size returns: 8 bytes per query row and q head, plus
 * 4 bytes per q head and 128-row query block with sinks) returns ATTN_ENOTSUP
 * before anything is launched (8 bytes per 128 packed query rows per kv head
 * are added for the dS scaling statistics).  Nothing in the scratch needs clearing
 * between calls (every byte a call reads, that call's kernels wrote first),
 * but all calls on one GPU share it: calls that can overlap on one GPU (two
 * streams, two threads) race and must be ordered by the caller.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
attn_status attn_bwd_noalloc(const attn_params *params, int64_t batch, int64_t seqlen_q, int64_t seqlen_k,
                             const void *q, const void *k, const void *v, const void *o, const float *lse,
                             const void *dout, void *dq, void *dk, void *dv, float *dsinks,
                             int32_t grad_dtype, void *stream);

/*
 * Forward over a KV cache (decode / chunked prefill; forward only).  q is
 * [B, seqlen_q, Hq, D]; slot b of the cache holds cache_seqlens[b] valid keys
 * (device int32 [B]): later keys are invisible and the causal / window band
 * is aligned to that used length (fa4-jax page, varlen semantics paragraph:
 * seqused_k).  Without block_table, k_cache and v_cache are
 * [B, cache_capacity, Hkv, D].  With block_table (device int32
 * [B, max_blocks_per_seq]) they are pages [num_blocks, page_block_size, Hkv, D]
 * and key j of slot b is row j % page_block_size of page
 * block_table[b][j / page_block_size] (vllm-project/flash-attention README on
 * the GitHub search page, flash_attn_with_kvcache: paged KV cache;
 * page_block_size here: any positive multiple of 64, the page's 256
 * included).  cache_seqlens and block_table contents are NOT checked: each
 * cache_seqlens[b] must be within [0, capacity] (capacity = cache_capacity,
 * or max_blocks_per_seq * page_block_size), and every page a used key needs
 * must exist.  o, lse as in attn_fwd; workspace from
 * attn_fwd_kvcache_workspace_size with the same cache arguments
 * (cache_capacity is ignored when block_table is given).
 */
attn_status attn_fwd_kvcache(const attn_params *params, int64_t batch, int64_t seqlen_q, const void *q,
                             const void *k_cache, const void *v_cache, const int32_t *cache_seqlens,
                             const int32_t *block_table, int32_t max_blocks_per_seq,
                             int32_t page_block_size, int64_t cache_capacity, void *o, float *lse,
                             void *workspace, size_t workspace_bytes, void *stream);
size_t attn_fwd_kvcache_workspace_size(const attn_params *params, int64_t batch, int64_t seqlen_q,
                                       const int32_t *block_table, int32_t max_blocks_per_seq,
                                       int32_t page_block_size, int64_t cache_capacity);

/*
 * In-place KV-cache append (vllm-project/flash-attention README on the
 * GitHub search page, flash_attn_with_kvcache: k, v are written into the
 * cache starting at cache_seqlens, keys rotated by rotary_cos / rotary_sin
 * at their positions).  New token i of slot b (k_new, v_new
 * [batch, seqlen_new, Hkv, D], params->dtype) goes to key position
 * cache_seqlens[b] + i of the slot: row cache_seqlens[b] + i of
 * k_cache[b] ([batch, cache_capacity, Hkv, D]), or, with a block table, row
 * p % page_block_size of page block_table[b][p / page_block_size] (pages
 * [num_blocks, page_block_size, Hkv, D]).  With rotary_dim > 0 the keys are
 * rotated first (see attn_rotary); values are copied as they are.  Positions
 * past the slot (the capacity, or max_blocks_per_seq pages) are dropped: the
 * caller keeps the cache large enough.  When seqlens_out is non-NULL it
 * receives cache_seqlens[b] + seqlen_new after the append, in stream order,
 * so it may be cache_seqlens itself.  All pointers are device memory,
 * 16-byte aligned; cache_seqlens and block_table contents are not checked.
 * Errors: ATTN_EINVAL for NULL tensors, sizes < 1, a bad page or rotary
 * setting; ATTN_EHIP for a launch failure.
 */
attn_status attn_kvcache_append(const attn_params *params, int64_t batch, int64_t seqlen_new, const void *k_new,
                                const void *v_new, void *k_cache, void *v_cache, const int32_t *cache_seqlens,
                                int32_t *seqlens_out, const int32_t *block_table, int32_t max_blocks_per_seq,
                                int32_t page_block_size, int64_t cache_capacity, const float *rotary_cos,
                                const float *rotary_sin, int32_t rotary_dim, int32_t rotary_interleaved,
                                int64_t seqlen_ro, void *stream);

/*
 * Rotary embedding of x [batch, seqlen, heads, D] (params->dtype) into out
 * (same shape; may be x): token i of batch b sits at position
 * positions[b] + i (per_token = 1) or positions[b] (per_token = 0; the
 * non-causal, non-local query rule of flash_attn_with_kvcache).  The first
 * rotary_dim dims (a multiple of 16, at most D) form rotary_dim / 2 pairs --
 * dims (2j, 2j+1) when rotary_interleaved, else (j, j + rotary_dim / 2), the
 * GPT-NeoX form -- and pair j at position p becomes
 * (a cos - b sin, a sin + b cos) with cos = rotary_cos[p][j],
 * sin = rotary_sin[p][j] (fp32 [seqlen_ro, rotary_dim / 2]), in fp32 and
 * rounded to nearest even; the other dims are copied.  Positions past the
 * table use its last row (the caller keeps seqlen_ro large enough).
 * Errors: as attn_kvcache_append.
 */
attn_status attn_rotary(const attn_params *params, int64_t batch, int64_t seqlen, int32_t heads, const void *x,
                        void *out, const int32_t *positions, int32_t per_token, const float *rotary_cos,
                        const float *rotary_sin, int32_t rotary_dim, int32_t rotary_interleaved, int64_t seqlen_ro,
                        void *stream);

/*
 * Forward, packed [T,H,D] with device int32 cu_seqlens_q/k [num_seqs+1].
 * total_q / total_k are the token counts (cu_seqlens_*[num_seqs]);
 * max_seqlen_q / max_seqlen_k bound every sequence's length.  lse is fp32
 * [Hq, total_q].  The forward needs no workspace:
 * attn_fwd_varlen_workspace_size returns 0, and workspace may be NULL.
 */
attn_status attn_fwd_varlen(const attn_params *params, int32_t num_seqs, int64_t total_q,
                            int64_t total_k, const int32_t *cu_seqlens_q,
                            const int32_t *cu_seqlens_k, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, const void *q, const void *k, const void *v,
                            void *o, float *lse, void *workspace, size_t workspace_bytes,
                            void *stream);
size_t attn_fwd_varlen_workspace_size(const attn_params *params, int32_t num_seqs, int64_t total_q,
                                      int64_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k);

/*
 * Backward, packed.  Same arguments as attn_fwd_varlen plus o, lse (fp32
 * [Hq, total_q]), dout, and the outputs dq, dk, dv, dsinks as in attn_bwd.
 * When the dK/dV grid has 2048 workgroups or more, max_seqlen_q is 1024 or
 * more, and the batch fits the tables' limits (at most 16384 blocks per kv
 * head in either grid, 8191 sequences), a short extra launch first builds,
 * in the workspace, one table per grid (dQ and dK/dV, 4 bytes per
 * workgroup) that orders the grid's blocks by their work under the mask,
 * largest first, so that the longest blocks of the batch start first
 * wherever their sequences sit in it.  The results do not depend on the
 * order; attn_bwd_varlen_workspace_size includes the tables when they are
 * built.
 */
attn_status attn_bwd_varlen(const attn_params *params, int32_t num_seqs, int64_t total_q,
                            int64_t total_k, const int32_t *cu_seqlens_q,
                            const int32_t *cu_seqlens_k, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, const void *q, const void *k, const void *v,
                            const void *o, const float *lse, const void *dout, void *dq,
                            void *dk, void *dv, float *dsinks, int32_t grad_dtype,
                            void *workspace, size_t workspace_bytes, void *stream);
size_t attn_bwd_varlen_workspace_size(const attn_params *params, int32_t num_seqs,
                                      int64_t total_q, int64_t total_k, int32_t max_seqlen_q,
                                      int32_t max_seqlen_k, int32_t grad_dtype);

/*
 * Kernel timing, for profiling.  While enabled, every kernel the library
 * launches is bracketed by a pair of HIP events recorded on the caller's
 * stream.  attn_timing_read synchronises on the recorded events and returns,
 * for one kernel, the number of launches and their total duration in
 * milliseconds since the last attn_timing_enable call; it returns
 * ATTN_EINVAL for an unknown kernel id.  attn_timing_select limits the
 * timing to the kernels whose bit (1 << attn_kernel_id) is set in
 * kernel_mask (the others launch with no events around them; the default
 * mask times every kernel); it returns ATTN_EINVAL for bits past
 * ATTN_KERNEL_COUNT.  Not thread safe: enable, run, read from one thread.
 * At most 16384 launches are recorded per enable (later ones are not timed;
 * attn_timing_read then reports ATTN_ENOTSUP).
 */
typedef enum {
    ATTN_KERNEL_FWD = 0,          /* fused forward */
    ATTN_KERNEL_FWD_COMBINE = 1,  /* split-KV merge */
    ATTN_KERNEL_BWD_DSINK = 2,    /* sums the dQ workgroups' sink-gradient partials into dsinks */
    ATTN_KERNEL_BWD_DQ = 3,       /* query-major backward: row statistics, dsinks, dQ */
    ATTN_KERNEL_BWD_DKDV = 4,     /* key-major backward: dK, dV */
    ATTN_KERNEL_ORDER = 5,        /* packed calls: the grids' dispatch-order tables */
    ATTN_KERNEL_COUNT = 6
} attn_kernel_id;
attn_status attn_timing_enable(int32_t on);
attn_status attn_timing_select(uint32_t kernel_mask);
attn_status attn_timing_read(int32_t kernel, int64_t *launches, double *total_ms);

/* Message describing the last non-OK status returned on this thread. */
const char *attn_last_error(void);

/* Library version, 100 * major + minor. */
int32_t attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN36_H */
