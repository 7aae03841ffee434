/*
 * sparse_attn.h: C ABI of a block-sparse attention library for AMD Instinct
 * MI355X (gfx950) with block routing and a dropped-block residual.
 *
 * The operation (per batch entry b and head h, tokens [N, d]):
 *
 *  1. Routing.  Mean-pool queries over query blocks of block_q tokens and keys
 *     and values over key blocks of block_k tokens (the last block of each may
 *     be short; its mean is over its actual tokens).  Score every key block J
 *     for every query block I with the block proxy s_IJ = scale * qbar_I . kbar_J
 *     and keep J when the proxy clears tau (Sol-Attn abstract: blocks are
 *     selected by comparing block proxy scores against a threshold; block
 *     centroids as in the PARK page, section 4.1).  The compared quantity r_IJ
 *     is either the proxy probability relative to the row's largest one,
 *     exp(s_IJ - max_J' s_IJ') (SA_TAU_RELATIVE), or the proxy probability
 *     softmax_J(s_I.)_J itself (SA_TAU_ABSOLUTE).  SA_TAU_TOPP keeps instead
 *     the shortest prefix of the ranking whose proxy probability mass reaches
 *     1 - tau (cumulative-mass retention, the dynamic budget the Sol-Attn
 *     abstract contrasts with fixed ones).  A top-k budget caps the kept count
 *     at max_keep (rank by r descending, ties by J ascending); if fewer than
 *     min_keep clear tau, the min_keep best-ranked blocks are kept.
 *     Key blocks that start before n_dense_prefix tokens are always kept, and
 *     a query block that starts before n_dense_prefix keeps every key block.
 *     The proxy map is never written to memory; only its per-row maximum and
 *     log-sum-exp are.
 *     With SA_FLAG_PAMA the proxy is per-query attention-mass aggregation
 *     (PARK page, section 5.1): A_IJ = mean over the queries i of block I of
 *     softmax_J(scale * q_i . kbar_J), each original query normalised over
 *     the key-block means on its own before the average; the scores compared
 *     are then s_IJ = ln A_IJ (so the softmax of a row is A itself, and
 *     SA_TAU_TOPP retains PARK's cumulative importance).  Its logits carry
 *     fp32-level error (split bf16 products).  A PAMA workgroup takes
 *     Q = 256 (bf16) or 128 (fp32) queries, G = Q / block_q query blocks;
 *     supported while (4 + G) * n_kb + Q floats plus a 26 KB staging tile fit
 *     in 128 KB of LDS (n_kb <= 3248 for bf16 at block_q = 64, 4330 at 128;
 *     4352 and 5222 for fp32).
 *     With SA_FLAG_FUSED (pass it to both calls) routing is fused into the
 *     attention pass, the Sol-Attn abstract's single pass: sparse_attn_route
 *     only pools and writes the proxy rows' maximum and log-sum-exp, and the
 *     cost and work order of the decisions to come (no lists), and
 *     sparse_attn_forward takes each query block's decisions at the start of
 *     its work item from s_IJ and those statistics, writes them to kv_mask and
 *     kv_count, and attends in the work order.  The
 *     decisions are the τ test of RELATIVE or ABSOLUTE; max_keep must be 0,
 *     min_keep 0 or 1 (with 1, a row where no block clears tau keeps its block
 *     of largest proxy score, lowest J among equal ones), no PAMA,
 *     n_kb <= 16384.  The dense prefix applies as above.
 *
 *  2. Exact pass.  One online-softmax pass over the kept key blocks:
 *     logits scale * q_i . k_t for every token t of a kept block (Sol-Attn
 *     abstract: routing, sparse computation and correction in one
 *     online-softmax pass).
 *
 *  3. Residual.  Each dropped block J enters the same running max and
 *     normaliser as a single logit scale * q_i . kbar_J + ln n_J carrying the
 *     value vbar_J, i.e. n_J tokens with the block-mean key and value (Sol-Attn
 *     abstract: the proxy of unselected blocks approximates their
 *     contribution; the block-mean key gives a lower bound on the block's
 *     log-mass, PARK page, appendix D.2).
 *
 *     o_i = (sum_t e^{a_it - M} v_t + sum_J e^{b_iJ - M} vbar_J) / Z,
 *     lse_i = M + ln Z.
 *
 * Conventions shared by every entry point
 *  - Q, K, V, O are [B, H, N, d] contiguous with d fastest, in the dtype of
 *    sa_params.dtype (bf16 or fp32).  Products run on bf16 matrix cores with
 *    fp32 accumulation; fp32 inputs enter them as bf16 pairs (the rounded
 *    value and its remainder), the softmax weights as bf16.  Routing
 *    (pooling, proxy, threshold) is fp32 throughout.  Products whose softmax
 *    weights are all below 2^-32 of the running reference of every row of a
 *    32-row group (at least 2^-32 below the row's normaliser) are skipped:
 *    the value products of such a 32-key half of an exact tile, and the whole
 *    fold of such a residual group.  Their sum is below half of the
 *    normaliser's last fp32 bit.
 *  - One head's keys (N * d elements) must span at most 2^32 - 1 bytes; larger
 *    is SA_ERR_UNSUPPORTED.
 *  - Every tensor pointer is a DEVICE pointer (hipMalloc or equivalent) of the
 *    current HIP device, 16-byte aligned (hipMalloc and torch allocations are;
 *    the kernels move 16-byte vectors; lse and perm need 4 bytes).  A
 *    misaligned pointer is SA_ERR_INVALID_ARG.  The caller owns and frees all
 *    memory; the library allocates nothing, frees nothing and never
 *    synchronises.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued asynchronously on it; results are ready once the caller
 *    synchronises that stream.
 *  - Errors: arguments are validated on the host before anything is enqueued;
 *    a negative sa_status is returned and nothing runs.  A failed launch
 *    returns SA_ERR_HIP.  sparse_attn_last_error() gives a message for the
 *    last failure on the calling thread.  No exception crosses the ABI.
 *  - Deterministic: identical inputs give bitwise identical outputs.
 *  - Thread-safe; concurrent calls on distinct streams and distinct output
 *    buffers do not interact.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sa_status {
    SA_OK = 0,
    SA_ERR_INVALID_ARG = -1,   /* a parameter or pointer is invalid                 */
    SA_ERR_UNSUPPORTED = -2,   /* valid but not implemented (d, block size, n_kb)    */
    SA_ERR_CAPACITY = -3,      /* kv_idx_cap smaller than sparse_attn_kv_idx_cap()   */
    SA_ERR_HIP = -4            /* the HIP runtime reported an error                  */
} sa_status;

typedef enum sa_dtype { SA_BF16 = 0, SA_F32 = 1 } sa_dtype;

typedef enum sa_tau_mode {
    SA_TAU_RELATIVE = 0,       /* keep r >= tau, r = exp(s_IJ - max_J' s_IJ')        */
    SA_TAU_ABSOLUTE = 1,       /* keep r >= tau, r = softmax_J(s_I.)_J               */
    SA_TAU_TOPP = 2            /* keep ranking positions whose preceding proxy mass
                                  is < 1 - tau                                       */
} sa_tau_mode;

enum {
    SA_FLAG_NO_RESIDUAL = 1,   /* forward: dropped blocks contribute nothing         */
    SA_FLAG_PAMA = 2,          /* route: PAMA proxy instead of the centroid proxy    */
    SA_FLAG_FUSED = 4          /* fused routing: decisions taken inside the forward  */
};

/* Problem statement: B, H, N, d, block sizes, tau and budget. */
typedef struct sa_params {
    int32_t B, H, N, d;        /* N >= 1; d in {64, 128}                            */
    int32_t block_q, block_k;  /* each in {64, 128}; N need not be a multiple        */
    float   tau;               /* >= 0; 0 keeps every block; > 1 (TOPP: >= 1) keeps
                                  only the floor and the prefix                      */
    int32_t tau_mode;          /* sa_tau_mode                                        */
    int32_t max_keep;          /* top-k cap on kept blocks per query block, 0 = none */
    int32_t min_keep;          /* floor when fewer clear tau (clamped to n_kb)       */
    int32_t n_dense_prefix;    /* leading always-attended tokens, 0..N               */
    float   scale;             /* logit scale; 0 => 1/sqrt(d)                        */
    int32_t dtype;             /* sa_dtype of Q, K, V, O                             */
    int32_t flags;             /* SA_FLAG_*                                          */
} sa_params;

/* Buffers written by sparse_attn_route and read by sparse_attn_forward.  With
 * n_qb = ceil(N / block_q), n_kb = ceil(N / block_k), words = ceil(n_kb / 32),
 * W = B * H * n_qb.  All are device memory,
 * sized by sparse_attn_route_sizes() (entry i of its output is the byte size of
 * buffer i in the order below).  A route may serve several forward calls (mask
 * reuse across calls): forward takes the keep mask, kept lists and block means
 * from the route and reads q, k, v anew. */
enum {
    SA_BUF_KV_COUNT = 0,  /* int32 [B,H,n_qb]            kept key blocks per query block   */
    SA_BUF_KV_IDX,        /* int32 [B,H,n_qb,kv_idx_cap] kept key-block indices, ascending;
                                                         entries past kv_count are unspecified */
    SA_BUF_KV_MASK,       /* uint32 [B,H,n_qb,words]     bit J%32 of word J/32: J kept     */
    SA_BUF_Q_MEAN,        /* fp32 [B,H,n_qb,d]           query block means                  */
    SA_BUF_K_MEAN,        /* fp32 [B,H,n_kb,d]           key block means                    */
    SA_BUF_V_MEAN,        /* fp32 [B,H,n_kb,d]           value block means                  */
    SA_BUF_KV_SPLIT,      /* bf16 [B,H,2,words,64,d]     residual tiles: for each group of 32
                                                         key blocks, 32 rows of block means
                                                         rounded to bf16, then 32 rows of their
                                                         bf16 remainders (keys, then values);
                                                         rows past n_kb are zero; the forward
                                                         of bf16 inputs reads the value
                                                         remainders of no tile             */
    SA_BUF_ROW_STATS,     /* fp32 [B,H,n_qb,2]           max_J s_IJ and log-sum-exp_J s_IJ  */
    SA_BUF_COST,          /* int32 [B,H,n_qb]            key/value tiles the forward visits */
    SA_BUF_WORK_ORDER,    /* int32 [W]                   work items b*H*n_qb + h*n_qb + I
                                                         by cost band floor(log2(cost)),
                                                         highest band first, ascending item
                                                         within a band; when 12288 <= W
                                                         <= 49152, n_qb <= 2048 and B*H <=
                                                         1024, head-major instead: heads by total cost
                                                         (highest first, lower index on
                                                         ties), then band (highest first),
                                                         then I                             */
    SA_BUF_K_BOUNDS,      /* fp32 [B,H,words,2]          for each residual tile, upper
                                                         bounds on the Euclidean norms of
                                                         [0] its 32 key means as the forward
                                                         forms them (bf16 part plus
                                                         remainder) and [1] its 32 key-mean
                                                         remainder rows; the forward drops
                                                         a tile whose logits they prove
                                                         negligible, unloaded ([0]) or after
                                                         its bf16 part ([1]); written by
                                                         centroid routes only: a route under
                                                         SA_FLAG_PAMA leaves it unset and
                                                         the forward of such a route does
                                                         not read it                       */
    SA_ROUTE_NBUF
};

typedef struct sa_route {
    int32_t  *kv_count;
    int32_t  *kv_idx;
    uint32_t *kv_mask;
    float    *q_mean;
    float    *k_mean;
    float    *v_mean;
    void     *kv_split;
    float    *row_stats;
    int32_t  *cost;
    int32_t  *work_order;
    float    *k_bounds;
    int32_t   kv_idx_cap;     /* row length of kv_idx, >= sparse_attn_kv_idx_cap(p) */
} sa_route;

/* Smallest valid kv_idx_cap for p: n_kb when there is no cap or a dense prefix
 * row exists, else min(n_kb, max(max_keep, min_keep) + prefix key blocks).
 * Returns a negative sa_status when p is invalid.  Host only; no HIP calls. */
int32_t sparse_attn_kv_idx_cap(const sa_params *p);

/* Byte sizes of the SA_ROUTE_NBUF route buffers for p and kv_idx_cap, written
 * to bytes[0..SA_ROUTE_NBUF-1].  Host only; no HIP calls. */
sa_status sparse_attn_route_sizes(const sa_params *p, int32_t kv_idx_cap, size_t *bytes);

/* Step 1 (routing).  Reads q, k, v once; writes every buffer of *r (k_bounds
 * only without SA_FLAG_PAMA, which may then be NULL).  Nothing of size
 * n_qb x n_kb is written except the kv_idx lists and the bit mask. */
sa_status sparse_attn_route(const sa_params *p, const void *q, const void *k, const void *v,
                            const sa_route *r, void *stream);

/* Steps 2 and 3.  Writes o [B,H,N,d] (dtype of p) and, when lse is not NULL,
 * lse [B,H,N] fp32 (natural log).  r must come from sparse_attn_route with
 * the same p (only SA_FLAG_NO_RESIDUAL may differ) on the same k and v.  The
 * route buffers are not validated on the device: entries of another route
 * (out-of-range counts, block indices or work items) are clamped to the
 * buffers' ranges, so that such a misuse reads nothing outside q, k, v and the
 * route, but its output is meaningless. */
sa_status sparse_attn_forward(const sa_params *p, const void *q, const void *k, const void *v,
                              const sa_route *r, void *o, float *lse, void *stream);

/* Dense softmax attention with the same kernels and conventions (every key
 * block kept, no residual); tau, budget and prefix fields are ignored. */
sa_status sparse_attn_dense_ref_gpu(const sa_params *p, const void *q, const void *k,
                                    const void *v, void *o, float *lse, void *stream);

/* Probe-fitted residual correction (SparsePR summary, section B), a second way
 * to correct the sparse output under the same route, in place of the block
 * residual:
 *   1. O_s: attention over the kept tokens only;
 *   2. probes: probes_per_block rows per query block, evenly spread (row
 *      I*block_q + floor((j + 1/2) m_I / probes_per_block)), attended densely;
 *   3. per (b, h), R = O_dense - O_s at the probes is fitted as R ~ b + x B,
 *      x = O_s (ridge regression with an unpenalised intercept, ridge
 *      lam = ridge * trace(Xc^T Xc) / d on the centred probe outputs Xc), and
 *      the map is projected on the `rank` leading right singular vectors of R;
 *   4. o = O_s + (b + O_s B) Pk on every row that is not a probe, O_dense on
 *      probe rows.
 * Intermediates live in the caller's workspace, of the size
 * sparse_attn_sparsepr_workspace_size() gives (host only, no HIP calls).  It
 * starts with, each piece padded to a multiple of 256 bytes: the gathered
 * probe queries [B,H,M,d] in q's dtype (M = n_qb * probes_per_block), the
 * probes' dense outputs [B,H,M,d] fp32, then O_s [B,H,N,d] fp32 (readable
 * after the call, for inspection); then the Gram matrices, the fitted map (b Pk
 * and the factors B Q and Q of B Pk) and the probe pass's per-key-range
 * outputs, in fp32.
 * probes_per_block in [1, 16], rank in [1, min(16, d)], ridge >= 0; the route
 * must not be fused.  o has the layout and dtype of q.  The workspace must not
 * be shared by concurrent calls. */
sa_status sparse_attn_sparsepr_workspace_size(const sa_params *p, int32_t probes_per_block, size_t *bytes);
sa_status sparse_attn_forward_sparsepr(const sa_params *p, const void *q, const void *k, const void *v,
                                       const sa_route *r, int32_t probes_per_block, int32_t rank, float ridge,
                                       void *workspace, size_t workspace_bytes, void *o, void *stream);

/* sparse_attn_forward_sparsepr without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * that must not call hipMalloc, harnesses that forbid it).  It allocates
 * nothing: the intermediates live in a static device array of
 * SA_SPARSEPR_STATIC_WORKSPACE_BYTES per GPU, which the library holds from its
 * first use on that GPU until the process ends.  The computation is
 * sparse_attn_forward_sparsepr's (the same kernels); when the layout that call
 * would use does not fit, the probe pass takes fewer key ranges (a different
 * summation order of the probes' dense outputs, nothing else).  A call that
 * does not fit even then returns SA_ERR_CAPACITY before any launch (for
 * Wan-1.3B-sized heads, N = 32760 and d = 128, about 12 heads at
 * probes_per_block = 4).  Every call on one GPU uses that GPU's one array:
 * calls that overlap on one GPU (concurrent streams, or threads) race and must
 * be serialised by the caller; no part of the array needs to start at zero,
 * and what an earlier call left in it does not matter.  Arguments, errors and
 * o as for sparse_attn_forward_sparsepr. */
#define SA_SPARSEPR_STATIC_WORKSPACE_BYTES ((size_t)256 << 20)
sa_status sparse_attn_forward_sparsepr_static(const sa_params *p, const void *q, const void *k, const void *v,
                                              const sa_route *r, int32_t probes_per_block, int32_t rank,
                                              float ridge, void *o, void *stream);

/* Token reordering (DFSAttn abstract: tokens reordered along a 3D Hilbert curve
 * before blocking, so that a block of consecutive tokens is compact in space
 * and time).  The library orders a T x Hh x W video token grid and permutes
 * token rows of [B, H, N, d] tensors; a caller reorders Q, K and V, runs route
 * and forward, and restores the output order with the inverse permutation. */

#define SA_HILBERT_MAX_BITS 9       /* grid sides up to 512 */

/* Hilbert order of the grid: perm[i] = raster index t*Hh*W + y*W + x of the
 * token at curve position i.  The curve is J. Skilling's (AIP Conf. Proc. 707,
 * 2004) on the enclosing 2^b cube, b = ceil(log2(max side)) (at least 1), with
 * the index formed from the bit planes of (t, y, x), most significant first;
 * the grid's tokens keep the order of their positions on it.  perm: host
 * memory of T*Hh*W int32, owned by the caller.  Host only; no HIP calls.
 * Errors: SA_ERR_INVALID_ARG (NULL perm, a side < 1), SA_ERR_UNSUPPORTED (a
 * side above 2^SA_HILBERT_MAX_BITS). */
sa_status sparse_attn_hilbert_order(int32_t T, int32_t Hh, int32_t W, int32_t *perm);

/* Row permutation of a [B, H, N, d] tensor (d in {64, 128}, dtype an sa_dtype)
 * on rows [n0, n0 + n_perm) of every (b, h); other rows are copied unchanged.
 *   inverse = 0 (gather):  out[b,h,n0+i,:] = in[b,h,n0+perm[i],:]
 *   inverse = 1 (scatter): out[b,h,n0+perm[i],:] = in[b,h,n0+i,:]
 * so a scatter with perm undoes a gather with it.  in, out: device memory, not
 * the same buffer; perm: device memory of n_perm int32 holding a permutation
 * of [0, n_perm) (an entry outside that range skips its row, leaving that
 * output row as it was).  Enqueued on `stream`; reads and writes every row
 * once. */
sa_status sparse_attn_permute_tokens(int32_t B, int32_t H, int32_t N, int32_t d, int32_t dtype, int32_t n0,
                                     int32_t n_perm, const int32_t *perm, int32_t inverse, const void *in,
                                     void *out, void *stream);

/* Static description of a status code. */
const char *sparse_attn_status_string(sa_status s);

/* Message of the last failure on the calling thread ("" if none). */
const char *sparse_attn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_ATTN_H */
