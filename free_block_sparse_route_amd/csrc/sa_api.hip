// C ABI: argument validation, buffer sizing and kernel launches.  Nothing here
// allocates, frees or synchronises; every launch goes to the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "sa_internal.h"
#include "sparse_attn.h"

// Workspace of the allocation-free probe-fitted entry point
// (sparse_attn_forward_sparsepr_static): one array per device, held until the
// process ends.  In host code its name is only a handle for the runtime; the
// device address of each GPU's copy comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[SA_SPARSEPR_STATIC_WORKSPACE_BYTES];

namespace {

thread_local char g_err[512] = "";

sa_status fail(sa_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
sa_status fail(sa_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

sa_status hip_fail(hipError_t e, const char *where) {
    return fail(SA_ERR_HIP, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
}

struct Dims {
    int n_qb, n_kb, words;
    int64_t BH;
};

Dims dims_of(const sa_params *p) {
    Dims d;
    d.n_qb = (p->N + p->block_q - 1) / p->block_q;
    d.n_kb = (p->N + p->block_k - 1) / p->block_k;
    d.words = (d.n_kb + 31) / 32;
    d.BH = (int64_t)p->B * p->H;
    return d;
}

// Parameter checks common to every entry point.  `routing` adds the checks of
// the routing fields.
sa_status check_params(const sa_params *p, bool routing) {
    if (!p) return fail(SA_ERR_INVALID_ARG, "params is NULL");
    if (p->B < 1 || p->H < 1 || p->N < 1)
        return fail(SA_ERR_INVALID_ARG, "B, H, N must be >= 1 (got %d, %d, %d)", p->B, p->H, p->N);
    if (p->d < 1) return fail(SA_ERR_INVALID_ARG, "d must be >= 1 (got %d)", p->d);
    if (p->block_q < 1 || p->block_k < 1)
        return fail(SA_ERR_INVALID_ARG, "block sizes must be >= 1 (got %d, %d)", p->block_q, p->block_k);
    if (p->dtype != SA_BF16 && p->dtype != SA_F32)
        return fail(SA_ERR_INVALID_ARG, "dtype %d is not an sa_dtype", p->dtype);
    if (!(p->scale >= 0.f) || isinf(p->scale))
        return fail(SA_ERR_INVALID_ARG, "scale must be finite and >= 0");
    if (p->flags & ~(SA_FLAG_NO_RESIDUAL | SA_FLAG_PAMA | SA_FLAG_FUSED))
        return fail(SA_ERR_INVALID_ARG, "unknown flag bits 0x%x", p->flags);
    const int64_t elems = (int64_t)p->B * p->H * p->N * p->d;
    if (elems > ((int64_t)1 << 40)) return fail(SA_ERR_INVALID_ARG, "tensor too large");
    if (routing) {
        if (!(p->tau >= 0.f)) return fail(SA_ERR_INVALID_ARG, "tau must be >= 0 and not NaN");
        if (p->tau_mode != SA_TAU_RELATIVE && p->tau_mode != SA_TAU_ABSOLUTE && p->tau_mode != SA_TAU_TOPP)
            return fail(SA_ERR_INVALID_ARG, "tau_mode %d is not an sa_tau_mode", p->tau_mode);
        if (p->max_keep < 0 || p->min_keep < 0)
            return fail(SA_ERR_INVALID_ARG, "max_keep and min_keep must be >= 0");
        if (p->n_dense_prefix < 0 || p->n_dense_prefix > p->N)
            return fail(SA_ERR_INVALID_ARG, "n_dense_prefix must be in [0, N]");
    }
    if (p->d != 64 && p->d != 128) return fail(SA_ERR_UNSUPPORTED, "d = %d (supported: 64, 128)", p->d);
    if ((p->block_q != 64 && p->block_q != 128) || (p->block_k != 64 && p->block_k != 128))
        return fail(SA_ERR_UNSUPPORTED, "block sizes %d x %d (supported: 64 or 128 each)", p->block_q,
                    p->block_k);
    // the attention kernels address one head's keys and values through a buffer
    // resource whose byte range is 32 bits wide
    const int64_t head_bytes = (int64_t)p->N * p->d * (p->dtype == SA_BF16 ? 2 : 4);
    if (head_bytes > (int64_t)UINT32_MAX)
        return fail(SA_ERR_UNSUPPORTED, "N * d * element size = %lld bytes per head exceeds 2^32 - 1",
                    (long long)head_bytes);
    const Dims d = dims_of(p);
    if (routing && d.n_kb > sa::kMaxKeyBlocks)
        return fail(SA_ERR_UNSUPPORTED, "n_kb = %d exceeds %d", d.n_kb, sa::kMaxKeyBlocks);
    if (routing && (p->flags & SA_FLAG_FUSED)) {
        // the decision of a block depends only on its own proxy and the row's
        // statistics (plus, for a floor of one block, the row's best block):
        // no cap, no ranking-based mode, no floor above one block
        if (p->flags & SA_FLAG_PAMA) return fail(SA_ERR_UNSUPPORTED, "fused routing with the PAMA proxy");
        if (p->tau_mode == SA_TAU_TOPP) return fail(SA_ERR_UNSUPPORTED, "fused routing with SA_TAU_TOPP");
        if (p->max_keep != 0) return fail(SA_ERR_UNSUPPORTED, "fused routing with max_keep");
        if (p->min_keep > 1) return fail(SA_ERR_UNSUPPORTED, "fused routing with min_keep = %d (at most 1)", p->min_keep);
        if (d.words > sa::kFusedMaxWords) return fail(SA_ERR_UNSUPPORTED, "fused routing: n_kb = %d too large", d.n_kb);
    }
    if (routing && (p->flags & SA_FLAG_PAMA) && sa::pama_lds_bytes(d.n_kb, p->block_q, p->dtype) > sa::kPamaLdsBudget)
        return fail(SA_ERR_UNSUPPORTED, "PAMA proxy: n_kb = %d too large for block_q = %d", d.n_kb, p->block_q);
    if (d.BH * d.n_qb > INT32_MAX / 2) return fail(SA_ERR_UNSUPPORTED, "too many work items");
    return SA_OK;
}

int32_t min_cap(const sa_params *p) {
    const Dims d = dims_of(p);
    // no cap, or a dense prefix (query block 0 then keeps every key block)
    if (p->max_keep == 0 || p->n_dense_prefix > 0) return d.n_kb;
    const int32_t floor_n = p->min_keep < d.n_kb ? p->min_keep : d.n_kb;
    const int32_t lim = p->max_keep > floor_n ? p->max_keep : floor_n;
    return lim < d.n_kb ? lim : d.n_kb;
}

// Host pointers (the route descriptor): not NULL.
sa_status check_host_ptr(const void *ptr, const char *name) {
    if (!ptr) return fail(SA_ERR_INVALID_ARG, "%s is NULL", name);
    return SA_OK;
}

// Device pointers: not NULL, 16-byte aligned (the kernels move 16-byte vectors).
sa_status check_ptr(const void *ptr, const char *name) {
    if (!ptr) return fail(SA_ERR_INVALID_ARG, "%s is NULL", name);
    if ((uintptr_t)ptr % 16 != 0) return fail(SA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return SA_OK;
}

}  // namespace

extern "C" {

int32_t sparse_attn_kv_idx_cap(const sa_params *p) {
    const sa_status s = check_params(p, true);
    if (s != SA_OK) return (int32_t)s;
    return min_cap(p);
}

sa_status sparse_attn_route_sizes(const sa_params *p, int32_t kv_idx_cap, size_t *bytes) {
    sa_status s = check_params(p, true);
    if (s != SA_OK) return s;
    if (!bytes) return fail(SA_ERR_INVALID_ARG, "bytes is NULL");
    if (kv_idx_cap < min_cap(p))
        return fail(SA_ERR_CAPACITY, "kv_idx_cap %d < required %d", kv_idx_cap, min_cap(p));
    const Dims d = dims_of(p);
    const size_t rows = (size_t)d.BH * d.n_qb;
    bytes[SA_BUF_KV_COUNT] = rows * 4;
    bytes[SA_BUF_KV_IDX] = rows * (size_t)kv_idx_cap * 4;
    bytes[SA_BUF_KV_MASK] = rows * (size_t)d.words * 4;
    bytes[SA_BUF_Q_MEAN] = rows * (size_t)p->d * 4;
    bytes[SA_BUF_K_MEAN] = (size_t)d.BH * d.n_kb * p->d * 4;
    bytes[SA_BUF_V_MEAN] = (size_t)d.BH * d.n_kb * p->d * 4;
    bytes[SA_BUF_KV_SPLIT] = (size_t)d.BH * 2 * d.words * 64 * p->d * 2;
    bytes[SA_BUF_ROW_STATS] = rows * 2 * 4;
    bytes[SA_BUF_COST] = rows * 4;
    bytes[SA_BUF_WORK_ORDER] = rows * 4;
    bytes[SA_BUF_K_BOUNDS] = (size_t)d.BH * d.words * 2 * 4;
    return SA_OK;
}

sa_status sparse_attn_route(const sa_params *p, const void *q, const void *k, const void *v,
                            const sa_route *r, void *stream) {
    sa_status s = check_params(p, true);
    if (s != SA_OK) return s;
    if ((s = check_ptr(q, "q")) || (s = check_ptr(k, "k")) || (s = check_ptr(v, "v")) ||
        (s = check_host_ptr(r, "route")))
        return s;
    if ((s = check_ptr(r->kv_count, "route.kv_count")) || (s = check_ptr(r->kv_idx, "route.kv_idx")) ||
        (s = check_ptr(r->kv_mask, "route.kv_mask")) || (s = check_ptr(r->q_mean, "route.q_mean")) ||
        (s = check_ptr(r->k_mean, "route.k_mean")) || (s = check_ptr(r->v_mean, "route.v_mean")) ||
        (s = check_ptr(r->kv_split, "route.kv_split")) || (s = check_ptr(r->row_stats, "route.row_stats")) || (s = check_ptr(r->cost, "route.cost")) ||
        (s = check_ptr(r->work_order, "route.work_order")) ||
        (!(p->flags & SA_FLAG_PAMA) && (s = check_ptr(r->k_bounds, "route.k_bounds"))))
        return s;
    if (r->kv_idx_cap < min_cap(p))
        return fail(SA_ERR_CAPACITY, "route.kv_idx_cap %d < required %d", r->kv_idx_cap, min_cap(p));
    const Dims d = dims_of(p);
    hipStream_t st = (hipStream_t)stream;

    sa::PoolArgs pa;
    pa.N = p->N; pa.block_q = p->block_q; pa.block_k = p->block_k;
    pa.n_qb = d.n_qb; pa.n_kb = d.n_kb;
    pa.q_mean = r->q_mean; pa.k_mean = r->k_mean; pa.v_mean = r->v_mean;
    pa.kv_split = (sa::bf16 *)r->kv_split; pa.words = d.words;
    // the select kernel pools the query blocks itself, except under the PAMA
    // proxy, whose kernel reads Q row by row
    pa.first = (p->flags & SA_FLAG_PAMA) ? 0 : 1;
    hipError_t e = sa::launch_pool(p->dtype, p->d, q, k, v, pa, (int)d.BH, st);
    if (e != hipSuccess) return hip_fail(e, "route: pool launch");

    sa::SelectArgs sa_;
    sa_.N = p->N; sa_.block_q = p->block_q; sa_.block_k = p->block_k;
    sa_.n_qb = d.n_qb; sa_.n_kb = d.n_kb; sa_.mask_words = d.words; sa_.kv_idx_cap = r->kv_idx_cap;
    sa_.exact_tile_rows = p->dtype == SA_BF16 ? 64 : 32;
    sa_.tau_mode = p->tau_mode; sa_.max_keep = p->max_keep; sa_.min_keep = p->min_keep;
    sa_.n_prefix = p->n_dense_prefix;
    sa_.scale = p->scale > 0.f ? p->scale : (float)(1.0 / sqrt((double)p->d));
    sa_.ln_tau = p->tau > 0.f ? (float)log((double)p->tau) : -INFINITY;
    sa_.topp_target = 1.f - p->tau;
    sa_.stats_only = (p->flags & SA_FLAG_FUSED) ? 1 : 0;
    sa_.q = q; sa_.q_bf16 = p->dtype == SA_BF16 ? 1 : 0;
    sa_.q_mean = r->q_mean; sa_.k_mean = r->k_mean;
    sa_.kv_count = r->kv_count; sa_.kv_idx = r->kv_idx; sa_.cost = r->cost;
    sa_.work_order = r->work_order; sa_.kv_mask = r->kv_mask;
    sa_.row_stats = r->row_stats;
    sa_.kv_split = (const sa::bf16 *)r->kv_split;
    sa_.k_bounds = r->k_bounds;
    e = sa::launch_select(p->d, sa_, (int)d.BH, st, p->dtype, (p->flags & SA_FLAG_PAMA) ? q : nullptr);
    if (e != hipSuccess) return hip_fail(e, "route: select launch");
    return SA_OK;
}

static sa_status run_flash(const sa_params *p, const void *q, const void *k, const void *v,
                           const sa_route *r, void *o, float *lse, void *stream, const char *who,
                           float *o32 = nullptr, bool no_residual = false) {
    const Dims d = dims_of(p);
    sa::FlashArgs fa;
    memset(&fa, 0, sizeof fa);
    fa.N = p->N; fa.Nq = p->N; fa.block_q = p->block_q; fa.block_k = p->block_k;
    fa.n_qb = d.n_qb; fa.n_kb = d.n_kb; fa.mask_words = d.words;
    const double scale = p->scale > 0.f ? (double)p->scale : 1.0 / sqrt((double)p->d);
    fa.scale_log2 = (float)(scale * 1.4426950408889634);
    fa.lse = lse;
    fa.o32 = o32;
    if (r) {
        fa.kv_idx_cap = r->kv_idx_cap;
        fa.residual = ((p->flags & SA_FLAG_NO_RESIDUAL) || no_residual) ? 0 : 1;
        // the residual-tile norm bounds of a centroid route (a PAMA route has none)
        fa.k_bounds = (fa.residual && !(p->flags & SA_FLAG_PAMA)) ? r->k_bounds : nullptr;
        fa.kv_count = r->kv_count; fa.kv_idx = r->kv_idx; fa.work_order = r->work_order;
        fa.kv_mask = r->kv_mask; fa.kv_split = (const sa::bf16 *)r->kv_split;
        if (p->flags & SA_FLAG_FUSED) {
            fa.kv_idx = nullptr;
            fa.kv_mask_out = r->kv_mask;
            fa.kv_count_out = r->kv_count;
            fa.q_mean = r->q_mean;
            fa.k_mean = r->k_mean;
            fa.row_stats = r->row_stats;
            fa.tau_mode = p->tau_mode;
            fa.n_prefix = p->n_dense_prefix;
            fa.min_keep = p->min_keep;
            fa.scale = (float)scale;
            fa.ln_tau = p->tau > 0.f ? (float)log((double)p->tau) : -INFINITY;
        }
    }
    hipError_t e = sa::launch_flash(p->dtype, p->d, p->block_q, q, k, v, o, fa, (int)d.BH,
                                    (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, who);
    return SA_OK;
}

sa_status sparse_attn_forward(const sa_params *p, const void *q, const void *k, const void *v,
                              const sa_route *r, void *o, float *lse, void *stream) {
    sa_status s = check_params(p, true);
    if (s != SA_OK) return s;
    if ((s = check_ptr(q, "q")) || (s = check_ptr(k, "k")) || (s = check_ptr(v, "v")) ||
        (s = check_ptr(o, "o")) || (s = check_host_ptr(r, "route")))
        return s;
    if ((s = check_ptr(r->kv_count, "route.kv_count")) || (s = check_ptr(r->kv_idx, "route.kv_idx")) ||
        (s = check_ptr(r->kv_mask, "route.kv_mask")) ||
        (s = check_ptr(r->kv_split, "route.kv_split")) ||
        (s = check_ptr(r->work_order, "route.work_order")) ||
        (!(p->flags & (SA_FLAG_PAMA | SA_FLAG_NO_RESIDUAL)) && (s = check_ptr(r->k_bounds, "route.k_bounds"))))
        return s;
    if ((p->flags & SA_FLAG_FUSED) &&
        ((s = check_ptr(r->q_mean, "route.q_mean")) || (s = check_ptr(r->k_mean, "route.k_mean")) ||
         (s = check_ptr(r->row_stats, "route.row_stats"))))
        return s;
    if (r->kv_idx_cap < min_cap(p))
        return fail(SA_ERR_CAPACITY, "route.kv_idx_cap %d < required %d", r->kv_idx_cap, min_cap(p));
    return run_flash(p, q, k, v, r, o, lse, stream, "forward: launch");
}

sa_status sparse_attn_dense_ref_gpu(const sa_params *p, const void *q, const void *k, const void *v,
                                    void *o, float *lse, void *stream) {
    sa_status s = check_params(p, false);
    if (s != SA_OK) return s;
    if ((s = check_ptr(q, "q")) || (s = check_ptr(k, "k")) || (s = check_ptr(v, "v")) ||
        (s = check_ptr(o, "o")))
        return s;
    return run_flash(p, q, k, v, nullptr, o, lse, stream, "dense: launch");
}

sa_status sparse_attn_hilbert_order(int32_t T, int32_t Hh, int32_t W, int32_t *perm) {
    if (!perm) return fail(SA_ERR_INVALID_ARG, "perm is NULL");
    if (T < 1 || Hh < 1 || W < 1) return fail(SA_ERR_INVALID_ARG, "grid %d x %d x %d: sides must be >= 1", T, Hh, W);
    int b = 1;
    const int side = T > Hh ? (T > W ? T : W) : (Hh > W ? Hh : W);
    while ((1 << b) < side) ++b;
    if (b > SA_HILBERT_MAX_BITS)
        return fail(SA_ERR_UNSUPPORTED, "grid side %d exceeds %d", side, 1 << SA_HILBERT_MAX_BITS);
    const int64_t n = sa::hilbert_fill(T, Hh, W, b, perm);
    if (n != (int64_t)T * Hh * W) return fail(SA_ERR_INVALID_ARG, "internal: %lld points", (long long)n);
    return SA_OK;
}

sa_status sparse_attn_permute_tokens(int32_t B, int32_t H, int32_t N, int32_t d, int32_t dtype, int32_t n0,
                                     int32_t n_perm, const int32_t *perm, int32_t inverse, const void *in,
                                     void *out, void *stream) {
    if (B < 1 || H < 1 || N < 1) return fail(SA_ERR_INVALID_ARG, "B, H, N must be >= 1 (got %d, %d, %d)", B, H, N);
    if (dtype != SA_BF16 && dtype != SA_F32) return fail(SA_ERR_INVALID_ARG, "dtype %d is not an sa_dtype", dtype);
    if (d != 64 && d != 128) return fail(SA_ERR_UNSUPPORTED, "d = %d (supported: 64, 128)", d);
    if (n0 < 0 || n_perm < 0 || (int64_t)n0 + n_perm > N)
        return fail(SA_ERR_INVALID_ARG, "rows [%d, %d + %d) outside [0, %d)", n0, n0, n_perm, N);
    if (inverse != 0 && inverse != 1) return fail(SA_ERR_INVALID_ARG, "inverse must be 0 or 1");
    sa_status s;
    if ((s = check_ptr(in, "in")) || (s = check_ptr(out, "out"))) return s;
    if (in == out) return fail(SA_ERR_INVALID_ARG, "in and out must not be the same buffer");
    if (n_perm > 0 && !perm) return fail(SA_ERR_INVALID_ARG, "perm is NULL");
    if ((int64_t)B * H * N * d > ((int64_t)1 << 40)) return fail(SA_ERR_INVALID_ARG, "tensor too large");
    if ((int64_t)B * H > 65535) return fail(SA_ERR_UNSUPPORTED, "B * H = %lld exceeds 65535", (long long)B * H);
    sa::PermuteArgs a;
    a.N = N;
    a.units = d * (dtype == SA_BF16 ? 2 : 4) / 16;
    a.n0 = n0;
    a.n_perm = n_perm;
    a.inverse = inverse;
    hipError_t e = sa::launch_permute(in, out, perm, a, B * H, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "permute: launch");
    return SA_OK;
}

// Probe-fitted residual: workspace pieces, each 256-byte aligned.
namespace {
struct PrLayout {
    size_t qp, od32, o32, scratch, part, cmean, cb_mat, cb_vec, osplit, lsplit, total;
    int M, n_chunks, kv_splits;
};
// limit_bytes > 0: fewer key ranges for the probe pass (down to one) while the
// workspace would exceed limit_bytes; the caller checks L.total against it.
PrLayout pr_layout(const sa_params *p, int per_block, size_t limit_bytes = 0) {
    const Dims d = dims_of(p);
    const size_t es = p->dtype == SA_BF16 ? 2 : 4;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    PrLayout L;
    L.M = d.n_qb * per_block;
    const size_t BH = (size_t)d.BH, D = (size_t)p->d;
    size_t off = 0;
    L.qp = off; off += up(BH * L.M * D * es);
    L.od32 = off; off += up(BH * L.M * D * 4);
    L.o32 = off; off += up(BH * (size_t)p->N * D * 4);
    L.scratch = off; off += up(BH * 3 * D * D * 4);
    L.n_chunks = (L.M + sa::kPrChunk - 1) / sa::kPrChunk;
    L.part = off; off += up(BH * L.n_chunks * 3 * D * D * 4);
    L.cmean = off; off += up(BH * L.n_chunks * 2 * D * 4);
    L.cb_mat = off; off += up(BH * D * D * 4);
    L.cb_vec = off; off += up(BH * D * 4);
    // The probe pass has few query blocks (P per block_q query rows): its key
    // tiles are split into ranges so that about 2048 workgroups run, each range
    // at least 8 tiles, at most 32 ranges; the ranges' outputs are merged.
    {
        const int64_t items = (int64_t)BH * ((L.M + p->block_q - 1) / p->block_q);
        const int64_t tiles = (p->N + (p->dtype == SA_BF16 ? 64 : 32) - 1) / (p->dtype == SA_BF16 ? 64 : 32);
        int64_t S = (2048 + items - 1) / items;
        S = S < 32 ? S : 32;
        S = S < tiles / 8 ? S : tiles / 8;
        L.kv_splits = S > 1 ? (int)S : 1;
    }
    const size_t fixed = off;
    for (;;) {
        off = fixed;
        L.osplit = off;
        if (L.kv_splits > 1) off += up((size_t)L.kv_splits * BH * L.M * D * 4);
        L.lsplit = off;
        if (L.kv_splits > 1) off += up((size_t)L.kv_splits * BH * L.M * 4);
        L.total = off;
        if (limit_bytes == 0 || L.total <= limit_bytes || L.kv_splits == 1) break;
        --L.kv_splits;
    }
    return L;
}

sa_status check_pr(const sa_params *p, int32_t per_block, int32_t rank, float ridge) {
    if (per_block < 1 || per_block > sa::kPrMaxPerBlock)
        return fail(SA_ERR_INVALID_ARG, "probes_per_block %d outside [1, %d]", per_block, sa::kPrMaxPerBlock);
    const int rmax = sa::kPrMaxRank < p->d ? sa::kPrMaxRank : p->d;
    if (rank < 1 || rank > rmax) return fail(SA_ERR_INVALID_ARG, "rank %d outside [1, %d]", rank, rmax);
    if (!(ridge >= 0.f) || isinf(ridge)) return fail(SA_ERR_INVALID_ARG, "ridge must be finite and >= 0");
    if (p->flags & SA_FLAG_FUSED) return fail(SA_ERR_UNSUPPORTED, "probe-fitted residual after fused routing");
    if (dims_of(p).n_qb * per_block < 2) return fail(SA_ERR_INVALID_ARG, "fewer than 2 probe rows");
    return SA_OK;
}
}  // namespace

sa_status sparse_attn_sparsepr_workspace_size(const sa_params *p, int32_t probes_per_block, size_t *bytes) {
    sa_status s = check_params(p, true);
    if (s != SA_OK) return s;
    if (!bytes) return fail(SA_ERR_INVALID_ARG, "bytes is NULL");
    if (probes_per_block < 1 || probes_per_block > sa::kPrMaxPerBlock)
        return fail(SA_ERR_INVALID_ARG, "probes_per_block %d outside [1, %d]", probes_per_block, sa::kPrMaxPerBlock);
    *bytes = pr_layout(p, probes_per_block).total;
    return SA_OK;
}

namespace {
// Argument checks of the probe-fitted residual entry points (the workspace aside).
sa_status check_sparsepr_call(const sa_params *p, const void *q, const void *k, const void *v, const sa_route *r,
                              int32_t probes_per_block, int32_t rank, float ridge, const void *o) {
    sa_status s = check_params(p, true);
    if (s != SA_OK) return s;
    if ((s = check_pr(p, probes_per_block, rank, ridge)) != SA_OK) return s;
    if ((s = check_ptr(q, "q")) || (s = check_ptr(k, "k")) || (s = check_ptr(v, "v")) ||
        (s = check_ptr(o, "o")) || (s = check_host_ptr(r, "route")))
        return s;
    if ((s = check_ptr(r->kv_count, "route.kv_count")) || (s = check_ptr(r->kv_idx, "route.kv_idx")) ||
        (s = check_ptr(r->kv_mask, "route.kv_mask")) || (s = check_ptr(r->kv_split, "route.kv_split")) ||
        (s = check_ptr(r->work_order, "route.work_order")))
        return s;
    if (r->kv_idx_cap < min_cap(p))
        return fail(SA_ERR_CAPACITY, "route.kv_idx_cap %d < required %d", r->kv_idx_cap, min_cap(p));
    return SA_OK;
}

// The probe-fitted residual's launches on a workspace laid out as L.
sa_status run_sparsepr(const sa_params *p, const void *q, const void *k, const void *v, const sa_route *r,
                       int32_t probes_per_block, int32_t rank, float ridge, const PrLayout &L, void *workspace,
                       void *o, void *stream) {
    sa_status s;
    const Dims d = dims_of(p);
    hipStream_t st = (hipStream_t)stream;
    unsigned char *ws = (unsigned char *)workspace;
    sa::PrArgs a;
    a.N = p->N; a.M = L.M; a.per_block = probes_per_block; a.block_q = p->block_q; a.rank = rank; a.ridge = ridge;
    a.O32 = (const float *)(ws + L.o32);
    a.Od32 = (const float *)(ws + L.od32);
    a.scratch = (float *)(ws + L.scratch);
    a.n_chunks = L.n_chunks;
    a.part = (float *)(ws + L.part);
    a.cmean = (float *)(ws + L.cmean);
    a.CB = (float *)(ws + L.cb_mat);
    a.kv_splits = L.kv_splits;
    a.Osplit = (const float *)(ws + L.osplit);
    a.Lsplit = (const float *)(ws + L.lsplit);
    a.Cb = (float *)(ws + L.cb_vec);
    // 1. sparse output over the kept tokens only, fp32
    if ((s = run_flash(p, q, k, v, r, nullptr, nullptr, stream, "sparsepr: sparse pass", (float *)(ws + L.o32),
                       true)) != SA_OK)
        return s;
    // 2. probe queries, gathered, attended densely in fp32
    hipError_t e = sa::launch_sparsepr_step(0, p->dtype, p->d, q, ws + L.qp, nullptr, a, (int)d.BH, st);
    if (e != hipSuccess) return hip_fail(e, "sparsepr: gather launch");
    sa::FlashArgs fa;
    memset(&fa, 0, sizeof fa);
    fa.N = p->N; fa.Nq = L.M; fa.block_q = p->block_q; fa.block_k = p->block_k;
    fa.n_qb = (L.M + p->block_q - 1) / p->block_q; fa.n_kb = d.n_kb; fa.mask_words = d.words;
    const double scale = p->scale > 0.f ? (double)p->scale : 1.0 / sqrt((double)p->d);
    fa.scale_log2 = (float)(scale * 1.4426950408889634);
    if (L.kv_splits > 1) {
        fa.kv_splits = L.kv_splits;
        fa.o32 = (float *)(ws + L.osplit);
        fa.lse = (float *)(ws + L.lsplit);
        fa.split_o = d.BH * (size_t)L.M * p->d;
        fa.split_l = d.BH * (size_t)L.M;
    } else {
        fa.o32 = (float *)(ws + L.od32);
    }
    e = sa::launch_flash(p->dtype, p->d, p->block_q, ws + L.qp, k, v, nullptr, fa, (int)d.BH, st);
    if (e != hipSuccess) return hip_fail(e, "sparsepr: probe pass launch");
    if (L.kv_splits > 1) {
        e = sa::launch_sparsepr_step(3, p->dtype, p->d, nullptr, nullptr, nullptr, a, (int)d.BH, st);
        if (e != hipSuccess) return hip_fail(e, "sparsepr: probe merge launch");
    }
    // 3. fit, 4. apply
    e = sa::launch_sparsepr_step(1, p->dtype, p->d, nullptr, nullptr, nullptr, a, (int)d.BH, st);
    if (e != hipSuccess) return hip_fail(e, "sparsepr: fit launch");
    e = sa::launch_sparsepr_step(2, p->dtype, p->d, nullptr, nullptr, o, a, (int)d.BH, st);
    if (e != hipSuccess) return hip_fail(e, "sparsepr: apply launch");
    return SA_OK;
}

constexpr size_t kStaticScratchBytes = SA_SPARSEPR_STATIC_WORKSPACE_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (looked up once per
// device, with that device current).
sa_status scratch_of_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "sparsepr (static workspace): hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(SA_ERR_UNSUPPORTED, "device ordinal %d >= %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "sparsepr (static workspace): hipGetSymbolAddress");
        if (!ptr || (uintptr_t)ptr % 256 != 0) return fail(SA_ERR_HIP, "sparsepr (static workspace): bad address");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SA_OK;
}
}  // namespace

sa_status sparse_attn_forward_sparsepr(const sa_params *p, const void *q, const void *k, const void *v,
                                       const sa_route *r, int32_t probes_per_block, int32_t rank, float ridge,
                                       void *workspace, size_t workspace_bytes, void *o, void *stream) {
    sa_status s = check_sparsepr_call(p, q, k, v, r, probes_per_block, rank, ridge, o);
    if (s != SA_OK) return s;
    if ((s = check_ptr(workspace, "workspace")) != SA_OK) return s;
    const PrLayout L = pr_layout(p, probes_per_block);
    if (workspace_bytes < L.total)
        return fail(SA_ERR_CAPACITY, "workspace %zu bytes < required %zu", workspace_bytes, L.total);
    return run_sparsepr(p, q, k, v, r, probes_per_block, rank, ridge, L, workspace, o, stream);
}

sa_status sparse_attn_forward_sparsepr_static(const sa_params *p, const void *q, const void *k, const void *v,
                                              const sa_route *r, int32_t probes_per_block, int32_t rank,
                                              float ridge, void *o, void *stream) {
    sa_status s = check_sparsepr_call(p, q, k, v, r, probes_per_block, rank, ridge, o);
    if (s != SA_OK) return s;
    const PrLayout L = pr_layout(p, probes_per_block, kStaticScratchBytes);
    if (L.total > kStaticScratchBytes)
        return fail(SA_ERR_CAPACITY,
                    "sparsepr (static workspace): this call needs %zu bytes of workspace, more than the %zu "
                    "bytes of the library's static array; use sparse_attn_forward_sparsepr with a workspace",
                    L.total, kStaticScratchBytes);
    void *ws = nullptr;
    if ((s = scratch_of_current_device(&ws)) != SA_OK) return s;
    return run_sparsepr(p, q, k, v, r, probes_per_block, rank, ridge, L, ws, o, stream);
}

const char *sparse_attn_status_string(sa_status s) {
    switch (s) {
        case SA_OK: return "ok";
        case SA_ERR_INVALID_ARG: return "invalid argument";
        case SA_ERR_UNSUPPORTED: return "unsupported configuration";
        case SA_ERR_CAPACITY: return "kv_idx capacity too small";
        case SA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *sparse_attn_last_error(void) { return g_err; }

}  // extern "C"
