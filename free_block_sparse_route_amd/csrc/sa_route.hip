// Routing kernels: block pooling, proxy scoring and block selection, and the
// cost-ordered work list for the attention kernel.
//
// pool    one workgroup per (b, h, 128-token span, tensor) reduces the span's
//         one or two blocks of K or V (and, for the PAMA proxy, Q) to fp32 means
//         with coalesced 16-byte loads (HBM-bound; the inputs are read exactly
//         once).  Block centroids: PARK page, section 4.1.
// select  one workgroup per (b, h, group of G query blocks) first pools its G
//         query blocks (so that these reads of Q overlap the latency-bound
//         proxy and selection work of other workgroups) and a share of the
//         head's residual-tile norm bounds, then the G proxy rows
//         s_IJ = scale * qbar_I . kbar_J are computed in fp32 into LDS (never
//         written to memory, Sol-Attn abstract: no materialised proxy map),
//         then one wave per row takes the row max / log-sum-exp, compares with
//         tau, applies the top-k cap or floor by an exact k-th-largest search
//         over order-preserving integer keys, forces the dense prefix and
//         compacts the kept blocks into an ascending index list and bit mask.
// order   work order for the attention kernel: a stable counting sort of the
//         query blocks by cost band floor(log2(cost)), cost = tiles the
//         attention kernel will visit, highest band first.  The dispatcher
//         issues workgroups roughly in order, so expensive blocks start early
//         and cheap ones fill the end (close to longest-processing-time-first
//         scheduling, which matters where a row may keep most key blocks),
//         while within a band the blocks stay in ascending order: neighbouring
//         query blocks keep mostly the same key blocks and meet in the L2.
#include <type_traits>

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

constexpr int kPoolThreads = 256;
constexpr int kSelectThreads = 512;       // 8 waves: a row per wave in flight on more SIMD slots
constexpr int kOrderThreads = 1024;
constexpr int kOrderTiles = 448;         // 32 x 448 counters: 56 KB of LDS
constexpr int kBands = 32;               // floor(log2(cost)) of a non-negative int32

// --------------------------------------------------------------------- pool
template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(const T *__restrict__ q,
                                                            const T *__restrict__ k,
                                                            const T *__restrict__ v,
                                                            PoolArgs a) {
    // one workgroup per 128-token span of one tensor: one block of 128 or two of 64
    const int which = blockIdx.z + a.first;  // 0 = q, 1 = k, 2 = v
    const int bh = blockIdx.y;
    const int bs = which == 0 ? a.block_q : a.block_k;
    const int nb = which == 0 ? a.n_qb : a.n_kb;
    const int r0 = blockIdx.x * 128;
    if (r0 >= a.N) return;
    const T *X = (which == 0 ? q : which == 1 ? k : v) + (size_t)bh * a.N * D;
    const int span = min(128, a.N - r0);

    constexpr int CH = D / 8;                 // 8-element chunks per row
    constexpr int RG = kPoolThreads / CH;     // row groups
    const int c = threadIdx.x % CH;
    const int g = threadIdx.x / CH;

    float acc[2][8];                          // the span's first and second block
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[b][i] = 0.f;
    // every load is issued before the first sum (a load under a branch would
    // wait for the one before it); rows past the span re-read the span's last
    // row and add nothing.  The loaded words stay raw until they are summed
    // (bf16: 4 registers per 8 elements instead of 8), so that more workgroups
    // fit a CU and more loads are in flight.  Loads and result stores carry the
    // non-temporal hint: the inputs stream through once (with the hint the
    // route took 1.035 instead of 1.10 ms on the stress shape, and the
    // attention pass after it was no slower).
    constexpr int IT = 128 / RG;
    constexpr int WPL = 8 * sizeof(T) / 4;    // 32-bit words per 8-element load
    uint32_t x[IT][WPL];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const T *src = X + (size_t)(r0 + min(g + it * RG, span - 1)) * D + c * 8;
#pragma unroll
        for (int h = 0; h < WPL / 4; ++h) {
            const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint32_t *>(src) + 4 * h));
#pragma unroll
            for (int e = 0; e < 4; ++e) x[it][4 * h + e] = w[e];
        }
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int r = g + it * RG;
        const bool in = r < span;
        const int b = r >= bs;                 // RG divides bs: uniform per iteration
        float y[8];
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                y[2 * i] = __uint_as_float(x[it][i] << 16);
                y[2 * i + 1] = __uint_as_float(x[it][i] & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = __uint_as_float(x[it][i]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[b][i] += in ? y[i] : 0.f;
    }
    // Row groups of one wave are combined with lane swaps (the lanes of a
    // feature chunk sit CH apart), the kernel's four waves through 4 KB of LDS;
    // then a thread finishes four consecutive features of a block and stores
    // them at once (16 bytes of fp32 means, 8 bytes each of the bf16 rows).
    static_assert(kPoolThreads == 4 * kWave && (CH == 16 || CH == 8), "lane layout");
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float x = acc[b][i];
            const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
            x = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
            const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
            x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
            if constexpr (CH == 8)        // lanes 8 apart within a row of 16: rotate by 8
                x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
            acc[b][i] = x;
        }
    __shared__ __attribute__((aligned(16))) float part[4][2][D];
    const int wave = threadIdx.x / kWave, lane = lane_id();
    if (lane < CH) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 8; ++i) part[wave][b][lane * 8 + i] = acc[b][i];
    }
    __syncthreads();
    const int nblk = (span + bs - 1) / bs;
    constexpr int Q4 = D / 4;                   // threads per block, four features each
    if ((int)threadIdx.x < nblk * Q4) {
        const int b = threadIdx.x / Q4, f = 4 * (threadIdx.x % Q4);
        const int J = (r0 + b * bs) / bs;
        const float inv = 1.f / (float)min(bs, a.N - J * bs);
        f32x4 m = *reinterpret_cast<const f32x4 *>(&part[0][b][f]);
#pragma unroll
        for (int w = 1; w < 4; ++w) m += *reinterpret_cast<const f32x4 *>(&part[w][b][f]);
        // (other blocks' rows left zeros in the sums)
        f32x4 mean;
#pragma unroll
        for (int e = 0; e < 4; ++e) mean[e] = m[e] * inv;
        float *dst = which == 0 ? a.q_mean : which == 1 ? a.k_mean : a.v_mean;
        __builtin_nontemporal_store(mean, reinterpret_cast<f32x4 *>(dst + ((size_t)bh * nb + J) * D + f));
        if (which != 0) {
            // residual tile rows: block J -> group J/32, row J%32 (bf16 of the mean)
            // and row 32 + J%32 (bf16 of what that rounding left)
            bf16 *sp = a.kv_split + (((size_t)bh * 2 + (which - 1)) * a.words + J / 32) * 64 * D;
            bf16x4 hi, lo;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hi[e] = (bf16)mean[e];
                lo[e] = (bf16)(mean[e] - (float)hi[e]);
            }
            __builtin_nontemporal_store(hi, reinterpret_cast<bf16x4 *>(sp + (size_t)(J % 32) * D + f));
            __builtin_nontemporal_store(lo, reinterpret_cast<bf16x4 *>(sp + (size_t)(32 + J % 32) * D + f));
            if (J == nb - 1) {
                const bf16x4 z = {};
                for (int r = J % 32 + 1; r < 32; ++r) {
                    *reinterpret_cast<bf16x4 *>(sp + (size_t)r * D + f) = z;
                    *reinterpret_cast<bf16x4 *>(sp + (size_t)(32 + r) * D + f) = z;
                }
            }
        }
    }
}

// --------------------------------------------------------------------- select
// e^x and ln x on the hardware base-2 exponential and logarithm (a few ulp;
// the proxy decisions carry a 1e-4 exemption band)
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
__device__ __forceinline__ float fast_log(float x) { return __builtin_amdgcn_logf(x) * 0.693147180559945309f; }

__device__ __forceinline__ uint64_t lanes_below() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Sum over the wave of small per-lane counts (exact: far below 2^24).
__device__ __forceinline__ int wave_count(int c) { return (int)wave_sum((float)c); }

// Number of row entries whose key is >= kmin (wave-uniform result).
__device__ __forceinline__ int count_ge(const float *S, int n, uint32_t kmin) {
    int cnt = 0;
    for (int base = 0; base < n; base += kWave) {
        const int J = base + lane_id();
        const bool p = J < n && orderable(S[J]) >= kmin;
        cnt += __popcll(__ballot(p));
    }
    return cnt;
}

// Proxy probability mass of the row entries whose key is >= kmin (wave-uniform).
__device__ __forceinline__ float mass_ge(const float *S, int n, uint32_t kmin, float lse) {
    float ms = 0.f;
    for (int J = lane_id(); J < n; J += kWave)
        if (orderable(S[J]) >= kmin) ms += fast_exp(S[J] - lse);
    return wave_sum(ms);
}

// Kept list, bit mask, count, statistics and cost of one proxy row read from
// LDS.  With ksel > 0 the row keeps the keys above T and the first take_eq keys
// equal to T in J order; otherwise the entries at or above thr (none for TOPP).
// Blocks of the dense prefix are always kept.
__device__ __forceinline__ void compact_row_lds(const float *S, int bh, int I, const SelectArgs &a, int ksel,
                                                uint32_t T, int take_eq, float thr, float m, float lse) {
    const int lane = lane_id();
    const int n = a.n_kb;
    const size_t row = (size_t)bh * a.n_qb + I;
    int32_t *idx = a.kv_idx + row * a.kv_idx_cap;
    uint32_t *mask = a.kv_mask + row * a.mask_words;
    const bool dense_row = (int64_t)I * a.block_q < a.n_prefix;
    const int last_cnt = a.N - (n - 1) * a.block_k;
    int kept = 0, eq_seen = 0, tiles = 0;
    for (int base = 0; base < n; base += kWave) {
        const int J = base + lane;
        const bool valid = J < n;
        const float sv = valid ? S[J] : 0.f;
        bool keep;
        if (ksel > 0) {
            const uint32_t key = orderable(sv);
            const bool eq = valid && key == T;
            const uint64_t be = __ballot(eq);
            const int rank = eq_seen + __popcll(be & lanes_below());
            eq_seen += __popcll(be);
            keep = valid && (key > T || (eq && rank < take_eq));
        } else {
            keep = valid && a.tau_mode != SA_TAU_TOPP && sv >= thr;   // TOPP: n_c = 0
        }
        keep = valid && (keep || dense_row || (int64_t)J * a.block_k < a.n_prefix);
        const uint64_t bk = __ballot(keep);
        if (keep) idx[kept + __popcll(bk & lanes_below())] = J;
        kept += __popcll(bk);
        const int w = base / 32;
        if (lane == 0 && w < a.mask_words) mask[w] = (uint32_t)bk;
        if (lane == 1 && w + 1 < a.mask_words) mask[w + 1] = (uint32_t)(bk >> 32);
        // cost: exact tiles of kept blocks, plus one residual tile per 32 pooled
        // blocks (one mask word) that holds a dropped block
        const int nj = (J == n - 1) ? last_cnt : a.block_k;
        tiles += keep ? (nj + a.exact_tile_rows - 1) / a.exact_tile_rows : 0;
        const uint64_t bd = __ballot(valid && !keep);
        if (lane == 0) tiles += ((uint32_t)bd != 0) + ((uint32_t)(bd >> 32) != 0);
    }
    tiles = (int)wave_sum((float)tiles);
    if (lane == 0) {
        a.kv_count[row] = kept;
        a.row_stats[row * 2 + 0] = m;
        a.row_stats[row * 2 + 1] = lse;
        a.cost[row] = tiles;
    }
}

// Rows longer than 20 * 64 key blocks: the same steps, reading the row from LDS.
__device__ __forceinline__ void select_row_lds(const float *S, int bh, int I, const SelectArgs &a) {
    const int lane = lane_id();
    const int n = a.n_kb;
    float m = -INFINITY;
    for (int J = lane; J < n; J += kWave) m = fmaxf(m, S[J]);
    m = wave_max(m);
    float z = 0.f;
    for (int J = lane; J < n; J += kWave) z += fast_exp(S[J] - m);
    z = wave_sum(z);
    const float lse = m + fast_log(z);
    const float thr = (a.tau_mode == SA_TAU_ABSOLUTE ? lse : m) + a.ln_tau;

    int n_c = 0;
    if (a.tau_mode == SA_TAU_TOPP) {
        // length of the ranking prefix whose preceding proxy mass stays below
        // the target (see the register version below)
        const float target = a.topp_target;
        if (target > 0.f) {
            uint32_t Ts = 0;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cand = Ts | (1u << bit);
                if (mass_ge(S, n, cand, lse) >= target) Ts = cand;
            }
            if (Ts == 0u) {
                n_c = n;
            } else {
                const float mgt = Ts == 0xffffffffu ? 0.f : mass_ge(S, n, Ts + 1, lse);
                const int ngt = Ts == 0xffffffffu ? 0 : count_ge(S, n, Ts + 1);
                const int neq = count_ge(S, n, Ts) - ngt;
                float peq = 0.f;
                for (int J = lane; J < n; J += kWave)
                    if (orderable(S[J]) == Ts) peq = fast_exp(S[J] - lse);
                peq = wave_max(peq);
                int teq = 1;
                while (teq < neq && mgt + (float)teq * peq < target) ++teq;
                n_c = ngt + teq;
            }
        }
    } else {
        for (int base = 0; base < n; base += kWave) {
            const int J = base + lane;
            n_c += __popcll(__ballot(J < n && S[J] >= thr));
        }
    }
    int ksel = 0;
    if (a.max_keep > 0 && n_c > a.max_keep) ksel = a.max_keep;
    else if (n_c < a.min_keep) ksel = min(a.min_keep, n);
    else if (a.tau_mode == SA_TAU_TOPP) ksel = n_c;         // a ranking prefix of n_c blocks

    // ksel-th largest key T, built bit by bit from the top: the largest T with
    // #{key >= T} >= ksel.  Equal keys beyond the budget are resolved by J.
    uint32_t T = 0;
    int take_eq = 0;
    if (ksel > 0) {
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            if (count_ge(S, n, cand) >= ksel) T = cand;
        }
        const int n_gt = (T == 0xffffffffu) ? 0 : count_ge(S, n, T + 1);
        take_eq = ksel - n_gt;
    }

    compact_row_lds(S, bh, I, a, ksel, T, take_eq, thr, m, lse);
}

// One proxy row: statistics, the tau test, the cap or floor, the kept list,
// bit mask and cost.  The lane holds scores J = lane + 64 i, i < R, in registers
// (R * 64 >= n_kb): every pass over the row, in particular the 32 counting
// passes of the cap's k-th-largest search, runs on registers.
template <int R>
__device__ __forceinline__ void select_row(const float *S, int bh, int I, const SelectArgs &a) {
    // Per-row copies the compiler cannot hoist out of the caller's loop over
    // rows: per-chunk conditions derived from them would otherwise stay live
    // across rows (as 64-bit lane masks) and spill.
    int lane = lane_id(), n = a.n_kb;
    asm volatile("" : "+v"(lane));
    asm volatile("" : "+s"(n));
    // Absent entries (J >= n) hold -inf: weight 0, and a key below every
    // finite score's, so no count or budget search that ends at a real key
    // includes them.  No per-entry validity mask is kept: held for every
    // chunk, such masks fill the scalar registers.
    float sv[R];
    uint32_t key[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int J = i * kWave + lane;
        sv[i] = J < n ? S[J] : -INFINITY;
        key[i] = orderable(sv[i]);
    }
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < R; ++i) m = fmaxf(m, sv[i]);
    m = wave_max(m);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i)
        z += fast_exp(sv[i] - m);
    z = wave_sum(z);
    const float lse = m + fast_log(z);
    // tau = 0 gives thr = -inf; clamped to the lowest finite value it keeps
    // every real entry and no absent one
    const float thr = fmaxf((a.tau_mode == SA_TAU_ABSOLUTE ? lse : m) + a.ln_tau, -3.40282347e38f);   // lowest finite float

    int n_c = 0;
    uint32_t T = 0;
    int take_eq = 0;
    bool topp_cut = false;      // T, take_eq already give the TOPP prefix
    if (a.tau_mode == SA_TAU_TOPP) {
        // ranking prefix whose preceding proxy mass stays below the target:
        // Ts = the largest key with mass(key >= Ts) >= target; blocks above Ts
        // are kept, then ties at Ts in J order while the mass before them is
        // below the target
        const float target = a.topp_target;
        float pv[R];
#pragma unroll
        for (int i = 0; i < R; ++i) pv[i] = fast_exp(sv[i] - lse);
        if (target > 0.f) {
            uint32_t Ts = 0;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cand = Ts | (1u << bit);
                float ms = 0.f;
#pragma unroll
                for (int i = 0; i < R; ++i) ms += key[i] >= cand ? pv[i] : 0.f;
                if (wave_sum(ms) >= target) Ts = cand;
            }
            if (Ts == 0u) {
                n_c = n;                                    // the whole row is needed
            } else {
                float mgt = 0.f, peq = 0.f;
                int ngt = 0, neq = 0;
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    mgt += key[i] > Ts ? pv[i] : 0.f;
                    peq = key[i] == Ts ? pv[i] : peq;
                    ngt += key[i] > Ts;
                    neq += key[i] == Ts;
                }
                mgt = wave_sum(mgt);
                ngt = wave_count(ngt);
                neq = wave_count(neq);
                peq = wave_max(peq);
                int teq = 1;
                while (teq < neq && mgt + (float)teq * peq < target) ++teq;
                n_c = ngt + teq;
                T = Ts;
                take_eq = teq;
                topp_cut = true;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < R; ++i) n_c += sv[i] >= thr;
        n_c = wave_count(n_c);
    }
    int ksel = 0;
    if (a.max_keep > 0 && n_c > a.max_keep) ksel = a.max_keep;
    else if (n_c < a.min_keep) ksel = min(a.min_keep, n);
    else if (a.tau_mode == SA_TAU_TOPP) ksel = n_c;         // a ranking prefix of n_c blocks

    // ksel-th largest key T, built bit by bit from the top: the largest T with
    // #{key >= T} >= ksel.  Every candidate is >= 1, so absent entries never
    // count.  Equal keys beyond the budget are resolved by J.
    if (ksel > 0 && !(topp_cut && ksel == n_c)) {
        T = 0;
        take_eq = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < R; ++i) cnt += key[i] >= cand;
            if (wave_count(cnt) >= ksel) T = cand;
        }
        int n_gt = 0;
        if (T != 0xffffffffu)
#pragma unroll
            for (int i = 0; i < R; ++i) n_gt += key[i] > T;
        take_eq = ksel - wave_count(n_gt);
    }

    // Equal keys at T split by the budget (rare): rank them in J order on the
    // LDS copy of the row.  Otherwise the kept set is every key >= T.
    if (ksel > 0) {
        int n_eq = 0;
#pragma unroll
        for (int i = 0; i < R; ++i) n_eq += key[i] == T;
        if (take_eq < wave_count(n_eq)) {
            compact_row_lds(S, bh, I, a, ksel, T, take_eq, thr, m, lse);
            return;
        }
    }
    const size_t row = (size_t)bh * a.n_qb + I;
    int32_t *idx = a.kv_idx + row * a.kv_idx_cap;
    uint32_t *mask = a.kv_mask + row * a.mask_words;
    int lv = lane, n_prefix = a.n_prefix, block_k = a.block_k;   // per-row copies, as above
    asm volatile("" : "+s"(n_prefix), "+s"(block_k));
    const bool dense_row = (int64_t)I * a.block_q < n_prefix;
    const int rows = a.exact_tile_rows;
    const int t_full = (block_k + rows - 1) / rows;
    const int t_last = (a.N - (n - 1) * block_k + rows - 1) / rows;
    int kept = 0, tiles = 0;
    uint32_t word = 0u;                 // lane w ends with mask word w
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int J = i * kWave + lv;
        // ksel > 0: T is a real entry's key, above every absent one
        bool keep = ksel > 0 ? key[i] >= T : a.tau_mode != SA_TAU_TOPP && sv[i] >= thr;   // TOPP: n_c = 0
        keep = keep || (dense_row && sv[i] > -INFINITY) || (int64_t)J * block_k < n_prefix;
        const uint64_t bk = __ballot(keep);
        if (keep) idx[kept + __popcll(bk & lanes_below())] = J;
        kept += __popcll(bk);
        word = lv == 2 * i ? (uint32_t)bk : lv == 2 * i + 1 ? (uint32_t)(bk >> 32) : word;
        // cost: exact tiles of the kept blocks
        tiles += keep ? (J == n - 1 ? t_last : t_full) : 0;
    }
    // plus one residual tile per mask word that holds a dropped block
    if (lv < a.mask_words) {
        mask[lv] = word;
        const int lim = n - 32 * lv;
        const uint32_t vmask = lim >= 32 ? ~0u : ((1u << lim) - 1u);
        tiles += (~word & vmask) != 0u;
    }
    tiles = (int)wave_sum((float)tiles);
    if (lane == 0) {
        a.kv_count[row] = kept;
        a.row_stats[row * 2 + 0] = m;
        a.row_stats[row * 2 + 1] = lse;
        a.cost[row] = tiles;
    }
}

// Pre-pass of fused routing: the row's maximum and log-sum-exp only.
__device__ __forceinline__ void row_stats_only(const float *S, int bh, int I, const SelectArgs &a) {
    const int lane = lane_id(), n = a.n_kb;
    float m = -INFINITY;
    for (int J = lane; J < n; J += kWave) m = fmaxf(m, S[J]);
    m = wave_max(m);
    float z = 0.f;
    for (int J = lane; J < n; J += kWave) z += fast_exp(S[J] - m);
    z = wave_sum(z);
    const float lse = m + fast_log(z);
    // The work order's cost of the row under the decisions the fused forward
    // will take (the same threshold test; a block within the rounding band may
    // be decided the other way there, which only moves the estimate by a tile):
    // exact tiles of the kept blocks plus one residual tile per mask word that
    // holds a dropped block.
    const float thr = fmaxf((a.tau_mode == SA_TAU_ABSOLUTE ? lse : m) + a.ln_tau, -3.40282347e38f);
    const bool dense_row = (int64_t)I * a.block_q < a.n_prefix;
    const int rows = a.exact_tile_rows;
    const int t_full = (a.block_k + rows - 1) / rows;
    const int t_last = (a.N - (n - 1) * a.block_k + rows - 1) / rows;
    // a floor of one block: when no block clears the threshold the forward keeps
    // the row's best block (the largest score, lowest J among equal ones)
    int floor_j = -1;
    if (a.min_keep > 0) {
        int npass = 0;
        for (int J = lane; J < n; J += kWave) npass += S[J] >= thr ? 1 : 0;
        if (wave_count(npass) == 0) {
            int jm = n;
            for (int J = lane; J < n; J += kWave) jm = (S[J] == m && J < jm) ? J : jm;
            floor_j = (int)wave_reduce((float)jm, [](float x, float y) { return fminf(x, y); });
        }
    }
    int tiles = 0;
    for (int base = 0; base < n; base += kWave) {
        const int J = base + lane;
        const bool keep = J < n && (S[J] >= thr || J == floor_j || dense_row || (int64_t)J * a.block_k < a.n_prefix);
        tiles += keep ? (J == n - 1 ? t_last : t_full) : 0;
        const uint64_t kb = __ballot(keep);
        // the chunk's two mask words: residual tile if a valid block is dropped
        const int lim0 = min(32, n - base), lim1 = min(32, max(0, n - base - 32));
        const uint32_t v0 = lim0 >= 32 ? ~0u : ((1u << lim0) - 1u);
        const uint32_t v1 = lim1 >= 32 ? ~0u : ((1u << lim1) - 1u);
        if (lane == 0) tiles += (~(uint32_t)kb & v0) != 0u;
        if (lane == 1 && lim1 > 0) tiles += (~(uint32_t)(kb >> 32) & v1) != 0u;
    }
    tiles = wave_count(tiles);
    if (lane == 0) {
        const size_t row = (size_t)bh * a.n_qb + I;
        a.row_stats[row * 2 + 0] = m;
        a.row_stats[row * 2 + 1] = lse;
        a.cost[row] = tiles;
    }
}

// The pointer passes through the empty statement as a global-memory pointer,
// so that the stores through it stay global stores (as a generic pointer they
// would become flat stores, which also count on the LDS counter: every later
// LDS wait would then wait for the stores too).
template <typename T>
__device__ __forceinline__ void launder_global(T *&p) {
    __attribute__((address_space(1))) T *g = (__attribute__((address_space(1))) T *)p;
    asm volatile("" : "+s"(g));
    p = (T *)g;
}

__device__ __forceinline__ void launder(SelectArgs &a) {
    asm volatile("" : "+s"(a.N), "+s"(a.block_q), "+s"(a.block_k), "+s"(a.n_qb), "+s"(a.n_kb), "+s"(a.mask_words));
    asm volatile("" : "+s"(a.kv_idx_cap), "+s"(a.exact_tile_rows), "+s"(a.tau_mode), "+s"(a.max_keep),
                 "+s"(a.min_keep), "+s"(a.n_prefix), "+s"(a.stats_only));
    asm volatile("" : "+s"(a.scale), "+s"(a.ln_tau), "+s"(a.topp_target));
    launder_global(a.kv_count);
    launder_global(a.kv_idx);
    launder_global(a.cost);
    launder_global(a.kv_mask);
    launder_global(a.row_stats);
}

// Query-block means inside the select kernel (PARK page, section 4.1), one
// block per wave at a time: a lane sums one 16-byte chunk of the rows of its row group (the wave
// loads kWave / CH rows at once, NB loads in flight per lane; rows past a
// ragged block re-read its last row and add nothing), and lane swaps combine
// the row groups, so that every lane ends with its chunk's sums.
template <typename T, int D>
struct BlockPool {
    static constexpr int EPC = 16 / (int)sizeof(T);     // elements per 16-byte chunk
    static constexpr int CH = D / EPC;                  // chunks per row: 8, 16 or 32
    static constexpr int RG = kWave / CH;               // rows per wave load
    static constexpr int NB = 64 / RG < 8 ? 64 / RG : 8;
    static_assert(CH == 8 || CH == 16 || CH == 32, "lane layout");
    static_assert(64 % (NB * RG) == 0, "a batch of loads divides a block");

    // sums of the rows of a block of bs rows at src (this lane's chunk), of
    // which the first span are present (kRagged: span < bs)
    template <bool kRagged>
    static __device__ __forceinline__ void sums(const T *__restrict__ src, int span, int bs, int rg,
                                                float (&acc)[EPC]) {
        for (int it0 = 0; it0 < bs; it0 += NB * RG) {
            u32x4 w[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int r = kRagged ? min(it0 + j * RG + rg, span - 1) : it0 + j * RG + rg;
                w[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + (size_t)r * D));
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const bool in = !kRagged || it0 + j * RG + rg < span;
                float y[EPC];
                if constexpr (sizeof(T) == 2) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        y[2 * i] = __uint_as_float(w[j][i] << 16);
                        y[2 * i + 1] = __uint_as_float(w[j][i] & 0xffff0000u);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[i] = __uint_as_float(w[j][i]);
                }
#pragma unroll
                for (int i = 0; i < EPC; ++i) acc[i] += in ? y[i] : 0.f;
            }
        }
    }

    // means of rows [r0, r0 + span) of X ([rows][D]), a block of bs rows
    static __device__ __forceinline__ void means(const T *__restrict__ X, int r0, int span, int bs,
                                                 float (&m)[EPC]) {
        const int lane = lane_id();
        const int c = lane % CH, rg = lane / CH;
        const T *src = X + (size_t)r0 * D + c * EPC;
        float acc[EPC];
#pragma unroll
        for (int i = 0; i < EPC; ++i) acc[i] = 0.f;
        // every block but a ragged last one is whole: no clamp, no masked adds
        if (span == bs) sums<false>(src, span, bs, rg, acc);
        else sums<true>(src, span, bs, rg, acc);
        // the row groups of a chunk sit CH lanes apart
        const float inv = 1.f / (float)span;
#pragma unroll
        for (int i = 0; i < EPC; ++i) {
            float x = acc[i];
            const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
            x = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
            if constexpr (CH <= 16) {
                const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
                x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
            }
            if constexpr (CH == 8)        // lanes 8 apart within a row of 16: rotate by 8
                x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
            m[i] = x * inv;
        }
    }

    // The group's g_cnt query blocks, wave w taking blocks w, w + 8, ...:
    // their means go to qs ([g][D] in LDS) and to q_mean.
    static __device__ __forceinline__ void run(const SelectArgs &a, int bh, int I0, int g_cnt, float *qs) {
        const int lane = lane_id(), wave = threadIdx.x / kWave;
        const int c = lane % CH;
        const T *X = (const T *)a.q + (size_t)bh * a.N * D;
        for (int g = wave; g < g_cnt; g += kSelectThreads / kWave) {
            const int r0 = (I0 + g) * a.block_q;
            float m[EPC];
            means(X, r0, min(a.block_q, a.N - r0), a.block_q, m);
            if (lane < CH) {
                float *dst = a.q_mean + ((size_t)bh * a.n_qb + I0 + g) * D + c * EPC;
#pragma unroll
                for (int h = 0; h < EPC / 4; ++h) {
                    const f32x4 x = {m[4 * h], m[4 * h + 1], m[4 * h + 2], m[4 * h + 3]};
                    *reinterpret_cast<f32x4 *>(qs + g * D + c * EPC + 4 * h) = x;
                    __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(dst + 4 * h));
                }
            }
        }
    }
};

// Bounds for the forward's early tests of residual tiles: for each residual
// tile of the head (group g of 32 key blocks), upper bounds on the Euclidean
// norms of its 32 key-mean remainder rows and of its 32 key means as the
// forward forms them (bf16 part plus remainder, both as the pool kernel stored
// them).  A wave per tile, the tiles dealt over the head's select workgroups:
// lane (r, half) sums the squares of half of row r in fp32 (the bf16 part plus
// remainder is exact in fp32), the two halves meet by a lane swap, the wave
// takes the largest row, and a bound is its square root raised by 2^-10 (over
// the rounding of the squares, the sums and the root).
template <int D>
__device__ __forceinline__ void residual_bounds(const SelectArgs &a, int bh, int grp, int n_grp) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int r = lane >> 1, hf = lane & 1;
    constexpr int NL = D / 16;                     // 16-byte loads per half row
    for (int g = grp + wave * n_grp; g < a.mask_words; g += (kSelectThreads / kWave) * n_grp) {
        const bf16 *hi_row = a.kv_split + ((size_t)bh * 2 * a.mask_words + g) * 64 * D + (size_t)r * D + hf * (D / 2);
        const bf16 *lo_row = hi_row + 32 * D;
        u32x4 wh[NL], wl[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            wh[j] = *reinterpret_cast<const u32x4 *>(hi_row + 8 * j);
            wl[j] = *reinterpret_cast<const u32x4 *>(lo_row + 8 * j);
        }
        float ss_lo = 0.f, ss_mean = 0.f;
#pragma unroll
        for (int j = 0; j < NL; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float l0 = __uint_as_float(wl[j][i] << 16), l1 = __uint_as_float(wl[j][i] & 0xffff0000u);
                const float m0 = __uint_as_float(wh[j][i] << 16) + l0;
                const float m1 = __uint_as_float(wh[j][i] & 0xffff0000u) + l1;
                ss_lo = fmaf(l0, l0, ss_lo);
                ss_lo = fmaf(l1, l1, ss_lo);
                ss_mean = fmaf(m0, m0, ss_mean);
                ss_mean = fmaf(m1, m1, ss_mean);
            }
        ss_lo += dpp_f(ss_lo, 0xB1);               // the row's other half (lane ^ 1)
        ss_mean += dpp_f(ss_mean, 0xB1);
        const float lo = wave_max(ss_lo), mean = wave_max(ss_mean);
        if (lane == 0) {
            const float2 b = {__builtin_sqrtf(mean) * (1.f + 1.f / 1024.f), __builtin_sqrtf(lo) * (1.f + 1.f / 1024.f)};
            *reinterpret_cast<float2 *>(a.k_bounds + ((size_t)bh * a.mask_words + g) * 2) = b;
        }
    }
}

// R: proxy row chunks of 64 held in registers (R * 64 >= n_kb), 0: longer rows
// are read from LDS.
template <int D, int G, int R>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(SelectArgs a) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    // one head's groups run on one die, which reads that head's key means once
    const int n_grp = (a.n_qb + G - 1) / G;
    const int task = die_task(blockIdx.x, (int)gridDim.x, n_grp);
    const int bh = task / n_grp;
    const int I0 = (task - bh * n_grp) * G;
    const int g_cnt = min(G, a.n_qb - I0);
    const int n = a.n_kb;
    float *S = smem;                                      // [G][n]
    float *qs = smem;                                     // [G][D] query means, before S is formed
    if (a.q_bf16) BlockPool<bf16, D>::run(a, bh, I0, g_cnt, qs);
    else BlockPool<float, D>::run(a, bh, I0, g_cnt, qs);
    residual_bounds<D>(a, bh, I0 / G, n_grp);
    __syncthreads();
    {
        // Proxy rows on the fp32 matrix cores (v_mfma_f32_16x16x4_f32, fp32
        // products and sums): a wave takes 16 key blocks at a time and forms
        // their scores against the group's (up to 16) query blocks.  Lane
        // (i16, kg) supplies key block i16 and query block i16 at features
        // kg * KS + s in MFMA step s (s even and odd on two accumulators);
        // result register r is key block 4 kg + r against query block i16.
        const int lane = lane_id();
        const int wave0 = threadIdx.x / kWave;
        const int i16 = lane & 15, kg = lane >> 4;
        constexpr int KS = D / 4;
        float qv[KS];
        {
            const bool ok = i16 < g_cnt;
            const float *src = qs + (ok ? i16 : 0) * D + kg * KS;
#pragma unroll
            for (int e = 0; e < KS; e += 4) {
                const f32x4 y = *reinterpret_cast<const f32x4 *>(src + e);   // row clamped: pooled
                const f32x4 x = ok ? y : f32x4{};
                qv[e] = x[0];
                qv[e + 1] = x[1];
                qv[e + 2] = x[2];
                qv[e + 3] = x[3];
            }
        }
        __syncthreads();                                  // S overwrites qs
        const float *kb = a.k_mean + (size_t)bh * n * D;
        const int n_sl = (n + 15) / 16;
        constexpr int kStride = kSelectThreads / kWave;
        // A slice past the last key block reads block 0 instead (in bounds): its
        // rows only form the scores of blocks J >= n_kb, which are never stored,
        // so the loaded values go to the products untouched (no select on them,
        // which would make the compiler wait for the loads where they are issued).
        auto load_slice = [&](int sl, float (&kv)[KS]) {
            const int J = sl * 16 + i16;
            const float *src = kb + (size_t)(J < n ? J : 0) * D + kg * KS;
#pragma unroll
            for (int e = 0; e < KS; e += 4) {
                const f32x4 y = *reinterpret_cast<const f32x4 *>(src + e);
                kv[e] = y[0];
                kv[e + 1] = y[1];
                kv[e + 2] = y[2];
                kv[e + 3] = y[3];
            }
        };
        auto scores = [&](int sl, const float (&kv)[KS]) {
            f32x4 acc0 = {}, acc1 = {};
#pragma unroll
            for (int e = 0; e < KS; e += 2) {
                acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[e], qv[e], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[e + 1], qv[e + 1], acc1, 0, 0, 0);
            }
            if (i16 < g_cnt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int Jr = sl * 16 + 4 * kg + r;
                    if (Jr < n) S[i16 * n + Jr] = (acc0[r] + acc1[r]) * a.scale;
                }
            }
        };
        // two slice buffers in turn: the next slice's keys are in flight while
        // the current one's products run (with a single buffer copied at the end
        // of each step the compiler waited for the next slice before the products)
        // The loads are unconditional (a slice past the last one reloads the last,
        // whose scores are not stored twice): a load under a branch makes the
        // compiler wait for every load in flight at the join.
        float ka[KS], kb2[KS];
        const int last = n_sl - 1;
        load_slice(min(wave0, last), ka);
        for (int sl = wave0; sl < n_sl; sl += 2 * kStride) {
            load_slice(min(sl + kStride, last), kb2);
            scores(sl, ka);
            if (sl + kStride >= n_sl) break;
            load_slice(min(sl + 2 * kStride, last), ka);
            scores(sl + kStride, kb2);
        }
    }
    __syncthreads();
    const int wave = threadIdx.x / kWave;
    for (int g = wave; g < g_cnt; g += kSelectThreads / kWave) {
        // A copy of the arguments the compiler must re-read every row, so that
        // nothing derived from them is hoisted out of this loop and held in
        // scalar registers across rows (it would spill).
        SelectArgs ar = a;
        launder(ar);
        const float *row = S + g * n;
        if (ar.stats_only) row_stats_only(row, bh, I0 + g, ar);
        else if constexpr (R > 0) select_row<R>(row, bh, I0 + g, ar);
        else select_row_lds(row, bh, I0 + g, ar);
    }
}

// --------------------------------------------------------------------- PAMA
// Per-query attention-mass aggregation (PARK page, section 5.1): the importance
// of key block J for query block I is the mean over the block's queries i of
// softmax_J(scale q_i . kbar_J); the selection then runs on s_IJ = ln A_IJ,
// whose softmax is A itself.  One workgroup per query block, a wave per 32
// queries; the logits of 32 key blocks at a time come from bf16 matrix cores
// with fp32 sums, every operand split into bf16 parts (the key means into
// three, fp32 queries into three; bf16 queries are exact) and every product of
// parts whose orders add up to at most 2 summed: the logits carry fp32-level
// error, which the decisions need.  Two passes over the key blocks: the first
// takes each query's maximum and normaliser (S^T = kbar q^T: a lane holds one
// query), the second recomputes the logits as S = q kbar^T (a lane holds one
// key block) and sums the normalised weights over the wave's queries.  The
// operand registers serve both products unchanged: the A and B operands of a
// 32x32x16 MFMA have the same lane layout.

template <typename T> struct QSplit { static constexpr int N = 1; };
template <> struct QSplit<float> { static constexpr int N = 3; };

// bf16 parts of 8 fp32 values: x = p[0] + p[1] + p[2] up to 2^-24 |x|
template <int NP>
__device__ __forceinline__ void split8(const float *x, bf16x8 (&p)[NP]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float r = x[e];
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const bf16 b = (bf16)r;
            p[k][e] = b;
            r -= (float)b;
        }
    }
}

constexpr int kPamaThreads = 256;       // 4 waves

// Query sets of 32 per wave: two for bf16 queries (the key operands read from
// LDS serve both sets' products), one for fp32 queries (their three bf16 parts
// fill the registers).
template <typename T> struct PamaShape {
    static constexpr int QS = QSplit<T>::N == 1 ? 2 : 1;
    static constexpr int QW = 32 * QS;                    // queries per wave
    static constexpr int QWG = (kPamaThreads / kWave) * QW;   // queries per workgroup
};

// Staging of one tile of 32 key-block means, split into three bf16 parts, in
// LDS: part p, row r at p * 32 * RS + r * RS bytes, RS = 2 D + 16 (the pad puts
// the 16 rows read by one ds_read_b128 quarter on distinct banks).  Every
// thread loads, splits and writes FPT consecutive features of one row; the
// waves then read their MFMA operands from the one staged copy.
template <int D>
struct PamaStage {
    static constexpr int FPT = 32 * D / kPamaThreads;   // features per thread
    static constexpr int TPR = D / FPT;                 // threads per row
    static constexpr int RS = 2 * D + 16;
    static constexpr int BYTES = 3 * 32 * RS;
    float x[FPT];

    __device__ __forceinline__ void load(const float *kb, int n_kb, int jt) {
        const int r = threadIdx.x / TPR, f = (threadIdx.x % TPR) * FPT;
        const int J = jt * 32 + r;
        const float *src = kb + (size_t)(J < n_kb ? J : 0) * D + f;
#pragma unroll
        for (int e = 0; e < FPT; e += 4) {
            const f32x4 v = J < n_kb ? *reinterpret_cast<const f32x4 *>(src + e) : f32x4{};
            x[e] = v[0];
            x[e + 1] = v[1];
            x[e + 2] = v[2];
            x[e + 3] = v[3];
        }
    }

    __device__ __forceinline__ void store(unsigned char *lds) const {
        const int r = threadIdx.x / TPR, f = (threadIdx.x % TPR) * FPT;
#pragma unroll
        for (int e = 0; e < FPT; e += 8) {
            bf16x8 p[3];
            split8<3>(x + e, p);
#pragma unroll
            for (int k = 0; k < 3; ++k)
                *reinterpret_cast<bf16x8 *>(lds + k * 32 * RS + r * RS + (f + e) * 2) = p[k];
        }
    }

    // operand of lane (h, l32) for step c, part k: row l32, features 16c + 8h..
    static __device__ __forceinline__ bf16x8 frag(const unsigned char *lds, int c, int k, int h, int l32) {
        return *reinterpret_cast<const bf16x8 *>(lds + k * 32 * RS + l32 * RS + (16 * c + 8 * h) * 2);
    }
};

// One workgroup per NB = QWG / BQ consecutive query blocks of a head; wave w
// holds the QW queries w QW .. of the group (all in one block, since QW <= BQ).
template <typename T, int D, int BQ, int R>
__global__ __launch_bounds__(kPamaThreads) void pama_kernel(const T *__restrict__ q, SelectArgs a) {
    using Sh = PamaShape<T>;
    constexpr int QS = Sh::QS, QW = Sh::QW, NB = Sh::QWG / BQ;
    constexpr int WAVES = kPamaThreads / kWave, WPB = BQ / QW;   // waves per query block
    static_assert(QW <= BQ && Sh::QWG % BQ == 0, "a wave's queries lie in one block");
    constexpr int NQ = QSplit<T>::N;
    constexpr int NS = D / 16;
    using St = PamaStage<D>;
    extern __shared__ __attribute__((aligned(16))) float smem[];
    const int n = a.n_kb;
    unsigned char *tile = reinterpret_cast<unsigned char *>(smem);
    float *part = smem + St::BYTES / 4;          // [WAVES][n]
    float *rows = part + WAVES * n;              // [NB][n]: ln A per block
    float *cq = rows + NB * n;                   // [QWG]: per-query log2 normaliser
    const int n_grp = (a.n_qb + NB - 1) / NB;
    const int task = die_task(blockIdx.x, (int)gridDim.x, n_grp);   // the groups of a head on one die
    const int bh = task / n_grp, I0 = (task - bh * n_grp) * NB;
    const int lane = lane_id(), h = lane >> 5, l32 = lane & 31;
    const int wave = threadIdx.x / kWave;
    const int wb = wave / WPB;                   // the wave's block within the group
    const int Iw = I0 + wb;
    const int q0 = Iw * a.block_q;
    const int m_w = Iw < a.n_qb ? min(a.block_q, a.N - q0) : 0;   // the block's actual rows
    const float c2 = a.scale * 1.44269504088896341f;          // logits in log2 units

    bf16x8 qf[QS][NS][NQ];       // lane (h, l32): query l32 of set s, features 16c + 8h..
#pragma unroll
    for (int s = 0; s < QS; ++s) {
        const int rb = (wave % WPB) * QW + s * 32 + l32;       // row within the block
        const bool ok = rb < m_w;
        const T *src = q + ((size_t)bh * a.N + (ok ? q0 + rb : 0)) * D + 8 * h;
#pragma unroll
        for (int c = 0; c < NS; ++c) {
            float x[8];
            Ld8<T>::load_f32(src + 16 * c, x);
            if (!ok)
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = 0.f;
            split8<NQ>(x, qf[s][c]);
        }
    }
    const float *kb = a.k_mean + (size_t)bh * n * D;
    const int n_jt = (n + 31) / 32;

    // One pass over the key-block tiles.  kSwap = false: S^T (lane: query l32
    // of set s, key blocks 8(r/4) + 4h + r%4); true: S (lane: key block l32,
    // queries 8(r/4) + 4h + r%4 of set s).  Products of parts with orders
    // a + b <= 2, smallest first.  The next tile's means are loaded while this
    // one is multiplied.
    auto pass = [&](auto swap, auto &&post) {
        constexpr bool kSwap = decltype(swap)::value;
        St st;
        st.load(kb, n, 0);
        for (int jt = 0; jt < n_jt; ++jt) {
            st.store(tile);
            __syncthreads();
            if (jt + 1 < n_jt) st.load(kb, n, jt + 1);
            f32x16 acc[QS];
#pragma unroll
            for (int s = 0; s < QS; ++s) acc[s] = f32x16{};
#pragma unroll
            for (int c = 0; c < NS; ++c) {
                bf16x8 kp[3];
#pragma unroll
                for (int k = 0; k < 3; ++k) kp[k] = St::frag(tile, c, k, h, l32);
#pragma unroll
                for (int ord = 2; ord >= 0; --ord) {
#pragma unroll
                    for (int qa = 0; qa < NQ; ++qa) {
                        const int kb_ = ord - qa;
                        if (kb_ < 0 || kb_ > 2) continue;
#pragma unroll
                        for (int s = 0; s < QS; ++s) {
                            if constexpr (kSwap)
                                acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[s][c][qa], kp[kb_], acc[s], 0, 0, 0);
                            else
                                acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kp[kb_], qf[s][c][qa], acc[s], 0, 0, 0);
                        }
                    }
                }
            }
            __syncthreads();                      // the tile is read; the next store may overwrite it
            post(jt, acc);
        }
    };

    // pass 1: per lane and set, running max and sum of 2^logit over its key blocks
    float m[QS], z[QS];
#pragma unroll
    for (int s = 0; s < QS; ++s) m[s] = -INFINITY, z[s] = 0.f;
    pass(std::false_type{}, [&](int jt, const f32x16 (&acc)[QS]) {
#pragma unroll
        for (int s = 0; s < QS; ++s) {
            float x[16];
            float mt = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int J = jt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                x[r] = J < n ? acc[s][r] * c2 : -INFINITY;
                mt = fmaxf(mt, x[r]);
            }
            if (mt > -INFINITY) {
                const float mn = fmaxf(m[s], mt);
                float zt = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) zt += __builtin_amdgcn_exp2f(x[r] - mn);
                z[s] = z[s] * __builtin_amdgcn_exp2f(m[s] - mn) + zt;       // m = -inf: z = 0
                m[s] = mn;
            }
        }
    });
#pragma unroll
    for (int s = 0; s < QS; ++s) {
        // combine the two lanes of each query: c = log2 of its normaliser
        const auto pm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m[s]), __float_as_uint(m[s]), false, false);
        const auto pz = __builtin_amdgcn_permlane32_swap(__float_as_uint(z[s]), __float_as_uint(z[s]), false, false);
        const float m0 = __uint_as_float(pm[0]), m1 = __uint_as_float(pm[1]);
        const float z0 = __uint_as_float(pz[0]), z1 = __uint_as_float(pz[1]);
        const float M = fmaxf(m0, m1);
        const float Z = (m0 > -INFINITY ? z0 * __builtin_amdgcn_exp2f(m0 - M) : 0.f) +
                        (m1 > -INFINITY ? z1 * __builtin_amdgcn_exp2f(m1 - M) : 0.f);
        const bool ok = (wave % WPB) * QW + s * 32 + l32 < m_w;
        if (h == 0) cq[wave * QW + s * 32 + l32] = ok ? M + __builtin_amdgcn_logf(Z) : INFINITY;
    }
    __syncthreads();
    // pass 2: normalised weights of each key block summed over the wave's queries
    float cr[QS][16];
#pragma unroll
    for (int s = 0; s < QS; ++s)
#pragma unroll
        for (int r = 0; r < 16; ++r) cr[s][r] = cq[wave * QW + s * 32 + 8 * (r >> 2) + 4 * h + (r & 3)];
    pass(std::true_type{}, [&](int jt, const f32x16 (&acc)[QS]) {
        float w = 0.f;
#pragma unroll
        for (int s = 0; s < QS; ++s)
#pragma unroll
            for (int r = 0; r < 16; ++r) w += __builtin_amdgcn_exp2f(acc[s][r] * c2 - cr[s][r]);   // invalid rows: 0
        const auto pw = __builtin_amdgcn_permlane32_swap(__float_as_uint(w), __float_as_uint(w), false, false);
        const float ws = __uint_as_float(pw[0]) + __uint_as_float(pw[1]);
        const int J = jt * 32 + l32;
        if (h == 0 && J < n) part[wave * n + J] = ws;
    });
    __syncthreads();
    for (int b = 0; b < NB; ++b) {
        const int I = I0 + b;
        if (I >= a.n_qb) break;
        const float inv_m = 1.f / (float)min(a.block_q, a.N - I * a.block_q);
        for (int J = threadIdx.x; J < n; J += kPamaThreads) {
            float A = 0.f;
#pragma unroll
            for (int w = 0; w < WPB; ++w) A += part[(b * WPB + w) * n + J];
            A *= inv_m;
            rows[b * n + J] = A > 0.f ? fast_log(A) : -1e30f;     // an underflowed importance stays a real, finite score
        }
    }
    __syncthreads();
    if (wave < NB && I0 + wave < a.n_qb) {
        if constexpr (R > 0) select_row<R>(rows + wave * n, bh, I0 + wave, a);
        else select_row_lds(rows + wave * n, bh, I0 + wave, a);
    }
}

template <typename T, int BQ>
static size_t pama_lds_bytes_t(int n_kb) {
    constexpr int NB = PamaShape<T>::QWG / BQ;
    return PamaStage<128>::BYTES + ((size_t)(kPamaThreads / kWave + NB) * n_kb + PamaShape<T>::QWG) * sizeof(float);
}

// d = 128 bound (the staging tile of d = 64 is smaller)
size_t pama_lds_bytes(int n_kb, int BQ, int dtype) {
    if (dtype == SA_BF16) return BQ == 128 ? pama_lds_bytes_t<bf16, 128>(n_kb) : pama_lds_bytes_t<bf16, 64>(n_kb);
    return BQ == 128 ? pama_lds_bytes_t<float, 128>(n_kb) : pama_lds_bytes_t<float, 64>(n_kb);
}

template <typename T, int D, int BQ, int R>
static hipError_t launch_pama_t(const void *q, const SelectArgs &a, int BH, hipStream_t st) {
    constexpr int NB = PamaShape<T>::QWG / BQ;
    const size_t lds = pama_lds_bytes_t<T, BQ>(a.n_kb);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)pama_kernel<T, D, BQ, R>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((pama_kernel<T, D, BQ, R>), dim3((a.n_qb + NB - 1) / NB * BH), dim3(kPamaThreads), lds, st,
                       (const T *)q, a);
    return hipGetLastError();
}

template <typename T, int D, int BQ>
static hipError_t launch_pama_b(const void *q, const SelectArgs &a, int BH, hipStream_t st) {
    const int chunks = (a.n_kb + kWave - 1) / kWave;
    if (chunks <= 4) return launch_pama_t<T, D, BQ, 4>(q, a, BH, st);
    if (chunks <= 8) return launch_pama_t<T, D, BQ, 8>(q, a, BH, st);
    if (chunks <= 16) return launch_pama_t<T, D, BQ, 16>(q, a, BH, st);
    if (chunks <= 20) return launch_pama_t<T, D, BQ, 20>(q, a, BH, st);
    return launch_pama_t<T, D, BQ, 0>(q, a, BH, st);
}

template <typename T>
static hipError_t launch_pama_dt(int D, const void *q, const SelectArgs &a, int BH, hipStream_t st) {
    if (D == 128) return a.block_q == 128 ? launch_pama_b<T, 128, 128>(q, a, BH, st)
                                          : launch_pama_b<T, 128, 64>(q, a, BH, st);
    return a.block_q == 128 ? launch_pama_b<T, 64, 128>(q, a, BH, st) : launch_pama_b<T, 64, 64>(q, a, BH, st);
}

// --------------------------------------------------------------------- order
__device__ __forceinline__ int cost_band(int32_t c) { return c > 1 ? 31 - __clz(c) : 0; }

// One workgroup of 16 waves.  The items are cut into at most kOrderTiles
// tiles of consecutive items (64 * m each); a wave owns whole tiles and reads
// them 64 items at a time (coalesced).  Pass 1 counts each tile's items per
// band row r = kBands-1-band (row 0: highest band); the exclusive prefix over
// the counts in (row, tile) order is where a tile's first item of row r goes;
// pass 2 places the items, ranking equal rows within 64 items by lane.  The
// order is therefore by row, then by item: a stable sort.
__global__ __launch_bounds__(kOrderThreads) void order_kernel(const int32_t *cost, int32_t *work_order, int W) {
    constexpr int NW = kOrderThreads / kWave;
    static_assert(kBands * 32 % kOrderThreads == 0, "scan split");
    __shared__ int32_t cnt[kBands * kOrderTiles];         // [row][tile]
    __shared__ int32_t part[NW];
    if (W <= 0) return;
    // tiles in use: one per 64 items, a multiple of 32 (so that the scan splits
    // evenly over the threads), at most kOrderTiles
    const int T = min(kOrderTiles, ((W + kWave - 1) / kWave + 31) / 32 * 32);
    const int kCells = kBands * T;
    const int kPer = kCells / kOrderThreads;
    const int t = threadIdx.x, lane = lane_id(), wave = t / kWave;
    const int m = (W + kWave * T - 1) / (kWave * T);      // 64-item chunks per tile
    const int span = kWave * m;
    const int n_tiles = (W + span - 1) / span;
    for (int e = t; e < kCells; e += kOrderThreads) cnt[e] = 0;
    __syncthreads();
    for (int tile = wave; tile < n_tiles; tile += NW) {
        for (int c = 0; c < m; ++c) {
            const int i = tile * span + c * kWave + lane;
            const int row = i < W ? kBands - 1 - cost_band(cost[i]) : -1;
            uint64_t left = __ballot(row >= 0);
            while (left) {
                const int r = __builtin_amdgcn_readlane(row, __builtin_ctzll(left));
                const uint64_t mr = __ballot(row == r);
                if (lane == 0) cnt[r * T + tile] += __popcll(mr);
                left &= ~mr;
            }
        }
    }
    __syncthreads();
    // exclusive scan of cnt: thread t takes kPer consecutive cells
    int32_t *mine = cnt + t * kPer;
    int sum = 0;
    for (int e = 0; e < kPer; ++e) sum += mine[e];
    int incl = sum;                                        // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) part[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += part[w];
    int run = before + incl - sum;
    for (int e = 0; e < kPer; ++e) {
        const int c = mine[e];
        mine[e] = run;
        run += c;
    }
    __syncthreads();
    for (int tile = wave; tile < n_tiles; tile += NW) {
        for (int c = 0; c < m; ++c) {
            const int i = tile * span + c * kWave + lane;
            const int row = i < W ? kBands - 1 - cost_band(cost[i]) : -1;
            uint64_t left = __ballot(row >= 0);
            while (left) {
                const int r = __builtin_amdgcn_readlane(row, __builtin_ctzll(left));
                const uint64_t mr = __ballot(row == r);
                const int base = cnt[r * T + tile];
                if (row == r) work_order[base + __popcll(mr & lanes_below())] = i;
                if (lane == 0) cnt[r * T + tile] = base + __popcll(mr);
                left &= ~mr;
            }
        }
    }
}

// Head-major work order, for long work lists: heads by total cost (highest
// first, lower index on ties), within a head by cost band (highest first) and
// then by query block.  A head's neighbouring query blocks, which keep mostly the
// same key blocks, then run together and share the key and value tiles in the
// dies' L2 and the Infinity Cache, while the heads' order keeps the most
// expensive work first.  One launch, one workgroup per head, no exchange between
// workgroups: every workgroup sums the costs of all heads itself (each wave whole
// heads, their loads issued first; W <= 48 * 1024 costs, read from the L2), ranks
// its own head among them, and one wave then sorts the head's items stably by
// band (costs held in registers, n_qb <= kHeadChunks * 64; band counts and
// running offsets in lane registers, lane r for band row r) into the head's slot
// rank * n_qb of the list.
constexpr int kHeadChunks = 32;
constexpr int kHeadMaxItems = 48 * 1024;

__global__ __launch_bounds__(kOrderThreads) void order_head_kernel(const int32_t *cost, int32_t *work_order, int BH,
                                                                   int n_qb) {
    __shared__ int32_t hcost[kOrderThreads];
    __shared__ int32_t rank_of;
    const int h = blockIdx.x, t = threadIdx.x, lane = lane_id(), wave = t / kWave;
    const int chunks = (n_qb + kWave - 1) / kWave;
    for (int g = wave; g < BH; g += kOrderThreads / kWave) {
        int c[kHeadChunks];
#pragma unroll
        for (int r = 0; r < kHeadChunks; ++r) {
            const int I = r * kWave + lane;
            c[r] = (r < chunks && I < n_qb) ? cost[(size_t)g * n_qb + I] : 0;
        }
        int sum = 0;
#pragma unroll
        for (int r = 0; r < kHeadChunks; ++r) sum += c[r];
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) sum += __shfl_xor(sum, o, kWave);
        if (lane == 0) hcost[g] = sum;
    }
    if (t == 0) rank_of = 0;
    __syncthreads();
    {
        const int ch = hcost[h];
        int before = 0;
        for (int g = t; g < BH; g += kOrderThreads) {
            const int cg = hcost[g];
            before += (cg > ch || (cg == ch && g < h)) ? 1 : 0;
        }
        before = (int)wave_sum((float)before);          // exact: at most 1024
        if (lane == 0 && before) atomicAdd(&rank_of, before);
    }
    __syncthreads();
    if (wave != 0) return;
    const int base_slot = rank_of * n_qb;
    int row[kHeadChunks];
#pragma unroll
    for (int r = 0; r < kHeadChunks; ++r) {
        const int I = r * kWave + lane;
        row[r] = (r < chunks && I < n_qb) ? cost[(size_t)h * n_qb + I] : -1;
    }
#pragma unroll
    for (int r = 0; r < kHeadChunks; ++r) row[r] = row[r] >= 0 ? kBands - 1 - cost_band(row[r]) : -1;
    int cnt = 0;                                    // lane r < kBands: items of band row r
#pragma unroll
    for (int r = 0; r < kHeadChunks; ++r) {
        if (r >= chunks) break;
        uint64_t left = __ballot(row[r] >= 0);
        while (left) {
            const int rr = __builtin_amdgcn_readlane(row[r], __builtin_ctzll(left));
            const uint64_t mr = __ballot(row[r] == rr);
            cnt += lane == rr ? __popcll(mr) : 0;
            left &= ~mr;
        }
    }
    // exclusive prefix over the band rows (lanes 0..kBands-1)
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < kBands; o <<= 1) {
        const int y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
    }
    int next = base_slot + incl - cnt;              // lane r: where band row r's next item goes
#pragma unroll
    for (int r = 0; r < kHeadChunks; ++r) {
        if (r >= chunks) break;
        uint64_t left = __ballot(row[r] >= 0);
        while (left) {
            const int rr = __builtin_amdgcn_readlane(row[r], __builtin_ctzll(left));
            const uint64_t mr = __ballot(row[r] == rr);
            const int base = __builtin_amdgcn_readlane(next, rr);
            if (row[r] == rr) work_order[base + __popcll(mr & lanes_below())] = h * n_qb + r * kWave + lane;
            next += lane == rr ? __popcll(mr) : 0;
            left &= ~mr;
        }
    }
}

// The head-major order serves long work lists (many items per workgroup slot of
// the attention kernel); shorter lists keep the global cost-band order, whose
// tail balances better.
constexpr int kHeadOrderMinItems = 16 * 768;

bool head_major_order(int BH, int n_qb) {
    const int64_t W = (int64_t)BH * n_qb;
    return W >= kHeadOrderMinItems && W <= kHeadMaxItems && n_qb <= kHeadChunks * kWave && BH <= kOrderThreads;
}

// --------------------------------------------------------------------- launch
template <typename T, int D>
static hipError_t launch_pool_t(const void *q, const void *k, const void *v, const PoolArgs &a,
                                int BH, hipStream_t st) {
    dim3 grid((a.N + 127) / 128, BH, 3 - a.first);
    hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(kPoolThreads), 0, st,
                       (const T *)q, (const T *)k, (const T *)v, a);
    return hipGetLastError();
}

hipError_t launch_pool(int dtype, int D, const void *q, const void *k, const void *v,
                       const PoolArgs &a, int BH, hipStream_t st) {
    if (dtype == SA_BF16) return D == 64 ? launch_pool_t<bf16, 64>(q, k, v, a, BH, st)
                                         : launch_pool_t<bf16, 128>(q, k, v, a, BH, st);
    return D == 64 ? launch_pool_t<float, 64>(q, k, v, a, BH, st)
                   : launch_pool_t<float, 128>(q, k, v, a, BH, st);
}

// Query blocks per select workgroup: as many proxy rows as the LDS budget
// holds (each workgroup reads all mean keys of its head once), at most 16.
int select_group(int n_kb, int D, int n_qb) {
    (void)D;
    static const int kG[] = {16, 12, 8, 4, 1};
    int i = 0;
    while (kG[i] > 1 && select_lds_bytes(kG[i], n_kb, D) > kSelectLdsBudget) ++i;
    while (kG[i] > 1 && kG[i + 1] >= n_qb) ++i;
    return kG[i];
}

size_t select_lds_bytes(int G, int n_kb, int D) {
    // the proxy rows, or the group's query means before them
    const size_t rows = ((size_t)G * n_kb + 3) / 4 * 4;
    return (rows > (size_t)G * D ? rows : (size_t)G * D) * sizeof(float);
}

template <int D, int G, int R>
static hipError_t launch_select_t(const SelectArgs &a, int BH, hipStream_t st) {
    const size_t lds = select_lds_bytes(G, a.n_kb, D);
    dim3 grid((a.n_qb + G - 1) / G * BH);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)select_kernel<D, G, R>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((select_kernel<D, G, R>), grid, dim3(kSelectThreads), lds, st, a);
    return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_select_g(const SelectArgs &a, int BH, hipStream_t st) {
    const int chunks = (a.n_kb + kWave - 1) / kWave;
    if (chunks <= 4) return launch_select_t<D, G, 4>(a, BH, st);
    if (chunks <= 8) return launch_select_t<D, G, 8>(a, BH, st);
    if (chunks <= 16) return launch_select_t<D, G, 16>(a, BH, st);
    if (chunks <= 20) return launch_select_t<D, G, 20>(a, BH, st);
    return launch_select_t<D, G, 0>(a, BH, st);
}

template <int D>
static hipError_t launch_select_d(const SelectArgs &a, int G, int BH, hipStream_t st) {
    switch (G) {
        case 16: return launch_select_g<D, 16>(a, BH, st);
        case 12: return launch_select_g<D, 12>(a, BH, st);
        case 8: return launch_select_g<D, 8>(a, BH, st);
        case 4: return launch_select_g<D, 4>(a, BH, st);
        default: return launch_select_g<D, 1>(a, BH, st);
    }
}

hipError_t launch_select(int D, const SelectArgs &a, int BH, hipStream_t st, int dtype, const void *q) {
    hipError_t e = hipSuccess;
    if (q) {
        e = dtype == SA_BF16 ? launch_pama_dt<bf16>(D, q, a, BH, st) : launch_pama_dt<float>(D, q, a, BH, st);
    } else {
        const int G = select_group(a.n_kb, D, a.n_qb);
        e = D == 64 ? launch_select_d<64>(a, G, BH, st) : launch_select_d<128>(a, G, BH, st);
    }
    if (e != hipSuccess) return e;
    // (fused routing too: its pre-pass writes the costs of the decisions the
    // forward will take)
    if (head_major_order(BH, a.n_qb)) {
        hipLaunchKernelGGL(order_head_kernel, dim3(BH), dim3(kOrderThreads), 0, st, (const int32_t *)a.cost,
                           a.work_order, BH, a.n_qb);
    } else
        hipLaunchKernelGGL(order_kernel, dim3(1), dim3(kOrderThreads), 0, st, (const int32_t *)a.cost, a.work_order,
                           BH * a.n_qb);
    return hipGetLastError();
}

}  // namespace sa
