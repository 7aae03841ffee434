// Routing kernels: block pooling, proxy scoring and block selection, and the
// cost-ordered work list for the attention kernel.
//
// pool    one workgroup per (b, h, 128-token span, tensor) reduces the span's
//         one or two blocks to fp32 means with coalesced 16-byte loads
//         (HBM-bound; the inputs are read exactly once).  Block centroids: PARK page,
//         section 4.1.
// select  one workgroup per (b, h, group of G query blocks): the G proxy rows
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
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

constexpr int kPoolThreads = 256;
constexpr int kSelectThreads = 256;
constexpr int kOrderThreads = 512;
constexpr int kBands = 32;               // floor(log2(cost)) of a non-negative int32

// --------------------------------------------------------------------- pool
template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(const T *__restrict__ q,
                                                            const T *__restrict__ k,
                                                            const T *__restrict__ v,
                                                            PoolArgs a) {
    // one workgroup per 128-token span of one tensor: one block of 128 or two of 64
    const int which = blockIdx.z;            // 0 = q, 1 = k, 2 = v
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
#pragma unroll
    for (int it = 0; it < 128 / RG; ++it) {
        const int r = g + it * RG;
        if (r < span) {
            float x[8];
            Ld8<T>::load_f32(X + (size_t)(r0 + r) * D + c * 8, x);
            const int b = r >= bs;             // RG divides bs: uniform per iteration
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[b][i] += x[i];
        }
    }
    __shared__ float part[2][RG * D];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 8; ++i) part[b][g * D + c * 8 + i] = acc[b][i];
    __syncthreads();
    const int nblk = (span + bs - 1) / bs;
    if (threadIdx.x < nblk * D) {
        const int b = threadIdx.x / D, col = threadIdx.x % D;
        const int J = (r0 + b * bs) / bs;
        const int cnt = min(bs, a.N - J * bs);
        float s = 0.f;                    // other blocks' rows left zeros here
        for (int gg = 0; gg < RG; ++gg) s += part[b][gg * D + col];
        const float m = s / (float)cnt;
        float *dst = which == 0 ? a.q_mean : which == 1 ? a.k_mean : a.v_mean;
        dst[((size_t)bh * nb + J) * D + col] = m;
        if (which != 0) {
            // residual tile rows: block J -> group J/32, row J%32 (bf16 of the mean)
            // and row 32 + J%32 (bf16 of what that rounding left)
            bf16 *sp = a.kv_split + (((size_t)bh * 2 + (which - 1)) * a.words + J / 32) * 64 * D;
            const bf16 hi = (bf16)m;
            sp[(size_t)(J % 32) * D + col] = hi;
            sp[(size_t)(32 + J % 32) * D + col] = (bf16)(m - (float)hi);
            if (J == nb - 1) {
                for (int r = J % 32 + 1; r < 32; ++r) {
                    sp[(size_t)r * D + col] = (bf16)0.f;
                    sp[(size_t)(32 + r) * D + col] = (bf16)0.f;
                }
            }
        }
    }
}

// --------------------------------------------------------------------- select
__device__ __forceinline__ uint64_t lanes_below() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

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
        if (orderable(S[J]) >= kmin) ms += expf(S[J] - lse);
    return wave_sum(ms);
}

// Rows longer than 20 * 64 key blocks: the same steps, reading the row from LDS.
__device__ __forceinline__ void select_row_lds(const float *S, int bh, int I, const SelectArgs &a) {
    const int lane = lane_id();
    const int n = a.n_kb;
    float m = -INFINITY;
    for (int J = lane; J < n; J += kWave) m = fmaxf(m, S[J]);
    m = wave_max(m);
    float z = 0.f;
    for (int J = lane; J < n; J += kWave) z += expf(S[J] - m);
    z = wave_sum(z);
    const float lse = m + logf(z);
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
                    if (orderable(S[J]) == Ts) peq = expf(S[J] - lse);
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

// One proxy row: statistics, the tau test, the cap or floor, the kept list,
// bit mask and cost.  The lane holds scores J = lane + 64 i, i < R, in registers
// (R * 64 >= n_kb): every pass over the row, in particular the 32 counting
// passes of the cap's k-th-largest search, runs on registers.
template <int R>
__device__ __forceinline__ void select_row(const float *S, int bh, int I, const SelectArgs &a) {
    const int lane = lane_id();
    const int n = a.n_kb;
    // absent entries (J >= n) hold -inf and key 0, below every real key
    float sv[R];
    uint32_t key[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int J = i * kWave + lane;
        sv[i] = J < n ? S[J] : -INFINITY;
        key[i] = J < n ? orderable(sv[i]) : 0u;
    }
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < R; ++i) m = fmaxf(m, sv[i]);
    m = wave_max(m);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i)
        if (key[i] != 0u) z += expf(sv[i] - m);
    z = wave_sum(z);
    const float lse = m + logf(z);
    const float thr = (a.tau_mode == SA_TAU_ABSOLUTE ? lse : m) + a.ln_tau;

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
        for (int i = 0; i < R; ++i) pv[i] = key[i] != 0u ? expf(sv[i] - lse) : 0.f;
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
                    ngt += __popcll(__ballot(key[i] > Ts));
                    neq += __popcll(__ballot(key[i] == Ts));
                }
                mgt = wave_sum(mgt);
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
        for (int i = 0; i < R; ++i) n_c += __popcll(__ballot(key[i] != 0u && sv[i] >= thr));
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
            for (int i = 0; i < R; ++i) cnt += __popcll(__ballot(key[i] >= cand));
            if (cnt >= ksel) T = cand;
        }
        int n_gt = 0;
        if (T != 0xffffffffu)
#pragma unroll
            for (int i = 0; i < R; ++i) n_gt += __popcll(__ballot(key[i] > T));
        take_eq = ksel - n_gt;
    }

    const size_t row = (size_t)bh * a.n_qb + I;
    int32_t *idx = a.kv_idx + row * a.kv_idx_cap;
    uint32_t *mask = a.kv_mask + row * a.mask_words;
    const bool dense_row = (int64_t)I * a.block_q < a.n_prefix;
    const int last_cnt = a.N - (n - 1) * a.block_k;
    int kept = 0, eq_seen = 0, tiles = 0;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int J = i * kWave + lane;
        const bool valid = key[i] != 0u;
        bool keep;
        if (ksel > 0) {
            const bool eq = valid && key[i] == T;
            const uint64_t be = __ballot(eq);
            const int rank = eq_seen + __popcll(be & lanes_below());
            eq_seen += __popcll(be);
            keep = valid && (key[i] > T || (eq && rank < take_eq));
        } else {
            keep = valid && a.tau_mode != SA_TAU_TOPP && sv[i] >= thr;   // TOPP: n_c = 0
        }
        keep = valid && (keep || dense_row || (int64_t)J * a.block_k < a.n_prefix);
        const uint64_t bk = __ballot(keep);
        if (keep) idx[kept + __popcll(bk & lanes_below())] = J;
        kept += __popcll(bk);
        const int w = 2 * i;
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

template <int D, int G>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(SelectArgs a) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    const int bh = blockIdx.y;
    const int I0 = blockIdx.x * G;
    const int g_cnt = min(G, a.n_qb - I0);
    const int n = a.n_kb;
    float *S = smem;                                      // [G][n]
    float *QB = smem + ((G * n + 3) & ~3);                // [G][D]
    for (int i = threadIdx.x; i < G * D; i += kSelectThreads)
        QB[i] = (i / D) < g_cnt ? a.q_mean[((size_t)bh * a.n_qb + I0) * D + i] : 0.f;
    __syncthreads();
    const float *kb = a.k_mean + (size_t)bh * n * D;
    for (int J = threadIdx.x; J < n; J += kSelectThreads) {
        float acc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = 0.f;
        const float *kr = kb + (size_t)J * D;
#pragma unroll 4
        for (int c = 0; c < D; c += 4) {
            const f32x4 kv = *reinterpret_cast<const f32x4 *>(kr + c);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const f32x4 qv = *reinterpret_cast<const f32x4 *>(QB + g * D + c);
                acc[g] = fmaf(qv[0], kv[0], acc[g]);
                acc[g] = fmaf(qv[1], kv[1], acc[g]);
                acc[g] = fmaf(qv[2], kv[2], acc[g]);
                acc[g] = fmaf(qv[3], kv[3], acc[g]);
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) S[g * n + J] = acc[g] * a.scale;
    }
    __syncthreads();
    const int wave = threadIdx.x / kWave;
    const int chunks = (n + kWave - 1) / kWave;        // uniform over the launch
    for (int g = wave; g < g_cnt; g += kSelectThreads / kWave) {
        const float *row = S + g * n;
        if (chunks <= 2) select_row<2>(row, bh, I0 + g, a);
        else if (chunks <= 4) select_row<4>(row, bh, I0 + g, a);
        else if (chunks <= 8) select_row<8>(row, bh, I0 + g, a);
        else if (chunks <= 16) select_row<16>(row, bh, I0 + g, a);
        else if (chunks <= 20) select_row<20>(row, bh, I0 + g, a);
        else select_row_lds(row, bh, I0 + g, a);
    }
}

// --------------------------------------------------------------------- order
__device__ __forceinline__ int cost_band(int32_t c) { return c > 1 ? 31 - __clz(c) : 0; }

// One workgroup.  Thread t owns the items of one contiguous chunk; cnt[r][t]
// counts its items in row r = kBands-1-band (row 0: highest band).  The
// exclusive prefix over cnt in (row, thread) order is then where thread t
// writes its first item of row r, which makes the sort stable.
__global__ __launch_bounds__(kOrderThreads) void order_kernel(const int32_t *cost, int32_t *work_order, int W) {
    __shared__ int32_t cnt[kBands * kOrderThreads];
    __shared__ int32_t part[kOrderThreads];
    const int t = threadIdx.x;
    const int chunk = (W + kOrderThreads - 1) / kOrderThreads;
    const int i0 = min(W, t * chunk), i1 = min(W, i0 + chunk);
    for (int r = 0; r < kBands; ++r) cnt[r * kOrderThreads + t] = 0;
    for (int i = i0; i < i1; ++i) ++cnt[(kBands - 1 - cost_band(cost[i])) * kOrderThreads + t];
    __syncthreads();
    // thread t scans the kBands consecutive entries [t*kBands, (t+1)*kBands) of cnt
    constexpr int kPer = kBands;   // kBands * kOrderThreads entries / kOrderThreads threads
    int32_t *mine = cnt + t * kPer;
    int sum = 0;
    for (int e = 0; e < kPer; ++e) sum += mine[e];
    part[t] = sum;
    __syncthreads();
    for (int off = 1; off < kOrderThreads; off <<= 1) {       // inclusive scan of part
        const int v = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    int run = t > 0 ? part[t - 1] : 0;
    for (int e = 0; e < kPer; ++e) {
        const int c = mine[e];
        mine[e] = run;
        run += c;
    }
    __syncthreads();
    for (int i = i0; i < i1; ++i) {
        const int slot = (kBands - 1 - cost_band(cost[i])) * kOrderThreads + t;
        work_order[cnt[slot]++] = i;
    }
}

// --------------------------------------------------------------------- launch
template <typename T, int D>
static hipError_t launch_pool_t(const void *q, const void *k, const void *v, const PoolArgs &a,
                                int BH, hipStream_t st) {
    dim3 grid((a.N + 127) / 128, BH, 3);
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

int select_group(int n_kb, int D, int n_qb) {
    int G = 8;
    while (G > 1 && ((size_t)G * n_kb + 4 + (size_t)G * D) * 4 > kSelectLdsBudget) G /= 2;
    while (G > 1 && G / 2 >= n_qb) G /= 2;
    return G;
}

size_t select_lds_bytes(int G, int n_kb, int D) {
    return (((size_t)G * n_kb + 3) / 4 * 4 + (size_t)G * D) * sizeof(float);
}

template <int D, int G>
static hipError_t launch_select_t(const SelectArgs &a, int BH, hipStream_t st) {
    const size_t lds = select_lds_bytes(G, a.n_kb, D);
    dim3 grid((a.n_qb + G - 1) / G, BH);
    hipLaunchKernelGGL((select_kernel<D, G>), grid, dim3(kSelectThreads), lds, st, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_select_d(const SelectArgs &a, int G, int BH, hipStream_t st) {
    switch (G) {
        case 8: return launch_select_t<D, 8>(a, BH, st);
        case 4: return launch_select_t<D, 4>(a, BH, st);
        case 2: return launch_select_t<D, 2>(a, BH, st);
        default: return launch_select_t<D, 1>(a, BH, st);
    }
}

hipError_t launch_select(int D, const SelectArgs &a, int BH, hipStream_t st) {
    const int G = select_group(a.n_kb, D, a.n_qb);
    hipError_t e = hipSuccess;
    e = D == 64 ? launch_select_d<64>(a, G, BH, st) : launch_select_d<128>(a, G, BH, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(order_kernel, dim3(1), dim3(kOrderThreads), 0, st, (const int32_t *)a.cost, a.work_order,
                       BH * a.n_qb);
    return hipGetLastError();
}

}  // namespace sa
