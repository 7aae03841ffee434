// Block-sparse attention with a dropped-block residual, one online-softmax pass
// (Sol-Attn abstract: dynamic routing, sparse computation and approximation
// correction in a single online-softmax pass).
//
// One workgroup per (b, h, query block).  Each wave owns 32 query rows and
// keeps them as the B operand of v_mfma_f32_32x32x16_bf16 for the whole pass.
// The kernel walks a stream of key/value tiles:
//   exact tiles     the tokens of the kept key blocks, in ascending block order
//                   (64 bf16 tokens, or 32 fp32 tokens in hi/lo split form)
//   residual tiles  32 block means (fp32, hi/lo split) with an additive logit
//                   bias of log2(n_J) for dropped blocks and -inf for kept
//                   ones; a tile whose 32 blocks are all kept is skipped
// and folds both kinds into the same running max and normaliser.
//
// Layout choice: scores are formed transposed, S^T = K Q^T, so that the MFMA
// accumulator gives each lane a single query row (lane & 31) and 32 of the
// tile's keys.  The output is formed transposed too, O^T = V^T P^T: the P^T
// operand is then exactly what each lane already holds after the softmax, and
// the per-row max, normaliser and rescale factor are per-lane scalars (the two
// lane halves holding the same row combine once per tile with one shuffle for
// the max, and once at the end for the normaliser).  K is staged row-major in
// LDS; V is staged transposed (V^T, keys contiguous per feature) with keys
// permuted inside each group of 16 so that every operand fetch is one 16-byte
// LDS read.  Both are padded by 16 bytes per row against bank conflicts and
// double-buffered: the global loads of tile t+1 are in flight while tile t is
// computed.
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

template <int D, int BQ>
struct FC {
    static constexpr int WAVES = BQ / 32;
    static constexpr int THREADS = WAVES * kWave;
    static constexpr int KSTR = D + 8;               // bf16 elements per K row in LDS
    static constexpr int VSTR = kTile + 8;           // bf16 elements per V^T row in LDS
    static constexpr int K_ELEMS = kTile * KSTR;
    static constexpr int V_ELEMS = D * VSTR;
    static constexpr int BUF = K_ELEMS + V_ELEMS;
    static constexpr size_t LDS = 2 * (size_t)BUF * sizeof(bf16);
    // 16-byte global chunks per tile: 64 bf16 rows or 32 fp32 rows of K (8D), and
    // the same for V in 4-row groups (2D); equal for both tile formats
    static constexpr int K_UNITS = 8 * D;
    static constexpr int V_UNITS = 2 * D;
    static constexpr int KU = (K_UNITS + THREADS - 1) / THREADS;
    static constexpr int VU = (V_UNITS + THREADS - 1) / THREADS;
    // waves per SIMD the register budget targets: two 128-row workgroups share a
    // CU; a 64-row workgroup (2 waves) gets the full register file
    static constexpr int WPE = BQ == 128 ? 2 : 1;
};

// Tile kinds.  A "split" tile covers 32 rows of fp32 data: LDS rows 0..31 hold
// the bf16 round-to-nearest part of each row and rows 32..63 the bf16 remainder
// (x - hi), for both K and V, so the same 64-column MFMA sequence yields
// hi + lo products: logits to about 2^-16 relative instead of 2^-9.
enum : int {
    kExact = 0,        // 64 bf16 tokens of a kept block
    kExactSplit = 1,   // 32 fp32 tokens of a kept block (fp32 inputs)
    kResidual = 2,     // 32 block means (fp32), dropped blocks only
};

struct TileDesc {
    int kind;
    int row0;      // first token (exact) or first pooled block (residual)
    int valid;     // rows of the tile that exist
    uint32_t kept; // residual: kept bits of the tile's 32 pooled blocks (1 past n_kb)
};

// The tile sequence of one work item; every thread steps it identically and
// every field is wave-uniform.
struct TileStream {
    const int32_t *list;
    const uint32_t *mask;
    int cnt, li, sub;
    int exact_rows, exact_kind;
    int dense_tiles, t;
    int rt, n_rt;

    __device__ bool next(TileDesc &o, const FlashArgs &a) {
        if (!list) {
            if (t < dense_tiles) {
                o.kind = exact_kind;
                o.row0 = t * exact_rows;
                o.valid = min(exact_rows, a.N - o.row0);
                ++t;
                return true;
            }
            return false;
        }
        while (li < cnt) {
            const int J = __builtin_amdgcn_readfirstlane(list[li]);
            const int b0 = J * a.block_k;
            const int b1 = min(b0 + a.block_k, a.N);
            const int tok0 = b0 + sub * exact_rows;
            ++sub;
            if (b0 + sub * exact_rows >= b1) {
                ++li;
                sub = 0;
            }
            if (tok0 < b1) {
                o.kind = exact_kind;
                o.row0 = tok0;
                o.valid = min(exact_rows, b1 - tok0);
                return true;
            }
        }
        while (rt < n_rt) {
            const int cur = rt++;
            const uint32_t bits = (uint32_t)__builtin_amdgcn_readfirstlane(mask[cur]);
            const int lim = a.n_kb - cur * 32;
            const uint32_t vmask = lim >= 32 ? ~0u : ((1u << lim) - 1u);
            if ((~bits & vmask) != 0) {
                o.kind = kResidual;
                o.row0 = cur * 32;
                o.valid = min(32, lim);
                o.kept = bits | ~vmask;
                return true;
            }
        }
        return false;
    }
};

template <int D, int BQ>
struct Staging {
    u32x4 k[FC<D, BQ>::KU];
    u32x4 v[FC<D, BQ>::VU][4];
};

// Buffer resource over `bytes` bytes at `base`: loads past the end return zero.
// Rows of a tile past its valid count only ever lie past the end of a head's
// tensor (blocks are multiples of the tile height except the last one), so the
// hardware range check supplies the zero fill.  All offsets go in the VGPR
// offset, which the range check covers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Per-thread byte offsets of a tile's 16-byte chunks inside the tile; they
// stay fixed for the whole pass (the tile position goes into the buffer
// resource's base), so the offset registers are never rewritten while loads
// are in flight.
template <int D, int BQ>
struct TileOffsets {
    int kb[FC<D, BQ>::KU];     // 64 bf16 rows: K unit u = (row u/(D/8), 8 columns)
    int vb[FC<D, BQ>::VU];     //               V unit u = (rows 4g..4g+3, 8 columns), row 4g
    int kf[FC<D, BQ>::KU];     // 32 fp32 rows: K unit u = (row u/(D/4), 4 columns)
    int vf[FC<D, BQ>::VU];     //               V unit u = (rows 4g..4g+3, 4 columns), row 4g

    __device__ void init() {
        using C = FC<D, BQ>;
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < C::KU; ++i) {
            const int u = tid + i * C::THREADS;
            kb[i] = (u / (D / 8)) * (D * 2) + (u % (D / 8)) * 16;
            kf[i] = (u / (D / 4)) * (D * 4) + (u % (D / 4)) * 16;
        }
#pragma unroll
        for (int i = 0; i < C::VU; ++i) {
            const int u = tid + i * C::THREADS;
            vb[i] = (4 * (u % 16)) * (D * 2) + (u / 16) * 16;
            vf[i] = (4 * (u % 8)) * (D * 4) + (u / 8) * 16;
        }
    }
};

template <int D, int BQ>
__device__ __forceinline__ void load_bf16(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                          const TileOffsets<D, BQ> &to, Staging<D, BQ> &st) {
    using C = FC<D, BQ>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::KU; ++i)
        if (C::K_UNITS % C::THREADS == 0 || tid + i * C::THREADS < C::K_UNITS) st.k[i] = bload(rk, to.kb[i]);
#pragma unroll
    for (int i = 0; i < C::VU; ++i)
        if (C::V_UNITS % C::THREADS == 0 || tid + i * C::THREADS < C::V_UNITS) {
#pragma unroll
            for (int r = 0; r < 4; ++r) st.v[i][r] = __builtin_amdgcn_raw_buffer_load_b128(rv, to.vb[i], r * (D * 2), 0);
        }
}

template <int D, int BQ>
__device__ __forceinline__ void load_f32(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                         const TileOffsets<D, BQ> &to, Staging<D, BQ> &st) {
    using C = FC<D, BQ>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::KU; ++i)
        if (C::K_UNITS % C::THREADS == 0 || tid + i * C::THREADS < C::K_UNITS) st.k[i] = bload(rk, to.kf[i]);
#pragma unroll
    for (int i = 0; i < C::VU; ++i)
        if (C::V_UNITS % C::THREADS == 0 || tid + i * C::THREADS < C::V_UNITS) {
#pragma unroll
            for (int r = 0; r < 4; ++r) st.v[i][r] = __builtin_amdgcn_raw_buffer_load_b128(rv, to.vf[i], r * (D * 4), 0);
        }
}

// V^T position of key 4g (the 4 keys 4g..4g+3 stay contiguous): bits 2 and 3 of
// the key offset inside its group of 16 are swapped, so that the 8 keys a lane
// contributes to one P^T operand are adjacent.
__device__ __forceinline__ int vt_pos(int g) { return 16 * (g >> 2) + 4 * (((g & 1) << 1) | ((g >> 1) & 1)); }

__device__ __forceinline__ bf16x4 bf16x4_of(float a, float b, float c, float d) {
    bf16x4 x;
    x[0] = (bf16)a; x[1] = (bf16)b; x[2] = (bf16)c; x[3] = (bf16)d;
    return x;
}

template <int D, int BQ>
__device__ __forceinline__ void store_bf16(bf16 *buf, const Staging<D, BQ> &st) {
    using C = FC<D, BQ>;
    const int tid = threadIdx.x;
    bf16 *Ks = buf;
    bf16 *Vt = buf + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::KU; ++i) {
        const int u = tid + i * C::THREADS;
        if (C::K_UNITS % C::THREADS == 0 || u < C::K_UNITS) {
            const int row = u / (D / 8), ch = u % (D / 8);
            *reinterpret_cast<u32x4 *>(Ks + row * C::KSTR + ch * 8) = st.k[i];
        }
    }
#pragma unroll
    for (int i = 0; i < C::VU; ++i) {
        const int u = tid + i * C::THREADS;
        if (C::V_UNITS % C::THREADS == 0 || u < C::V_UNITS) {
            const int g = u % 16, c = u / 16;
            const int pos = vt_pos(g);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // bf16 j of each row: 16-bit half (j & 1) of 32-bit word j / 2
                const int sh = 16 * (j & 1);
                u32x2 x;
                x[0] = ((st.v[i][0][j >> 1] >> sh) & 0xffffu) | (((st.v[i][1][j >> 1] >> sh) & 0xffffu) << 16);
                x[1] = ((st.v[i][2][j >> 1] >> sh) & 0xffffu) | (((st.v[i][3][j >> 1] >> sh) & 0xffffu) << 16);
                *reinterpret_cast<u32x2 *>(Vt + (8 * c + j) * C::VSTR + pos) = x;
            }
        }
    }
}

template <int D, int BQ>
__device__ __forceinline__ void store_split(bf16 *buf, const Staging<D, BQ> &st) {
    using C = FC<D, BQ>;
    const int tid = threadIdx.x;
    bf16 *Ks = buf;
    bf16 *Vt = buf + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::KU; ++i) {
        const int u = tid + i * C::THREADS;
        if (C::K_UNITS % C::THREADS == 0 || u < C::K_UNITS) {
            const int row = u / (D / 4), c4 = u % (D / 4);
            float x[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = __uint_as_float(st.k[i][e]);
                lo[e] = x[e] - (float)(bf16)x[e];
            }
            *reinterpret_cast<bf16x4 *>(Ks + row * C::KSTR + c4 * 4) = bf16x4_of(x[0], x[1], x[2], x[3]);
            *reinterpret_cast<bf16x4 *>(Ks + (row + 32) * C::KSTR + c4 * 4) = bf16x4_of(lo[0], lo[1], lo[2], lo[3]);
        }
    }
#pragma unroll
    for (int i = 0; i < C::VU; ++i) {
        const int u = tid + i * C::THREADS;
        if (C::V_UNITS % C::THREADS == 0 || u < C::V_UNITS) {
            const int g = u % 8, c = u / 8;
            const int pos = vt_pos(g);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float x[4], lo[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    x[r] = __uint_as_float(st.v[i][r][j]);
                    lo[r] = x[r] - (float)(bf16)x[r];
                }
                bf16 *row = Vt + (4 * c + j) * C::VSTR;
                *reinterpret_cast<bf16x4 *>(row + pos) = bf16x4_of(x[0], x[1], x[2], x[3]);
                *reinterpret_cast<bf16x4 *>(row + pos + 32) = bf16x4_of(lo[0], lo[1], lo[2], lo[3]);
            }
        }
    }
}

template <typename T> struct Store4;
template <> struct Store4<bf16> {
    static __device__ __forceinline__ void st(bf16 *p, float a, float b, float c, float d) {
        *reinterpret_cast<bf16x4 *>(p) = bf16x4_of(a, b, c, d);
    }
};
template <> struct Store4<float> {
    static __device__ __forceinline__ void st(float *p, float a, float b, float c, float d) {
        f32x4 x = {a, b, c, d};
        *reinterpret_cast<f32x4 *>(p) = x;
    }
};

// Key/value rows and fp32 block means of one (b, h).
template <typename T>
struct HeadSrc {
    const T *k, *v;
    const float *km, *vm;
    int n_rows, n_means;
};

// Issue the global loads of tile t: a buffer resource starting at the tile's
// first row and ending at the end of the head, so rows past the end read zero.
template <typename T, int D, int BQ>
__device__ __forceinline__ void issue_tile(const TileDesc &t, const HeadSrc<T> &hs, const TileOffsets<D, BQ> &to,
                                           Staging<D, BQ> &st) {
    if (t.kind == kResidual) {
        const uint32_t bytes = (uint32_t)(hs.n_means - t.row0) * (D * 4);
        load_f32<D, BQ>(buffer_rsrc(hs.km + (size_t)t.row0 * D, bytes), buffer_rsrc(hs.vm + (size_t)t.row0 * D, bytes),
                        to, st);
    } else {
        const uint32_t bytes = (uint32_t)(hs.n_rows - t.row0) * (D * sizeof(T));
        const auto rk = buffer_rsrc(hs.k + (size_t)t.row0 * D, bytes);
        const auto rv = buffer_rsrc(hs.v + (size_t)t.row0 * D, bytes);
        if constexpr (sizeof(T) == 2) load_bf16<D, BQ>(rk, rv, to, st);
        else load_f32<D, BQ>(rk, rv, to, st);
    }
}

// kSparse: kept-list and residual tiles from a route; otherwise every key tile (dense).
template <typename T, int D, int BQ, bool kSparse>
__global__ __launch_bounds__((FC<D, BQ>::THREADS)) __attribute__((amdgpu_waves_per_eu(FC<D, BQ>::WPE, FC<D, BQ>::WPE))) void flash_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, T *__restrict__ o,
    FlashArgs a) {
    using C = FC<D, BQ>;
    constexpr bool kF32 = sizeof(T) == 4;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    bf16 *lds = reinterpret_cast<bf16 *>(smem_raw);

    const int item = kSparse ? __builtin_amdgcn_readfirstlane(a.work_order[blockIdx.x]) : (int)blockIdx.x;
    const int bh = item / a.n_qb;
    const int I = item - bh * a.n_qb;
    const int lane = lane_id();
    const int h = lane >> 5, l32 = lane & 31;
    const int wave = threadIdx.x / kWave;
    const size_t head = (size_t)bh * a.N * D;
    const int qrow = I * a.block_q + wave * 32 + l32;
    const bool row_ok = qrow < a.N;

    // this wave's 32 query rows, as B operands (lane: row l32, features 16c + 8h + 0..7);
    // fp32 inputs also keep the bf16 remainder of each query element
    bf16x8 qf[D / 16];
    bf16x8 ql[kF32 ? D / 16 : 1];
    {
        const bf16x8 zero = {};
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            if constexpr (kF32) {
                float x[8];
                if (row_ok) Ld8<float>::load_f32(reinterpret_cast<const float *>(q) + head + (size_t)qrow * D + 16 * c + 8 * h, x);
                else
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    qf[c][e] = (bf16)x[e];
                    ql[c][e] = (bf16)(x[e] - (float)qf[c][e]);
                }
            } else {
                qf[c] = row_ok ? Ld8<T>::load(q + head + (size_t)qrow * D + 16 * c + 8 * h) : zero;
            }
        }
    }

    TileStream ts;
    ts.t = 0; ts.li = 0; ts.sub = 0; ts.rt = 0;
    ts.exact_rows = kF32 ? 32 : 64;
    ts.exact_kind = kF32 ? kExactSplit : kExact;
    ts.dense_tiles = (a.N + ts.exact_rows - 1) / ts.exact_rows;
    const size_t row_id = (size_t)bh * a.n_qb + I;
    if constexpr (kSparse) {
        ts.list = a.kv_idx + row_id * a.kv_idx_cap;
        ts.cnt = __builtin_amdgcn_readfirstlane(a.kv_count[row_id]);
        ts.mask = a.kv_mask + row_id * a.mask_words;
        ts.n_rt = a.residual ? a.mask_words : 0;
    } else {
        ts.list = nullptr;
        ts.mask = nullptr;
        ts.cnt = 0;
        ts.n_rt = 0;
    }
    HeadSrc<T> hs;
    hs.k = k + head;
    hs.v = v + head;
    hs.km = kSparse ? a.k_mean + (size_t)bh * a.n_kb * D : nullptr;
    hs.vm = kSparse ? a.v_mean + (size_t)bh * a.n_kb * D : nullptr;
    hs.n_rows = a.N;
    hs.n_means = a.n_kb;
    TileOffsets<D, BQ> to;
    to.init();
    const float lg_bk = log2f((float)a.block_k);
    const float lg_last = log2f((float)(a.N - (a.n_kb - 1) * a.block_k));

    f32x16 acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
    float m_ref = -INFINITY, l_run = 0.f;   // softmax reference (log2 units) and normaliser

    Staging<D, BQ> st;
    TileDesc cur, nxt;
    bool have = ts.next(cur, a);
    if (have) {
        issue_tile<T, D, BQ>(cur, hs, to, st);
        if (cur.kind == kExact) store_bf16<D, BQ>(lds, st);
        else store_split<D, BQ>(lds, st);
    }
    __syncthreads();
    int buf = 0;
    while (have) {
        const bool have_next = ts.next(nxt, a);
        // Nothing is in flight here (the previous tile's loads were consumed by
        // its LDS stores).  Saying so explicitly keeps the compiler from placing
        // its loop-entry wait after the prefetch below, which would expose the
        // prefetch latency on every tile.
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt/lgkmcnt untouched
        if (have_next) issue_tile<T, D, BQ>(nxt, hs, to, st);
        const bf16 *Ks = lds + buf * C::BUF;
        const bf16 *Vt = Ks + C::K_ELEMS;

        // S^T for LDS key rows 0..31 (s[0]) and 32..63 (s[1])
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            const bf16x8 k0 = *reinterpret_cast<const bf16x8 *>(Ks + l32 * C::KSTR + 16 * c + 8 * h);
            const bf16x8 k1 = *reinterpret_cast<const bf16x8 *>(Ks + (32 + l32) * C::KSTR + 16 * c + 8 * h);
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[c], s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[c], s[1], 0, 0, 0);
            if constexpr (kF32) s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, ql[c], s[0], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);

        // accumulator register r of lane (h, l32) in block b holds LDS key row
        // 32b + 8(r/4) + 4h + r%4
        const bool split = cur.kind != kExact;
        const float c = a.scale_log2;
        float mx = -INFINITY;       // this lane's tile maximum, log2 units
        if (!split) {
            if (cur.valid < kTile) {            // partial tile (uniform): drop absent keys
                const int lim = cur.valid - 4 * h;
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (32 * b + 8 * (r >> 2) + (r & 3) >= lim) s[b][r] = -INFINITY;
            }
            float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                m0 = fmaxf(m0, s[0][r]);
                m1 = fmaxf(m1, s[1][r]);
            }
            mx = fmaxf(m0, m1) * c;             // c > 0
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kv = 8 * (r >> 2) + 4 * h + (r & 3);
                float x = (s[0][r] + s[1][r]) * c;
                if (cur.kind == kResidual) {
                    const bool drop = ((cur.kept >> kv) & 1u) == 0;
                    x = drop ? x + (cur.row0 + kv == a.n_kb - 1 ? lg_last : lg_bk) : -INFINITY;
                } else {
                    x = kv < cur.valid ? x : -INFINITY;
                }
                s[0][r] = x;
                mx = fmaxf(mx, x);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        // Lazy rescaling: the reference m_ref moves only when some row of the wave
        // exceeds it by more than 8 (log2 units), so weights stay <= 2^8 and the
        // accumulator rescale is skipped on most tiles.  The result is the same
        // softmax: numerator and normaliser share the reference.
        if (__ballot(mx > m_ref + 8.f) != 0) {
            const float m_new = fmaxf(m_ref, mx);
            const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
            m_ref = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
        }
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
        float ps0 = 0.f, ps1 = 0.f;
        // P^T operands: step j takes registers 8(j&1)..8(j&1)+7 of block j/2; a
        // split tile feeds the same weights to its hi (keys 0..31) and lo (32..63) halves
        bf16x8 pb[4];
        if (!split) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[b][r], c, -m_use));
                    if (r & 1) ps1 += p; else ps0 += p;
                    pb[2 * b + (r >> 3)][r & 7] = (bf16)p;
                }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(s[0][r] - m_use);
                if (r & 1) ps1 += p; else ps0 += p;
                pb[r >> 3][r & 7] = (bf16)p;
            }
            pb[2] = pb[0];
            pb[3] = pb[1];
        }
        l_run += ps0 + ps1;
        __builtin_amdgcn_sched_barrier(0);

#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8 va = *reinterpret_cast<const bf16x8 *>(Vt + (32 * db + l32) * C::VSTR + 16 * j + 8 * h);
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[j], acc[db], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);

        if (have_next) {
            bf16 *dst = lds + (buf ^ 1) * C::BUF;
            if (nxt.kind == kExact) store_bf16<D, BQ>(dst, st);
            else store_split<D, BQ>(dst, st);
        }
        __syncthreads();
        buf ^= 1;
        cur = nxt;
        have = have_next;
    }

    // epilogue: O^T accumulator register r of block db holds feature 32db + 8(r/4) + 4h + r%4
    const float lt = l_run + __shfl_xor(l_run, 32, kWave);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (row_ok) {
        T *orow = o + head + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                Store4<T>::st(orow + 32 * db + 8 * g + 4 * h, acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv,
                              acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
        if (a.lse && h == 0)
            a.lse[(size_t)bh * a.N + qrow] = lt > 0.f ? (m_ref + log2f(lt)) * 0.69314718055994531f : -INFINITY;
    }
}

template <typename T, int D, int BQ, bool kSparse>
static hipError_t launch_flash_t(const void *q, const void *k, const void *v, void *o,
                                 const FlashArgs &a, int BH, hipStream_t st) {
    using C = FC<D, BQ>;
    static bool attr_set = false;
    auto kern = flash_kernel<T, D, BQ, kSparse>;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)C::LDS);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int items = BH * a.n_qb;
    hipLaunchKernelGGL(kern, dim3(items), dim3(C::THREADS), C::LDS, st, (const T *)q, (const T *)k,
                       (const T *)v, (T *)o, a);
    return hipGetLastError();
}

template <typename T, int D, int BQ>
static hipError_t launch_flash_s(const void *q, const void *k, const void *v, void *o, const FlashArgs &a,
                                 int BH, hipStream_t st) {
    return a.kv_idx ? launch_flash_t<T, D, BQ, true>(q, k, v, o, a, BH, st)
                    : launch_flash_t<T, D, BQ, false>(q, k, v, o, a, BH, st);
}

template <typename T>
static hipError_t launch_flash_dt(int D, int BQ, const void *q, const void *k, const void *v, void *o,
                                  const FlashArgs &a, int BH, hipStream_t st) {
    if (D == 128) return BQ == 128 ? launch_flash_s<T, 128, 128>(q, k, v, o, a, BH, st)
                                   : launch_flash_s<T, 128, 64>(q, k, v, o, a, BH, st);
    return BQ == 128 ? launch_flash_s<T, 64, 128>(q, k, v, o, a, BH, st)
                     : launch_flash_s<T, 64, 64>(q, k, v, o, a, BH, st);
}

hipError_t launch_flash(int dtype, int D, int BQ, const void *q, const void *k, const void *v,
                        void *o, const FlashArgs &a, int BH, hipStream_t st) {
    if (dtype == SA_BF16) return launch_flash_dt<bf16>(D, BQ, q, k, v, o, a, BH, st);
    return launch_flash_dt<float>(D, BQ, q, k, v, o, a, BH, st);
}

}  // namespace sa
