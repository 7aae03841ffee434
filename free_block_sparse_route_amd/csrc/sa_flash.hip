// Block-sparse attention with a dropped-block residual, one online-softmax pass
// (Sol-Attn abstract: dynamic routing, sparse computation and approximation
// correction in a single online-softmax pass).
//
// One workgroup per (b, h, query block).  Each wave owns 32 query rows and
// keeps them as the B operand of v_mfma_f32_32x32x16_bf16 for the whole pass.
// The kernel walks a stream of 64-row key/value tiles:
//   exact tiles     the tokens of the kept key blocks, in ascending block order
//                   (64 bf16 tokens, or 32 fp32 tokens in hi/lo split form)
//   residual tiles  32 block means in hi/lo split form (prepared by routing)
//                   with an additive logit bias of log2(n_J) for dropped blocks
//                   and -inf for kept ones; a tile whose 32 blocks are all kept
//                   is skipped
// and folds both kinds into the same running max and normaliser.  A split tile
// holds bf16(x) in rows 0..31 and bf16(x - bf16(x)) in rows 32..63, so the same
// 64-column MFMA sequence yields hi + lo products (about 2^-16 relative).
//
// Products are formed transposed: S^T = K Q^T and O^T = V^T P^T.  The MFMA
// accumulator then gives each lane one query row (lane & 31) and 32 of the
// tile's keys, P^T is exactly what each lane holds after the softmax, and the
// row max, normaliser and rescale factor are per-lane scalars.
//
// LDS: K and V tiles row-major (features contiguous), two stages in two arrays.  bf16 tiles
// go straight from memory into LDS with buffer->LDS loads (no registers, no
// LDS store instructions); the buffer range check zero-fills rows past the end
// of a head.  16-byte chunks are XOR-swizzled per row: for K so that 16 lanes
// reading one feature chunk of 16 rows hit distinct banks, for V so that the
// transposing reads (ds_read_b64_tr_b16) that build V^T operands spread over
// all banks.
#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D, int BQ>
struct FC {
    static constexpr int WAVES = BQ / 32;
    static constexpr int THREADS = WAVES * kWave;
    static constexpr int RB = D * 2;                    // bytes per LDS row (bf16)
    static constexpr int NC = D / 8;                    // 16-byte chunks per row
    static constexpr int TILE = kTile * RB;             // bytes of one K or V tile
    static constexpr int STAGE = 2 * TILE;              // K then V
    static constexpr int PPW = TILE / 1024 / WAVES;     // 1 KB buffer->LDS pieces per wave per tile
    static constexpr int SU = 32 * (D / 4) / THREADS;   // 16-byte fp32 units per thread per tile
    // waves per SIMD the register budget targets: two 128-row workgroups share a
    // CU; a 64-row workgroup (2 waves) gets the full register file
    static constexpr int WPE = BQ == 128 ? 2 : 1;
};

// chunk position = logical chunk ^ swizzle(row)
template <int D> __device__ __forceinline__ int swz_k(int r) { return r & (D / 8 - 1); }
template <int D> __device__ __forceinline__ int swz_v(int r) {
    return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

enum : int {
    kExact = 0,        // 64 bf16 tokens of a kept block
    kExactSplit = 1,   // 32 fp32 tokens of a kept block (fp32 inputs)
    kResidual = 2,     // 32 block means, split, dropped blocks only
};

struct TileDesc {
    int kind;
    int row0;      // first token (exact) or first pooled block (residual)
    int valid;     // rows of the tile that exist
    uint32_t kept; // residual: kept bits of the tile's 32 pooled blocks (1 past n_kb)
};

// The tile sequence of one work item; every thread steps it identically and
// every field is wave-uniform.  The kept-block index and the mask word are
// fetched one step ahead, so their memory latency is hidden behind a tile
// instead of delaying the next tile's loads.
struct TileStream {
    const int32_t *list;
    const uint32_t *mask;
    int cnt, li, sub;
    int exact_rows, exact_kind;
    int dense_tiles, t;
    int rt, n_rt;
    int J_cur, J_pf;          // kept blocks li and li + 1
    uint32_t w_cur, w_pf;     // mask words rt and rt + 1

    __device__ void prime() {
        J_cur = cnt > 0 ? __builtin_amdgcn_readfirstlane(list[0]) : 0;
        J_pf = cnt > 1 ? __builtin_amdgcn_readfirstlane(list[1]) : 0;
        w_cur = n_rt > 0 ? (uint32_t)__builtin_amdgcn_readfirstlane(mask[0]) : 0u;
        w_pf = n_rt > 1 ? (uint32_t)__builtin_amdgcn_readfirstlane(mask[1]) : 0u;
    }

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
            const int b0 = J_cur * a.block_k;
            const int b1 = min(b0 + a.block_k, a.N);
            const int tok0 = b0 + sub * exact_rows;
            ++sub;
            if (b0 + sub * exact_rows >= b1) {
                ++li;
                sub = 0;
                J_cur = J_pf;
                J_pf = li + 1 < cnt ? __builtin_amdgcn_readfirstlane(list[li + 1]) : 0;
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
            const uint32_t bits = w_cur;
            w_cur = w_pf;
            w_pf = rt + 1 < n_rt ? (uint32_t)__builtin_amdgcn_readfirstlane(mask[rt + 1]) : 0u;
            const int lim = a.n_kb - cur * 32;
            const uint32_t vmask = lim >= 32 ? ~0u : ((1u << lim) - 1u);
            if ((~bits & vmask) != 0) {
                o.kind = kResidual;
                o.row0 = cur * 32;
                o.valid = kTile;
                o.kept = bits | ~vmask;
                return true;
            }
        }
        return false;
    }
};

// Buffer resource over `bytes` bytes at `base`: loads past the end return zero
// (also when they go straight to LDS).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// Per-lane constants of the pass: source offsets of the buffer->LDS pieces (a
// wave's piece i covers LDS bytes [(w + WAVES i) KB, +1 KB) of a tile, lane l
// its 16 bytes at l*16, holding the swizzled chunk of that slot), and the LDS
// read bases of the K and V^T operands.
template <int D, int BQ>
struct Lanes {
    int ksrc[FC<D, BQ>::PPW], vsrc[FC<D, BQ>::PPW];
    int kread[D / 16];         // K operand of step c: row l32, features 16c + 8h (swizzled)
    int vread[D / 32];         // V^T operand of feature block db (rows 4h + (i>>2))

    __device__ void init(int wave, int lane) {
        using C = FC<D, BQ>;
        constexpr int RPK = 1024 / C::RB;              // rows per 1 KB piece
        constexpr int SPR = C::RB / 16;                // 16-byte slots per row
#pragma unroll
        for (int i = 0; i < C::PPW; ++i) {
            const int q = wave + C::WAVES * i;
            const int r = q * RPK + lane / SPR;
            const int p = lane % SPR;
            ksrc[i] = r * C::RB + 16 * (p ^ swz_k<D>(r));
            vsrc[i] = r * C::RB + 16 * (p ^ swz_v<D>(r));
        }
        const int h = lane >> 5, l32 = lane & 31;
        const int fk = swz_k<D>(l32);      // equal for rows l32 and 32 + l32
#pragma unroll
        for (int c = 0; c < D / 16; ++c) kread[c] = l32 * C::RB + 16 * ((2 * c + h) ^ fk);
        const int G = lane >> 4, i = lane & 15;
        const int vrow = 4 * h + (i >> 2);
        const int cl = 2 * (G & 1) + ((i & 3) >> 1);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            vread[db] = vrow * C::RB + 16 * ((4 * db + cl) ^ swz_v<D>(vrow)) + 8 * (i & 1);
    }
};

// fp32 split tiles go through registers: K/V unit u = (row u/(D/4), 4 features)
template <int D, int BQ>
struct Staging {
    u32x4 k[FC<D, BQ>::SU];
    u32x4 v[FC<D, BQ>::SU];
};

template <int D, int BQ>
__device__ __forceinline__ void load_split(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, Staging<D, BQ> &st) {
    using C = FC<D, BQ>;
#pragma unroll
    for (int i = 0; i < C::SU; ++i) {
        const int u = threadIdx.x + i * C::THREADS;
        const int off = (u / (D / 4)) * (D * 4) + (u % (D / 4)) * 16;
        st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
        st.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    }
}

__device__ __forceinline__ bf16x4 bf16x4_of(float a, float b, float c, float d) {
    bf16x4 x;
    x[0] = (bf16)a; x[1] = (bf16)b; x[2] = (bf16)c; x[3] = (bf16)d;
    return x;
}

template <int D, int BQ>
__device__ __forceinline__ void store_split(unsigned char *stage, const Staging<D, BQ> &st) {
    using C = FC<D, BQ>;
#pragma unroll
    for (int i = 0; i < C::SU; ++i) {
        const int u = threadIdx.x + i * C::THREADS;
        const int row = u / (D / 4), c4 = u % (D / 4);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const u32x4 w = t == 0 ? st.k[i] : st.v[i];
            const int pos = (c4 >> 1) ^ (t == 0 ? swz_k<D>(row) : swz_v<D>(row));
            unsigned char *base = stage + t * C::TILE + 16 * pos + 8 * (c4 & 1);
            float x[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = __uint_as_float(w[e]);
                lo[e] = x[e] - (float)(bf16)x[e];
            }
            *reinterpret_cast<bf16x4 *>(base + row * C::RB) = bf16x4_of(x[0], x[1], x[2], x[3]);
            *reinterpret_cast<bf16x4 *>(base + (row + 32) * C::RB) = bf16x4_of(lo[0], lo[1], lo[2], lo[3]);
        }
    }
}

// 16 bytes per lane from a buffer straight into LDS at lds_base + 16 * lane.
__device__ __forceinline__ void buffer_to_lds(__amdgpu_buffer_rsrc_t r, unsigned char *lds_base, int voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_base, 16, voffset, 0, 0,
                                             0);
#endif
}

// One buffer->LDS piece per (i, tensor): 1 KB of the tile at the wave's slot.
template <int D, int BQ>
__device__ __forceinline__ void load_direct(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                            unsigned char *stage, const Lanes<D, BQ> &ln, int wave) {
    using C = FC<D, BQ>;
#pragma unroll
    for (int i = 0; i < C::PPW; ++i) {
        const int piece = (wave + C::WAVES * i) * 1024;
        buffer_to_lds(rk, stage + piece, ln.ksrc[i]);
        buffer_to_lds(rv, stage + C::TILE + piece, ln.vsrc[i]);
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

// Key/value rows and residual tiles of one (b, h).
template <typename T>
struct HeadSrc {
    const T *k, *v;
    const bf16 *ks, *vs;      // split block means: 64-row tiles
    int n_rows;
};

// Start the loads of tile t into `stage`: direct for bf16 tiles, into `st` for
// fp32 split tiles (stored by store_split once the current tile is done).
template <typename T, int D, int BQ>
__device__ __forceinline__ void issue_tile(const TileDesc &t, const HeadSrc<T> &hs, const Lanes<D, BQ> &ln,
                                           unsigned char *stage, int wave, Staging<D, BQ> &st) {
    if (t.kind == kResidual) {
        const size_t off = (size_t)(t.row0 / 32) * kTile * D;
        load_direct<D, BQ>(buffer_rsrc(hs.ks + off, kTile * D * 2), buffer_rsrc(hs.vs + off, kTile * D * 2), stage, ln,
                           wave);
    } else {
        const uint32_t bytes = (uint32_t)(hs.n_rows - t.row0) * (D * sizeof(T));
        const auto rk = buffer_rsrc(hs.k + (size_t)t.row0 * D, bytes);
        const auto rv = buffer_rsrc(hs.v + (size_t)t.row0 * D, bytes);
        if constexpr (sizeof(T) == 2) load_direct<D, BQ>(rk, rv, stage, ln, wave);
        else load_split<D, BQ>(rk, rv, st);
    }
}

// One work item: the query block I of head bh = item / n_qb, from its first
// tile to its output rows.  kSparse: kept-list and residual tiles from a route;
// otherwise every key tile (dense).
template <typename T, int D, int BQ, bool kSparse>
__device__ __forceinline__ void run_item(int item, const T *__restrict__ q, const T *__restrict__ k,
                                         const T *__restrict__ v, T *__restrict__ o, const FlashArgs &a,
                                         unsigned char *lds0, unsigned char *lds1) {
    using C = FC<D, BQ>;
    constexpr bool kF32 = sizeof(T) == 4;
    const int bh = item / a.n_qb;
    const int I = item - bh * a.n_qb;
    const int lane = lane_id();
    const int h = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const size_t head = (size_t)bh * a.N * D;
    const int qrow = I * a.block_q + wave * 32 + l32;
    const bool row_ok = qrow < a.N;

    Lanes<D, BQ> ln;
    ln.init(wave, lane);

    // this wave's 32 query rows as B operands: in step c the lane holds features
    // 16c + 8h + 0..7 of row l32; fp32 inputs also keep the bf16 remainder
    bf16x8 qf[D / 16];
    bf16x8 ql[kF32 ? D / 16 : 1];
    {
        const bf16x8 zero = {};
#pragma unroll
        for (int c2 = 0; c2 < D / 16; ++c2) {
            const size_t off = head + (size_t)qrow * D + 16 * c2 + 8 * h;
            if constexpr (kF32) {
                float x[8];
                if (row_ok) Ld8<float>::load_f32(reinterpret_cast<const float *>(q) + off, x);
                else
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    qf[c2][e] = (bf16)x[e];
                    ql[c2][e] = (bf16)(x[e] - (float)qf[c2][e]);
                }
            } else {
                qf[c2] = row_ok ? Ld8<T>::load(q + off) : zero;
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
        ts.n_rt = (a.residual && ts.cnt < a.n_kb) ? a.mask_words : 0;   // all kept: no residual
    } else {
        ts.list = nullptr;
        ts.mask = nullptr;
        ts.cnt = 0;
        ts.n_rt = 0;
    }
    ts.prime();
    HeadSrc<T> hs;
    hs.k = k + head;
    hs.v = v + head;
    hs.ks = kSparse ? a.kv_split + (size_t)bh * 2 * a.mask_words * kTile * D : nullptr;
    hs.vs = kSparse ? hs.ks + (size_t)a.mask_words * kTile * D : nullptr;
    hs.n_rows = a.N;
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
        issue_tile<T, D, BQ>(cur, hs, ln, lds0, wave, st);
        if constexpr (kF32) {
            if (cur.kind == kExactSplit) store_split<D, BQ>(lds0, st);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): this thread's loads have landed
    __syncthreads();
    // One pipeline step: compute the tile in cur_stage while the next tile streams
    // into nxt_stage.  The loop below alternates two distinct LDS arrays so that
    // every LDS access names its stage statically: the compiler can then see that
    // reads of the current stage do not alias the buffer->LDS loads in flight.
    auto step = [&](const unsigned char *cur_stage, unsigned char *nxt_stage) -> bool {
        const bool have_next = ts.next(nxt, a);
        // Nothing is in flight here.  Saying so explicitly keeps the compiler from
        // placing its loop-entry wait after the prefetch below.
        __builtin_amdgcn_s_waitcnt(0x0F70);
        if (have_next) issue_tile<T, D, BQ>(nxt, hs, ln, nxt_stage, wave, st);
        const unsigned char *Ks = cur_stage;
        const unsigned char *Vs = cur_stage + C::TILE;

        // S^T for LDS key rows 0..31 (s[0]) and 32..63 (s[1])
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int c2 = 0; c2 < D / 16; ++c2) {
            const bf16x8 k0 = *reinterpret_cast<const bf16x8 *>(Ks + ln.kread[c2]);
            const bf16x8 k1 = *reinterpret_cast<const bf16x8 *>(Ks + ln.kread[c2] + 32 * C::RB);
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[c2], s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[c2], s[1], 0, 0, 0);
            if constexpr (kF32) s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, ql[c2], s[0], 0, 0, 0);
        }

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

        // O^T += V^T P^T: the V^T operand of step j (keys 16j..16j+15) comes from two
        // transposing reads: keys 16j + 4h + e and 16j + 8 + 4h + e (e = 0..3)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(Vs + ln.vread[db] + 16 * j * C::RB));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(Vs + ln.vread[db] + (16 * j + 8) * C::RB));
                // whole-vector reinterpretation: per-element bit casts of __bf16 vector
                // elements are mis-compiled by this toolchain (splat of element 0)
                const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                const bf16x8 va = __builtin_bit_cast(bf16x8, both);
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[j], acc[db], 0, 0, 0);
            }
        }

        if constexpr (kF32) {
            if (have_next && nxt.kind == kExactSplit) store_split<D, BQ>(nxt_stage, st);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the next tile has landed in LDS
        __syncthreads();
        cur = nxt;
        return have_next;
    };
    while (have) {
        have = step(lds0, lds1);
        if (!have) break;
        have = step(lds1, lds0);
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

// Workgroup i runs on GPU die i % 8: the dispatcher deals workgroups to the 8
// dies (XCDs) in turn.  In each group of 8 * kDieRun consecutive workgroups, die
// x takes the kDieRun consecutive work positions x * kDieRun + 0..kDieRun-1 of
// the group, so that neighbouring query blocks, which keep mostly the same key
// blocks, meet in one die's L2, while the order of the work list holds at the
// scale of a group.  The last, partial group keeps the plain order.
constexpr int kDieRun = 16;

__device__ __forceinline__ int grid_position(int i, int W) {
    constexpr int kGroup = 8 * kDieRun;
    const int base = i - i % kGroup;
    if (base + kGroup > W) return i;
    const int r = i - base;
    return base + (r & 7) * kDieRun + (r >> 3);
}

// One workgroup per work item (query block); kSparse takes the item from the
// route's work order, the dense path in plain order.
template <typename T, int D, int BQ, bool kSparse>
__global__ __launch_bounds__((FC<D, BQ>::THREADS)) __attribute__((amdgpu_waves_per_eu(FC<D, BQ>::WPE, FC<D, BQ>::WPE))) void flash_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, T *__restrict__ o,
    FlashArgs a) {
    using C = FC<D, BQ>;
    __shared__ __attribute__((aligned(1024))) unsigned char lds0[C::STAGE];
    __shared__ __attribute__((aligned(1024))) unsigned char lds1[C::STAGE];
    const int p = grid_position(blockIdx.x, a.n_items);
    const int item = kSparse ? __builtin_amdgcn_readfirstlane(a.work_order[p]) : p;
    run_item<T, D, BQ, kSparse>(item, q, k, v, o, a, lds0, lds1);
}

template <typename T, int D, int BQ, bool kSparse>
static hipError_t launch_flash_t(const void *q, const void *k, const void *v, void *o,
                                 const FlashArgs &a, int BH, hipStream_t st) {
    using C = FC<D, BQ>;
    auto kern = flash_kernel<T, D, BQ, kSparse>;
    FlashArgs args = a;
    args.n_items = BH * a.n_qb;
    hipLaunchKernelGGL(kern, dim3(args.n_items), dim3(C::THREADS), 0, st, (const T *)q, (const T *)k,
                       (const T *)v, (T *)o, args);
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
