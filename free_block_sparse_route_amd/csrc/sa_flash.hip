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
#include <type_traits>

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
};

// Waves per SIMD the register budget targets.  bf16, 128-row workgroups: three
// share a CU (48 KB of LDS each: K double-buffered, V single-buffered).  fp32
// rows need more registers: two 128-row workgroups (64 KB of LDS each).  A
// 64-row workgroup (2 waves): two waves per SIMD for bf16, so that the three
// workgroups the LDS admits can share a CU (with the whole register file one
// wave per SIMD left room for two); fp32 rows keep the whole file.
template <typename T, int BQ>
constexpr int kWavesPerEU = BQ == 128 ? (sizeof(T) == 2 ? 3 : 2) : (sizeof(T) == 2 ? 2 : 1);

// chunk position = logical chunk ^ swizzle(row)
template <int D> __device__ __forceinline__ int swz_k(int r) { return r & (D / 8 - 1); }
template <int D> __device__ __forceinline__ int swz_v(int r) {
    return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

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
    float lo;      // residual: bound on the norms of its key-mean remainder rows (inf: none)
    float kmax;    // residual: bound on the norms of its key means (inf: none)
};

// The tile sequence of one work item; every thread steps it identically and
// every field is wave-uniform.  The kept list and the mask words are read
// through the scalar cache (constant address space: the route wrote them before
// this kernel started and nothing changes them during it), one entry ahead of
// use, so that the read is in flight during a whole step and no step waits on
// the vector-memory counter, which also counts the tile loads in flight.
struct TileStream {
    const kconst<int32_t> *list;
    const kconst<uint32_t> *mask;
    const kconst<f32x2> *bounds;   // the head's residual-tile norm bounds, or null
    int cnt, li, sub;
    int exact_rows, exact_kind;
    int dense_tiles, t;
    int rt, n_rt;
    int J_cur, J_pf;          // kept blocks li and li + 1
    uint32_t w_cur, w_pf;     // mask words rt and rt + 1

    // A list entry outside [0, n_kb) (a route that does not belong to this
    // call) is clamped, so that no tile is read outside the head.
    static __device__ __forceinline__ int clampJ(int J, int n_kb) { return min(max(J, 0), n_kb - 1); }

    __device__ void prime(const FlashArgs &a) {
        J_cur = cnt > 0 ? clampJ(list[0], a.n_kb) : 0;
        J_pf = cnt > 1 ? clampJ(list[1], a.n_kb) : 0;
        w_cur = n_rt > 0 ? mask[0] : 0u;
        w_pf = n_rt > 1 ? mask[1] : 0u;
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
                J_pf = clampJ(list[min(li + 1, cnt - 1)], a.n_kb);   // unconditional: the load lands in J_pf's register
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
            w_pf = mask[min(rt + 1, n_rt - 1)];
            const int lim = a.n_kb - cur * 32;
            const uint32_t vmask = lim >= 32 ? ~0u : ((1u << lim) - 1u);
            if ((~bits & vmask) != 0) {
                o.kind = kResidual;
                o.row0 = cur * 32;
                o.valid = kTile;
                o.kept = bits | ~vmask;
                const f32x2 bd = bounds ? (f32x2)bounds[cur] : f32x2{INFINITY, INFINITY};
                o.kmax = bd.x;
                o.lo = bd.y;
                return true;
            }
        }
        return false;
    }
};

// Fused routing: the kept blocks come from this work item's decision words in
// LDS (bit J % 32 of word J / 32), in ascending J, then one residual tile per
// word that holds a dropped block: the same tile order as a route's lists.
struct BitStream {
    const uint32_t *lw;       // decision words in LDS
    const kconst<f32x2> *bounds;   // the head's residual-tile norm bounds, or null
    int words, wi, sub, rt, n_rt;
    int exact_rows, exact_kind;
    uint32_t bits;            // kept bits of word wi not yet visited

    __device__ uint32_t word(int w) const { return (uint32_t)__builtin_amdgcn_readfirstlane((int)lw[w]); }

    __device__ void prime(const FlashArgs &) {
        wi = 0;
        sub = 0;
        rt = 0;
        bits = words > 0 ? word(0) : 0u;
    }

    __device__ bool next(TileDesc &o, const FlashArgs &a) {
        while (wi < words) {
            if (bits == 0u) {
                if (++wi < words) bits = word(wi);
                continue;
            }
            const int J = wi * 32 + __builtin_ctz(bits);
            const int b0 = J * a.block_k;
            const int b1 = min(b0 + a.block_k, a.N);
            const int tok0 = b0 + sub * exact_rows;
            ++sub;
            if (b0 + sub * exact_rows >= b1) {
                bits &= bits - 1u;
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
            const uint32_t kept = word(cur);
            const int lim = a.n_kb - cur * 32;
            const uint32_t vmask = lim >= 32 ? ~0u : ((1u << lim) - 1u);
            if ((~kept & vmask) != 0) {
                o.kind = kResidual;
                o.row0 = cur * 32;
                o.valid = kTile;
                o.kept = kept | ~vmask;
                const f32x2 bd = bounds ? (f32x2)bounds[cur] : f32x2{INFINITY, INFINITY};
                o.kmax = bd.x;
                o.lo = bd.y;
                return true;
            }
        }
        return false;
    }
};

// Decision words of one query block under fused routing, taken at the start of
// its work item (Sol-Attn abstract: blocks are selected against the threshold
// inside the attention pass; the pre-pass supplies only the proxy row's maximum
// and log-sum-exp).  Every thread scores key blocks J = t, t + THREADS, ...:
// s = scale * qbar_I . kbar_J in fp32 (the query mean through the scalar cache),
// kept when s clears the threshold the route's row statistics give, or when
// the dense prefix covers it.  With a floor of one block (min_keep = 1) and no
// block clearing the threshold, the block of largest s (lowest J among equal
// ones) is kept as well: the first block of the ranking, as in the unfused
// route.  Writes the words to LDS and to the route's mask, the count to the
// route; returns the count (uniform).
constexpr int kFusedWords = 512;           // n_kb <= 16368
template <int D, int BQ>
__device__ __forceinline__ int fused_route(int bh, int I, const FlashArgs &a, uint32_t *fw) {
    using C = FC<D, BQ>;
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int n = a.n_kb, words = a.mask_words;
    const size_t row = (size_t)bh * a.n_qb + I;
    const float thr = (a.tau_mode == SA_TAU_ABSOLUTE ? a.row_stats[row * 2 + 1] : a.row_stats[row * 2]) + a.ln_tau;
    const bool dense_row = (int64_t)I * a.block_q < a.n_prefix;
    const kconst<float> *qb = (const kconst<float> *)(a.q_mean + row * D);
    const float *kb = a.k_mean + (size_t)bh * n * D;
    float best = -INFINITY;                // this thread's largest score and its block
    int best_j = n;
    int npass = 0;                         // blocks that clear the threshold
    for (int base = 0; base < n; base += C::THREADS) {
        const int J = base + (int)threadIdx.x;
        bool keep = false;
        if (J < n) {
            const float *kr = kb + (size_t)J * D;
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < D; c += 4) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(kr + c);
#pragma unroll
                for (int e = 0; e < 4; ++e) s4[e] = fmaf(qb[c + e], x[e], s4[e]);
            }
            const float sc = ((s4[0] + s4[1]) + (s4[2] + s4[3])) * a.scale;
            const bool pass = sc >= thr;
            npass += pass ? 1 : 0;
            if (sc > best || best_j == n) {   // J rises along the loop: ties keep the lower J
                best = sc;
                best_j = J;
            }
            keep = pass || dense_row || (int64_t)J * a.block_k < a.n_prefix;
        }
        const uint64_t b = __ballot(keep);
        const int w = (base + wave * kWave) / 32;
        if (lane == 0 && w < words) fw[w] = (uint32_t)b;
        if (lane == 1 && w + 1 < words) fw[w + 1] = (uint32_t)(b >> 32);
    }
    uint32_t *part = fw + kFusedWords;     // per-wave partial results: [4][WAVES]
    npass = (int)wave_sum((float)npass);
    if (lane == 0) part[C::WAVES + wave] = (uint32_t)npass;
    __syncthreads();
    int total_pass = 0;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) total_pass += (int)part[C::WAVES + w];
    total_pass = __builtin_amdgcn_readfirstlane(total_pass);
    if (a.min_keep > 0 && total_pass == 0) {
        // the floor: the block of largest score, lowest index among equal ones
        const float m = wave_max(best);
        const float jm = wave_reduce(best == m ? (float)best_j : (float)n, [](float x, float y) { return fminf(x, y); });
        if (lane == 0) {
            part[2 * C::WAVES + wave] = __float_as_uint(m);
            part[3 * C::WAVES + wave] = (uint32_t)(int)jm;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            float bm = -INFINITY;
            int bj = n;
            for (int w = 0; w < C::WAVES; ++w) {
                const float mw = __uint_as_float(part[2 * C::WAVES + w]);
                const int jw = (int)part[3 * C::WAVES + w];
                if (jw < n && (bj == n || mw > bm || (mw == bm && jw < bj))) {
                    bm = mw;
                    bj = jw;
                }
            }
            if (bj < n) fw[bj / 32] |= 1u << (bj % 32);
        }
        __syncthreads();
    }
    int cnt = 0;
    for (int w = threadIdx.x; w < words; w += C::THREADS) {
        const uint32_t x = fw[w];
        a.kv_mask_out[row * words + w] = x;
        cnt += __popc(x);
    }
    cnt = (int)wave_sum((float)cnt);
    if (lane == 0) part[wave] = (uint32_t)cnt;
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) total += (int)part[w];
    if (threadIdx.x == 0) a.kv_count_out[row] = total;
    return __builtin_amdgcn_readfirstlane(total);
}

// Buffer resource over `bytes` bytes at `base`: loads past the end return zero
// (also when they go straight to LDS).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// Per-lane constants of the pass: source offsets of the buffer->LDS pieces (a
// wave's piece i covers LDS bytes [(w + WAVES i) KB, +1 KB) of a tile, lane l
// its 16 bytes at l*16, holding the swizzled chunk of that slot), and the LDS
// read bases of the K and V^T operands.  When the rows of piece i + 1 lie a
// whole number of swizzle periods past those of piece i (kFold), the offsets of
// piece i are those of piece 0 plus i * kPieceStride and only piece 0's are kept.
template <int D, int BQ>
struct Lanes {
    static constexpr int kRowsPerStep = FC<D, BQ>::WAVES * (1024 / FC<D, BQ>::RB);
    static constexpr bool kFold = kRowsPerStep % (D / 8) == 0 && kRowsPerStep % 4 == 0;
    static constexpr int kPieceStride = kRowsPerStep * FC<D, BQ>::RB;
    static constexpr int NSRC = kFold ? 1 : FC<D, BQ>::PPW;
    int ksrc[NSRC], vsrc[NSRC];
    int kread[D / 16];         // K operand of step c: row l32, features 16c + 8h (swizzled)
    int vread[D / 32];         // V^T operand of feature block db (rows 4h + (i>>2))

    __device__ void init(int wave, int lane) {
        using C = FC<D, BQ>;
        constexpr int RPK = 1024 / C::RB;              // rows per 1 KB piece
        constexpr int SPR = C::RB / 16;                // 16-byte slots per row
#pragma unroll
        for (int i = 0; i < NSRC; ++i) {
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
__device__ __forceinline__ void store_split(unsigned char *Kst, unsigned char *Vst, const Staging<D, BQ> &st) {
    using C = FC<D, BQ>;
#pragma unroll
    for (int i = 0; i < C::SU; ++i) {
        const int u = threadIdx.x + i * C::THREADS;
        const int row = u / (D / 4), c4 = u % (D / 4);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const u32x4 w = t == 0 ? st.k[i] : st.v[i];
            const int pos = (c4 >> 1) ^ (t == 0 ? swz_k<D>(row) : swz_v<D>(row));
            unsigned char *base = (t == 0 ? Kst : Vst) + 16 * pos + 8 * (c4 & 1);
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
__device__ __forceinline__ void buffer_to_lds(__amdgpu_buffer_rsrc_t r, unsigned char *lds_base, int voffset,
                                              int soffset) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_base, 16, voffset,
                                             soffset, 0, 0);
#endif
}

// One tile of K or V: the wave's buffer->LDS pieces, 1 KB each, at its slots.
template <int D, int BQ>
__device__ __forceinline__ void load_direct(__amdgpu_buffer_rsrc_t r, unsigned char *dst, const int *src, int wave) {
    using C = FC<D, BQ>;
    using L = Lanes<D, BQ>;
#pragma unroll
    for (int i = 0; i < C::PPW; ++i) {
        if constexpr (L::kFold) buffer_to_lds(r, dst + (wave + C::WAVES * i) * 1024, src[0], i * L::kPieceStride);
        else buffer_to_lds(r, dst + (wave + C::WAVES * i) * 1024, src[i], 0);
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

// Buffer resource of the K (value = false) or V rows of tile t.
template <typename T, int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const TileDesc &t, const HeadSrc<T> &hs, bool value) {
    if (t.kind == kResidual) {
        // the value half of a residual tile uses only its 32 rows of bf16 means:
        // the loads of the 32 remainder rows fall outside the range and fetch
        // nothing (they land as zeros)
        const size_t off = (size_t)(t.row0 / 32) * kTile * D;
        return buffer_rsrc((value ? hs.vs : hs.ks) + off, (value ? kTile / 2 : kTile) * D * 2);
    }
    const uint32_t bytes = (uint32_t)(hs.n_rows - t.row0) * (D * sizeof(T));
    return buffer_rsrc((value ? hs.v : hs.k) + (size_t)t.row0 * D, bytes);
}

// Start the loads of tile t: straight to LDS for bf16 rows and residual tiles,
// into `st` for fp32 rows (stored by store_split once the current tile is done).
template <typename T, int D, int BQ>
__device__ __forceinline__ void issue_tile(const TileDesc &t, const HeadSrc<T> &hs, const Lanes<D, BQ> &ln,
                                           unsigned char *Kst, unsigned char *Vst, int wave, Staging<D, BQ> &st) {
    const auto rk = tile_rsrc<T, D>(t, hs, false);
    const auto rv = tile_rsrc<T, D>(t, hs, true);
    if (sizeof(T) == 2 || t.kind == kResidual) {
        load_direct<D, BQ>(rk, Kst, ln.ksrc, wave);
        load_direct<D, BQ>(rv, Vst, ln.vsrc, wave);
    } else {
        load_split<D, BQ>(rk, rv, st);
    }
}

// S^T = K Q^T over one tile: s[0] holds LDS key rows 0..31, s[1] rows 32..63.
// The K operands are read two steps ahead of the MFMAs that take them.
template <int D, int BQ, bool kF32>
__device__ __forceinline__ void qk_tile(const unsigned char *Ks, const Lanes<D, BQ> &ln, const bf16x8 *qf,
                                        const bf16x8 *ql, f32x16 (&s)[2]) {
    using C = FC<D, BQ>;
    constexpr int NS = D / 16;
    bf16x8 k0v[NS], k1v[NS];
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
        k0v[c2] = *reinterpret_cast<const bf16x8 *>(Ks + ln.kread[c2]);
        k1v[c2] = *reinterpret_cast<const bf16x8 *>(Ks + ln.kread[c2] + 32 * C::RB);
    }
#pragma unroll
    for (int c2 = 0; c2 < NS; ++c2) {
        if (c2 + 2 < NS) {
            k0v[c2 + 2] = *reinterpret_cast<const bf16x8 *>(Ks + ln.kread[c2 + 2]);
            k1v[c2 + 2] = *reinterpret_cast<const bf16x8 *>(Ks + ln.kread[c2 + 2] + 32 * C::RB);
        }
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0v[c2], qf[c2], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1v[c2], qf[c2], s[1], 0, 0, 0);
        if constexpr (kF32) s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0v[c2], ql[c2], s[0], 0, 0, 0);
    }
}

// S^T for the 32 LDS key rows 32hb.. of a tile (one accumulator block); the K
// operands are read two steps ahead of the MFMAs that take them.
template <int D, int BQ>
__device__ __forceinline__ f32x16 qk_half(const unsigned char *Ks, int hb, const Lanes<D, BQ> &ln, const bf16x8 *qf) {
    using C = FC<D, BQ>;
    constexpr int NS = D / 16;
    const unsigned char *base = Ks + 32 * hb * C::RB;
    bf16x8 kv[NS];
    f32x16 s = {};
    kv[0] = *reinterpret_cast<const bf16x8 *>(base + ln.kread[0]);
    kv[1] = *reinterpret_cast<const bf16x8 *>(base + ln.kread[1]);
#pragma unroll
    for (int c2 = 0; c2 < NS; ++c2) {
        if (c2 + 2 < NS) kv[c2 + 2] = *reinterpret_cast<const bf16x8 *>(base + ln.kread[c2 + 2]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv[c2], qf[c2], s, 0, 0, 0);
    }
    return s;
}

// O^T += V^T P^T over the 32 keys 32hb.. of a tile: steps j = 2hb + n / NB with
// P^T operands pa (j even) and pc (j odd), features 32(n % NB)..; V^T operands
// read two steps ahead.
template <int D, int BQ>
__device__ __forceinline__ void pv_half(const unsigned char *Vs, int hb, const Lanes<D, BQ> &ln, const bf16x8 &pa,
                                        const bf16x8 &pc, f32x16 (&acc)[D / 32]) {
    using C = FC<D, BQ>;
    constexpr int NB = D / 32, NP = 2 * NB;
    bf16x8 vop[NP];
    auto vload = [&](int n) -> bf16x8 {
        const int db = n % NB, j = 2 * hb + n / NB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(Vs + ln.vread[db] + 16 * j * C::RB));
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(Vs + ln.vread[db] + (16 * j + 8) * C::RB));
        const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, both);
    };
    vop[0] = vload(0);
    vop[1] = vload(1);
#pragma unroll
    for (int n = 0; n < NP; ++n) {
        if (n + 2 < NP) vop[n + 2] = vload(n + 2);
        acc[n % NB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[n], n < NB ? pa : pc, acc[n % NB], 0, 0, 0);
    }
}

// max over the two lanes (l, l ^ 32) that hold one query row
__device__ __forceinline__ float row_pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lazy rescaling: the reference m_ref of the online softmax moves only when
// some row of the wave exceeds it by more than kLazy (log2 units), so the
// accumulator rescale is skipped on almost every tile.  Weights stay below
// 2^kLazy; fp32 sums and bf16 weights keep their relative precision at any
// such scale, and with at most 2^24 keys a row's sums stay below 2^(kLazy+30),
// far from overflow.  Numerator and normaliser share the reference, so the
// softmax is unchanged.
constexpr float kLazy = 32.f;
constexpr float kLazyWeight = 4294967296.f;     // 2^kLazy

// Online-softmax state of the wave's 32 rows (per lane: its row, log2 units).
template <int D>
struct SoftState {
    f32x16 acc[D / 32];
    float m_ref, l_run;

    __device__ __forceinline__ float m_use() const { return m_ref == -INFINITY ? 0.f : m_ref; }

    // After weights were formed against m_use(): the reference must move if
    // one of them may exceed 2^kLazy (their sum shows it, as do an overflow
    // and a NaN) or if there is no reference yet.  Rare: the first tile of a
    // row, and a rise of the logits by more than kLazy.
    __device__ __forceinline__ bool needs_move(float psum) const {
        return !(psum <= kLazyWeight) || m_ref == -INFINITY;
    }

    // New reference from this tile's row maxima (row_max: both lanes of a row
    // agree); rescales the normaliser and returns the factor for the accumulator.
    __device__ __forceinline__ float move_ref_l(float row_max) {
        const float m_new = fmaxf(m_ref, row_max);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        m_ref = m_new;
        l_run *= alpha;
        return alpha;
    }
    __device__ __forceinline__ void scale_acc(float alpha) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
    }
    __device__ __forceinline__ void move_ref(float row_max) { scale_acc(move_ref_l(row_max)); }
};

// An empty instruction that reads x: x must be computed before this point.
__device__ __forceinline__ void pin(const bf16x8 &x) {
    const u32x4 w = __builtin_bit_cast(u32x4, x);
    asm volatile("" ::"v"(w));
}
__device__ __forceinline__ void pin(float x) { asm volatile("" ::"v"(x)); }

// Lane maximum of one accumulator block (32 keys of a full exact tile), log2 units.
__device__ __forceinline__ float half_max(const f32x16 &s, float c) {
    float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
        m0 = fmaxf(m0, s[r]);
        m1 = fmaxf(m1, s[r + 1]);
    }
    return fmaxf(m0, m1) * c;           // c > 0
}

// Weights of one accumulator block against the reference m_use: the P^T
// operands of its two steps and their sum.  Straight-line code, so that it can
// share a scheduling region with MFMAs.
__device__ __forceinline__ void weights_half(const f32x16 &s, float c, float m_use, bf16x8 &pa, bf16x8 &pc,
                                             float &psum) {
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[r], c, -m_use));
        if (r & 1) ps1 += p; else ps0 += p;
        if (r < 8) pa[r] = (bf16)p; else pc[r - 8] = (bf16)p;
    }
    psum = ps0 + ps1;
}

// Keys of an accumulator block at or past `lim` (lane-relative) are absent.
__device__ __forceinline__ void drop_absent(f32x16 &s, int lim) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) >= lim) s[r] = -INFINITY;
}

// Negligible weights.  The reference m_ref of a row is set from a row maximum
// (whose weight is then 1) and only moves up, so the row's normaliser is at
// least 1 from its first tile on.  A weight below 2^-32 of the reference is
// below 2^-32 of the normaliser: 32 of them add less than 2^-27 to it, below
// half of its last bit, and their values move the accumulator as little.  The
// products with such weights are skipped when they hold for all 32 rows of a
// wave: the P V of an exact half-tile (its weights still enter the normaliser),
// and the whole fold of a residual tile (kNegligible: its logits lie more than
// 32 below the reference).
constexpr float kNegligible = 32.f;
constexpr float kNegligibleWeight = 2.3283064365386963e-10f;    // 2^-32

// An exact tile in four scheduling regions: S^T of key rows 0..31; S^T of rows
// 32..63 while the weights of rows 0..31 are formed; P V of keys 0..31 while
// the weights of keys 32..63 are formed; P V of keys 32..63.  The MFMAs of one
// half run while the exponentials of the other are computed.  The weights of a
// half are formed against the current reference without a row maximum; when
// one may pass 2^kLazy (seen in their sum) the reference moves to the half's
// row maximum and they are formed again (rare).  The P V of a half whose
// weights are all negligible for every row of the wave (below kNegligibleWeight)
// is not formed; their sum still enters the normaliser.  Rows at
// or past `valid` (a partial last tile) are dropped.  wait_v() runs before the
// first read of Vs.  Accumulator register r of lane (h, l32) holds key row
// 8(r/4) + 4h + r%4 of its 32-row block.
template <int D, int BQ, typename WaitV>
__device__ __forceinline__ void tile_exact(const unsigned char *Ks, const unsigned char *Vs, const Lanes<D, BQ> &ln,
                                           const bf16x8 *qf, float c, int valid, int h, SoftState<D> &sm,
                                           WaitV &&wait_v) {
    constexpr int NS = D / 16, NB = D / 32;
    f32x16 s0 = qk_half<D, BQ>(Ks, 0, ln, qf);
    if (valid < kTile) drop_absent(s0, valid - 4 * h);
    bf16x8 p0, p1, p2, p3;
    float ps_a, ps_b;
    f32x16 s1 = qk_half<D, BQ>(Ks, 1, ln, qf);
    weights_half(s0, c, sm.m_use(), p0, p1, ps_a);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int m = 0; m < NS; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 48 / NS, 0);
        if (m + 2 < NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    // keep the weights in this region: without a use here the compiler sinks
    // them past the branches below, away from the MFMAs they should overlap
    pin(p0);
    pin(p1);
    pin(ps_a);
    if (__ballot(sm.needs_move(ps_a)) != 0) {
        // rare path: the logits are formed again from the keys still in LDS,
        // so that none stays live across the scheduled region above
        f32x16 r0 = qk_half<D, BQ>(Ks, 0, ln, qf);
        if (valid < kTile) drop_absent(r0, valid - 4 * h);
        sm.move_ref(row_pair_max(half_max(r0, c)));
        weights_half(r0, c, sm.m_use(), p0, p1, ps_a);
    }
    sm.l_run += ps_a;
    if (valid < kTile) drop_absent(s1, valid - 32 - 4 * h);
    wait_v();                           // this tile's values are in LDS from here on
    pv_half<D, BQ>(Vs, 0, ln, p0, p1, sm.acc);
    weights_half(s1, c, sm.m_use(), p2, p3, ps_b);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
    for (int m = 0; m < 2 * NB; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x002, 24 / NB, 1);
        if (m + 2 < 2 * NB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    pin(p2);
    pin(p3);
    pin(ps_b);
    if (__ballot(sm.needs_move(ps_b)) != 0) {
        // the weights of keys 0..31 were formed against the old reference: the
        // accumulator is rescaled after their P V has been added
        f32x16 r1 = qk_half<D, BQ>(Ks, 1, ln, qf);
        if (valid < kTile) drop_absent(r1, valid - 32 - 4 * h);
        sm.scale_acc(sm.move_ref_l(row_pair_max(half_max(r1, c))));
        weights_half(r1, c, sm.m_use(), p2, p3, ps_b);
    }
    sm.l_run += ps_b;
    if (__ballot(!(ps_b < kNegligibleWeight)) != 0) pv_half<D, BQ>(Vs, 1, ln, p2, p3, sm.acc);
}

// A split tile (fp32 rows or residual block means): S^T of its hi rows (0..31)
// plus its lo rows (32..63) gives the logits of its 32 keys; residual tiles add
// the logit bias log2(n_J) of dropped blocks and drop kept ones, fp32 tiles drop
// absent rows.  The P^T operands pa, pc serve the 32 keys of either half.
// Updates the state and returns true, or returns false for a negligible
// residual tile (state unchanged, pa and pc unset).  The lane's keys are 4h + kr,
// kr = 8(r/4) + r%4: the lane part is folded into per-tile values so that each
// register tests a constant kr.
template <int D>
__device__ __forceinline__ bool weights_split(f32x16 &s0, const f32x16 &s1, const TileDesc &cur, float c,
                                              float lg_bk, float lg_last, int n_kb, int h, SoftState<D> &sm,
                                              bf16x8 &pa, bf16x8 &pc) {
    const uint32_t kh = cur.kept >> (4 * h);
    const int last = n_kb - 1 - cur.row0 - 4 * h;
    const int vlim = cur.valid - 4 * h;
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int kr = 8 * (r >> 2) + (r & 3);
        float x = (s0[r] + s1[r]) * c;
        if (cur.kind == kResidual) {
            const bool drop = ((kh >> kr) & 1u) == 0;
            x = drop ? x + (kr == last ? lg_last : lg_bk) : -INFINITY;
        } else {
            x = kr < vlim ? x : -INFINITY;
        }
        s0[r] = x;
        mx = fmaxf(mx, x);
    }
    if (__ballot(mx > sm.m_ref + kLazy) != 0) sm.move_ref(row_pair_max(mx));
    // (a row with no reference yet, m_ref = -inf, never counts as negligible)
    if (cur.kind == kResidual && __ballot(!(mx < sm.m_ref - kNegligible)) == 0) return false;
    const float m_use = sm.m_use();
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s0[r] - m_use);
        if (r & 1) ps1 += p; else ps0 += p;
        if (r < 8) pa[r] = (bf16)p; else pc[r - 8] = (bf16)p;
    }
    sm.l_run += ps0 + ps1;
    return true;
}

// Early test of a residual tile from the bf16 part of its key means alone: the
// remainder rows add c q_i . lo_J to a logit, at most qnc * t.lo in size
// (Cauchy-Schwarz, with the bounds of both norms).  Returns true when even
// with that added (and a slack over the fp32 rounding of the full logit) every
// dropped block's logit lies more than kNegligible below the reference for
// all 32 rows of the wave: weights_split would then find the tile negligible,
// so it is skipped without forming the remainder part.
template <int D>
__device__ __forceinline__ bool residual_negligible(const f32x16 &s0, const TileDesc &t, float c, float lg_bk,
                                                    float lg_last, int n_kb, int h, const SoftState<D> &sm,
                                                    float qnc) {
    const float margin = qnc * t.lo;
    if (!(margin < INFINITY)) return false;        // no bound for this tile
    const uint32_t kh = t.kept >> (4 * h);
    const int last = n_kb - 1 - t.row0 - 4 * h;
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int kr = 8 * (r >> 2) + (r & 3);
        const bool drop = ((kh >> kr) & 1u) == 0;
        mx = fmaxf(mx, drop ? s0[r] * c + (kr == last ? lg_last : lg_bk) : -INFINITY);
    }
    const float ub = mx == -INFINITY ? -INFINITY
                                     : mx + margin * (1.f + 1.f / 256.f) + fabsf(mx) * (1.f / 1048576.f) + 1.f / 64.f;
    return __ballot(!(ub < sm.m_ref - kNegligible)) == 0;
}

// Test of a residual tile from norms alone, before any of its products: a
// dropped block's logit c q_i . kbar_J + log2 n_J is at most qnc * t.kmax +
// log2 block_k (Cauchy-Schwarz with the bounds of both norms; the last block's
// bias is the smaller).  True when that, with a slack over the fp32 rounding
// of the logit, lies more than kNegligible below the reference of every row
// of the wave: residual_negligible would then hold as well, so the tile is
// skipped without changing any result.
template <int D>
__device__ __forceinline__ bool residual_negligible_by_norms(const TileDesc &t, float qnc, float lg_bk,
                                                             const SoftState<D> &sm) {
    const float ub = qnc * t.kmax * (1.f + 1.f / 256.f) + lg_bk + 1.f / 64.f;
    if (!(ub < INFINITY)) return false;             // no bound for this tile
    return __ballot(!(ub < sm.m_ref - kNegligible)) == 0;
}

// One work item: the query block I of head bh = item / n_qb, from its first
// tile to its output rows.  kSparse: kept-list and residual tiles from a route;
// otherwise every key tile (dense).  LDS: K0/V0 and K1/V1, one tile each.
template <typename T, int D, int BQ, bool kSparse, bool kFused>
__device__ __forceinline__ void run_item(int item, const T *__restrict__ q, const T *__restrict__ k,
                                         const T *__restrict__ v, T *__restrict__ o, const FlashArgs &a,
                                         unsigned char *K0, unsigned char *V0, unsigned char *K1, unsigned char *V1,
                                         uint32_t *fw) {
    using C = FC<D, BQ>;
    constexpr bool kF32 = sizeof(T) == 4;
    // dense path with split key ranges: item = query block * kv_splits + split
    const int kv_part = kSparse ? 0 : item % a.kv_splits;
    if constexpr (!kSparse) item /= a.kv_splits;
    const int bh = item / a.n_qb;
    const int I = item - bh * a.n_qb;
    const int lane = lane_id();
    const int h = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const size_t head = (size_t)bh * a.N * D;            // keys and values
    const size_t qhead = (size_t)bh * a.Nq * D;          // queries and outputs
    const int qrow = I * a.block_q + wave * 32 + l32;
    const bool row_ok = qrow < a.Nq;

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
            const size_t off = qhead + (size_t)qrow * D + 16 * c2 + 8 * h;
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

    using Stream = std::conditional_t<kFused, BitStream, TileStream>;
    Stream ts;
    ts.exact_rows = kF32 ? 32 : 64;
    ts.exact_kind = kF32 ? kExactSplit : kExact;
    const size_t row_id = (size_t)bh * a.n_qb + I;
    if constexpr (kFused) {
        const int cnt = fused_route<D, BQ>(bh, I, a, fw);
        ts.lw = fw;
        ts.words = a.mask_words;
        ts.n_rt = (a.residual && cnt < a.n_kb) ? a.mask_words : 0;   // all kept: no residual
    } else {
        ts.li = 0; ts.sub = 0; ts.rt = 0;
        {
            const int tiles = (a.N + ts.exact_rows - 1) / ts.exact_rows;
            ts.t = (int)((int64_t)kv_part * tiles / a.kv_splits);         // this range's key tiles
            ts.dense_tiles = (int)((int64_t)(kv_part + 1) * tiles / a.kv_splits);
        }
        if constexpr (kSparse) {
            ts.list = (const kconst<int32_t> *)(a.kv_idx + row_id * a.kv_idx_cap);
            // at most the list's capacity and n_kb: a count beyond them (a route
            // that does not belong to this call) cannot run the stream off the list
            ts.cnt = min(max(__builtin_amdgcn_readfirstlane(a.kv_count[row_id]), 0), min(a.kv_idx_cap, a.n_kb));
            ts.mask = (const kconst<uint32_t> *)(a.kv_mask + row_id * a.mask_words);
            ts.n_rt = (a.residual && ts.cnt < a.n_kb) ? a.mask_words : 0;   // all kept: no residual
        } else {
            ts.list = nullptr;
            ts.mask = nullptr;
            ts.cnt = 0;
            ts.n_rt = 0;
        }
    }
    // bf16 residual tiles may be found negligible before their remainder part
    // is formed (residual_negligible): the route's per-tile bounds
    ts.bounds = (kSparse && !kF32 && a.k_bounds)
                    ? (const kconst<f32x2> *)(a.k_bounds + (size_t)bh * a.mask_words * 2)
                    : nullptr;
    ts.prime(a);
    HeadSrc<T> hs;
    hs.k = k + head;
    hs.v = v + head;
    hs.ks = kSparse ? a.kv_split + (size_t)bh * 2 * a.mask_words * kTile * D : nullptr;
    hs.vs = kSparse ? hs.ks + (size_t)a.mask_words * kTile * D : nullptr;
    hs.n_rows = a.N;
    const float lg_bk = log2f((float)a.block_k);
    const float lg_last = log2f((float)(a.N - (a.n_kb - 1) * a.block_k));
    const float c = a.scale_log2;
    // c times an upper bound on the norms of the wave's 32 query rows (raised by
    // 2^-10 over the rounding of the sums and the root): with a tile's bound
    // on its remainder rows it bounds what they add to any logit of the tile
    float qnc = INFINITY;
    if constexpr (kSparse && !kF32) {
        if (a.k_bounds) {
            float ss = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < D / 16; ++c2)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = (float)qf[c2][e];
                    ss = fmaf(x, x, ss);
                }
            const float m = wave_max(row_pair_sum(ss));
            qnc = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(__builtin_sqrtf(m)))) *
                  (1.f + 1.f / 1024.f) * c;
        }
    }

    SoftState<D> sm;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) sm.acc[i] = f32x16{};
    sm.m_ref = -INFINITY;
    sm.l_run = 0.f;
    Staging<D, BQ> st;

    TileDesc cur, nxt;
    bool have = ts.next(cur, a);
    if constexpr (kF32) {
        if (have) {
            issue_tile<T, D, BQ>(cur, hs, ln, K0, V0, wave, st);
            if (cur.kind == kExactSplit) store_split<D, BQ>(K0, V0, st);
        }
    } else {
        // bf16: K is double-buffered; the single V buffer takes a tile's values
        // at the start of that tile's step
        if (have) load_direct<D, BQ>(tile_rsrc<T, D>(cur, hs, false), K0, ln.ksrc, wave);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): this thread's loads have landed
    __syncthreads();
    // One pipeline step: compute the tile in (Kc, Vc) while the next tile streams
    // into Kn (and Vn for fp32 rows).  The loops below alternate two sets of LDS
    // arrays so that every LDS access names its buffer statically: the compiler
    // can then see that reads of the current tile do not alias the buffer->LDS
    // loads in flight.  bf16: the step starts the loads of the current tile's
    // values (first) and the next tile's keys; wait_v lets the values land.
    auto step = [&](const unsigned char *Kc, const unsigned char *Vc, unsigned char *Kn, unsigned char *Vn,
                    auto &&compute) -> bool {
        const bool have_next = ts.next(nxt, a);
        // Nothing is in flight here.  Saying so explicitly keeps the compiler from
        // placing its loop-entry wait after the prefetch below.
        __builtin_amdgcn_s_waitcnt(0x0F70);
        if constexpr (kF32) {
            if (have_next) issue_tile<T, D, BQ>(nxt, hs, ln, Kn, Vn, wave, st);
        } else {
            load_direct<D, BQ>(tile_rsrc<T, D>(cur, hs, true), const_cast<unsigned char *>(Vc), ln.vsrc, wave);
            if (have_next) load_direct<D, BQ>(tile_rsrc<T, D>(nxt, hs, false), Kn, ln.ksrc, wave);
        }
        auto wait_v = [&]() {
            if constexpr (!kF32) {
                // the PPW value pieces were issued before the PPW key pieces
                static_assert(C::PPW <= 15, "vmcnt field");
                if (have_next) __builtin_amdgcn_s_waitcnt(0x0F70 | C::PPW);
                else __builtin_amdgcn_s_waitcnt(0x0F70);
                __syncthreads();
            }
        };
        compute(Kc, Vc, wait_v);
        if constexpr (kF32) {
            if (have_next && nxt.kind == kExactSplit) store_split<D, BQ>(Kn, Vn, st);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the next keys have landed in LDS
        __syncthreads();
        cur = nxt;
        return have_next;
    };
    auto exact = [&](const unsigned char *Kc, const unsigned char *Vc, auto &wait_v) {
        tile_exact<D, BQ>(Kc, Vc, ln, qf, c, cur.valid, h, sm, wait_v);
    };
    auto split = [&](const unsigned char *Kc, const unsigned char *Vc, auto &wait_v) {
        f32x16 s0, s1;
        bf16x8 pa, pc;
        bool fold;
        if constexpr (kF32) {
            f32x16 s2[2];
            qk_tile<D, BQ, true>(Kc, ln, qf, ql, s2);
            s0 = s2[0];
            s1 = s2[1];
            fold = weights_split<D>(s0, s1, cur, c, lg_bk, lg_last, a.n_kb, h, sm, pa, pc);
        } else {
            // bf16 split tiles are residual tiles: first a test from the
            // norms alone, then the key means' bf16 part, and the remainder
            // part only if the tile may still matter
            fold = !residual_negligible_by_norms<D>(cur, qnc, lg_bk, sm);
            if (fold) {
                s0 = qk_half<D, BQ>(Kc, 0, ln, qf);
                fold = !residual_negligible<D>(s0, cur, c, lg_bk, lg_last, a.n_kb, h, sm, qnc);
            }
            if (fold) {
                s1 = qk_half<D, BQ>(Kc, 1, ln, qf);
                fold = weights_split<D>(s0, s1, cur, c, lg_bk, lg_last, a.n_kb, h, sm, pa, pc);
            }
        }
        wait_v();                       // every wave takes the workgroup barrier
        if (fold) {
            pv_half<D, BQ>(Vc, 0, ln, pa, pc, sm.acc);
            // Residual tiles take their block-mean values in bf16 (the hi rows): the
            // rounding moves an output by at most 2^-9 of the mean's magnitude times
            // the dropped blocks' weight, unlike a key-mean rounding, which the
            // exponential amplifies.  fp32 rows keep both halves.
            if (cur.kind == kExactSplit) pv_half<D, BQ>(Vc, 1, ln, pa, pc, sm.acc);
        }
    };
    // The stream gives the exact tiles of the kept blocks first, then the split
    // tiles (all tiles of fp32 inputs, the residual tiles of bf16 ones).
    bool odd = false;        // the current tile sits in (K1, V1)
    if constexpr (!kF32) {
        while (have && cur.kind == kExact) {
            have = step(K0, V0, K1, V1, exact);
            if (!have || cur.kind != kExact) {
                odd = true;
                break;
            }
            have = step(K1, V1, K0, V0, exact);
        }
    }
    if (have && odd) have = step(K1, V1, K0, V0, split);
    while (have) {
        have = step(K0, V0, K1, V1, split);
        if (!have) break;
        have = step(K1, V1, K0, V0, split);
    }

    // epilogue: O^T accumulator register r of block db holds feature 32db + 8(r/4) + 4h + r%4
    const float lt = row_pair_sum(sm.l_run);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    // The row index is formed again from the lane number rather than kept from
    // the prologue: held across the tile loops it does not fit the register
    // budget of three waves per SIMD and goes to scratch memory.
    int l32e = lane_id() & 31;
    asm volatile("" : "+v"(l32e));
    const int qrow_e = I * a.block_q + wave * 32 + l32e;
    if (qrow_e < a.Nq) {
        if (a.o32) {                     // fp32 output (an intermediate of a later step)
            float *orow = a.o32 + kv_part * a.split_o + qhead + (size_t)qrow_e * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    Store4<float>::st(orow + 32 * db + 8 * g + 4 * h, sm.acc[db][4 * g] * inv,
                                      sm.acc[db][4 * g + 1] * inv, sm.acc[db][4 * g + 2] * inv,
                                      sm.acc[db][4 * g + 3] * inv);
        } else {
            T *orow = o + qhead + (size_t)qrow_e * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    Store4<T>::st(orow + 32 * db + 8 * g + 4 * h, sm.acc[db][4 * g] * inv,
                                  sm.acc[db][4 * g + 1] * inv, sm.acc[db][4 * g + 2] * inv,
                                  sm.acc[db][4 * g + 3] * inv);
        }
        if (a.lse && h == 0)
            a.lse[kv_part * a.split_l + (size_t)bh * a.Nq + qrow_e] = lt > 0.f ? (sm.m_ref + log2f(lt)) * 0.69314718055994531f : -INFINITY;
    }
}

// Workgroup i runs on GPU die i % 8: the dispatcher deals workgroups to the 8
// dies (XCDs) in turn.  In each group of 8 * run consecutive workgroups, die x
// takes the run consecutive work positions x * run + 0..run-1 of the group, so
// that neighbouring query blocks, which keep mostly the same key blocks, meet in
// one die's L2, while the order of the work list holds at the scale of a group.
// The last, partial group keeps the plain order.  Runs of 32 for lists ordered
// by cost band alone, 64 for head-major lists (measured best for each).
constexpr int kDieRunLog2 = 5;
constexpr int kDieRunHeadMajorLog2 = 6;

__device__ __forceinline__ int grid_position(int i, int W, int run_log2) {
    const int group = 8 << run_log2;
    const int base = i & ~(group - 1);
    if (base + group > W) return i;
    const int r = i - base;
    return base + ((r & 7) << run_log2) + (r >> 3);
}

// One workgroup per work item (query block); kSparse takes the item from the
// route's work order, the dense path in plain order.
template <typename T, int D, int BQ, bool kSparse, bool kFused>
__global__ __launch_bounds__((FC<D, BQ>::THREADS)) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<T, BQ>, kWavesPerEU<T, BQ>))) void flash_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, T *__restrict__ o,
    FlashArgs a) {
    using C = FC<D, BQ>;
    const int p = grid_position(blockIdx.x, a.n_items, a.die_run_log2);
    // sparse paths take the route's cost-ordered work list (under fused routing
    // the pre-pass costs the decisions the forward takes)
    // (an entry outside [0, n_items) is clamped: a route that does not belong to
    // this call gives a wrong result, never a read outside the tensors)
    const int item = kSparse ? min(max(__builtin_amdgcn_readfirstlane(a.work_order[p]), 0), a.n_items - 1) : p;
    __shared__ __attribute__((aligned(1024))) unsigned char K0[C::TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char K1[C::TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char V0[C::TILE];
    uint32_t *fw = nullptr;
    if constexpr (kFused) {
        __shared__ uint32_t FW[kFusedWords + 4 * C::WAVES];
        fw = FW;
    }
    if constexpr (sizeof(T) == 2) {
        run_item<T, D, BQ, kSparse, kFused>(item, q, k, v, o, a, K0, V0, K1, V0, fw);
    } else {
        __shared__ __attribute__((aligned(1024))) unsigned char V1[C::TILE];
        run_item<T, D, BQ, kSparse, kFused>(item, q, k, v, o, a, K0, V0, K1, V1, fw);
    }
}

template <typename T, int D, int BQ, bool kSparse, bool kFused>
static hipError_t launch_flash_t(const void *q, const void *k, const void *v, void *o,
                                 const FlashArgs &a, int BH, hipStream_t st) {
    using C = FC<D, BQ>;
    auto kern = flash_kernel<T, D, BQ, kSparse, kFused>;
    FlashArgs args = a;
    if (args.kv_splits < 1 || kSparse) args.kv_splits = 1;
    args.n_items = BH * a.n_qb * args.kv_splits;
    args.die_run_log2 = kSparse && head_major_order(BH, a.n_qb) ? kDieRunHeadMajorLog2 : kDieRunLog2;
    hipLaunchKernelGGL(kern, dim3(args.n_items), dim3(C::THREADS), 0, st, (const T *)q, (const T *)k,
                       (const T *)v, (T *)o, args);
    return hipGetLastError();
}

template <typename T, int D, int BQ>
static hipError_t launch_flash_s(const void *q, const void *k, const void *v, void *o, const FlashArgs &a,
                                 int BH, hipStream_t st) {
    if (a.kv_mask_out) return launch_flash_t<T, D, BQ, true, true>(q, k, v, o, a, BH, st);
    return a.kv_idx ? launch_flash_t<T, D, BQ, true, false>(q, k, v, o, a, BH, st)
                    : launch_flash_t<T, D, BQ, false, false>(q, k, v, o, a, BH, st);
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
