// Probe-fitted residual correction (SparsePR summary, section B): a second way
// to correct the sparse output, beside the proxy-reuse residual of the forward.
//
//   1. the sparse output O_s over the kept tokens only, in fp32 (forward kernel,
//      no block residual);
//   2. probe rows, P per query block evenly spread (row I*bq + floor((j+1/2) m_I / P)),
//      gathered and attended densely (forward kernel, dense path, the key tiles
//      split into ranges whose rows merge by their log-sum-exp), in fp32;
//   3. per (b, h) and chunk of kPrChunk probes, one workgroup forms the chunk's
//      means and centred Gram matrices; then per (b, h) one workgroup combines
//      the chunks (the centred scatter of a union is the sum of the chunks'
//      plus n_c (m_c - m)(m_c - m)^T per chunk, which keeps the centring exact
//      in fp32) and fits R = O_d - O_s at the probes as an affine map of
//      x = O_s, B = (G + lam I)^-1 H with a ridge lam = ridge * trace / d and
//      the intercept b = rm - xm B, projected on the k leading eigenvectors Q
//      of R^T R (the right singular vectors of R; subspace iteration on 2k
//      columns, then Rayleigh-Ritz), Pk = Q Q^T.  Only W = B Q is formed, by
//      a Cholesky solve with the k columns of H Q; the fit leaves W, Q and
//      C_b = (rm Q - xm W) Q^T;
//   4. every row not probed takes O_s + C_b + (O_s W) Q^T (= O_s B Pk + b Pk
//      + O_s), probed rows take O_d.
//
// Steps 3 and 4 are small: d x d matrices per head and one d x d product per row.
#include <math.h>
#include <stdint.h>

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

constexpr int kPrThreads = 256;
constexpr int kPrIters = 40;             // subspace iterations on k columns (no room to double them)
constexpr int kPrItersOver = 6;          // subspace iterations on 2k columns
constexpr int kPrJacobiSweeps = 4;       // Jacobi sweeps of the Rayleigh-Ritz step
constexpr int kFitThreads = 512;         // the fit: two waves per SIMD hide its LDS latencies (1024 is slower)

__device__ __forceinline__ int probe_row(int j, const PrArgs &a) {
    const int I = j / a.per_block, jj = j - I * a.per_block;
    const int m = min(a.block_q, a.N - I * a.block_q);
    return I * a.block_q + (2 * jj + 1) * m / (2 * a.per_block);
}

// ------------------------------------------------------------------ gather
template <typename T>
__global__ __launch_bounds__(kPrThreads) void probe_gather_kernel(const T *__restrict__ q, T *__restrict__ qp,
                                                                   PrArgs a, int D) {
    const int bh = blockIdx.y;
    const int units = D * (int)sizeof(T) / 16;
    const int u = threadIdx.x % units, step = kPrThreads / units;
    const uint4 *src = reinterpret_cast<const uint4 *>(q) + (size_t)bh * a.N * units;
    uint4 *dst = reinterpret_cast<uint4 *>(qp) + (size_t)bh * a.M * units;
    const int j_end = min(a.M, (int)(blockIdx.x + 1) * 64);
    for (int j = blockIdx.x * 64 + threadIdx.x / units; j < j_end; j += step)
        dst[(size_t)j * units + u] = src[(size_t)probe_row(j, a) * units + u];
}

// ------------------------------------------------------------------ fit
// Lower triangle of a D x D matrix, packed by rows.
__device__ __forceinline__ int tri(int i, int j) { return i * (i + 1) / 2 + j; }

// sum over k = k0, k0 + step, ... < k1 of x[k * sx] * y[k * sy] (LDS), with eight
// independent partial sums so that the reads are issued ahead of their use
__device__ __forceinline__ float lds_dot(const float *x, int sx, const float *y, int sy, int k0, int k1, int step) {
    float p[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int k = k0;
    for (; k + 7 * step < k1; k += 8 * step) {
        float xv[8], yv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            xv[u] = x[(k + u * step) * sx];
            yv[u] = y[(k + u * step) * sy];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) p[u] = fmaf(xv[u], yv[u], p[u]);
    }
    for (; k < k1; k += step) p[0] = fmaf(x[k * sx], y[k * sy], p[0]);
    return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

// One chunk of kPrChunk probes of one (b, h): its means of x and r and, with
// xc = x - xm and rc = r - rm (chunk means), G = sum xc xc^T, H = sum xc rc^T
// and S = sum r r^T = sum rc rc^T + n rm rm^T.  The centred rows are staged in
// LDS 32 probes at a time; thread (bi, bj) accumulates the BE x BE blocks
// (bi, bj) of the three matrices in registers.
template <int D>
__global__ __launch_bounds__(kPrThreads) void pr_gram_kernel(PrArgs a) {
    constexpr int BE = D / 16;                            // block edge: 16 x 16 blocks
    constexpr int JS = 32;                                // probes per staging step
    static_assert(BE % 4 == 0, "blocks of whole float4s");
    const int c = blockIdx.x, bh = blockIdx.y;
    const int jb = c * kPrChunk, je = min(a.M, jb + kPrChunk);
    __shared__ __attribute__((aligned(16))) float XC[JS * D];
    __shared__ __attribute__((aligned(16))) float RC[JS * D];
    __shared__ float ps[kPrThreads / D][2][D];
    __shared__ float xm[D], rm[D];
    const float *Os = a.O32 + (size_t)bh * a.N * D;
    const float *Od = a.Od32 + (size_t)bh * a.M * D;
    {
        constexpr int NP = kPrThreads / D;                // threads per feature
        const int f = threadIdx.x % D, part = threadIdx.x / D;
        float sx = 0.f, sr = 0.f;
#pragma unroll 8
        for (int j = jb + part; j < je; j += NP) {
            const float x = Os[(size_t)probe_row(j, a) * D + f];
            sx += x;
            sr += Od[(size_t)j * D + f] - x;
        }
        ps[part][0][f] = sx;
        ps[part][1][f] = sr;
    }
    __syncthreads();
    const float n_rows = (float)(je - jb);
    if (threadIdx.x < D) {
        float sx = 0.f, sr = 0.f;
#pragma unroll
        for (int q = 0; q < kPrThreads / D; ++q) {
            sx += ps[q][0][threadIdx.x];
            sr += ps[q][1][threadIdx.x];
        }
        xm[threadIdx.x] = sx / n_rows;
        rm[threadIdx.x] = sr / n_rows;
        float *cm = a.cmean + ((size_t)bh * a.n_chunks + c) * 2 * D;
        cm[threadIdx.x] = sx / n_rows;
        cm[D + threadIdx.x] = sr / n_rows;
    }
    const int bi = threadIdx.x / 16, bj = threadIdx.x % 16;
    float g[BE][BE], hm[BE][BE], sm[BE][BE];
#pragma unroll
    for (int u = 0; u < BE; ++u)
#pragma unroll
        for (int v = 0; v < BE; ++v) g[u][v] = hm[u][v] = sm[u][v] = 0.f;
    for (int j0 = jb; j0 < je; j0 += JS) {
        __syncthreads();                                  // the means are in; the last step's rows are read
        for (int e = threadIdx.x; e < JS * D; e += kPrThreads) {
            const int j = j0 + e / D, f = e % D;
            float xc = 0.f, rc = 0.f;
            if (j < je) {
                const float x = Os[(size_t)probe_row(j, a) * D + f];
                xc = x - xm[f];
                rc = (Od[(size_t)j * D + f] - x) - rm[f];
            }
            XC[e] = xc;
            RC[e] = rc;
        }
        __syncthreads();
        const int jn = min(JS, je - j0);
        for (int jj = 0; jj < jn; ++jj) {
            float xa[BE], ra[BE], xb[BE], rb[BE];
#pragma unroll
            for (int q = 0; q < BE; q += 4) {
                const f32x4 x4a = *reinterpret_cast<const f32x4 *>(XC + jj * D + bi * BE + q);
                const f32x4 r4a = *reinterpret_cast<const f32x4 *>(RC + jj * D + bi * BE + q);
                const f32x4 x4b = *reinterpret_cast<const f32x4 *>(XC + jj * D + bj * BE + q);
                const f32x4 r4b = *reinterpret_cast<const f32x4 *>(RC + jj * D + bj * BE + q);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    xa[q + w] = x4a[w];
                    ra[q + w] = r4a[w];
                    xb[q + w] = x4b[w];
                    rb[q + w] = r4b[w];
                }
            }
#pragma unroll
            for (int u = 0; u < BE; ++u)
#pragma unroll
                for (int v = 0; v < BE; ++v) {
                    g[u][v] = fmaf(xa[u], xb[v], g[u][v]);
                    hm[u][v] = fmaf(xa[u], rb[v], hm[u][v]);
                    sm[u][v] = fmaf(ra[u], rb[v], sm[u][v]);
                }
        }
    }
    float *out = a.part + ((size_t)bh * a.n_chunks + c) * 3 * D * D;
#pragma unroll
    for (int u = 0; u < BE; ++u) {
        const int i = bi * BE + u;
#pragma unroll
        for (int v = 0; v < BE; ++v) {
            const int j = bj * BE + v;
            out[i * D + j] = g[u][v];
            out[D * D + i * D + j] = hm[u][v];
            out[2 * D * D + i * D + j] = sm[u][v] + n_rows * rm[i] * rm[j];
        }
    }
}

// LDS of the fit, one pool: packed R^T R (subspace phase), then the packed
// factor; the means; 32 solution columns; the subspace basis.
template <int D>
struct FitLds {
    static constexpr int kTri = D * (D + 1) / 2;
    static constexpr int kRegion = 32 * D > 2 * 16 * D ? 32 * D : 2 * 16 * D;   // >= D * kPrMaxRank too
    static_assert(kRegion >= D * kPrMaxRank, "basis fits the region");
    static_assert(kRegion >= D * kPrMaxRank + 2 * kPrMaxRank * kPrMaxRank + kPrMaxRank,
                  "Rayleigh-Ritz: S Q, the small matrix, its rotations and their order fit the region");
    static constexpr int kFloats = kTri + 2 * D + 64 + kRegion + D * kPrMaxRank;
};

template <int D>
__global__ __launch_bounds__(kFitThreads) void pr_fit_kernel(PrArgs a) {
    using FL = FitLds<D>;
    const int bh = blockIdx.x;
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    __shared__ float pool[FL::kFloats];
    float *L = pool;                         // packed lower triangle
    float *xm = pool + FL::kTri, *rm = xm + D;
    float *red = rm + D;                     // 64 floats of small values
    float *wb = red + 16;
    float *reg = red + 64;                   // the solve's 32 columns
    float *Qs = reg + FL::kRegion;           // the subspace basis, Qs[i * KP + c]
    float *Gm = a.scratch + (size_t)bh * 3 * D * D;      // centred X^T X, then X^T R, then R^T R
    float *Hm = Gm + D * D;
    float *Sm = Hm + D * D;
    float *Bm = a.CB + (size_t)bh * D * D;
    float *bv = a.Cb + (size_t)bh * D;
    const float invM = 1.f / (float)a.M;

    // means of x and r over the probes: the chunks' means weighted by their rows
    const int C = a.n_chunks;
    const float *cmean = a.cmean + (size_t)bh * C * 2 * D;
    const float *part = a.part + (size_t)bh * C * 3 * D * D;
    auto rows_of = [&](int c) { return (float)(min(a.M, (c + 1) * kPrChunk) - c * kPrChunk); };
    if (threadIdx.x < D) {
        float sx = 0.f, sr = 0.f;
        for (int c = 0; c < C; ++c) {
            const float n = rows_of(c);
            sx += n * cmean[(size_t)c * 2 * D + threadIdx.x];
            sr += n * cmean[(size_t)c * 2 * D + D + threadIdx.x];
        }
        xm[threadIdx.x] = sx * invM;
        rm[threadIdx.x] = sr * invM;
    }
    __syncthreads();
    // G = sum_c (G_c + n_c dx_c dx_c^T), H = sum_c (H_c + n_c dx_c dr_c^T), S = sum_c S_c,
    // with dx_c = xm_c - xm and dr_c = rm_c - rm
    // (four entries e, e + 256, ... per thread, so that their loads overlap)
    constexpr int EU = 4;
    static_assert(D * D % (EU * kFitThreads) == 0, "entries split evenly");
    for (int e0 = threadIdx.x; e0 < D * D; e0 += EU * kFitThreads) {
        float g[EU], hh[EU], sv[EU];
#pragma unroll
        for (int u = 0; u < EU; ++u) g[u] = hh[u] = sv[u] = 0.f;
        const int j = e0 % D;                             // the same column for the four entries
        for (int c = 0; c < C; ++c) {
            const float *pc = part + (size_t)c * 3 * D * D;
            const float *mc = cmean + (size_t)c * 2 * D;
            const float n = rows_of(c);
            const float dxj = mc[j] - xm[j], drj = mc[D + j] - rm[j];
#pragma unroll
            for (int u = 0; u < EU; ++u) {
                const int e = e0 + u * kFitThreads, i = e / D;
                const float dxi = mc[i] - xm[i];
                g[u] += pc[e] + n * dxi * dxj;
                hh[u] += pc[D * D + e] + n * dxi * drj;
                sv[u] += pc[2 * D * D + e];
            }
        }
#pragma unroll
        for (int u = 0; u < EU; ++u) {
            const int e = e0 + u * kFitThreads;
            Gm[e] = g[u];
            Hm[e] = hh[u];
            Sm[e] = sv[u];
        }
    }
    __threadfence_block();
    __syncthreads();

    // ridge relative to the scale of the centred Gram matrix
    float tr = 0.f;
    for (int i = threadIdx.x; i < D; i += kFitThreads) tr += Gm[i * D + i];
    tr = wave_sum(tr);
    if (lane == 0) red[wave] = tr;
    __syncthreads();
    float trace = 0.f;
#pragma unroll
    for (int w = 0; w < kFitThreads / kWave; ++w) trace += red[w];
    const float lam = a.ridge * trace / (float)D;

    // Only B Pk = B Q Q^T is needed (Q: the k leading eigenvectors of R^T R), and
    // B Q = (G + lam I)^-1 (H Q): the subspace comes first, then a solve with k
    // right-hand sides instead of D.

    // Leading eigenvectors of S = R^T R: subspace iteration on K2 = min(2k, 16)
    // columns from a fixed start (S packed into LDS), then Rayleigh-Ritz: the
    // k leading eigenvectors of the K2 x K2 matrix Q^T S Q (Jacobi rotations)
    // carried back, Q_k = Q U_k.  With twice the columns the k-th direction
    // separates at the rate lambda_{2k+1} / lambda_k per step instead of
    // lambda_{k+1} / lambda_k; without room for them (k > 8) more steps are taken.
    float *Sp = L;
    const int K = a.rank;
    const int K2 = min(2 * K, kPrMaxRank);
    const int KI = (K2 + 3) & ~3;                         // row stride of the iterated basis
    const int KP = (K + 3) & ~3;                          // row stride of the final basis (zero past K)
    const int n_iter = K2 >= 2 * K ? kPrItersOver : kPrIters;
#pragma unroll 16
    for (int e = threadIdx.x; e < D * D; e += kFitThreads) {
        const int i = e / D, j = e - (e / D) * D;
        if (j <= i) Sp[tri(i, j)] = Sm[e];
    }
    for (int e = threadIdx.x; e < D * KI; e += kFitThreads) {
        const int i = e / KI, c = e - (e / KI) * KI;
        const int f = i * K2 + c;                         // the start's entry (i, c)
        uint32_t hsh = (uint32_t)f * 2654435761u + 0x9e3779b9u;
        hsh ^= hsh >> 15;
        hsh *= 2246822519u;
        hsh ^= hsh >> 13;
        Qs[e] = c < K2 ? (float)(hsh & 0xffff) / 32768.f - 1.f : 0.f;
    }
    __syncthreads();
    // Z = S Q into dst (stride KI): thread (i, part) forms row i over a part of
    // the l range for every column (each S entry read once), the parts meet by
    // lane swaps.  Ends with a barrier.
    auto s_times_q = [&](float *dst) {
        constexpr int TPR = kFitThreads / D;             // threads per row (a power of two)
        const int i = threadIdx.x / TPR, part = threadIdx.x % TPR;
        f32x4 z[kPrMaxRank / 4];
#pragma unroll
        for (int g = 0; g < kPrMaxRank / 4; ++g) z[g] = f32x4{};
        const int l0 = part * (D / TPR), l1 = l0 + D / TPR;
        const int G4 = KI / 4;
#pragma unroll 8
        for (int l = l0; l < l1; ++l) {
            const float sv = l <= i ? Sp[tri(i, l)] : Sp[tri(l, i)];
            const f32x4 *ql = reinterpret_cast<const f32x4 *>(Qs + l * KI);
#pragma unroll
            for (int g = 0; g < kPrMaxRank / 4; ++g)
                if (g < G4) z[g] += sv * ql[g];
        }
#pragma unroll
        for (int g = 0; g < kPrMaxRank / 4; ++g) {
            if (g < G4) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    float v = z[g][u];
#pragma unroll
                    for (int sh = 1; sh < TPR; sh <<= 1) v += __shfl_xor(v, sh, kWave);
                    z[g][u] = v;
                }
            }
        }
        __syncthreads();
        if (part == 0)
#pragma unroll
            for (int g = 0; g < kPrMaxRank / 4; ++g)
                if (g < G4) *reinterpret_cast<f32x4 *>(dst + i * KI + 4 * g) = z[g];
        __syncthreads();
    };
    for (int it = 0; it <= n_iter; ++it) {
        if (it > 0) s_times_q(Qs);
        // modified Gram-Schmidt on the columns, by one wave, in registers: lane
        // l holds rows l, l + 64, ..  In fp32 one pass leaves the basis
        // orthogonal only to about eps times the spread of the column norms
        // (up to 1e-3 here), which would carry into Pk = Q Q^T; the last
        // iteration, whose basis the Rayleigh-Ritz step uses, orthogonalises
        // twice (a second pass restores orthogonality to rounding).
        if (wave == 0) {
            constexpr int RL = D / kWave;                 // rows per lane
            float qv[RL][kPrMaxRank];
#pragma unroll
            for (int r = 0; r < RL; ++r)
#pragma unroll
                for (int c = 0; c < kPrMaxRank; ++c) qv[r][c] = c < K2 ? Qs[(lane + r * kWave) * KI + c] : 0.f;
            const int passes = it == n_iter ? 2 : 1;
            for (int pass = 0; pass < passes; ++pass)
#pragma unroll
            for (int c = 0; c < kPrMaxRank; ++c) {
                if (c >= K2) break;
#pragma unroll
                for (int pcol = 0; pcol < c; ++pcol) {
                    float dp = 0.f;
#pragma unroll
                    for (int r = 0; r < RL; ++r) dp = fmaf(qv[r][pcol], qv[r][c], dp);
                    dp = wave_sum(dp);
#pragma unroll
                    for (int r = 0; r < RL; ++r) qv[r][c] = fmaf(-dp, qv[r][pcol], qv[r][c]);
                }
                float nn = 0.f;
#pragma unroll
                for (int r = 0; r < RL; ++r) nn = fmaf(qv[r][c], qv[r][c], nn);
                nn = wave_sum(nn);
                const float inv = nn > 0.f ? 1.f / sqrtf(nn) : 0.f;
#pragma unroll
                for (int r = 0; r < RL; ++r) qv[r][c] *= inv;
            }
#pragma unroll
            for (int r = 0; r < RL; ++r)
#pragma unroll
                for (int c = 0; c < kPrMaxRank; ++c)
                    if (c < K2) Qs[(lane + r * kWave) * KI + c] = qv[r][c];
        }
        __syncthreads();
    }
    // Rayleigh-Ritz.  The T region holds Z = S Q, then Hr = Q^T Z (K2 x K2,
    // stride 16), Ur (the rotations, K2 x K2, stride 16) and the order of the
    // Ritz values.
    {
        float *Z = reg;
        float *Hr = reg + D * kPrMaxRank;
        float *Ur = Hr + kPrMaxRank * kPrMaxRank;
        int *sel = reinterpret_cast<int *>(Ur + kPrMaxRank * kPrMaxRank);
        s_times_q(Z);
        for (int e = threadIdx.x; e < K2 * K2; e += kFitThreads) {
            const int r = e / K2, c = e - (e / K2) * K2;
            float h = 0.f;
#pragma unroll 8
            for (int l = 0; l < D; ++l) h = fmaf(Qs[l * KI + r], Z[l * KI + c], h);
            Hr[r * kPrMaxRank + c] = h;
        }
        __syncthreads();
        if (wave == 0) {
            // symmetrise (rounding), then cyclic Jacobi: lane j < K2 updates
            // entries (j, p), (j, q) and their mirrors, and row j of U
            if (lane < K2)
                for (int c = 0; c < lane; ++c) {
                    const float m = 0.5f * (Hr[lane * kPrMaxRank + c] + Hr[c * kPrMaxRank + lane]);
                    Hr[lane * kPrMaxRank + c] = m;
                    Hr[c * kPrMaxRank + lane] = m;
                }
            float u[kPrMaxRank];
#pragma unroll
            for (int c = 0; c < kPrMaxRank; ++c) u[c] = c == lane ? 1.f : 0.f;
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
            for (int sweep = 0; sweep < kPrJacobiSweeps; ++sweep) {
#pragma unroll
                for (int pp = 0; pp < kPrMaxRank - 1; ++pp) {
#pragma unroll
                    for (int qq = pp + 1; qq < kPrMaxRank; ++qq) {
                        if (qq >= K2) break;
                        const float hpq = Hr[pp * kPrMaxRank + qq];
                        const float hpp = Hr[pp * kPrMaxRank + pp], hqq = Hr[qq * kPrMaxRank + qq];
                        // converged pairs (off-diagonal below fp32 resolution of the diagonal) are skipped
                        if (!(fabsf(hpq) > 1e-7f * (fabsf(hpp) + fabsf(hqq)))) continue;
                        const float theta = (hqq - hpp) / (2.f * hpq);
                        const float t = (theta >= 0.f ? 1.f : -1.f) / (fabsf(theta) + sqrtf(theta * theta + 1.f));
                        const float c = 1.f / sqrtf(t * t + 1.f), sn = t * c;
                        if (lane < K2 && lane != pp && lane != qq) {
                            const float hjp = Hr[lane * kPrMaxRank + pp], hjq = Hr[lane * kPrMaxRank + qq];
                            const float np = c * hjp - sn * hjq, nq = sn * hjp + c * hjq;
                            Hr[lane * kPrMaxRank + pp] = np;
                            Hr[lane * kPrMaxRank + qq] = nq;
                            Hr[pp * kPrMaxRank + lane] = np;
                            Hr[qq * kPrMaxRank + lane] = nq;
                        }
                        if (lane == 0) {
                            Hr[pp * kPrMaxRank + pp] = hpp - t * hpq;
                            Hr[qq * kPrMaxRank + qq] = hqq + t * hpq;
                            Hr[pp * kPrMaxRank + qq] = 0.f;
                            Hr[qq * kPrMaxRank + pp] = 0.f;
                        }
                        const float up = u[pp], uq = u[qq];
                        u[pp] = c * up - sn * uq;
                        u[qq] = sn * up + c * uq;
                        __builtin_amdgcn_s_waitcnt(0xc07f);
                        __builtin_amdgcn_wave_barrier();
                    }
                }
            }
            // lane j: row j of U; rank of the Ritz value j (largest first, ties by index)
            if (lane < K2) {
#pragma unroll
                for (int c = 0; c < kPrMaxRank; ++c)
                    if (c < K2) Ur[lane * kPrMaxRank + c] = u[c];
                const float dj = Hr[lane * kPrMaxRank + lane];
                int rank = 0;
                for (int m = 0; m < K2; ++m) {
                    const float dm = Hr[m * kPrMaxRank + m];
                    rank += dm > dj || (dm == dj && m < lane);
                }
                if (rank < K) sel[rank] = lane;
            }
        }
        __syncthreads();
        // Q_k = Q U_k into Z (stride KP), then back into Qs
        for (int e = threadIdx.x; e < D * KP; e += kFitThreads) {
            const int i = e / KP, r = e - (e / KP) * KP;
            float v = 0.f;
            if (r < K) {
                const int j = sel[r];
                for (int m = 0; m < K2; ++m) v = fmaf(Qs[i * KI + m], Ur[m * kPrMaxRank + j], v);
            }
            Z[e] = v;
        }
        __syncthreads();
        for (int e = threadIdx.x; e < D * KP; e += kFitThreads) Qs[e] = Z[e];
        __syncthreads();
    }

    // G + lam I, packed over S (no longer needed)
#pragma unroll 16
    for (int e = threadIdx.x; e < D * D; e += kFitThreads) {
        const int i = e / D, j = e - (e / D) * D;
        if (j <= i) L[tri(i, j)] = Gm[e] + (i == j ? lam : 0.f);
    }
    // right-hand sides T = H Q (columns c < K of the 32-column region, the rest zero)
    float *T = reg;                                       // T[i * 32 + c]
    for (int e = threadIdx.x; e < D * 32; e += kFitThreads) {
        const int i = e / 32, c = e - (e / 32) * 32;
        float v = 0.f;
        if (c < K) {
            const float *hrow = Hm + (size_t)i * D;
#pragma unroll 8
            for (int l = 0; l < D; ++l) v = fmaf(hrow[l], Qs[l * KP + c], v);
        }
        T[e] = v;
    }
    __syncthreads();

    // Cholesky G + lam I = L L^T, left-looking, in place (row i of the packed
    // triangle holds L[i][0..j-1] and the matrix entries from j on): column j
    // needs its diagonal, a dot product of row j with itself (wave 0), then for
    // every row below it a dot product with row j (two threads per row, a half
    // of the terms each).
    for (int j = 0; j < D; ++j) {
        const float *Lj = L + tri(j, 0);
        if (wave == 0) {
            float dsum = 0.f;
            for (int k = lane; k < j; k += kWave) dsum = fmaf(Lj[k], Lj[k], dsum);
            dsum = wave_sum(dsum);
            if (lane == 0) L[tri(j, j)] = sqrtf(fmaxf(L[tri(j, j)] - dsum, 1e-30f));
        }
        __syncthreads();
        const float djj = L[tri(j, j)];
        for (int t = threadIdx.x; t < 2 * (D - 1 - j); t += kFitThreads) {
            const int i = j + 1 + (t >> 1), half = t & 1;
            const float *Li = L + tri(i, 0);
            float p[4] = {0.f, 0.f, 0.f, 0.f};
            int k = half;
            for (; k + 6 < j; k += 8) {
#pragma unroll
                for (int u = 0; u < 4; ++u) p[u] = fmaf(Li[k + 2 * u], Lj[k + 2 * u], p[u]);
            }
            for (; k < j; k += 2) p[0] = fmaf(Li[k], Lj[k], p[0]);
            float sdot = (p[0] + p[1]) + (p[2] + p[3]);
            sdot += __shfl_xor(sdot, 1, kWave);
            if (half == 0) L[tri(i, j)] = (L[tri(i, j)] - sdot) / djj;
        }
        __syncthreads();
    }

    // W = (L L^T)^-1 T in place, by one wave: lane (part, c) takes column c
    // (< 16 >= K) and the terms k = part mod 4 of each dot product; the four
    // parts meet by lane swaps
    if (wave == 0) {
        const int c = lane & 15, part = lane >> 4;
        auto meet = [&](float v) {
            v += __shfl_xor(v, 16, kWave);
            v += __shfl_xor(v, 32, kWave);
            return v;
        };
        for (int i = 0; i < D; ++i) {                     // forward: L y = t
            const float *Li = L + tri(i, 0);
            const float s = meet(lds_dot(Li, 1, T + c, 32, part, i, 4));
            if (part == 0) T[i * 32 + c] = (T[i * 32 + c] - s) / Li[i];
            __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): this wave's LDS writes are done
            __builtin_amdgcn_wave_barrier();
        }
        for (int i = D - 1; i >= 0; --i) {                // backward: L^T w = y
            float p[4] = {0.f, 0.f, 0.f, 0.f};
            int k = i + 1 + part;
            for (; k + 12 < D; k += 16) {
                float lv[4], tv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    lv[u] = L[tri(k + 4 * u, i)];
                    tv[u] = T[(k + 4 * u) * 32 + c];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) p[u] = fmaf(lv[u], tv[u], p[u]);
            }
            for (; k < D; k += 4) p[0] = fmaf(L[tri(k, i)], T[k * 32 + c], p[0]);
            const float s = meet((p[0] + p[1]) + (p[2] + p[3]));
            if (part == 0) T[i * 32 + c] = (T[i * 32 + c] - s) / L[tri(i, i)];
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
        }
    }
    __syncthreads();

    // W = B Q sits in T; b Q = rm Q - xm W; then C_B = W Q^T, C_b = (b Q) Q^T
    if (threadIdx.x < K) {
        const int c = threadIdx.x;
        float s = 0.f;
#pragma unroll 16
        for (int l = 0; l < D; ++l) s += rm[l] * Qs[l * KP + c] - xm[l] * T[l * 32 + c];
        wb[c] = s;
    }
    __syncthreads();
    // the map's factors for the apply: W = B Q, then Q, both D x KP (zero past K)
    for (int e = threadIdx.x; e < D * KP; e += kFitThreads) {
        const int i = e / KP, c = e - (e / KP) * KP;
        Bm[e] = c < K ? T[i * 32 + c] : 0.f;
        Bm[D * KP + e] = Qs[e];
    }
    if (threadIdx.x < D) {
        float s = 0.f;
        for (int c = 0; c < K; ++c) s += wb[c] * Qs[threadIdx.x * KP + c];
        bv[threadIdx.x] = s;
    }
}

// ------------------------------------------------------------------ apply
// Four consecutive outputs in one store.
template <typename T> struct Store4;
template <> struct Store4<bf16> {
    static __device__ __forceinline__ void st(bf16 *dst, const float *v) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)v[e];
        *reinterpret_cast<bf16x4 *>(dst) = w;
    }
};
template <> struct Store4<float> {
    static __device__ __forceinline__ void st(float *dst, const float *v) {
        *reinterpret_cast<f32x4 *>(dst) = f32x4{v[0], v[1], v[2], v[3]};
    }
};

// Every row takes O_s + C_b + O_s C_B with C_B = W Q^T of rank k: y = x W (k
// values), then x + C_b + y Q^T; a row per four threads, D / 4 columns each in
// groups of four, group g of thread p at columns 4 (p + 4 g) .. (the four
// threads of a row read 64 contiguous bytes per load; the k partial sums of y
// meet by lane swaps).  HBM-bound: one read of O_s and one write of O.
// G4: groups of four rank columns, (k + 3) / 4.
template <typename T, int D, int G4>
__global__ __launch_bounds__(kPrThreads) void pr_apply_kernel(T *__restrict__ o, PrArgs a) {
    constexpr int TPR = 4;                    // threads per row
    constexpr int CPT = D / TPR;              // columns per thread
    constexpr int RPB = kPrThreads / TPR;     // rows per workgroup
    const int bh = blockIdx.y;
    constexpr int KP = 4 * G4;
    __shared__ __attribute__((aligned(16))) float Ws[D * kPrMaxRank];
    __shared__ __attribute__((aligned(16))) float Qs[D * kPrMaxRank];
    __shared__ float Cbs[D];
    __shared__ int probe_off[2 * kPrMaxPerBlock];         // probe rows (offsets in block) of the two blocks met
    const float *F = a.CB + (size_t)bh * D * D;           // W [D][KP], then Q [D][KP]
    const int I0 = blockIdx.x * RPB / a.block_q;          // first query block of this workgroup's rows
    if (threadIdx.x < 2 * a.per_block) {
        const int I = I0 + threadIdx.x / a.per_block, jj = threadIdx.x % a.per_block;
        const int mI = max(0, min(a.block_q, a.N - I * a.block_q));
        probe_off[threadIdx.x] = mI > 0 ? (2 * jj + 1) * mI / (2 * a.per_block) : -1;
    }
    for (int e = threadIdx.x; e < D * KP; e += kPrThreads) {
        Ws[e] = F[e];
        Qs[e] = F[D * KP + e];
    }
    for (int e = threadIdx.x; e < D; e += kPrThreads) Cbs[e] = a.Cb[(size_t)bh * D + e];
    __syncthreads();
    const int r = blockIdx.x * RPB + threadIdx.x / TPR;
    const int pt = threadIdx.x % TPR;
    auto col = [&](int c) { return 4 * (pt + TPR * (c >> 2)) + (c & 3); };   // thread's c-th column
    if (r >= a.N) return;
    const float *xr = a.O32 + ((size_t)bh * a.N + r) * D;
    float x[CPT];
#pragma unroll
    for (int q = 0; q < CPT; q += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(xr + col(q));
#pragma unroll
        for (int w = 0; w < 4; ++w) x[q + w] = v[w];
    }
    // W and Q rows in groups of four (KP = 4 G4; columns past K are zero)
    f32x4 y[G4];
#pragma unroll
    for (int g = 0; g < G4; ++g) y[g] = f32x4{};
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const f32x4 *wr = reinterpret_cast<const f32x4 *>(Ws + col(c) * KP);
#pragma unroll
        for (int g = 0; g < G4; ++g) y[g] += x[c] * wr[g];
    }
#pragma unroll
    for (int g = 0; g < G4; ++g) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            y[g][u] += __shfl_xor(y[g][u], 1, kWave);
            y[g][u] += __shfl_xor(y[g][u], 2, kWave);
        }
    }
    // probed rows take their dense values (the rows of a workgroup meet at most
    // two query blocks: RPB <= block_q)
    const int I = r / a.block_q, off = r - I * a.block_q;
    const int* po = probe_off + (I - I0) * a.per_block;
    int probe = -1;
    for (int jj = 0; jj < a.per_block; ++jj)
        if (po[jj] == off) probe = I * a.per_block + jj;
    T *orow = o + ((size_t)bh * a.N + r) * D;
    float out[CPT];
    if (probe >= 0) {
        const float *od = a.Od32 + ((size_t)bh * a.M + probe) * D;
#pragma unroll
        for (int c = 0; c < CPT; ++c) out[c] = od[col(c)];
    } else {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const f32x4 *qr = reinterpret_cast<const f32x4 *>(Qs + col(c) * KP);
            f32x4 t = f32x4{};
#pragma unroll
            for (int g = 0; g < G4; ++g) t += y[g] * qr[g];
            out[c] = x[c] + Cbs[col(c)] + ((t[0] + t[1]) + (t[2] + t[3]));
        }
    }
#pragma unroll
    for (int q = 0; q < CPT; q += 4) Store4<T>::st(orow + col(q), out + q);
}

// ------------------------------------------------------------------ merge
// The probe pass's key ranges s give normalised rows O_s with log-sum-exp l_s;
// the row over all keys is sum_s exp(l_s - l) O_s with l = log sum_s exp(l_s).
// One row per wave, D / 64 features per lane.
template <int D>
__global__ __launch_bounds__(kPrThreads) void pr_merge_kernel(PrArgs a, int rows) {
    constexpr int RPB = kPrThreads / kWave;               // rows per workgroup (a wave each)
    constexpr int FPL = D / kWave;                        // features per lane
    const int row = blockIdx.x * RPB + threadIdx.x / kWave;
    if (row >= rows) return;
    const int lane = lane_id();
    const int S = a.kv_splits;
    float lmax = -INFINITY;
    for (int sp = 0; sp < S; ++sp) lmax = fmaxf(lmax, a.Lsplit[(size_t)sp * rows + row]);
    float wsum = 0.f, acc[FPL];
#pragma unroll
    for (int f = 0; f < FPL; ++f) acc[f] = 0.f;
    for (int sp = 0; sp < S; ++sp) {
        const float l = a.Lsplit[(size_t)sp * rows + row];
        const float w = l == -INFINITY ? 0.f : expf(l - lmax);
        wsum += w;
        const float *src = a.Osplit + ((size_t)sp * rows + row) * D;
#pragma unroll
        for (int f = 0; f < FPL; ++f) acc[f] = fmaf(w, src[lane + f * kWave], acc[f]);
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    float *dst = const_cast<float *>(a.Od32) + (size_t)row * D;
#pragma unroll
    for (int f = 0; f < FPL; ++f) dst[lane + f * kWave] = acc[f] * inv;
}

// ------------------------------------------------------------------ launch
template <int D>
static hipError_t launch_pr_d(int dtype, const void *q, void *qp, void *o, const PrArgs &a, int BH, int step,
                              hipStream_t st) {
    if (step == 0) {
        dim3 grid((a.M + 63) / 64, BH);
        if (dtype == SA_BF16)
            hipLaunchKernelGGL(probe_gather_kernel<bf16>, grid, dim3(kPrThreads), 0, st, (const bf16 *)q, (bf16 *)qp, a, D);
        else
            hipLaunchKernelGGL(probe_gather_kernel<float>, grid, dim3(kPrThreads), 0, st, (const float *)q, (float *)qp, a, D);
    } else if (step == 1) {
        hipLaunchKernelGGL(pr_gram_kernel<D>, dim3(a.n_chunks, BH), dim3(kPrThreads), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(pr_fit_kernel<D>, dim3(BH), dim3(kFitThreads), 0, st, a);
    } else if (step == 3) {
        const int rows = BH * a.M;
        constexpr int RPB = kPrThreads / kWave;
        hipLaunchKernelGGL(pr_merge_kernel<D>, dim3((rows + RPB - 1) / RPB), dim3(kPrThreads), 0, st, a, rows);
    } else {
        dim3 grid((a.N + kPrThreads / 4 - 1) / (kPrThreads / 4), BH);
        auto go = [&](auto g4) {
            constexpr int G4 = decltype(g4)::value;
            if (dtype == SA_BF16)
                hipLaunchKernelGGL((pr_apply_kernel<bf16, D, G4>), grid, dim3(kPrThreads), 0, st, (bf16 *)o, a);
            else
                hipLaunchKernelGGL((pr_apply_kernel<float, D, G4>), grid, dim3(kPrThreads), 0, st, (float *)o, a);
        };
        switch ((a.rank + 3) / 4) {       // the rank is 1 .. 16
            case 1: go(std::integral_constant<int, 1>{}); break;
            case 2: go(std::integral_constant<int, 2>{}); break;
            case 3: go(std::integral_constant<int, 3>{}); break;
            default: go(std::integral_constant<int, 4>{}); break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_sparsepr_step(int step, int dtype, int D, const void *q, void *qp, void *o, const PrArgs &a,
                                int BH, hipStream_t st) {
    return D == 128 ? launch_pr_d<128>(dtype, q, qp, o, a, BH, step, st)
                    : launch_pr_d<64>(dtype, q, qp, o, a, BH, step, st);
}

}  // namespace sa
