// Probe-fitted residual correction (SparsePR summary, section B): a second way
// to correct the sparse output, beside the proxy-reuse residual of the forward.
//
//   1. the sparse output O_s over the kept tokens only, in fp32 (forward kernel,
//      no block residual);
//   2. probe rows, P per query block evenly spread (row I*bq + floor((j+1/2) m_I / P)),
//      gathered and attended densely (forward kernel, dense path), in fp32;
//   3. per (b, h), one workgroup fits R = O_d - O_s at the probes as an affine
//      map of x = O_s: centred Gram matrices, a ridge lam = ridge * trace / d,
//      a Cholesky solve for B, the intercept b = rm - xm B; the k leading
//      eigenvectors of R^T R (the right singular vectors of R) by subspace
//      iteration; and the projected map C_B = B Pk, C_b = b Pk, Pk = V_k V_k^T;
//   4. every row not probed takes O_s + C_b + O_s C_B, probed rows take O_d.
//
// Steps 3 and 4 are small: d x d matrices per head and one d x d product per row.
#include <math.h>
#include <stdint.h>

#include "sa_device.h"
#include "sa_internal.h"

namespace sa {

constexpr int kPrThreads = 256;
constexpr int kPrIters = 60;             // subspace iterations

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

// sum over the probes of A[j][r] * B[j][c] for the D x D entries a thread owns
// (row r, columns c0 .. c0 + D/2 - 1); A, B in {0: x - xm, 1: r - rm, 2: r}.
// Probe rows are staged in LDS 16 at a time.
template <int D>
__device__ void gram(const PrArgs &a, int bh, const float *xm, const float *rm, int ka, int kb, float *out,
                     float *SA, float *SB) {
    constexpr int H = D / 2, JS = 16;
    const int r = threadIdx.x / 2, c0 = (threadIdx.x & 1) * H;
    const bool active = threadIdx.x < 2 * D;
    float acc[H];
#pragma unroll
    for (int c = 0; c < H; ++c) acc[c] = 0.f;
    const float *Os = a.O32 + (size_t)bh * a.N * D;
    const float *Od = a.Od32 + (size_t)bh * a.M * D;
    auto val = [&](int k, int j, int f) -> float {
        const float x = Os[(size_t)probe_row(j, a) * D + f];
        if (k == 0) return x - xm[f];
        const float rr = Od[(size_t)j * D + f] - x;
        return k == 1 ? rr - rm[f] : rr;
    };
    for (int j0 = 0; j0 < a.M; j0 += JS) {
        __syncthreads();
        for (int e = threadIdx.x; e < JS * D; e += kPrThreads) {
            const int j = j0 + e / D, f = e % D;
            SA[e] = j < a.M ? val(ka, j, f) : 0.f;
            SB[e] = j < a.M ? val(kb, j, f) : 0.f;
        }
        __syncthreads();
        if (active)
            for (int jj = 0; jj < JS; ++jj) {
                const float ar = SA[jj * D + r];
#pragma unroll
                for (int c = 0; c < H; ++c) acc[c] = fmaf(ar, SB[jj * D + c0 + c], acc[c]);
            }
    }
    if (active)
#pragma unroll
        for (int c = 0; c < H; ++c) out[r * D + c0 + c] = acc[c];
}

template <int D>
__global__ __launch_bounds__(kPrThreads) void pr_fit_kernel(PrArgs a) {
    const int bh = blockIdx.x;
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    __shared__ float xm[D], rm[D];
    __shared__ float L[D * (D + 1) / 2];
    __shared__ float Qs[D * kPrMaxRank];
    __shared__ float red[kPrThreads / kWave];
    __shared__ float SA[16 * D], SB[16 * D];
    float *Gm = a.scratch + (size_t)bh * 3 * D * D;      // centred X^T X, then X^T R, then R^T R
    float *Hm = Gm + D * D;
    float *Sm = Hm + D * D;
    float *Bm = a.CB + (size_t)bh * D * D;
    float *bv = a.Cb + (size_t)bh * D;
    const float *Os = a.O32 + (size_t)bh * a.N * D;
    const float *Od = a.Od32 + (size_t)bh * a.M * D;
    const float invM = 1.f / (float)a.M;

    // means of x and r over the probes
    if (threadIdx.x < D) {
        float sx = 0.f, sr = 0.f;
        for (int j = 0; j < a.M; ++j) {
            const float x = Os[(size_t)probe_row(j, a) * D + threadIdx.x];
            sx += x;
            sr += Od[(size_t)j * D + threadIdx.x] - x;
        }
        xm[threadIdx.x] = sx * invM;
        rm[threadIdx.x] = sr * invM;
    }
    __syncthreads();
    gram<D>(a, bh, xm, rm, 0, 0, Gm, SA, SB);
    gram<D>(a, bh, xm, rm, 0, 1, Hm, SA, SB);
    gram<D>(a, bh, xm, rm, 2, 2, Sm, SA, SB);
    __threadfence_block();
    __syncthreads();

    // ridge relative to the scale of the centred Gram matrix
    float tr = 0.f;
    for (int i = threadIdx.x; i < D; i += kPrThreads) tr += Gm[i * D + i];
    tr = wave_sum(tr);
    if (lane == 0) red[wave] = tr;
    __syncthreads();
    float trace = 0.f;
#pragma unroll
    for (int w = 0; w < kPrThreads / kWave; ++w) trace += red[w];
    const float lam = a.ridge * trace / (float)D;
    for (int e = threadIdx.x; e < D * (D + 1) / 2; e += kPrThreads) {
        int i = (int)((sqrtf(8.f * e + 1.f) - 1.f) * 0.5f);
        while (tri(i + 1, 0) <= e) ++i;
        while (tri(i, 0) > e) --i;
        const int j = e - tri(i, 0);
        L[e] = Gm[i * D + j] + (i == j ? lam : 0.f);
    }
    __syncthreads();

    // Cholesky G + lam I = L L^T, by one wave (LDS operations of a wave are in order)
    if (wave == 0) {
        for (int j = 0; j < D; ++j) {
            const float djj = sqrtf(fmaxf(L[tri(j, j)], 1e-30f));
            for (int i = j + 1 + lane; i < D; i += kWave) L[tri(i, j)] /= djj;
            if (lane == 0) L[tri(j, j)] = djj;
            __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): this wave's LDS writes are done
            __builtin_amdgcn_wave_barrier();
            // trailing update of the lower triangle below row j
            const int n = D - j - 1;
            for (int e = lane; e < n * (n + 1) / 2; e += kWave) {
                int ii = (int)((sqrtf(8.f * e + 1.f) - 1.f) * 0.5f);
                while ((ii + 1) * (ii + 2) / 2 <= e) ++ii;
                while (ii * (ii + 1) / 2 > e) --ii;
                const int kk = e - ii * (ii + 1) / 2;
                const int i = j + 1 + ii, k = j + 1 + kk;
                L[tri(i, k)] -= L[tri(i, j)] * L[tri(k, j)];
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
        }
    }
    __syncthreads();

    // B = (L L^T)^-1 H, a column per thread: forward then backward substitution
    if (threadIdx.x < D) {
        const int c = threadIdx.x;
        for (int i = 0; i < D; ++i) {
            float y = Hm[i * D + c];
            for (int k = 0; k < i; ++k) y -= L[tri(i, k)] * Bm[k * D + c];
            Bm[i * D + c] = y / L[tri(i, i)];
        }
        for (int i = D - 1; i >= 0; --i) {
            float y = Bm[i * D + c];
            for (int k = i + 1; k < D; ++k) y -= L[tri(k, i)] * Bm[k * D + c];
            Bm[i * D + c] = y / L[tri(i, i)];
        }
    }
    __threadfence_block();
    __syncthreads();
    // intercept b = rm - xm B
    if (threadIdx.x < D) {
        float s = rm[threadIdx.x];
        for (int i = 0; i < D; ++i) s -= xm[i] * Bm[i * D + threadIdx.x];
        bv[threadIdx.x] = s;
    }

    // leading eigenvectors of S = R^T R by subspace iteration from a fixed start
    const int K = a.rank;
    for (int e = threadIdx.x; e < D * K; e += kPrThreads) {
        uint32_t hsh = (uint32_t)e * 2654435761u + 0x9e3779b9u;
        hsh ^= hsh >> 15;
        hsh *= 2246822519u;
        hsh ^= hsh >> 13;
        Qs[e] = (float)(hsh & 0xffff) / 32768.f - 1.f;      // Qs[i * K + c]
    }
    __syncthreads();
    for (int it = 0; it <= kPrIters; ++it) {
        if (it > 0) {
            // Z = S Q into registers, then back to Qs
            float z[(D * kPrMaxRank + kPrThreads - 1) / kPrThreads];
            int n_own = 0;
            for (int e = threadIdx.x; e < D * K; e += kPrThreads) {
                const int i = e / K, c = e - (e / K) * K;
                float s = 0.f;
                for (int l = 0; l < D; ++l) s += Sm[i * D + l] * Qs[l * K + c];
                z[n_own++] = s;
            }
            __syncthreads();
            n_own = 0;
            for (int e = threadIdx.x; e < D * K; e += kPrThreads) Qs[e] = z[n_own++];
            __syncthreads();
        }
        // modified Gram-Schmidt on the columns, by one wave
        if (wave == 0) {
            for (int c = 0; c < K; ++c) {
                for (int pcol = 0; pcol < c; ++pcol) {
                    float dp = 0.f;
                    for (int i = lane; i < D; i += kWave) dp += Qs[i * K + pcol] * Qs[i * K + c];
                    dp = wave_sum(dp);
                    for (int i = lane; i < D; i += kWave) Qs[i * K + c] -= dp * Qs[i * K + pcol];
                }
                float nn = 0.f;
                for (int i = lane; i < D; i += kWave) nn += Qs[i * K + c] * Qs[i * K + c];
                nn = wave_sum(nn);
                const float inv = nn > 0.f ? 1.f / sqrtf(nn) : 0.f;
                for (int i = lane; i < D; i += kWave) Qs[i * K + c] *= inv;
                __builtin_amdgcn_s_waitcnt(0xc07f);
                __builtin_amdgcn_wave_barrier();
            }
        }
        __syncthreads();
    }

    // W = B Q (D x K) in the rows of L (no longer needed), then C_B = W Q^T, C_b = (b Q) Q^T
    float *W = L;
    for (int e = threadIdx.x; e < D * K; e += kPrThreads) {
        const int i = e / K, c = e - (e / K) * K;
        float s = 0.f;
        for (int l = 0; l < D; ++l) s += Bm[i * D + l] * Qs[l * K + c];
        W[e] = s;
    }
    __shared__ float wb[kPrMaxRank];
    if (threadIdx.x < K) {
        float s = 0.f;
        for (int l = 0; l < D; ++l) s += bv[l] * Qs[l * K + threadIdx.x];
        wb[threadIdx.x] = s;
    }
    __threadfence_block();
    __syncthreads();
    for (int e = threadIdx.x; e < D * D; e += kPrThreads) {
        const int i = e / D, j = e - (e / D) * D;
        float s = 0.f;
        for (int c = 0; c < K; ++c) s += W[i * K + c] * Qs[j * K + c];
        Bm[e] = s;
    }
    if (threadIdx.x < D) {
        float s = 0.f;
        for (int c = 0; c < K; ++c) s += wb[c] * Qs[threadIdx.x * K + c];
        bv[threadIdx.x] = s;
    }
}

// ------------------------------------------------------------------ apply
// 64 rows per workgroup; thread t: row t / 4, output columns (t % 4) * D/4 ..
template <typename T, int D>
__global__ __launch_bounds__(kPrThreads) void pr_apply_kernel(T *__restrict__ o, PrArgs a) {
    constexpr int CW = D / 4;                 // columns per thread
    constexpr int KC = 32;                    // rows of C_B per staging step
    const int bh = blockIdx.y;
    const int r0 = blockIdx.x * 64;
    __shared__ float X[64 * D];
    __shared__ float Cs[KC * D];
    const float *Os = a.O32 + (size_t)bh * a.N * D;
    const float *CB = a.CB + (size_t)bh * D * D;
    const float *Cb = a.Cb + (size_t)bh * D;
    for (int e = threadIdx.x; e < 64 * D; e += kPrThreads) {
        const int r = r0 + e / D;
        X[e] = r < a.N ? Os[(size_t)r * D + (e % D)] : 0.f;
    }
    const int rl = threadIdx.x / 4, c0 = (threadIdx.x % 4) * CW;
    float acc[CW];
#pragma unroll
    for (int c = 0; c < CW; ++c) acc[c] = Cb[c0 + c];
    for (int k0 = 0; k0 < D; k0 += KC) {
        __syncthreads();
        for (int e = threadIdx.x; e < KC * D; e += kPrThreads) Cs[e] = CB[(size_t)k0 * D + e];
        __syncthreads();
        for (int kk = 0; kk < KC; ++kk) {
            const float x = X[rl * D + k0 + kk];
#pragma unroll
            for (int c = 0; c < CW; ++c) acc[c] = fmaf(x, Cs[kk * D + c0 + c], acc[c]);
        }
    }
    const int r = r0 + rl;
    if (r >= a.N) return;
    // probed rows take their dense values
    const int I = r / a.block_q, off = r - I * a.block_q;
    const int m = min(a.block_q, a.N - I * a.block_q);
    int probe = -1;
    for (int jj = 0; jj < a.per_block; ++jj)
        if ((2 * jj + 1) * m / (2 * a.per_block) == off) probe = I * a.per_block + jj;
    T *orow = o + ((size_t)bh * a.N + r) * D + c0;
    if (probe >= 0) {
        const float *od = a.Od32 + ((size_t)bh * a.M + probe) * D + c0;
#pragma unroll
        for (int c = 0; c < CW; ++c) orow[c] = (T)od[c];
    } else {
#pragma unroll
        for (int c = 0; c < CW; ++c) orow[c] = (T)(X[rl * D + c0 + c] + acc[c]);
    }
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
        hipLaunchKernelGGL(pr_fit_kernel<D>, dim3(BH), dim3(kPrThreads), 0, st, a);
    } else {
        dim3 grid((a.N + 63) / 64, BH);
        if (dtype == SA_BF16)
            hipLaunchKernelGGL((pr_apply_kernel<bf16, D>), grid, dim3(kPrThreads), 0, st, (bf16 *)o, a);
        else
            hipLaunchKernelGGL((pr_apply_kernel<float, D>), grid, dim3(kPrThreads), 0, st, (float *)o, a);
    }
    return hipGetLastError();
}

hipError_t launch_sparsepr_step(int step, int dtype, int D, const void *q, void *qp, void *o, const PrArgs &a,
                                int BH, hipStream_t st) {
    return D == 128 ? launch_pr_d<128>(dtype, q, qp, o, a, BH, step, st)
                    : launch_pr_d<64>(dtype, q, qp, o, a, BH, step, st);
}

}  // namespace sa
