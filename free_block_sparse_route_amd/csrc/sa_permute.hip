// Token reordering: the Hilbert order of a video token grid (host) and the
// row permutation that applies it to [B, H, N, d] tensors on the GPU and
// undoes it (DFSAttn abstract: tokens are reordered along a 3D Hilbert curve
// so that blocks of consecutive tokens are compact in space and time).
//
// Curve: J. Skilling, "Programming the Hilbert curve", AIP Conf. Proc. 707
// (2004).  A point's index is the bit interleave (most significant bit plane
// first, axes t, y, x) of its "transposed" form; the order of the grid's
// tokens is the order of their indices on the enclosing 2^b cube.  The host
// walks the curve index by index, maps each index back to its point (Gray
// decode, then the undo of the excess work) and emits the points that lie in
// the grid, so the order needs no sort and no memory beyond the output.
//
// Permutation: one 16-byte unit per thread, rows of d elements; gather writes
// consecutive output rows (coalesced writes, row-wise reads), scatter reads
// consecutive input rows.  HBM-bound: every row is read once and written once.
#include <stdint.h>

#include "sa_internal.h"

namespace sa {

// Point (t, y, x) of Hilbert index h on the 2^b cube.
void hilbert_point(uint64_t h, int b, uint32_t X[3]) {
    X[0] = X[1] = X[2] = 0;
    for (int p = 0; p < b; ++p)
        for (int i = 0; i < 3; ++i) X[i] |= (uint32_t)((h >> (3 * p + 2 - i)) & 1u) << p;
    // Gray decode
    uint32_t t = X[2] >> 1;
    for (int i = 2; i > 0; --i) X[i] ^= X[i - 1];
    X[0] ^= t;
    // undo the excess work, low planes first
    const uint32_t top = 1u << b;
    for (uint32_t Q = 2; Q != top; Q <<= 1) {
        const uint32_t P = Q - 1;
        for (int i = 2; i >= 0; --i) {
            if (X[i] & Q) {
                X[0] ^= P;
            } else {
                t = (X[0] ^ X[i]) & P;
                X[0] ^= t;
                X[i] ^= t;
            }
        }
    }
}

int64_t hilbert_fill(int T, int Hh, int W, int b, int32_t *perm) {
    const uint64_t total = 1ull << (3 * b);
    int64_t k = 0;
    uint32_t X[3];
    for (uint64_t h = 0; h < total; ++h) {
        hilbert_point(h, b, X);
        if (X[0] < (uint32_t)T && X[1] < (uint32_t)Hh && X[2] < (uint32_t)W)
            perm[k++] = (int32_t)(((int64_t)X[0] * Hh + X[1]) * W + X[2]);
    }
    return k;
}

constexpr int kPermThreads = 256;
constexpr int kPermRows = 64;            // rows per workgroup

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const uint4 *__restrict__ in, uint4 *__restrict__ out,
                                                               const int32_t *__restrict__ perm, PermuteArgs a) {
    constexpr int kMaxIt = 8;                 // rows per thread: 64 rows / (256 threads / units), units >= 4
    const int bh = blockIdx.y;
    const int units = a.units;
    const int u = threadIdx.x % units;
    const int step = kPermThreads / units;
    const int r0 = blockIdx.x * kPermRows + threadIdx.x / units;
    const int r_end = min(a.N, (int)(blockIdx.x + 1) * kPermRows);
    const size_t head = (size_t)bh * a.N * units;
    // every row's permutation entry, then every row's load, then the stores:
    // the loads of a thread are all in flight together.  Rows are read and
    // written once, with the non-temporal hint (on one Hunyuan tensor: 0.25
    // instead of 0.27 ms, 5.9 TB/s, against one row at a time without it).
    int src[kMaxIt], dst[kMaxIt];
#pragma unroll
    for (int k = 0; k < kMaxIt; ++k) {
        const int r = r0 + k * step;
        int other = r, ok = r < r_end;
        const int i = r - a.n0;
        if (ok && i >= 0 && i < a.n_perm) {
            const int p = perm[i];
            ok = p >= 0 && p < a.n_perm;                     // not a permutation entry: row left as is
            other = a.n0 + p;
        }
        src[k] = ok ? (a.inverse ? r : other) : -1;
        dst[k] = ok ? (a.inverse ? other : r) : -1;
    }
    typedef unsigned int w4 __attribute__((ext_vector_type(4)));
    const w4 *iw = reinterpret_cast<const w4 *>(in);
    w4 *ow = reinterpret_cast<w4 *>(out);
    w4 v[kMaxIt];
#pragma unroll
    for (int k = 0; k < kMaxIt; ++k)
        v[k] = __builtin_nontemporal_load(iw + head + (size_t)(src[k] < 0 ? 0 : src[k]) * units + u);
#pragma unroll
    for (int k = 0; k < kMaxIt; ++k)
        if (dst[k] >= 0) __builtin_nontemporal_store(v[k], ow + head + (size_t)dst[k] * units + u);
}

hipError_t launch_permute(const void *in, void *out, const int32_t *perm, const PermuteArgs &a, int BH,
                          hipStream_t st) {
    dim3 grid((a.N + kPermRows - 1) / kPermRows, BH);
    hipLaunchKernelGGL(permute_kernel, grid, dim3(kPermThreads), 0, st, (const uint4 *)in, (uint4 *)out, perm, a);
    return hipGetLastError();
}

}  // namespace sa
