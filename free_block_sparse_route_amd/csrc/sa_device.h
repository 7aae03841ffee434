// Device helpers shared by the routing and attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_attn.h"

namespace sa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kTile = 64;          // key/value rows per attention tile

// Eight consecutive input elements as bf16 (fp32 inputs rounded to nearest even).
template <typename T> struct Ld8;
template <> struct Ld8<bf16> {
    static __device__ __forceinline__ bf16x8 load(const bf16 *p) {
        return *reinterpret_cast<const bf16x8 *>(p);
    }
    static __device__ __forceinline__ void load_f32(const bf16 *p, float *out) {
        u32x4 w = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct Ld8<float> {
    static __device__ __forceinline__ bf16x8 load(const float *p) {
        f32x4 a = *reinterpret_cast<const f32x4 *>(p);
        f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
        bf16x8 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r[i] = (bf16)a[i];
            r[4 + i] = (bf16)b[i];
        }
        return r;
    }
    static __device__ __forceinline__ void load_f32(const float *p, float *out) {
        f32x4 a = *reinterpret_cast<const f32x4 *>(p);
        f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[i] = a[i];
            out[4 + i] = b[i];
        }
    }
};

// Order-preserving map of fp32 to uint32 (larger float => larger key).
__device__ __forceinline__ uint32_t orderable(float x) {
    uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace sa
