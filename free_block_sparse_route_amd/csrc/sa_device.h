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

// Wave-wide reductions on the VALU, every lane receiving the result: DPP
// swaps lanes within quads (xor 1, xor 2), mirrors within 8 and 16 lanes, and
// v_permlane16/32_swap exchange rows and halves.  Each step combines two
// values that every lane of the pair sees in the same order, so all lanes end
// with bit-identical results.  Call from wave-uniform control flow only.
__device__ __forceinline__ float dpp_f(float x, int ctrl) {
    switch (ctrl) {   // the control must be a constant of the builtin
        case 0xB1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
        case 0x4E: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
        case 0x141: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
        default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
    }
}

template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
    v = op(v, dpp_f(v, 0xB1));        // quad_perm [1,0,3,2]
    v = op(v, dpp_f(v, 0x4E));        // quad_perm [2,3,0,1]
    v = op(v, dpp_f(v, 0x141));       // row_half_mirror: the other quad of 8
    v = op(v, dpp_f(v, 0x140));       // row_mirror: the other 8 of 16
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

__device__ __forceinline__ float wave_max(float v) {
    return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}

__device__ __forceinline__ float wave_sum(float v) {
    return wave_reduce(v, [](float x, float y) { return x + y; });
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Workgroup i of a launch runs on GPU die (XCD) i % 8: the dispatcher deals
// workgroups to the 8 dies in turn.  die_task maps launch slot i of W to a
// task so that, in each group of 8 * run consecutive slots, die x takes the
// run consecutive tasks x * run .. x * run + run - 1 of the group; the last,
// partial group keeps the plain order.  Tasks that share data (the work of
// one head) then meet in one die's L2.  A bijection on 0..W-1.
__device__ __forceinline__ int die_task(int i, int W, int run) {
    const int span = 8 * run;
    const int base = i - i % span;
    if (base + span > W) return i;
    const int r = i - base;
    return base + (r & 7) * run + (r >> 3);
}

// Constant address space: loads through it at a wave-uniform address go
// through the scalar cache.  Only for memory that nothing writes while the
// kernel runs (buffers a previous kernel wrote).
template <typename X> using kconst = __attribute__((address_space(4))) X;

}  // namespace sa
