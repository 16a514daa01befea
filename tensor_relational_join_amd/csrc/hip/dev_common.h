// dev_common.h -- device helpers shared by the libja kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../ja_tables.h"
#include "ja.h"

namespace ja {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// bfloat16 bits -> float (exact widening).
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16 bits, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two floats -> two bfloat16 packed in one dword (lo = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) { return f32_to_bf16(a) | (f32_to_bf16(b) << 16); }

// Workgroup index -> work-item index such that each XCD (workgroups are
// dealt to the 8 XCDs round-robin) receives a contiguous range of the work
// list, keeping neighbouring tiles in one L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    const int x = bid & 7, k = bid >> 3;
    const int q = n >> 3, r = n & 7;
    return x * q + (x < r ? x : r) + k;
}

}  // namespace ja
