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

// float -> bfloat16 bits, round to nearest, ties to even; NaN stays NaN
// (the hardware conversion, v_cvt_pk_bf16_f32, two values per instruction).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two floats -> two bfloat16 packed in one dword (lo = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// IEEE half bits <-> float: exact widening; narrowing rounds to nearest even
// (the default rounding mode of v_cvt_f16_f32 and v_cvt_pk_f16_f32).
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    const f16x2_t v = {(_Float16)a, (_Float16)b};  // v_cvt_pk_f16_f32
    return __builtin_bit_cast(uint32_t, v);
}

// The 16-bit element formats the kernels read and write: F16 selects IEEE
// half, otherwise bfloat16.
template <bool F16>
__device__ __forceinline__ float h16_to_f32(uint32_t h) {
    if constexpr (F16)
        return f16_to_f32(h);
    else
        return bf16_to_f32(h);
}
template <bool F16>
__device__ __forceinline__ uint32_t f32_to_h16(float f) {
    if constexpr (F16)
        return f32_to_f16(f);
    else
        return f32_to_bf16(f);
}
template <bool F16>
__device__ __forceinline__ uint32_t pack_h16x2(float a, float b) {
    if constexpr (F16)
        return pack_f16x2(a, b);
    else
        return pack_bf16x2(a, b);
}
// low / high 16-bit element of a dword, widened to float
template <bool F16>
__device__ __forceinline__ float h16lo_to_f32(uint32_t w) {
    return F16 ? f16_to_f32(w & 0xffffu) : bf16lo_to_f32(w);
}
template <bool F16>
__device__ __forceinline__ float h16hi_to_f32(uint32_t w) {
    return F16 ? f16_to_f32(w >> 16) : bf16hi_to_f32(w);
}

// 16x16x32 MFMA on 16-byte fragments of 8 elements in either format.
template <bool F16>
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Streaming 16-byte accesses with the non-temporal hint, for data a kernel
// touches once.  On MI355X a plain cold copy of 2 x 67 MB rises from about
// 4.0 to 5.4 TB/s with both hinted and a 1:1 join over 2 x 180 MB in, 180 MB
// out from 5.9 to 6.2 TB/s with its loads hinted.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(void* p, uint4 v) {
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ float4 ld_nt_f4(const float* p) {
    const uint4 v = ld_nt(p);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

// silu(g) u = g u / (1 + e^-g), with the hardware reciprocal (v_rcp_f32,
// within 1 ulp in fp32) instead of an IEEE division: the result is rounded
// to a 16-bit format next, whose unit roundoff is 2^16 times larger.
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Workgroup index -> work-item index such that each XCD (workgroups are
// dealt to the 8 XCDs round-robin) receives a contiguous range of the work
// list, keeping neighbouring tiles in one L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    const int x = bid & 7, k = bid >> 3;
    const int q = n >> 3, r = n & 7;
    return x * q + (x < r ? x : r) + k;
}

}  // namespace ja
