// calib.hip -- measurement aids: the matrix-core throughput this GPU
// sustains on a loop of nothing but bf16 MFMAs (no memory traffic, no LDS, no
// barriers), and the HBM bandwidth a plain streaming copy reaches -- the
// ceilings the kernels are compared against beside the published peaks.
#include "dev_common.h"

namespace ja {

typedef __bf16 cal_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float cal_f32x16_t __attribute__((ext_vector_type(16)));

constexpr int CAL_THREADS = 256;  // 4 wavefronts
constexpr int CAL_CHAINS = 4;     // independent accumulators per wavefront

// Every wavefront runs `iters` rounds of CAL_CHAINS independent
// v_mfma_f32_32x32x16_bf16 (32,768 flops each); the accumulators' sum is
// written so that no MFMA is dead code.
__global__ __launch_bounds__(CAL_THREADS) void mfma_loop_kernel(int32_t iters, float* __restrict__ sink) {
    cal_bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(1.0f / 256.0f);
        b[i] = (__bf16)((float)((threadIdx.x + i) & 7) / 1024.0f);
    }
    cal_f32x16_t acc[CAL_CHAINS];
#pragma unroll
    for (int c = 0; c < CAL_CHAINS; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < CAL_CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CAL_CHAINS; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    sink[blockIdx.x * CAL_THREADS + threadIdx.x] = s;
}

hipError_t launch_mfma_loop(int32_t workgroups, int32_t iters, float* sink, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(CAL_THREADS), 0, stream, iters, sink);
    return hipGetLastError();
}

// A streaming copy of n16 16-byte vectors: each thread moves COPY_UNROLL
// vectors, all loaded before any is stored, loads and stores non-temporal,
// one pass with no grid-stride loop (the fastest plain copy among those
// tried on MI355X: unroll 2 to 8, grids of 4 to 32 workgroups per compute
// unit, with and without the hint).
constexpr int COPY_UNROLL = 4;

__global__ __launch_bounds__(CAL_THREADS) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                           int64_t n16) {
    const int64_t base = (int64_t)blockIdx.x * CAL_THREADS * COPY_UNROLL + threadIdx.x;
    uint4 v[COPY_UNROLL];
#pragma unroll
    for (int j = 0; j < COPY_UNROLL; ++j) {
        const int64_t i = base + (int64_t)j * CAL_THREADS;
        if (i < n16) v[j] = ld_nt(src + i);
    }
#pragma unroll
    for (int j = 0; j < COPY_UNROLL; ++j) {
        const int64_t i = base + (int64_t)j * CAL_THREADS;
        if (i < n16) st_nt(dst + i, v[j]);
    }
}

hipError_t launch_copy(const void* src, void* dst, int64_t n16, hipStream_t stream) {
    if (n16 <= 0) return hipSuccess;
    const int64_t grid = (n16 + CAL_THREADS * COPY_UNROLL - 1) / (CAL_THREADS * COPY_UNROLL);
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(CAL_THREADS), 0, stream, (const uint4*)src, (uint4*)dst,
                       n16);
    return hipGetLastError();
}

}  // namespace ja
