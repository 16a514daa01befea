// calib.hip -- a measurement aid: the matrix-core throughput this GPU
// sustains on a loop of nothing but bf16 MFMAs (no memory traffic, no LDS, no
// barriers), the ceiling the contraction and attention kernels are compared
// against beside the published peak.
#include <hip/hip_runtime.h>
#include <stdint.h>

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

}  // namespace ja
