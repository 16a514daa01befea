// calib.cpp -- host side of the measurement aid in hip/calib.hip.
#include "ja_host.h"

namespace ja {
hipError_t launch_mfma_loop(int32_t workgroups, int32_t iters, float* sink, hipStream_t stream);
hipError_t launch_copy(const void* src, void* dst, int64_t n16, hipStream_t stream);
}

using namespace ja;

extern "C" {

ja_status ja_calibrate_mfma(int32_t workgroups, int32_t iters, float* sink, double* flops, void* stream) {
    if (!sink) return fail(JA_ERR_ARG, "sink is NULL");
    if (workgroups < 1 || iters < 1) return fail(JA_ERR_ARG, "workgroups and iterations must be positive");
    if ((uintptr_t)sink & 3) return fail(JA_ERR_ARG, "sink must be 4-byte aligned");
    if (flops) *flops = (double)workgroups * 4.0 * (double)iters * 4.0 * 32768.0;
    JA_TRY_HIP(launch_mfma_loop(workgroups, iters, sink, (hipStream_t)stream));
    return JA_OK;
}

ja_status ja_calibrate_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst) return fail(JA_ERR_ARG, "NULL buffer");
    if (((uintptr_t)src | (uintptr_t)dst | bytes) & 15) return fail(JA_ERR_ARG, "buffers and size must be 16-byte multiples");
    JA_TRY_HIP(launch_copy(src, dst, (int64_t)(bytes / 16), (hipStream_t)stream));
    return JA_OK;
}

}  // extern "C"
