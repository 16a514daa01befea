// noalloc.hip -- the one-shot join-agg for callers that cannot allocate device
// memory (serving loops, harnesses that forbid hipMalloc).  The plan tables
// are still copied in with a synchronous host-to-device copy, so a call
// cannot be recorded into a stream capture.
//
// ja_einsum takes a caller-owned workspace for the plan's device tables and
// the run's scratch.  ja_einsum_noalloc puts both in `scratch`, a static
// device array of JA_NOALLOC_SCRATCH_BYTES that every GPU the library runs
// on holds for the life of the process; the caller passes only inputs and
// outputs.  Plans that do not fit are refused.  Every call on a GPU shares
// that GPU's array and leaves its contents behind (the kernels need nothing
// in it zeroed: the tables are copied in by each call and every scratch word
// a kernel reads is written earlier in the same call), so two calls that
// overlap on one GPU -- on different streams, or from different host threads
// -- race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../host/ja_host.h"

namespace {

static __device__ __align__(256) uint8_t scratch[JA_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_dev[MAX_DEVICES];  // the array's device address on each GPU, looked up once

// The device address of `scratch` on the current GPU.  The array's name is
// only a host-side stand-in; the address each GPU placed its copy at comes
// from hipGetSymbolAddress, called once per device with that device current.
ja_status scratch_ptr(void** out) {
    int dev = -1;
    JA_TRY_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= MAX_DEVICES) return ja::fail(JA_ERR_UNSUPPORTED, "device index beyond 63");
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return ja::hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return ja::fail(JA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        scratch_dev[dev] = p;
    }
    *out = scratch_dev[dev];
    return JA_OK;
}

}  // namespace

extern "C" ja_status ja_einsum_noalloc(const ja_spec* s, const ja_decomp* d, const ja_relation_desc* const* in,
                                       const void* const* in_ptrs, int32_t n_in, const ja_relation_desc* out,
                                       void* out_ptr, void* stream) {
    ja_plan* p = nullptr;
    ja_status st = ja_plan_create(s, d, in, n_in, out, &p);
    if (st) return st;
    size_t tb = 0, wb = 0;
    ja_plan_device_bytes(p, &tb, &wb);
    const size_t tb_al = (tb + 255) & ~(size_t)255;
    if (tb_al + wb > JA_NOALLOC_SCRATCH_BYTES) {
        ja_plan_destroy(p);
        return ja::fail(JA_ERR_WORKSPACE,
                        "the plan needs " + std::to_string(tb_al + wb) + " bytes of device scratch; the static scratch holds " +
                            std::to_string((size_t)JA_NOALLOC_SCRATCH_BYTES) + " (ja_einsum takes a workspace of any size)");
    }
    void* ws = nullptr;
    st = scratch_ptr(&ws);
    if (!st) st = ja_plan_upload(p, ws, tb, stream);
    if (!st) st = ja_plan_run(p, in_ptrs, out_ptr, wb ? (uint8_t*)ws + tb_al : nullptr, stream);
    ja_plan_destroy(p);
    return st;
}
