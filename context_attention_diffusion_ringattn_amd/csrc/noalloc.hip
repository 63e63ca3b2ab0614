// noalloc.hip -- ringattn_forward_noalloc: ringattn_forward for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops
// that forbid allocation).  The split workspace of its launch plan lives in
// `scratch`, a fixed device array of kScratchBytes that each GPU the library
// runs on holds until the process ends; plans needing more are not chosen.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "ringattn.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // == RINGATTN_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == RINGATTN_NOALLOC_SCRATCH_BYTES, "scratch size mismatch");

// The split workspace of ringattn_forward_noalloc.  In host code `scratch`
// names a host-side stand-in, not device memory: host code only ever uses the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` per device, set on first use

// Device address of `scratch` on the current device (looked up once per
// device, with that device current); nullptr after reporting an error.
void *scratch_on_current_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        ringattn::report_error(RINGATTN_EHIP, e != hipSuccess ? hipGetErrorString(e) : "device index out of range");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            ringattn::report_error(RINGATTN_EHIP, e != hipSuccess ? hipGetErrorString(e) : "no scratch address");
            return nullptr;
        }
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" int ringattn_forward_noalloc(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                        const int64_t *chunk_offsets, int32_t n_chunks, int64_t kv_chunk_stride,
                                        float *out, float *lse, float scale, const ringattn_shape *shape,
                                        const ringattn_plan *plan, void *stream) {
    size_t need = 0;
    int st = ringattn::forward_check(q, k, v, chunk_offsets, n_chunks, kv_chunk_stride, out, lse, scale, shape, plan,
                                     kScratchBytes, &need);
    if (st != RINGATTN_OK) return st;
    void *ws = nullptr;
    if (need > 0 && !(ws = scratch_on_current_device())) return RINGATTN_EHIP;
    return ringattn::forward_impl(q, k, v, chunk_offsets, n_chunks, kv_chunk_stride, out, lse, scale, shape, plan, ws,
                                  need > 0 ? kScratchBytes : 0, kScratchBytes, (hipStream_t)stream);
}
