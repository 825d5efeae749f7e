// qsa_static.hip -- qsa_select_sparse_decode_static: the fused selection + attention call for
// callers that cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc). The split workspace (a region of completion
// counters, then the split partials) comes from `scratch`, a device array the library holds
// on every GPU it runs on until the process ends, instead of from the caller.
//
// In host code `scratch` names a host-side stand-in of the array, not a device address. The
// device address of each GPU's copy is looked up once per device with hipGetSymbolAddress,
// with that device current, and kept per device; only that address reaches a kernel.
#include <atomic>
#include <mutex>

#include "qsa_internal.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)8 << 20;   // counters + partials of one call
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// This device's copy of `scratch` (the current device), looked up on its first use.
hipError_t scratch_ptr(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" {

qsa_status qsa_select_sparse_decode_static(const qsa_shape *sh, const qsa_paged *pg, const uint16_t *q,
                                           const float *scores, int32_t *selected, uint16_t *out, float *lse,
                                           const uint16_t *gate, int32_t num_splits, void *stream)
{
    if (sh && pg && sh->topk + sh->window > 0 && !scores && sh->num_rows > 0 && sh->num_requests > 0)
        return QSA_ERR_INVALID_ARG;
    const size_t need = qsa_workspace_bytes(sh, num_splits);
    void *ws = nullptr;
    if (need > 0) {
        if (need > kScratchBytes) return QSA_ERR_WORKSPACE_TOO_SMALL;
        if (scratch_ptr(&ws) != hipSuccess) return QSA_ERR_HIP;
    }
    // the counters are cleared first: the array holds whatever the last call on this GPU left
    return qsa::decode_call(sh, pg, q, scores, selected, out, lse, gate, num_splits, ws, need > 0 ? kScratchBytes : 0,
                            stream, true);
}

}  // extern "C"
