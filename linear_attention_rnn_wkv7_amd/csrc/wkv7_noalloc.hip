// wkv7_backward_noalloc: wkv7_backward without a caller workspace, for
// callers that cannot allocate device memory.  Its workspace is a fixed
// file-scope device array, one per GPU, held until the process ends.
//
// The workspace holds only data a call writes before it reads it (the
// chunk form's per-head flags, the step scan's sub-checkpoints, a split
// sequence's per-segment flags and state gradients, and the recomputed
// checkpoint record when none is handed over), so nothing is cleared
// between calls.  Calls that overlap on one GPU share the array and race.

#include <atomic>

#include "wkv7.h"
#include "wkv7_internal.h"

namespace {

constexpr size_t kScratchBytes = WKV7_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this GPU's copy of `scratch`, looked up once per device
// (with that device current) and kept; in host code the array's own name is
// not a device address.
int scratch_ptr(size_t need, void **ptr)
{
    static std::atomic<void *> cache[wkv7::kMaxDevices];
    if (need > kScratchBytes) return WKV7_ERR_WORKSPACE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= wkv7::kMaxDevices) return WKV7_ERR_HIP;
    void *p = cache[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return WKV7_ERR_HIP;
        cache[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return WKV7_OK;
}

}  // namespace

extern "C" {

int wkv7_backward_noalloc(const wkv7_shape *shape, const void *r, const void *w, const void *k,
                          const void *v, const void *a, const void *b, const float *s0,
                          const void *dy, const float *dsT, const float *ckpt,
                          float *dr, float *dw, float *dk, float *dv, float *da, float *db,
                          float *ds0, hipStream_t stream)
{
    return wkv7::backward_entry(shape, r, w, k, v, a, b, s0, dy, dsT, ckpt, dr, dw, dk, dv, da, db,
                                ds0, nullptr, 0, scratch_ptr, stream);
}

}  // extern "C"
