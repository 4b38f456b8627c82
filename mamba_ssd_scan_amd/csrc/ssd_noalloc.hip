// ssd_noalloc.hip -- ssd_prefill for callers that cannot allocate device memory (code under
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the scratch that
// ssd_prefill takes from the caller's workspace lives here in a file-scope device array.
//
// The array is `scratch`, kScratchBytes long, one copy per GPU the library runs on, held
// until the process ends.  In host code its name is only a stand-in for the device symbol,
// so its address on a device is taken once per device with hipGetSymbolAddress (with that
// device current) and kept in `g_scratch`; every use below goes through that address.
// Calls on one GPU share its array: calls that overlap in time on one GPU (different
// streams with no ordering between them) race.  Every prefill clears the parts of its
// scratch that must start at zero itself, so the previous call's contents do no harm.
#include <hip/hip_runtime.h>

#include <atomic>

#include "ssd.h"

namespace {

constexpr size_t kScratchBytes = SSD_PREFILL_NOALLOC_MAX_BYTES;  // per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on each device (0: not taken yet).  Taking it twice on one
// device from two threads stores the same address: the race is benign.
std::atomic<void *> g_scratch[kMaxDevices];

int scratch_of_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SSD_ERR_HIP;
    if (dev >= kMaxDevices) return SSD_ERR_UNSUPPORTED;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSD_ERR_HIP;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return SSD_OK;
}

}  // namespace

extern "C" int ssd_prefill_noalloc(const void *x, const void *dt, const float *A, const void *Bm, const void *Cm,
                                   const float *D, const float *initial_state, float *final_state, float *y,
                                   ssd_dtype_t in_dtype, int batch, int seqlen, int nheads, int headdim, int dstate,
                                   int ngroups, int chunk, void *hip_stream)
{
    if (seqlen > 0) {
        const size_t need = ssd_prefill_workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups, chunk);
        if (need > kScratchBytes) return SSD_ERR_WORKSPACE;  // (0 = invalid shape: the prefill reports it)
    }
    void *ws = nullptr;
    const int st = scratch_of_current_device(&ws);
    if (st != SSD_OK) return st;
    // The three-launch path: it has no waits between workgroups (nothing to report through
    // ssd_prefill_check, which would need the scratch address) and its result equals
    // ssd_prefill's on every path bit for bit.
    return ssd_prefill_forced(x, dt, A, Bm, Cm, D, nullptr, 0, nullptr, initial_state, final_state, y, in_dtype,
                              SSD_F32, batch, seqlen, nheads, headdim, dstate, ngroups, chunk, 0, 0, 0, 0, ws,
                              kScratchBytes, hip_stream, SSD_PATH_STAGED, -1);
}
