// noalloc.hip -- greedy verify for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  Same kernels and results as mtp_verify_greedy; its key
// scratch lives in a file-scope device array instead of a context.
//
// The array is a per-device object of the loaded code: each GPU the library
// runs on holds its own copy until the process ends.  Host code never uses
// the array's name as an address (on the host it is only a stand-in): the
// device address is looked up once per device, with that device current,
// through hipGetSymbolAddress, and only that address reaches kernels.
#include <cstdio>
#include <mutex>

#include "mtp_internal.h"

namespace mtp {

// argmax keys, one per verified row (n_seq * (n_draft + 1) rows per call)
static __device__ __align__(256) uint64_t scratch[MTP_NOALLOC_MAX_ROWS];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
uint64_t *g_scratch[kMaxDevices] = {};
}  // namespace

// Device address of this device's scratch array (looked up on the first call
// on the current device).  Returns hipSuccess and *out, or the lookup's error.
hipError_t noalloc_scratch(uint64_t **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = (uint64_t *)p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace mtp
