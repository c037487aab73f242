// ssm_scan_fwd_noalloc: the forward scan for callers that cannot allocate
// (code under HIP graph capture, tight serving loops).  The scan's scratch --
// job ticket, error word, per-tile progress words and the carried states of
// the segment hand-off -- lives in one file-scope device array instead of a
// caller-provided workspace.  Each GPU holds its own copy of the array until
// the process ends; calls that overlap on one GPU share it and race.
#include <mutex>

#include "ssm_kernels.h"
#include "ssm_scan.h"

namespace ssm {
namespace {

static __device__ __align__(256) unsigned char scratch[SSM_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_addr[kMaxDevices];   // device address of `scratch`, per device (null: not resolved yet)

}  // namespace

// The device address of this device's `scratch`.  The array's name in host
// code is only a stand-in for the symbol: its address is resolved once per
// device, with that device current, and kept.
hipError_t noalloc_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_addr[dev] = p;
    }
    *out = g_addr[dev];
    return hipSuccess;
}

}  // namespace ssm
