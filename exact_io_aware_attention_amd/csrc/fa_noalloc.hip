// fa_bwd_noalloc: the bf16 backward with its row-statistics scratch in a
// static device array of the library instead of a caller-provided
// workspace, for callers that cannot allocate device memory (code under
// stream capture, tight serving loops, harnesses that forbid allocation).
//
// The array is file-scope device memory of the code object: each GPU the
// library runs on holds its own copy, at its own address, until the process
// ends. Host code never passes the array's name to a kernel (in host code
// that name is only a stand-in for the symbol, not a device address): the
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and kept.
//
// Every call on one GPU shares that GPU's array. The backward's preprocessing
// kernel writes every scratch entry the later kernels read, so nothing needs
// clearing between calls; but two calls that overlap in time on one GPU (on
// different streams, or from different host threads) race on it.
#include <mutex>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on first use,
// with the device current). Returns the HIP status of the lookup.
hipError_t scratch_for_current_device(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (ptr == nullptr)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

namespace fa {

hipError_t noalloc_scratch(size_t bytes, void **out)
{
    if (bytes > kScratchBytes)
        return hipErrorInvalidValue;
    return scratch_for_current_device(out);
}

}  // namespace fa
