// Library-held scratch memory for w4a16_gemm_noalloc, the product form for
// callers that cannot allocate device memory (code under graph capture, tight
// serving loops).  The K-split partial sums that w4a16_gemm takes from a
// caller workspace live here instead, in one fixed array per GPU.
//
// In host code `scratch` names a host-side stand-in, never the device memory:
// its device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and kept, and only that address is handed to
// kernels.  Every call on a GPU shares that GPU's array, so calls that overlap
// on one GPU (other streams, other threads) race; calls in order on one
// stream do not.  Nothing in it needs clearing: every split writes its whole
// partial tile before the split sum reads it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

static __device__ __align__(256) unsigned char scratch[w4::kNoAllocScratchBytes];

namespace w4 {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace w4
