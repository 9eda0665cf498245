// static_scratch.hip -- the device scratch of ds_indexer_score_topk_noalloc:
// one file-scope array per GPU, so that the call allocates nothing.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up here, once per device (with that device
// current), and only that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.hpp"

namespace dsi {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 256;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices] = {};

} // namespace

hipError_t static_scratch(int device, void **ptr)
{
    *ptr = nullptr;
    if (device < 0 || device >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return e != hipSuccess ? e : hipErrorInvalidSymbol;
        scratch_ptr[device] = p;
    }
    *ptr = scratch_ptr[device];
    return hipSuccess;
}

} // namespace dsi
