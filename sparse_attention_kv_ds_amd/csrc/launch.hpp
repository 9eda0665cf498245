// launch.hpp -- the kernel launch helper used by the launchers of the .hip sources.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdlib.h>

#include "internal.hpp"

namespace dsi {

// DS_INDEXER_DEBUG set to anything but "" or "0": every launch is followed by
// a synchronisation of its stream and a check of the result, so that a failing
// kernel is reported (DS_ERR_HIP) by the call that launched it rather than by
// a later one.  For tests and debugging: the synchronisation stalls the host,
// and it is not allowed under stream capture.  Read at every launch, so that
// a process can switch it.
inline bool debug_sync()
{
    const char *v = getenv("DS_INDEXER_DEBUG");
    return v != nullptr && v[0] != 0 && !(v[0] == '0' && v[1] == 0);
}

// the result of a launch that returned `e`, checked to completion in debug mode
inline hipError_t after_launch(hipError_t e, hipStream_t st)
{
    if (e != hipSuccess || !debug_sync())
        return e;
    e = hipStreamSynchronize(st);
    return e != hipSuccess ? e : hipGetLastError();
}

// Launch `kernel` on `st`, converting each argument to the kernel's parameter
// type; with `tm`, record its events on this launch (`first` / `last`: this
// launch opens / closes the timed step).
template <class... P, class... A>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                         Timing *tm, bool first, bool last, A &&...args)
{
    hipEvent_t e0 = tm && first ? tm->start : nullptr;
    hipEvent_t e1 = tm && last ? tm->stop : nullptr;
    // the runtime's last-error slot may still hold the result of an unrelated
    // earlier call (a query answered "not ready", say): clear it, so that the
    // check below reports this launch only
    (void)hipGetLastError();
    if (e0 || e1)
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, st, e0, e1, 0u,
                              static_cast<P>(args)...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, st, static_cast<P>(args)...);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess && tm) {
        tm->started |= e0 != nullptr;
        tm->stopped |= e1 != nullptr;
    }
    return after_launch(e, st);
}

} // namespace dsi
