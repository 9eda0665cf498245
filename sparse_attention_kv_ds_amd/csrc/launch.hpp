// launch.hpp -- the kernel launch helper used by the launchers of the .hip sources.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace dsi {

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
    return e;
}

} // namespace dsi
