// ecmd_launch.h -- the one way the library enqueues a kernel (host code).
//
// A launch normally goes through hipLaunchKernel.  A timed launch
// (cmd_launch_timed) asks for two caller-owned HIP events to be recorded by
// the dispatches themselves (the HIP extension hipExtLaunchKernel /
// hipExtModuleLaunchKernel): the first dispatch records `start` when it
// begins and every dispatch records `stop` when it ends, so after the launch
// the events bracket exactly the kernel execution of all its dispatches -- the
// interval a kernel-trace profiler reports -- without the command processor's
// time between a separate event packet and the dispatch.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime_api.h>

namespace ecmd {

struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
// The events of the timed launch in progress on this thread (none normally).
LaunchEvents &launch_events();

// Enqueue kernel fn (a __global__ function's address) with its by-value
// arguments on stream; returns a hipError_t.
template <class... A>
int launch_kernel(const void *fn, dim3 grid, dim3 block, unsigned lds_bytes, void *stream, const A &...args)
{
    void *params[] = {const_cast<void *>(static_cast<const void *>(&args))...};
    LaunchEvents &ev = launch_events();
    hipError_t e;
    if (ev.start || ev.stop) {
        e = hipExtLaunchKernel(fn, grid, block, params, lds_bytes, (hipStream_t)stream, ev.start, ev.stop, 0);
        ev.start = nullptr;   // only the first dispatch starts the interval
    } else {
        e = hipLaunchKernel(fn, grid, block, params, lds_bytes, (hipStream_t)stream);
    }
    if (e != hipSuccess) (void)hipGetLastError();   // the status is returned; leave no sticky error
    return (int)e;
}

// The same for a kernel of a loaded module (run-time compiled kernels):
// grid work-groups of block work-items.
int launch_module(hipFunction_t fn, unsigned grid, unsigned block, unsigned lds_bytes, void *stream, void **params);

}  // namespace ecmd
