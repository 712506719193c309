// Kernel launch with optional dispatch timestamps (HIP device sources only).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace gsa {

// Launches kernel on stream.  When events is non-null, events[i0] and
// events[i1] (each nullable; an index < 0 means none) take the start and end
// timestamps of this dispatch itself, so that the elapsed time between them is
// the kernel's execution time with no launch gap.
template <class F, class... Args>
inline void launch_timed(F kernel, dim3 grid, dim3 block, unsigned lds, void* stream,
                         void* const* events, int i0, int i1, Args... args) {
  hipEvent_t e0 = events && i0 >= 0 ? (hipEvent_t)events[i0] : nullptr;
  hipEvent_t e1 = events && i1 >= 0 ? (hipEvent_t)events[i1] : nullptr;
  if (e0 || e1)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, (hipStream_t)stream, e0, e1, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, (hipStream_t)stream, args...);
}

}  // namespace gsa
