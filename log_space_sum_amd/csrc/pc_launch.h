// pc_launch.h -- the one launch path of every kernel of the library.
//
// When a handle times its kernels, the runtime installs an EventSink for the
// calling thread around each group of launches.  Every launch then asks the
// sink for a fresh event pair and hands it to hipExtLaunchKernelGGL, which
// stamps the two events from the kernel's own dispatch packet: the measured
// interval is the kernel's execution alone, the interval a kernel trace
// reports, without the queueing gap that an event recorded before the launch
// would add.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

namespace pc {

struct EventSink {
  // A start/stop event pair for the next launch (created on first use).
  virtual void acquire(hipEvent_t* start, hipEvent_t* stop) = 0;
  virtual ~EventSink() = default;
};

// The calling thread's sink, or null when nothing is timed.
EventSink*& event_sink();

template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, size_t lds_bytes, hipStream_t s, Args... args) {
  if (EventSink* sink = event_sink()) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    sink->acquire(&e0, &e1);
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds_bytes, s, e0, e1, 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds_bytes, s, args...);
  }
}

}  // namespace pc
