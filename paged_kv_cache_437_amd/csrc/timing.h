// Opt-in per-kernel timing with HIP events (internal).  While enabled, each launch
// made by the library carries a pair of events that its own dispatch records
// (hipExtLaunchKernelGGL), so they time the kernel alone, without marker packets
// of their own before and after it.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace pkv {

// Cheap no-ops while timing is off.  timing_begin opens a pair of events for the
// calling thread's next launch on `stream` (none while the stream is being captured
// into a graph); timing_start / timing_stop return them (null when none is open), to
// be passed to that launch; timing_end files them for collection if the launch was
// accepted, else returns them to the pool.
void timing_begin(const char* kernel, hipStream_t stream);
hipEvent_t timing_start();
hipEvent_t timing_stop();
void timing_end(hipStream_t stream);

}  // namespace pkv
