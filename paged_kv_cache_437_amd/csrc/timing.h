// Opt-in per-kernel timing with HIP events (internal).  While enabled, each launch
// made by the library is bracketed by a pair of events recorded on its stream.
#pragma once

#include <hip/hip_runtime.h>

namespace pkv {

// Cheap no-ops while timing is off.
void timing_begin(const char* kernel, hipStream_t stream);
void timing_end(hipStream_t stream);

}  // namespace pkv
