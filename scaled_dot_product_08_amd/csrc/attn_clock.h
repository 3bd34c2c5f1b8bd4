// Internal interface of the clock-sampling kernel (measurement support).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa08 {

// Writes {shader-clock counter, 100 MHz real-time counter} to dst[0], dst[1].
hipError_t launch_clock_sample(uint64_t* dst, hipStream_t stream);

}  // namespace sdpa08
