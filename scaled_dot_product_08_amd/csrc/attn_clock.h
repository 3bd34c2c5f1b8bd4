// Internal interface of the clock-sampling kernel (measurement support).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa08 {

constexpr int kClockXcds = 8;           // XCDs of the device
constexpr int kClockCusPerXcd = 128;    // slots per XCD: HW_ID's (engine, array, CU) fields
constexpr int kClockSlots = kClockXcds * kClockCusPerXcd;

// For every CU slot s (XCD x, HW_ID bits [14:8] c; s = 128 x + c):
// dst[2s] = its shader-clock counter, dst[2s + 1] = the 100 MHz real-time
// counter, read by a wave running on that CU. Slots of absent CUs are left
// as they were.
hipError_t launch_clock_sample(uint64_t* dst, hipStream_t stream);

}  // namespace sdpa08
