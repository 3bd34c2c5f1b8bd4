// Clock sampling for measurements. Waves on every CU record that CU's
// shader-clock counter (s_memtime: cycles of the CU's shader clock; it stops
// while the CU is clock-gated, so counters of different CUs drift apart) and
// the constant 100 MHz real-time counter (s_memrealtime) into device memory,
// at the slot of the CU they run on (hardware registers XCC_ID and HW_ID).
// Two samples are compared per CU: over a busy region between them,
// (dt_shader / dt_real) * 100 MHz is that CU's average shader clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_clock.h"

namespace sdpa08 {
namespace {

// s_getreg_b32 operands: hardware register 20 (XCC_ID) bits [3:0], and
// register 4 (HW_ID) bits [14:8]: CU id [11:8], shader-array id [12], shader
// engine id [14:13].
constexpr int kXccIdReg = (3 << 11) | (0 << 6) | 20;
constexpr int kHwIdCuReg = (6 << 11) | (8 << 6) | 4;

__global__ __launch_bounds__(64) void clock_sample_kernel(uint64_t* dst) {
  const uint64_t t = __builtin_amdgcn_s_memtime();
  const uint64_t r = __builtin_amdgcn_s_memrealtime();
  const int xcc = __builtin_amdgcn_s_getreg(kXccIdReg) & (kClockXcds - 1);
  const int cu = __builtin_amdgcn_s_getreg(kHwIdCuReg) & (kClockCusPerXcd - 1);
  const int slot = xcc * kClockCusPerXcd + cu;
  if (threadIdx.x < 2) dst[2 * slot + threadIdx.x] = threadIdx.x == 0 ? t : r;
}

}  // namespace

hipError_t launch_clock_sample(uint64_t* dst, hipStream_t stream) {
  // Eight workgroups per slot: enough that every CU runs at least one. After a
  // barrier the device is idle and they all read their counters within
  // microseconds. (A kernel may start on CUs that the previous kernel of the
  // stream has already released, so a sample meant to follow that kernel must
  // come after a barrier, such as an event record, on the stream.)
  hipLaunchKernelGGL(clock_sample_kernel, dim3(8 * kClockSlots), dim3(64), 0, stream, dst);
  return hipGetLastError();
}

}  // namespace sdpa08
