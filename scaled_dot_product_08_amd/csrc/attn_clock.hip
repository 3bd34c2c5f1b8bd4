// Clock sampling for measurements. One wave records the shader-clock counter
// (s_memtime, counting cycles of the shader clock of the XCD it runs on) and
// the constant-rate real-time counter (s_memrealtime, 100 MHz) into device
// memory. Two samples enqueued on a stream around a timed region give the
// average shader clock over that region: (dt_shader / dt_real) * 100 MHz.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_clock.h"

namespace sdpa08 {
namespace {

__global__ __launch_bounds__(64) void clock_sample_kernel(uint64_t* dst) {
  const uint64_t t = __builtin_amdgcn_s_memtime();
  const uint64_t r = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x < 2) dst[threadIdx.x] = threadIdx.x == 0 ? t : r;
}

}  // namespace

hipError_t launch_clock_sample(uint64_t* dst, hipStream_t stream) {
  hipLaunchKernelGGL(clock_sample_kernel, dim3(1), dim3(64), 0, stream, dst);
  return hipGetLastError();
}

}  // namespace sdpa08
