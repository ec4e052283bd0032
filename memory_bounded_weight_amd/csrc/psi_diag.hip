// psi_diag.hip -- transport-control delay kernel.
//
// [PSI] sec. II-D and sec. IV-C separate transport correctness from
// arithmetic: reuse of a page must follow the copy and consumer
// dependencies whatever the timing.  With PSI_ARENA_JITTER the arena
// enqueues this kernel before every page or bias copy (on its copy stream:
// a consumer that did not wait for the copy would read stale bytes) and
// before every kernel launch (on the compute stream: a copy that did not
// wait for the previous consumer would overwrite a page still in use), for
// a deterministic pseudo-random 0-63 us, so that a missing wait would show
// up as changed bits.  One wave spins on the constant 100 MHz real-time counter; the loop
// is bounded by the requested duration.
#include "psi_internal.h"

namespace psi {
namespace {

__global__ __launch_bounds__(64) void delay_kernel(uint64_t ticks) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(1);
}

}  // namespace

hipError_t launch_delay(uint32_t microseconds, hipStream_t s) {
  if (microseconds == 0) return hipSuccess;
  hipLaunchKernelGGL(delay_kernel, dim3(1), dim3(64), 0, s, (uint64_t)microseconds * 100u);
  return hipGetLastError();
}

}  // namespace psi
