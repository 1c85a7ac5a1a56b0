// k_dynamic_bf16_rows.hip -- the persistent dynamic megakernel, bf16, DOWN
// tiles writing fp32 output rows summed by combine tasks (larger layers).
#include "launch.hpp"
#include "sched.hpp"

namespace moe {

hipError_t launch_dynamic_bf16_rows(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL((k_dynamic<bf16_t, false>), dim3(p.workers), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t occupancy_dynamic_bf16(int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k_dynamic<bf16_t, false>, kThreads, 0);
}

}  // namespace moe
