// k_static_bf16.hip -- the static-partition persistent megakernel, bf16
// (baseline: the same tasks pre-assigned round-robin, barriers between stages).
#include "launch.hpp"
#include "sched.hpp"

namespace moe {

hipError_t launch_static_bf16(bool scatter, const Params& p, hipStream_t s) {
  if (scatter)
    hipLaunchKernelGGL((k_static<bf16_t, true>), dim3(p.workers), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((k_static<bf16_t, false>), dim3(p.workers), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t occupancy_static_bf16(int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k_static<bf16_t, false>, kThreads, 0);
}

}  // namespace moe
