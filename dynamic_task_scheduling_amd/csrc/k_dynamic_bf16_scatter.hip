// k_dynamic_bf16_scatter.hip -- the persistent dynamic megakernel, bf16,
// scatter-add combine in the DOWN epilogue (layers with few routed rows).
#include "launch.hpp"
#include "sched.hpp"

namespace moe {

hipError_t launch_dynamic_bf16_scatter(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL((k_dynamic<bf16_t, true>), dim3(p.workers), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
