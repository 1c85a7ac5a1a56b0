// k_dynamic_layers_bf16_scatter.hip -- several bf16 layers in one persistent
// launch, scatter-add combine (layers with few routed rows).
#include "launch.hpp"
#include "sched.hpp"

namespace moe {

hipError_t launch_dynamic_layers_bf16_scatter(const Params* layers, int n, int workers,
                                              hipStream_t s) {
  hipLaunchKernelGGL((k_dynamic_layers<bf16_t, true>), dim3(workers), dim3(kThreads), 0, s, layers, n);
  return hipGetLastError();
}

}  // namespace moe
