// k_dynamic_layers_bf16_rows.hip -- several bf16 layers in one persistent
// launch, DOWN tiles writing output rows summed by combine tasks.
#include "launch.hpp"
#include "sched.hpp"

namespace moe {

hipError_t launch_dynamic_layers_bf16_scatter(const Params* layers, int n, int workers,
                                              hipStream_t s);

hipError_t launch_dynamic_layers_bf16(bool scatter, const Params* layers, int n, int workers,
                                      hipStream_t s) {
  if (scatter) return launch_dynamic_layers_bf16_scatter(layers, n, workers, s);
  hipLaunchKernelGGL((k_dynamic_layers<bf16_t, false>), dim3(workers), dim3(kThreads), 0, s, layers, n);
  return hipGetLastError();
}

}  // namespace moe
