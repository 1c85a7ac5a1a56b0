// k_f32.hip -- every kernel of the fp32 path (register-staged fp32 tiles):
// persistent dynamic and static megakernels, and the per-stage launches.
#include "launch.hpp"
#include "sched.hpp"

namespace moe {

hipError_t launch_dynamic_f32(bool scatter, const Params& p, hipStream_t s) {
  if (scatter)
    hipLaunchKernelGGL((k_dynamic<float, true>), dim3(p.workers), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((k_dynamic<float, false>), dim3(p.workers), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_dynamic_layers_f32(bool scatter, const Params* layers, int n, int workers,
                                     hipStream_t s) {
  if (scatter)
    hipLaunchKernelGGL((k_dynamic_layers<float, true>), dim3(workers), dim3(kThreads), 0, s, layers, n);
  else
    hipLaunchKernelGGL((k_dynamic_layers<float, false>), dim3(workers), dim3(kThreads), 0, s, layers, n);
  return hipGetLastError();
}

hipError_t launch_static_f32(bool scatter, const Params& p, hipStream_t s) {
  if (scatter)
    hipLaunchKernelGGL((k_static<float, true>), dim3(p.workers), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((k_static<float, false>), dim3(p.workers), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_stages_f32(const Params& p, hipStream_t s) {
  return launch_stage_sequence<float>(p, s);
}

hipError_t launch_route_only_f32(const Params& p, hipStream_t s) {
  return launch_route_sequence<float>(p, s);
}

hipError_t occupancy_dynamic_f32(int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k_dynamic<float, false>, kThreads, 0);
}

hipError_t occupancy_static_f32(int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k_static<float, false>, kThreads, 0);
}

}  // namespace moe
