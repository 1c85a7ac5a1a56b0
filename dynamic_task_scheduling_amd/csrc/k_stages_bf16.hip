// k_stages_bf16.hip -- one launch per stage, bf16 (the multi-kernel
// baseline), and the routing-only sequence used on caller logits.
#include "launch.hpp"
#include "sched.hpp"

namespace moe {

hipError_t launch_stages_bf16(const Params& p, hipStream_t s) {
  return launch_stage_sequence<bf16_t>(p, s);
}

hipError_t launch_route_only_bf16(const Params& p, hipStream_t s) {
  return launch_route_sequence<bf16_t>(p, s);
}

}  // namespace moe
