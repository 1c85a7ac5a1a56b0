// launch.hpp -- host-side launchers of the device kernels.
//
// Each kernel family is compiled in a translation unit of its own (k_*.hip),
// so the library builds in parallel; the host code in moe.hip reaches the
// kernels only through these functions.  Every launcher enqueues on stream
// `s` and returns the launch status (hipGetLastError after the launches).
#pragma once
#include <hip/hip_runtime.h>

#include "params.hpp"

namespace moe {

// Persistent dynamic megakernel (one workgroup per worker, p.workers of
// them); `scatter` selects the instantiation with the scatter-add combine.
hipError_t launch_dynamic_bf16_scatter(const Params& p, hipStream_t s);
hipError_t launch_dynamic_bf16_rows(const Params& p, hipStream_t s);
hipError_t launch_dynamic_f32(bool scatter, const Params& p, hipStream_t s);

// Several layers in one persistent launch; `layers` is a device array of n
// parameter blocks (all of one element type and combine mode).
hipError_t launch_dynamic_layers_bf16(bool scatter, const Params* layers, int n, int workers,
                                      hipStream_t s);
hipError_t launch_dynamic_layers_f32(bool scatter, const Params* layers, int n, int workers,
                                     hipStream_t s);

// Persistent static-partition megakernel.
hipError_t launch_static_bf16(bool scatter, const Params& p, hipStream_t s);
hipError_t launch_static_f32(bool scatter, const Params& p, hipStream_t s);

// One ordinary launch per stage (the multi-kernel baseline).
hipError_t launch_stages_bf16(const Params& p, hipStream_t s);
hipError_t launch_stages_f32(const Params& p, hipStream_t s);

// Routing from given logits: top-k, build, positions (p.route_from_logits).
hipError_t launch_route_only_bf16(const Params& p, hipStream_t s);
hipError_t launch_route_only_f32(const Params& p, hipStream_t s);

// Resident workgroups per CU of the persistent kernels.
hipError_t occupancy_dynamic_bf16(int* blocks);
hipError_t occupancy_static_bf16(int* blocks);
hipError_t occupancy_dynamic_f32(int* blocks);
hipError_t occupancy_static_f32(int* blocks);

}  // namespace moe
