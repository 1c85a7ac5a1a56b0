// common.hpp -- shared device helpers for the gfx950 MoE megakernel library:
// element types, bf16 rounding, scoped atomics and fences, the watchdog
// clock, and the launch-parameter block every kernel receives.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define DEV __device__ __forceinline__

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace moe {

constexpr int kThreads = 256;   // 4 wave64 per workgroup
constexpr int kBN = 128;        // output columns per GEMM task
constexpr int kTB = 32;         // tokens per router / position tile
constexpr int kMaxK = 8;        // top-k limit
constexpr int kMaxE = 256;      // router width limit

// ---------------------------------------------------------------- element
DEV float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
DEV bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename Elem> struct ElemTraits;
template <> struct ElemTraits<bf16_t> {
  static constexpr bool kBf16 = true;
  static constexpr int kBK = 64;           // K depth of one LDS stage
  static DEV float to_f(bf16_t v) { return bf2f(v); }
  static DEV bf16_t from_f(float v) { return f2bf(v); }
};
template <> struct ElemTraits<float> {
  static constexpr bool kBf16 = false;
  static constexpr int kBK = 32;
  static DEV float to_f(float v) { return v; }
  static DEV float from_f(float v) { return v; }
};

// ------------------------------------------------------- atomics / fences
// Cross-task publication on gfx950.  Each XCD has its own L2, so a value a
// task writes must leave that L2 before a consumer on another XCD reads it.
// The generic agent-scope release/acquire would write back the producer's
// whole L2 and invalidate the consumer's whole L2 on every task -- measured
// at 20-30% of the layer time.  This library instead relies on a property of
// its own data flow: every inter-task buffer (routing tables, row-tile table,
// gathered rows Xp, hidden rows H, zeroed y rows) is written once per launch
// and read only after all of its writers have been published, so no reader
// can hold a stale copy from this launch (kernel boundaries order launches).
// Producers therefore store that data with agent-coherent (sc1, write-
// through) stores and drain them (vmcnt(0)) before the atomic that
// publishes; consumers read with plain loads and need no invalidation.
// The dependency counters and queue words themselves are relaxed atomics.
// This holds at cache-line granularity too: every region one task writes
// and another reads (a row block of Xp, H or y, a token tile of the routing
// tables, a router partial tile) starts and ends on a 128-byte boundary, so
// a reader never caches a line that a later writer still changes.
DEV void publish_fence() {
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xf << 8));   // vmcnt(0): stores done
  asm volatile("" ::: "memory");
}
DEV void consume_fence() { asm volatile("" ::: "memory"); }

// Agent-coherent (write-through) stores for inter-task data.
DEV void st_wt(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV void st_wt(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A pointer the caller knows is the same in every lane, moved into scalar
// registers (so buffer descriptors built from it need no per-lane loop).
template <typename T>
DEV T* uniform_ptr(T* ptr) {
  const uint64_t b = (uint64_t)(uintptr_t)ptr;
  return (T*)(uintptr_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b));
}

typedef unsigned int u32x4_t __attribute__((__vector_size__(16)));
// 16 bytes at base + byte_off; base must be 16-byte aligned, byte_off < 2^31.
// base must be the same in every lane of the wave (the buffer descriptor is
// scalar): a per-lane base makes the compiler loop over its distinct values.
// Per-lane addressing goes into byte_off.
DEV void st_wt16(void* base, uint32_t byte_off, uint4 v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
  const u32x4_t d = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(d, r, byte_off, 0, 16 /* sc1 */);
}
// The same with the non-temporal hint, for data written once and read once
// much later, which should not displace cached lines that other tasks reuse.
DEV void st_wt16_stream(void* base, uint32_t byte_off, uint4 v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
  const u32x4_t d = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(d, r, byte_off, 0, 16 | 2 /* sc1 nt */);
}

// 16 bytes read with the non-temporal hint: data read once, which should
// not displace cached lines that other tasks reuse.
DEV float4 ld_stream4(const float* p) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// 16 bytes read coherently with device-scope atomics from every XCD (four
// agent-scope relaxed atomic loads): for data other workgroups may have
// updated with atomics after this XCD's L2 could have cached a line of it.
DEV float4 ld_coherent4(const float* p) {
  float4 v;
  v.x = __hip_atomic_load(p + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.y = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.z = __hip_atomic_load(p + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.w = __hip_atomic_load(p + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}

DEV int ld_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV void st_relaxed(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV int add_relaxed(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV int cas_relaxed(int* p, int expected, int desired) {
  __hip_atomic_compare_exchange_strong(p, &expected, desired, __ATOMIC_RELAXED,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return expected;
}

// threadIdx.x through an empty volatile asm: the persistent loop runs many
// tile shapes, and lane-dependent address math must not be hoisted out of it
// (that would keep every shape's per-lane offsets live across all tasks).
DEV int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}
// The thread index as every task body and scheduler step reads it: opaque at
// each use, so no lane-dependent value is computed once before the
// persistent loop and kept (or spilled) across all task types.
DEV int tidx() { return opaque_tid(); }

// Cross-lane exchange inside a wave (ds_bpermute), with the lane index taken
// from tidx() so that no lane-index arithmetic is hoisted out of the
// persistent loop.  xor: the value of lane (lane ^ o); up: of lane (lane - o),
// or the lane's own value for lanes below o.
DEV float wave_xor(float v, int o) {
  const int lane = tidx() & 63;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(((lane ^ o) & 63) << 2, __float_as_int(v)));
}
DEV int wave_xor_i(int v, int o) {
  const int lane = tidx() & 63;
  return __builtin_amdgcn_ds_bpermute(((lane ^ o) & 63) << 2, v);
}
DEV int wave_up(int v, int o) {
  const int lane = tidx() & 63;
  return __builtin_amdgcn_ds_bpermute((lane >= o ? lane - o : lane) << 2, v);
}

// A value every lane of the wave holds (a workgroup-wide result broadcast
// through LDS), read from the first lane into a scalar register, so that the
// branches and addresses that depend on it are scalar.
DEV int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Constant-rate device clock (100 MHz on CDNA3/CDNA4) for watchdogs and
// the optional task trace.
DEV uint64_t rtc() { return __builtin_amdgcn_s_memrealtime(); }

// XCD (XCC) id of the executing wave: HW_REG_XCC_ID, bits [3:0].
DEV int xcc_id() {
  return __builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (3 << 11)) & 0xf;
}

}  // namespace moe
