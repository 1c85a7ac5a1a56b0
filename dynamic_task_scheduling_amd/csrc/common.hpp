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
// Inter-task visibility on gfx950: every XCD has its own L2, so producer and
// consumer on different XCDs need an agent-scope release (write back) and
// acquire (invalidate).  The compiler lowers these to the right cache
// maintenance for the memory model.
DEV void fence_release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
DEV void fence_acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

DEV int ld_acquire(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
DEV int ld_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV void st_relaxed(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV void st_release(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
DEV int add_relaxed(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV int add_acqrel(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
DEV int cas_relaxed(int* p, int expected, int desired) {
  __hip_atomic_compare_exchange_strong(p, &expected, desired, __ATOMIC_RELAXED,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return expected;
}

// Constant-rate device clock (100 MHz on CDNA3/CDNA4) for watchdogs and
// the optional task trace.
DEV uint64_t rtc() { return __builtin_amdgcn_s_memrealtime(); }

// XCD (XCC) id of the executing wave: HW_REG_XCC_ID, bits [3:0].
DEV int xcc_id() {
  return __builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (3 << 11)) & 0xf;
}

}  // namespace moe
