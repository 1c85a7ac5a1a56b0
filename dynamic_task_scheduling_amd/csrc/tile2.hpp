// tile2.hpp -- bf16 GEMM tile for gfx950 with a multi-stage LDS ring fed by
// direct global->LDS loads.
//
// C[BM, 128] (x NB matrices sharing A) = A[BM, K] * B[K, 128], bf16 in,
// fp32 accumulate, v_mfma_f32_16x16x32_bf16.
//
// Why: a task's K loop is bound by memory latency, not MFMA, unless several
// K stages are in flight.  The 16-byte global_load_lds form (new on gfx950)
// writes straight into LDS without staging in VGPRs, so S-1 stages (S = 3 or
// 4, up to 144 KB of the 160 KB LDS) can be outstanding while the MFMAs
// consume the oldest one.
//
// LDS layouts (one stage):
//   A: BM rows x 128 bytes (64 bf16 of K).  16-byte chunk c of row m sits at
//      position c ^ (m & 7): the 16 rows one fragment read touches fall on 8
//      distinct bank groups.
//   B: 64 rows (K) x 256 bytes (128 bf16 of N), the weights' natural row-major
//      layout; chunk c of row k at c ^ 2*(k & 3).  The MFMA B operand needs
//      8 consecutive K per lane, which ds_read_b64_tr_b16 delivers: each 16-lane
//      group reads a 4 (K) x 16 (N) block and every lane receives one column.
// A lane of a global_load_lds instruction writes its 16 bytes at
// base + 16 * lane, so the swizzles are applied to the global addresses.
#pragma once
#include <type_traits>

#include "common.hpp"

namespace moe {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] and
// vmcnt[5:4] at bits 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// One 16-byte global->LDS load per lane into [lds_base + 16*lane].  Issued
// through inline asm on purpose: the compiler's wait-count pass cannot tell
// which ring stage an LDS read touches and, seeing LDS DMA in flight, waits
// for all of it before LDS reads and barriers, which would leave a single
// stage in flight.  The ring tracks completion itself with s_waitcnt vmcnt
// (loads retire in order), so compiler-issued loads stay correctly ordered:
// extra outstanding DMA only makes the compiler's own waits stricter.  The
// asm declares no memory clobber; ordering against LDS reads comes from the
// barrier + compiler fence in the K loop.
DEV void dma16(const void* gptr, uint32_t lds_base) {
  // m0 is a reserved register: save and restore it around the load.
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(gptr));
}

DEV uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const LDS_AS void*)p;
}

// MF selects the MFMA: 16 = v_mfma_f32_16x16x32_bf16, 32 =
// v_mfma_f32_32x32x16_bf16.  The 32x32 form keeps the matrix pipe far busier
// with one wave per SIMD (measured 2.1 vs 1.35 PFLOP/s on gfx950) and halves
// LDS fragment traffic per flop.
// CLAMP_B: B has only `b_cols` valid columns (a multiple of 8, row stride
// ldb >= b_cols); 16-byte chunks past them reload chunk 0 of the same row, so
// every load stays inside B and only the (discarded) padded output columns
// see duplicated values.  Used by the router, whose width E may be < 128.
template <int BM, int NB, int S, int MF = 32, bool CLAMP_B = false>
struct Tile2 {
  static constexpr int BN = kBN;
  static constexpr int BK = 64;
  static constexpr int WM = (BM >= 64) ? 2 : 1;
  static constexpr int WN = 4 / WM;
  static constexpr int WTM = BM / WM;
  static constexpr int WTN = BN / WN;
  static constexpr int FM = WTM / MF;
  static constexpr int FN = WTN / MF;
  static_assert(MF == 16 || MF == 32, "MFMA shape");
  static_assert(FM >= 1 && FN >= 1, "wave tile");
  static constexpr int A_BYTES = BM * 128;
  static constexpr int B_BYTES = BK * 256;
  static constexpr int STAGE = A_BYTES + NB * B_BYTES;
  static constexpr int LDS_BYTES = S * STAGE;
  static constexpr int A_INST = BM / 32;           // per wave per stage
  static constexpr int B_INST = 4;                 // per wave per stage per matrix
  static constexpr int LOADS = A_INST + NB * B_INST;
  static_assert(S >= 2 && S <= 8, "stages");
  static_assert((S - 2) * LOADS < 64, "vmcnt range");

  typedef float f32x16_t __attribute__((ext_vector_type(16)));
  using Frag = typename std::conditional<MF == 32, f32x16_t, f32x4_t>::type;
  static constexpr int FRAG = MF == 32 ? 16 : 4;   // accumulator values per lane
  using Acc = Frag[NB][FM][FN];

  struct Args {
    const bf16_t* A;    // row 0 of the tile, K column 0
    int lda;
    int a_rows;         // valid rows (>= 1); later rows repeat the last one
    const bf16_t* B[NB];  // K row 0, column n0 of the tile
    int ldb;
    int K;              // multiple of 64
    int b_cols;         // CLAMP_B only: valid columns of B (multiple of 8)
  };

  static DEV void issue(const Args& g, int kt, char* stage) {
    const int tid_ = opaque_tid();
    const int wave = tid_ >> 6, lane = tid_ & 63;
    const int k0 = kt * BK;
#pragma unroll
    for (int ii = 0; ii < A_INST; ++ii) {
      const int i = wave * A_INST + ii;            // rows 8i .. 8i+7
      const int m = 8 * i + (lane >> 3);
      const int c = (lane & 7) ^ (m & 7);
      const int mr = m < g.a_rows ? m : g.a_rows - 1;
      const bf16_t* src = g.A + (size_t)mr * g.lda + k0 + c * 8;
      dma16(src, __builtin_amdgcn_readfirstlane(lds_addr(stage + i * 1024)));
    }
#pragma unroll
    for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
      for (int ii = 0; ii < B_INST; ++ii) {
        const int i = wave * B_INST + ii;          // K rows 4i .. 4i+3
        const int k = 4 * i + (lane >> 4);
        int c = (lane & 15) ^ (2 * (k & 3));
        if constexpr (CLAMP_B) c = (c * 8 < g.b_cols) ? c : 0;
        const bf16_t* src = g.B[mtx] + (size_t)(k0 + k) * g.ldb + c * 8;
        dma16(src, __builtin_amdgcn_readfirstlane(
                       lds_addr(stage + A_BYTES + mtx * B_BYTES + i * 1024)));
      }
  }

  static DEV void compute(const char* stage, Acc& acc) {
    const int tid_ = opaque_tid();
    const int lane = tid_ & 63;
    const int wave = tid_ >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int l16 = lane & 15, lg = lane >> 4;
    if constexpr (MF == 16) {
      // A lane: row lane%16, K 8*(lane/16)..+7; B lane: column lane%16, same K.
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t a[FM];
        bf16x8_t b[NB][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          const int m = wm * WTM + fm * 16 + l16;
          const int c = kk * 4 + lg;
          a[fm] = *reinterpret_cast<const LDS_AS bf16x8_t*>(
              (const LDS_AS char*)stage + m * 128 + ((c ^ (m & 7)) << 4));
        }
#pragma unroll
        for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const int n = wn * WTN + fn * 16 + 4 * (l16 & 3);
            b[mtx][fn] = read_b(stage, mtx, n, kk * 32 + 8 * lg + (l16 >> 2));
          }
#pragma unroll
        for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
              acc[mtx][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[mtx][fn],
                                                                         acc[mtx][fm][fn], 0, 0, 0);
      }
    } else {
      // A lane: row lane%32, K 8*(lane/32)..+7.  B lane: column lane%32, same
      // K; 16-lane group g reads columns 16*(g&1).., K rows 8*(g>>1)..
      const int l32 = lane & 31, lh = lane >> 5;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8_t a[FM];
        bf16x8_t b[NB][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          const int m = wm * WTM + fm * 32 + l32;
          const int c = kk * 2 + lh;
          a[fm] = *reinterpret_cast<const LDS_AS bf16x8_t*>(
              (const LDS_AS char*)stage + m * 128 + ((c ^ (m & 7)) << 4));
        }
#pragma unroll
        for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const int n = wn * WTN + fn * 32 + 16 * (lg & 1) + 4 * (l16 & 3);
            b[mtx][fn] = read_b(stage, mtx, n, kk * 16 + 8 * (lg >> 1) + (l16 >> 2));
          }
#pragma unroll
        for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
              acc[mtx][fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fm], b[mtx][fn],
                                                                         acc[mtx][fm][fn], 0, 0, 0);
      }
    }
  }

  // Eight consecutive K (rows k0, k0+4's quads) of B column block starting at
  // n for this lane, via two transposing LDS reads: rows k0..k0+3 and
  // k0+4..k0+7 of the 4 x 16 block each 16-lane group addresses.
  static DEV bf16x8_t read_b(const char* stage, int mtx, int n, int k0) {
    const int c = n >> 3, half = (n >> 2) & 1;
    bf16x4_t v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = k0 + 4 * h;
      const LDS_AS char* p = (const LDS_AS char*)stage + A_BYTES + mtx * B_BYTES + k * 256 +
                             ((c ^ (2 * (k & 3))) << 4) + half * 8;
      v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t*)p);
    }
    return __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
  }

  // Wait until at most `newer` stages of loads (those issued after the
  // stage about to be consumed) are still in flight.
  template <int N>
  static DEV void wait_newer(int newer) {
    if constexpr (N > 0) {
      if (newer >= N) { wait_vmcnt<N * LOADS>(); return; }
      wait_newer<N - 1>(newer);
    } else {
      wait_vmcnt<0>();
    }
  }
  static DEV void wait_stage(int newer) { wait_newer<S - 2>(newer); }

  // Full K loop; ends with a barrier so the caller may reuse `smem`.
  static DEV void run(const Args& g, char* smem, Acc& acc) {
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[m][fm][fn] = Frag{};
    const int nk = g.K / BK;
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < nk) issue(g, s, smem + s * STAGE);
    for (int kt = 0; kt < nk; ++kt) {
      // stages issued after k-tile kt: kt+1 .. min(kt+S-2, nk-1)
      const int newer = min(S - 2, nk - 1 - kt);
      wait_stage(newer);
      // every wave's loads of stage kt have landed; no hardware fence needed
      // (LDS reads of the stage about to be refilled were consumed by
      // MFMAs), only a compiler fence so LDS reads stay after the barrier
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (kt + S - 1 < nk) issue(g, kt + S - 1, smem + ((kt + S - 1) % S) * STAGE);
      compute(smem + (kt % S) * STAGE, acc);
    }
    __syncthreads();
  }

  // Visit every accumulator position: fn(row, col, fm, fn, i).  16x16
  // result: lane holds column lane%16, rows 4*(lane/16)+i.  32x32 result:
  // column lane%32, rows 8*(i/4) + 4*(lane/32) + i%4.
  template <typename F>
  static DEV void for_each(F&& fn) {
    const int tid_ = opaque_tid();
    const int lane = tid_ & 63;
    const int wave = tid_ >> 6;
    const int wm = wave / WN, wn = wave % WN;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fnn = 0; fnn < FN; ++fnn)
#pragma unroll
        for (int i = 0; i < FRAG; ++i) {
          int row, col;
          if constexpr (MF == 16) {
            row = wm * WTM + fm * 16 + (lane >> 4) * 4 + i;
            col = wn * WTN + fnn * 16 + (lane & 15);
          } else {
            row = wm * WTM + fm * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
            col = wn * WTN + fnn * 32 + (lane & 31);
          }
          fn(row, col, fm, fnn, i);
        }
  }
};

}  // namespace moe
