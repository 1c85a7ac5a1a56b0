// tile2.hpp -- bf16 GEMM tile for gfx950 with a multi-stage LDS ring fed by
// direct global->LDS loads.
//
// C[BM, 128] (x NB matrices sharing A) = A[BM, K] * B[K, 128], bf16 in,
// fp32 accumulate, v_mfma_f32_32x32x16_bf16.
//
// Why: a task's K loop is bound by memory latency, not MFMA, unless several
// K stages are in flight.  The 16-byte global_load_lds form (new on gfx950)
// writes straight into LDS without staging in VGPRs, so S-1 stages (S = 3 or
// 4, up to 144 KB of the 160 KB LDS) can be outstanding while the MFMAs
// consume the oldest one.
//
// LDS layouts (one stage):
//   A: BM rows x 128 bytes (64 bf16 of K).  16-byte chunk c of row m sits at
//      position c ^ swz_a128(m): the 16 rows one 16-lane phase of a fragment
//      read touches fall on 16 distinct 16-byte bank groups.
//   B: 64 rows (K) x 256 bytes (128 bf16 of N), the weights' natural row-major
//      layout; chunk c of row k at c ^ swz_b(k).  The MFMA B operand needs
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

// LDS swizzles.  gfx950's LDS has 64 banks of 4 bytes (256 bytes per clock):
// a 16-byte-per-lane read is served 16 lanes at a time and an 8-byte-per-lane
// read 32 lanes at a time, so the lanes served together must fall on 16
// distinct 16-byte bank groups of a 256-byte line.  Each function gives the
// XOR applied to the 16-byte chunk index of a row.
//   swz_a128: A rows of 128 bytes (8 chunks): a fragment read takes one chunk
//             of 16 consecutive rows, two rows per 256-byte line.
//   swz_a64:  A rows of 64 bytes (4 chunks): four rows per line.
//   swz_b:    B rows of 256 bytes (16 chunks): a transposing read takes two
//             chunks of 4 consecutive rows per 16 lanes, 32 lanes together
//             read four chunks of 4 rows.
DEV int swz_a128(int m) { return (m >> 1) & 7; }
DEV int swz_a64(int m) { return (m >> 2) & 3; }
DEV int swz_b(int k) { return 4 * (k & 3); }

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
  // m0 is a reserved register: save and restore it around the load.  s_nop 0
  // is the one wait state an SALU write of M0 needs before an LDS DMA.
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(gptr));
}

DEV uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const LDS_AS void*)p;
}

// One 16-byte global->LDS load per lane from sbase + voff (a uniform 64-bit
// base in SGPRs plus a 32-bit per-lane offset), landing at
// [lds_base + 16*lane].  The per-lane offsets of a tile are computed once;
// each K stage only moves the uniform base.
DEV void dma16s(uint32_t voff, uint64_t base, uint32_t lds_base) {
  const uint64_t sbase =
      ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) << 32) |
      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(voff), "s"(sbase));
}

// The same with the non-temporal hint, for data that should not displace
// cached lines other tasks reuse.
DEV void dma16s_nt(uint32_t voff, uint64_t base, uint32_t lds_base) {
  const uint64_t sbase =
      ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) << 32) |
      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(voff), "s"(sbase));
}

// C[BM, 128] (x NB matrices sharing A) = A[BM, K] * B[K, 128], bf16 in, fp32
// accumulate, v_mfma_f32_32x32x16_bf16 (the 32x32 form keeps the matrix pipe
// far busier with one wave per SIMD than 16x16x32, and halves LDS fragment
// traffic per flop).
//
// The K loop is software-pipelined at two levels: S-1 ring stages of
// direct-to-LDS loads are in flight, and inside a stage the fragments of
// step kk+1 are read from LDS into a second register set while the MFMAs of
// step kk run (the last step of a stage prefetches step 0 of the next stage
// after the barrier), so the matrix pipe never waits on an LDS read it could
// have issued earlier.  Lane addresses are computed once per tile.
//
// CLAMP_B: B has only `b_cols` valid columns (a multiple of 8, row stride
// ldb >= b_cols); 16-byte chunks past them reload chunk 0 of the same row, so
// every load stays inside B and only the (discarded) padded output columns
// see duplicated values.  Used by the router, whose width E may be < 128.
//
// NT_B: B's loads carry the non-temporal hint (weights this tile streams
// once; see GemmSel).
template <int BM, int NB, int S, int MF = 32, bool CLAMP_B = false, bool NT_B = false>
struct Tile2 {
  static_assert(MF == 32, "32x32x16 MFMA tile");
  static constexpr int BN = kBN;
  static constexpr int BK = 64;
  static constexpr int WM = (BM >= 64) ? 2 : 1;
  static constexpr int WN = 4 / WM;
  static constexpr int WTM = BM / WM;
  static constexpr int WTN = BN / WN;
  static constexpr int FM = WTM / 32;
  static constexpr int FN = WTN / 32;
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
  using Frag = f32x16_t;
  static constexpr int FRAG = 16;                  // accumulator values per lane
  using Acc = Frag[NB][FM][FN];

  struct Args {
    const bf16_t* A;    // row 0 of the tile, K column 0
    int lda;
    int a_rows;         // valid rows (>= 1); later rows repeat the last one
    const bf16_t* B[NB];  // K row 0, column n0 of the tile
    int ldb;
    int K;              // multiple of 64
    int b_cols;         // CLAMP_B only: valid columns of B (multiple of 8)
    // row gather: tile row m is A row a_idx[m] (a_idx[m] * lda * 2 < 2^32
    // bytes); nullptr: row m is A row m
    const int* a_idx = nullptr;
  };

  // Per-lane constants of one tile run.
  struct Lane {
    uint32_t a_src[A_INST];   // A DMA source byte offsets (stage 0)
    uint32_t b_src[B_INST];   // B DMA source byte offsets (stage 0; every matrix)
    uint32_t a_rd[FM][4];     // A fragment LDS offsets in a stage, per K step
    uint32_t b_rd[FN];        // B fragment LDS offset in a stage (step, half, matrix: immediates)
    uint32_t a_dst, b_dst;    // this wave's first DMA destination in a stage (uniform)
  };

  struct Frags {
    bf16x8_t a[FM];
    bf16x8_t b[NB][FN];
  };

  static DEV void make_lane(const Args& g, int tid, Lane& L) {
    const int wave = tid >> 6, lane = tid & 63;
    // DMA sources.  A: rows 8i..8i+7, chunk c of row m at c ^ swz_a128(m).
#pragma unroll
    for (int ii = 0; ii < A_INST; ++ii) {
      const int i = wave * A_INST + ii;
      const int m = 8 * i + (lane >> 3);
      const int c = (lane & 7) ^ swz_a128(m);
      const int mr = m < g.a_rows ? m : g.a_rows - 1;
      const int sr = g.a_idx ? g.a_idx[mr] : mr;
      L.a_src[ii] = (uint32_t)sr * (uint32_t)g.lda * 2u + (uint32_t)c * 16u;
    }
    // B: K rows 4i..4i+3, chunk c of row k at c ^ swz_b(k).
#pragma unroll
    for (int ii = 0; ii < B_INST; ++ii) {
      const int i = wave * B_INST + ii;
      const int k = 4 * i + (lane >> 4);
      int c = (lane & 15) ^ swz_b(k);
      if constexpr (CLAMP_B) c = (c * 8 < g.b_cols) ? c : 0;
      L.b_src[ii] = (uint32_t)k * (uint32_t)g.ldb * 2u + (uint32_t)c * 16u;
    }
    L.a_dst = (uint32_t)(wave * A_INST) * 1024u;
    L.b_dst = (uint32_t)A_BYTES + (uint32_t)(wave * B_INST) * 1024u;
    // Fragment reads.  A lane: row lane%32, K 8*(lane/32)..+7 of the step.
    // B lane: column lane%32 via two transposing reads of 4 K rows each;
    // 16-lane group g covers columns 16*(g&1).., K rows 8*(g>>1)..
    const int wm = wave / WN, wn = wave % WN;
    const int l16 = lane & 15, lg = lane >> 4, l32 = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int m = wm * WTM + fm * 32 + l32;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int c = kk * 2 + lh;
        L.a_rd[fm][kk] = (uint32_t)(m * 128 + ((c ^ swz_a128(m)) << 4));
      }
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int n = wn * WTN + fn * 32 + 16 * (lg & 1) + 4 * (l16 & 3);
      const int kl = 8 * (lg >> 1) + (l16 >> 2);
      const int c = n >> 3, half = (n >> 2) & 1;
      L.b_rd[fn] = (uint32_t)(A_BYTES + kl * 256 + ((c ^ swz_b(kl)) << 4) + half * 8);
    }
  }

  static DEV void issue(const Lane& L, uint64_t a_base, const uint64_t* b_base, uint32_t stage) {
#pragma unroll
    for (int ii = 0; ii < A_INST; ++ii)
      dma16s(L.a_src[ii], a_base, __builtin_amdgcn_readfirstlane(stage + L.a_dst + ii * 1024));
#pragma unroll
    for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
      for (int ii = 0; ii < B_INST; ++ii) {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(stage + L.b_dst + mtx * B_BYTES + ii * 1024);
        if constexpr (NT_B) dma16s_nt(L.b_src[ii], b_base[mtx], dst);
        else dma16s(L.b_src[ii], b_base[mtx], dst);
      }
  }

  template <int KK>
  static DEV void load_frags(const Lane& L, uint32_t stage, Frags& f) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      f.a[fm] = *reinterpret_cast<const LDS_AS bf16x8_t*>((uintptr_t)(stage + L.a_rd[fm][KK]));
#pragma unroll
    for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const uint32_t b = stage + L.b_rd[fn] + mtx * B_BYTES + KK * 4096;
        const bf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t*)(uintptr_t)b);
        const bf16x4_t v1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t*)(uintptr_t)(b + 1024));
        f.b[mtx][fn] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
  }

  static DEV void mfmas(const Frags& f, Acc& acc) {
#pragma unroll
    for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[mtx][fm][fn] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[fm], f.b[mtx][fn], acc[mtx][fm][fn], 0, 0, 0);
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

  // Every wave's loads of the next stage have landed and every wave has
  // finished reading the stage the next DMA refills: LDS reads drained,
  // then a barrier, then a compiler fence so later LDS reads stay after it.
  static DEV void stage_barrier(int newer) {
    wait_stage(newer);
    __builtin_amdgcn_s_waitcnt((0x3f & 0xf) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // Full K loop; ends with a barrier so the caller may reuse `smem`.
  static DEV void run(const Args& g, char* smem, Acc& acc) {
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[m][fm][fn] = Frag{};
    Lane L;
    make_lane(g, opaque_tid(), L);
    const uint32_t base = lds_addr(smem);
    const uint64_t a0 = (uint64_t)(uintptr_t)g.A;
    uint64_t b0[NB];
#pragma unroll
    for (int m = 0; m < NB; ++m) b0[m] = (uint64_t)(uintptr_t)g.B[m];
    const uint64_t b_step = (uint64_t)BK * (uint64_t)g.ldb * 2u;
    const int nk = g.K / BK;
    auto issue_stage = [&](int kt, uint32_t stage) __attribute__((always_inline)) {
      uint64_t bb[NB];
#pragma unroll
      for (int m = 0; m < NB; ++m) bb[m] = b0[m] + (uint64_t)kt * b_step;
      issue(L, a0 + (uint64_t)kt * (BK * 2), bb, stage);
    };
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < nk) issue_stage(s, base + s * STAGE);
    stage_barrier(min(S - 2, nk - 1));
    Frags f0, f1;
    load_frags<0>(L, base, f0);
    uint32_t cur = base;                         // slot of stage kt
    uint32_t refill = base + (S - 1) * STAGE;    // slot of stage kt + S - 1
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + S - 1 < nk) issue_stage(kt + S - 1, refill);
      load_frags<1>(L, cur, f1);
      mfmas(f0, acc);
      load_frags<2>(L, cur, f0);
      mfmas(f1, acc);
      load_frags<3>(L, cur, f1);
      mfmas(f0, acc);
      const uint32_t next = (cur + STAGE == base + S * STAGE) ? base : cur + STAGE;
      if (kt + 1 < nk) {
        stage_barrier(min(S - 2, nk - 2 - kt));
        load_frags<0>(L, next, f0);
      }
      mfmas(f1, acc);
      refill = cur;
      cur = next;
    }
    __syncthreads();
  }

  // Visit every accumulator position: fn(row, col, fm, fn, i).  32x32
  // result: column lane%32, rows 8*(i/4) + 4*(lane/32) + i%4.
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
          const int row = wm * WTM + fm * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
          const int col = wn * WTN + fnn * 32 + (lane & 31);
          fn(row, col, fm, fnn, i);
        }
  }
};

}  // namespace moe
