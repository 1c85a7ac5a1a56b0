// tile3.hpp -- 256-row bf16 GEMM tile for gfx950 with global->LDS loads
// interleaved into the MFMA stream.
//
// C[256, 128] (x NB matrices sharing A) = A[256, K] * B[K, 128], bf16 in,
// fp32 accumulate, v_mfma_f32_32x32x16_bf16.  Four waves in a 2 x 2 grid;
// each wave owns 128 rows x 64 columns of every matrix (FM = 4, FN = 2), the
// shape that reads the fewest LDS bytes per MFMA with 256 accumulators.
//
// Why a second tile: with the loads of a K stage issued in one burst, a wave
// sits on its queued global_load_lds instructions while its matrix pipe
// idles (measured: the loads alone doubled the MFMA-only loop time).  Here a
// stage is 32 deep, the ring holds S = 4 stages (6 with one B matrix), and
// the loads are issued one at a time between the MFMAs, so the matrix pipe
// keeps running while the address unit drains them.  A slot is refilled as
// soon as the barrier that frees it has passed (half of the next stage's
// loads go out in the same iteration), so S - 2 whole stages are in flight
// whenever a wave waits: the deeper the ring of outstanding loads, the more
// memory latency the tile hides (measured: with every CU streaming from
// HBM, a tile's load latency grows with the device's total traffic).
// The loop body has no data-dependent branch: past the last stage the ring
// re-reads the last stage into the slot that is free anyway, so the
// outstanding-load count before each wait is a constant.
//
// Issue cost of the loads: a global_load_lds takes its LDS address from M0.
// Writing M0 before every load (and restoring it after) made each load cost
// about 27 issue cycles of the wave's MFMA stream, against about 8 with M0
// left alone.  So the LDS bytes one wave fills in a stage are one contiguous
// region, M0 is set once per stage to the middle of that region, and each
// load reaches its 1 KB slice through the instruction's signed 13-bit offset,
// which the hardware adds to both the global and the LDS address (the global
// side is pre-compensated in the per-lane offsets and the SGPR bases).
//
// LDS layout (one stage): four per-wave regions of LOADS KB; region w holds
//   A rows 64 w .. 64 w + 63 (64 bytes = 32 bf16 of K each), then for each B
//   matrix the K rows 8 w .. 8 w + 7 (256 bytes = 128 bf16 of N each).
//   16-byte chunk c of A row m sits at c ^ swz_a64(m): the sixteen rows one
//   16-lane phase of a fragment read touches fall on sixteen distinct
//   16-byte bank groups.  Chunk c of B row k sits at c ^ swz_b(k), read with
//   ds_read_b64_tr_b16 into the K-contiguous MFMA operand (as in tile2.hpp).
//   Every row starts at a multiple of 64 (A) or 256 (B) bytes, so the bank
//   pattern is that of a plain row-major stage.
#pragma once
#include "tile2.hpp"

namespace moe {

DEV uint64_t uniform_u64(uint64_t v) {
  return ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
}

// One 16-byte global->LDS load per lane from sbase + voff + OFF to the LDS
// address M0 + OFF (+ 16 * lane), M0 left as the caller set it.  Only the
// 256-row tile's K loop, which contains nothing else that reads or writes
// M0, issues these between its set_m0 and restore_m0.
template <int OFF>
DEV void dma16_m0(uint32_t voff, uint64_t sbase) {
  static_assert(OFF >= -4096 && OFF < 4096, "13-bit signed instruction offset");
  // sbase is wave-uniform by construction; re-asserting it keeps the
  // operand in SGPRs where the compiler's uniformity analysis loses track
  // (a no-op for a value already in SGPRs)
  asm volatile("global_load_lds_dwordx4 %0, %1 offset:%2" ::"v"(voff), "s"(uniform_u64(sbase)),
               "i"(OFF));
}

// The same load, first setting M0 = lds (wave-uniform).  s_nop 0 is the one
// wait state an SALU write of M0 needs before an LDS DMA reads it.
template <int OFF>
DEV void dma16_set_m0(uint32_t lds, uint32_t voff, uint64_t sbase) {
  static_assert(OFF >= -4096 && OFF < 4096, "13-bit signed instruction offset");
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%3" ::"s"(lds),
               "v"(voff), "s"(uniform_u64(sbase)), "i"(OFF));
}

DEV uint32_t save_m0() {
  uint32_t v;
  asm volatile("s_mov_b32 %0, m0" : "=s"(v));
  return v;
}
DEV void restore_m0(uint32_t v) { asm volatile("s_mov_b32 m0, %0" ::"s"(v)); }

template <int NB>
struct Tile3 {
  static constexpr int BM = 256;
  static constexpr int BN = kBN;
  static constexpr int BK = 32;
  static constexpr int WM = 2, WN = 2;
  static constexpr int WTM = 128, WTN = 64;
  static constexpr int FM = 4, FN = 2;
  static constexpr int A_BYTES = BM * 64;            // 16 KB
  static constexpr int B_BYTES = BK * 256;           // 8 KB per matrix
  static constexpr int STAGE = A_BYTES + NB * B_BYTES;
  static constexpr int S = (147456 / STAGE) > 6 ? 6 : (147456 / STAGE);
  static constexpr int LDS_BYTES = S * STAGE;
  static constexpr int A_INST = 4;                   // per wave per stage (1 KB each)
  static constexpr int B_INST = 2;                   // per wave per stage per matrix
  static constexpr int LOADS = A_INST + NB * B_INST;
  static constexpr int REG = LOADS * 1024;           // one wave's region of a stage
  static constexpr int M0_OFF = 4096;                // M0 = region + M0_OFF
  static_assert(4 * REG == STAGE && LOADS <= 8, "regions / offset range");
  static constexpr int MF_PER_KK = NB * FM * FN;     // MFMAs per 16-deep step
  // A stage's loads go out in two parts: loads 0 .. LOADS0 - 1 in the
  // second half of one iteration (right after the barrier that frees the
  // slot), the rest in the first half of the next.
  static constexpr int LOADS0 = (LOADS + 1) / 2;
  static constexpr int LOADS1 = LOADS - LOADS0;
  // loads still allowed in flight when stage kt + 1 must have landed: the
  // S - 2 stages after it
  static constexpr int NEWER = (S - 2) * LOADS;
  static_assert(S >= 3 && NEWER < 64, "ring depth / vmcnt range");
  static_assert(LOADS0 <= MF_PER_KK, "one load slot per MFMA");

  typedef float f32x16_t __attribute__((ext_vector_type(16)));
  using Frag = f32x16_t;
  static constexpr int FRAG = 16;
  using Acc = Frag[NB][FM][FN];

  struct Args {
    const bf16_t* A;    // row 0 of the tile, K column 0
    int lda;
    int a_rows;         // valid rows (>= 1); later rows repeat the last one
    const bf16_t* B[NB];
    int ldb;
    int K;              // multiple of 32
    // row gather: tile row m is A row a_idx[m] (a_idx[m] * lda * 2 < 2^32
    // bytes); nullptr: row m is A row m
    const int* a_idx = nullptr;
  };

  // Instruction offset of load j: its slice of the region, relative to M0.
  static constexpr int load_off(int j) { return j * 1024 - M0_OFF; }

  struct Lane {
    // per-lane global offsets, less the instruction offset of their load
    // and plus kBaseBias (the SGPR bases are lowered by it, keeping these
    // non-negative)
    uint32_t a_src[A_INST];
    uint32_t b_src[B_INST];
    uint32_t a_rd[FM][2];
    uint32_t b_rd[FN];
    uint32_t m0;             // wave-uniform: region + M0_OFF within a stage
  };
  static constexpr int kBaseBias = 8192;

  struct Frags {
    bf16x8_t a[FM];
    bf16x8_t b[NB][FN];
  };

  static DEV void make_lane(const Args& g, int tid, Lane& L) {
    const int wave = tid >> 6, lane = tid & 63;
    // A: instruction i covers rows 16 i .. 16 i + 15; lane -> row l / 4,
    // LDS chunk l % 4, which holds global chunk (l % 4) ^ swz_a64(m).
#pragma unroll
    for (int ii = 0; ii < A_INST; ++ii) {
      const int i = wave * A_INST + ii;
      const int m = 16 * i + (lane >> 2);
      const int c = (lane & 3) ^ swz_a64(m);
      const int mr = m < g.a_rows ? m : g.a_rows - 1;
      const int sr = g.a_idx ? g.a_idx[mr] : mr;
      L.a_src[ii] = (uint32_t)sr * (uint32_t)g.lda * 2u + (uint32_t)c * 16u +
                    (uint32_t)(kBaseBias - load_off(ii));
    }
    // B: instruction i covers K rows 4 i .. 4 i + 3.  The offset of matrix
    // mtx's loads beyond the first matrix's goes into its SGPR base.
#pragma unroll
    for (int ii = 0; ii < B_INST; ++ii) {
      const int i = wave * B_INST + ii;
      const int k = 4 * i + (lane >> 4);
      const int c = (lane & 15) ^ swz_b(k);
      L.b_src[ii] = (uint32_t)k * (uint32_t)g.ldb * 2u + (uint32_t)c * 16u +
                    (uint32_t)(kBaseBias - load_off(A_INST + ii));
    }
    L.m0 = __builtin_amdgcn_readfirstlane((uint32_t)(wave * REG + M0_OFF));
    const int wm = wave / WN, wn = wave % WN;
    const int l16 = lane & 15, lg = lane >> 4, l32 = lane & 31, lh = lane >> 5;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int m = wm * WTM + fm * 32 + l32;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int c = kk * 2 + lh;
        L.a_rd[fm][kk] = (uint32_t)((m >> 6) * REG + (m & 63) * 64 + ((c ^ swz_a64(m)) << 4));
      }
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int n = wn * WTN + fn * 32 + 16 * (lg & 1) + 4 * (l16 & 3);
      const int kl = 8 * (lg >> 1) + (l16 >> 2);
      const int c = n >> 3, half = (n >> 2) & 1;
      L.b_rd[fn] = (uint32_t)((kl >> 3) * REG + A_INST * 1024 + (kl & 7) * 256 +
                              ((c ^ swz_b(kl)) << 4) + half * 8);
    }
  }

  // Load J (0 <= J < LOADS) of a stage: A instructions first, then each B
  // matrix's; load J fills 1 KB slice J of the wave's region.  Load 0 sets
  // M0 for the stage (`stage` is the uniform LDS address of the ring slot);
  // the others rely on it.  a_base / b_base are the biased SGPR bases.
  template <int J>
  static DEV void issue_one(const Lane& L, uint64_t a_base, const uint64_t* b_base,
                            uint32_t stage) {
    if constexpr (J == 0) {
      dma16_set_m0<load_off(0)>(stage + L.m0, L.a_src[0], a_base);
    } else if constexpr (J < A_INST) {
      dma16_m0<load_off(J)>(L.a_src[J], a_base);
    } else {
      constexpr int mtx = (J - A_INST) / B_INST, ii = (J - A_INST) % B_INST;
      dma16_m0<load_off(J)>(L.b_src[ii], b_base[mtx]);
    }
  }

  template <int J0, int NJ>
  static DEV void issue_range(const Lane& L, uint64_t a_base, const uint64_t* b_base,
                              uint32_t stage) {
    if constexpr (NJ > 0) {
      issue_one<J0>(L, a_base, b_base, stage);
      issue_range<J0 + 1, NJ - 1>(L, a_base, b_base, stage);
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
        const uint32_t b = stage + L.b_rd[fn] + mtx * (B_INST * 1024) + KK * (2 * REG);
        const bf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t*)(uintptr_t)b);
        const bf16x4_t v1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t*)(uintptr_t)(b + 1024));
        f.b[mtx][fn] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
  }

  static DEV void mfma_one(const Frags& f, Acc& acc, int i) {
    const int mtx = i / (FM * FN), fm = (i / FN) % FM, fn = i % FN;
    acc[mtx][fm][fn] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[fm], f.b[mtx][fn], acc[mtx][fm][fn], 0, 0, 0);
  }

  static DEV void mfmas(const Frags& f, Acc& acc) {
#pragma unroll
    for (int i = 0; i < MF_PER_KK; ++i) mfma_one(f, acc, i);
  }

  // The MFMAs of one step with loads J0 .. J0 + NJ - 1 of a stage spread
  // evenly between them; sched_barrier keeps the compiler from regrouping
  // them.
  template <int J0, int NJ, int I = 0>
  static DEV void mfmas_with_loads(const Frags& f, Acc& acc, const Lane& L, uint64_t a_base,
                                   const uint64_t* b_base, uint32_t stage) {
    if constexpr (I < MF_PER_KK) {
      mfma_one(f, acc, I);
      // load j goes after MFMA j * MF_PER_KK / NJ
      constexpr int j = (I * NJ + MF_PER_KK - 1) / MF_PER_KK;
      if constexpr (j < NJ && j * MF_PER_KK / NJ == I) {
        __builtin_amdgcn_sched_barrier(0);
        issue_one<J0 + j>(L, a_base, b_base, stage);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfmas_with_loads<J0, NJ, I + 1>(f, acc, L, a_base, b_base, stage);
    }
  }

  // Stage kt + 1 has landed (later loads may still be in flight) and every
  // wave is done reading the slot the next loads refill.
  static DEV void stage_barrier() {
    wait_vmcnt<NEWER>();
    __builtin_amdgcn_s_waitcnt((0x3f & 0xf) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // Full K loop; ends with every load drained and a barrier, so the caller
  // may reuse `smem`.
  static DEV void run(const Args& g, char* smem, Acc& acc) {
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[m][fm][fn] = Frag{};
    Lane L;
    make_lane(g, opaque_tid(), L);
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(smem));
    // SGPR bases lowered by the bias the per-lane offsets carry (and, for
    // B matrix m, by its loads' extra instruction offset)
    const uint64_t a0 = uniform_u64((uint64_t)(uintptr_t)g.A) - (uint64_t)kBaseBias;
    uint64_t b0[NB];
#pragma unroll
    for (int m = 0; m < NB; ++m)
      b0[m] = uniform_u64((uint64_t)(uintptr_t)g.B[m]) - (uint64_t)(kBaseBias + m * B_INST * 1024);
    const uint32_t m0_saved = save_m0();
    const uint64_t b_step = (uint64_t)BK * (uint64_t)g.ldb * 2u;
    const int nk = g.K / BK;
    // stage kt's global bases (stages past the end re-read the last one)
    auto bases = [&](int kt, uint64_t& a, uint64_t* b) __attribute__((always_inline)) {
      const int kc = kt < nk ? kt : nk - 1;
      a = a0 + (uint64_t)kc * (BK * 2);
#pragma unroll
      for (int m = 0; m < NB; ++m) b[m] = b0[m] + (uint64_t)kc * b_step;
    };
    // prologue: stages 0 .. S - 2 whole, the first part of stage S - 1
#pragma unroll
    for (int s = 0; s < S - 1; ++s) {
      uint64_t a, b[NB];
      bases(s, a, b);
      issue_range<0, LOADS>(L, a, b, base + s * STAGE);
    }
    {
      uint64_t a, b[NB];
      bases(S - 1, a, b);
      issue_range<0, LOADS0>(L, a, b, base + (S - 1) * STAGE);
    }
    // stage 0 landed: the later prologue loads may be in flight
    wait_vmcnt<(S - 2) * LOADS + LOADS0>();
    __builtin_amdgcn_s_waitcnt((0x3f & 0xf) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    Frags f0, f1;
    load_frags<0>(L, base, f0);
    uint32_t cur = base;                          // slot of stage kt
    uint32_t fill = base + (S - 1) * STAGE;       // slot of stage kt + S - 1
    for (int kt = 0; kt < nk; ++kt) {
      uint64_t a, b[NB];
      // first half: the second part of stage kt + S - 1 (its slot's M0 is set)
      bases(kt + S - 1, a, b);
      load_frags<1>(L, cur, f1);
      mfmas_with_loads<LOADS0, LOADS1>(f0, acc, L, a, b, fill);
      const uint32_t next = (cur + STAGE == base + S * STAGE) ? base : cur + STAGE;
      stage_barrier();
      // stage kt's slot is free: the first part of stage kt + S goes there
      load_frags<0>(L, next, f0);
      __builtin_amdgcn_sched_barrier(0);
      bases(kt + S, a, b);
      mfmas_with_loads<0, LOADS0>(f1, acc, L, a, b, cur);
      fill = cur;
      cur = next;
    }
    wait_vmcnt<0>();
    restore_m0(m0_saved);
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
