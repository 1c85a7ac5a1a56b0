// tile.hpp -- one output tile of C[BM, 128] = A[BM, K] * B[K, 128] on gfx950.
//
// Used by every GEMM-shaped task: the router logits, the expert UP tiles
// (two B matrices -- gate and up -- sharing one A tile) and the DOWN tiles.
// The pages split each expert's GEMMs into row-block x column-block tasks so
// an idle CU can always find one (xxqk.cn/news/665650 section 2.2;
// m.xxqk.cn/news/657744 section 2.1); this is the body of such a task.
//
// Layout: A is row-major with K contiguous (token rows); B is row-major
// [K, N] with N contiguous (the weight layouts [d,f] and [f,d]).  bf16 MFMA
// wants K contiguous in both operands, so B rows are loaded 8 (k) x 4 (n) per
// thread and transposed in registers before they reach LDS.
//
// Workgroup = 4 wave64, arranged WM x WN over the tile; each wave owns a
// (BM/WM) x (128/WN) block of 16x16 accumulators.  K advances BK per stage;
// two LDS stages: global loads for stage k+1 are issued before the MFMAs of
// stage k and land in LDS after them.
#pragma once
#include "common.hpp"

namespace moe {

template <typename Elem, int BM, int NB>
struct Tile {
  using TR = ElemTraits<Elem>;
  static constexpr bool kBf16 = TR::kBf16;
  static constexpr int BN = kBN;
  static constexpr int BK = TR::kBK;
  static constexpr int WM = (BM >= 64) ? 2 : 1;
  static constexpr int WN = 4 / WM;
  static constexpr int WTM = BM / WM;
  static constexpr int WTN = BN / WN;
  static constexpr int FM = WTM / 16;
  static constexpr int FN = WTN / 16;
  static constexpr int KSTEP = kBf16 ? 32 : 4;   // K of one MFMA
  // LDS geometry, in elements.  Row padding keeps 16 consecutive rows of a
  // fragment read on distinct banks.
  static constexpr int A_LD = kBf16 ? BK + 8 : BK + 4;
  static constexpr int A_ELEMS = BM * A_LD;
  static constexpr int B_LD = kBf16 ? BK + 8 : BN + 4;   // bf16: [BN][BK] ; fp32: [BK][BN]
  static constexpr int B_ELEMS = kBf16 ? BN * B_LD : BK * B_LD;
  static constexpr int STAGE = A_ELEMS + NB * B_ELEMS;
  static constexpr int LDS_BYTES = 2 * STAGE * (int)sizeof(Elem);
  static constexpr int A_CHUNKS = BM * 8 / kThreads;     // 16-byte chunks / thread
  static constexpr int EPC = 16 / (int)sizeof(Elem);    // elements per chunk
  static_assert(BM == 32 || BM == 64 || BM == 128, "BM");
  static_assert(A_CHUNKS >= 1, "A chunks");

  using Acc = f32x4_t[NB][FM][FN];

  struct Args {
    const Elem* A;      // row 0 of the tile, column 0 of K
    int lda;
    int a_rows;         // valid rows (rest read as zero)
    const Elem* B[NB];  // row 0 of K, column n0 of the tile
    int ldb;
    int n_valid;        // valid columns in [0, 128)
    int K;              // multiple of BK
    // row gather: tile row m is A row a_idx[m]; nullptr: row m is A row m
    const int* a_idx = nullptr;
  };

  struct Regs {
    uint4 a[A_CHUNKS];
    // bf16: 8 rows x 4 columns per matrix (8-byte loads); fp32: 4 x 16 bytes
    uint2 b16[kBf16 ? NB : 1][kBf16 ? 8 : 1];
    uint4 b32[kBf16 ? 1 : NB][kBf16 ? 1 : 4];
  };

  static DEV void load(const Args& g, int kt, Regs& r) {
    const int tid = opaque_tid();
    const int k0 = kt * BK;
#pragma unroll
    for (int p = 0; p < A_CHUNKS; ++p) {
      const int row = (tid >> 3) + 32 * p;
      const int c = tid & 7;
      if (row < g.a_rows)
        r.a[p] = *reinterpret_cast<const uint4*>(g.A + (size_t)(g.a_idx ? g.a_idx[row] : row) * g.lda +
                                                 k0 + c * EPC);
      else
        r.a[p] = make_uint4(0, 0, 0, 0);
    }
    if constexpr (kBf16) {
      const int nq = tid & 31, kq = tid >> 5;
      const int n = nq * 4;
      const bool full = (n + 4 <= g.n_valid) && ((g.ldb & 3) == 0);
#pragma unroll
      for (int m = 0; m < NB; ++m) {
        const bf16_t* bp = reinterpret_cast<const bf16_t*>(g.B[m]) + (size_t)(k0 + kq * 8) * g.ldb + n;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (full) {
            r.b16[m][i] = *reinterpret_cast<const uint2*>(bp + (size_t)i * g.ldb);
          } else {
            uint32_t v[4];
#pragma unroll
            for (int c = 0; c < 4; ++c)
              v[c] = (n + c < g.n_valid) ? bp[(size_t)i * g.ldb + c] : 0u;
            r.b16[m][i] = make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
          }
        }
      }
    } else {
      const int c = tid & 31;
      const int n = c * 4;
      const bool full = (n + 4 <= g.n_valid) && ((g.ldb & 3) == 0);
#pragma unroll
      for (int m = 0; m < NB; ++m) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int row = (tid >> 5) + 8 * p;
          const float* bp = reinterpret_cast<const float*>(g.B[m]) + (size_t)(k0 + row) * g.ldb + n;
          if (full) {
            r.b32[m][p] = *reinterpret_cast<const uint4*>(bp);
          } else {
            uint32_t v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
              v[q] = (n + q < g.n_valid) ? __float_as_uint(bp[q]) : 0u;
            r.b32[m][p] = make_uint4(v[0], v[1], v[2], v[3]);
          }
        }
      }
    }
  }

  static DEV void store(const Regs& r, Elem* stage) {
    const int tid = opaque_tid();
#pragma unroll
    for (int p = 0; p < A_CHUNKS; ++p) {
      const int row = (tid >> 3) + 32 * p;
      const int c = tid & 7;
      *reinterpret_cast<uint4*>(stage + row * A_LD + c * EPC) = r.a[p];
    }
    if constexpr (kBf16) {
      const int nq = tid & 31, kq = tid >> 5;
#pragma unroll
      for (int m = 0; m < NB; ++m) {
        Elem* bs = stage + A_ELEMS + m * B_ELEMS;
        // 8 rows (k) x 4 columns (n) -> 4 columns of 8 consecutive k.
        uint32_t col[4][4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {          // pairs of rows 2h, 2h+1
          const uint2 lo = r.b16[m][2 * h], hi = r.b16[m][2 * h + 1];
          col[0][h] = (lo.x & 0xffffu) | (hi.x << 16);
          col[1][h] = (lo.x >> 16) | (hi.x & 0xffff0000u);
          col[2][h] = (lo.y & 0xffffu) | (hi.y << 16);
          col[3][h] = (lo.y >> 16) | (hi.y & 0xffff0000u);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *reinterpret_cast<uint4*>(bs + (nq * 4 + c) * B_LD + kq * 8) =
              make_uint4(col[c][0], col[c][1], col[c][2], col[c][3]);
      }
    } else {
      const int c = tid & 31;
#pragma unroll
      for (int m = 0; m < NB; ++m) {
        Elem* bs = stage + A_ELEMS + m * B_ELEMS;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int row = (tid >> 5) + 8 * p;
          *reinterpret_cast<uint4*>(bs + row * B_LD + c * 4) = r.b32[m][p];
        }
      }
    }
  }

  static DEV void compute(const Elem* stage, Acc& acc) {
    const int tid_ = opaque_tid();
    const int lane = tid_ & 63;
    const int wave = tid_ >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int l16 = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < BK / KSTEP; ++kk) {
      if constexpr (kBf16) {
        bf16x8_t a[FM];
        bf16x8_t b[NB][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          a[fm] = *reinterpret_cast<const bf16x8_t*>(
              stage + (wm * WTM + fm * 16 + l16) * A_LD + kk * 32 + lg * 8);
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            b[m][fn] = *reinterpret_cast<const bf16x8_t*>(
                stage + A_ELEMS + m * B_ELEMS + (wn * WTN + fn * 16 + l16) * B_LD + kk * 32 + lg * 8);
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
              acc[m][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fm], b[m][fn], acc[m][fm][fn], 0, 0, 0);
      } else {
        float a[FM];
        float b[NB][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          a[fm] = stage[(wm * WTM + fm * 16 + l16) * A_LD + kk * 4 + lg];
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            b[m][fn] = stage[A_ELEMS + m * B_ELEMS + (kk * 4 + lg) * B_LD + wn * WTN + fn * 16 + l16];
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
              acc[m][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[fm], b[m][fn], acc[m][fm][fn], 0, 0, 0);
      }
    }
  }

  // Full K loop.  `smem` holds 2 stages (LDS_BYTES).  Ends with a barrier,
  // so the caller may reuse `smem` right away.
  static DEV void run(const Args& g, Elem* smem, Acc& acc) {
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[m][fm][fn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nk = g.K / BK;
    Regs r;
    load(g, 0, r);
    store(r, smem);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      Elem* cur = smem + (kt & 1) * STAGE;
      Elem* nxt = smem + ((kt + 1) & 1) * STAGE;
      if (kt + 1 < nk) load(g, kt + 1, r);
      compute(cur, acc);
      if (kt + 1 < nk) store(r, nxt);
      __syncthreads();
    }
  }

  // Visit every accumulator position: fn(row, col, fm, fn, i) with row in
  // [0,BM), col in [0,128); the value of matrix m is acc[m][fm][fn][i].
  // 16x16 MFMA result layout: a lane holds column lane%16 and rows
  // 4*(lane/16) .. +3 of its fragment.
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
        for (int i = 0; i < 4; ++i) {
          const int row = wm * WTM + fm * 16 + (lane >> 4) * 4 + i;
          const int col = wn * WTN + fnn * 16 + (lane & 15);
          fn(row, col, fm, fnn, i);
        }
  }
};

}  // namespace moe
