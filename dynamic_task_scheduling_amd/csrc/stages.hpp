// stages.hpp -- bodies of the MoE-layer tasks.  Every scheduling mode
// (persistent dynamic, persistent static, one launch per stage) runs exactly
// these functions; only who runs them, and when, differs -- the control the
// pages insist on when comparing schedulers (xxqk.cn/news/665650 s3.1: change
// only the scheduling policy, never the operators).
//
// Each function is called by all 256 threads of a workgroup and returns with
// the workgroup converged.  None of them publishes its results: the caller
// owns fences and dependency counters.
#pragma once
#include "common.hpp"
#include "params.hpp"
#include "tile.hpp"
#include "tile2.hpp"
#include "tile3.hpp"

namespace moe {

// Task bodies are compiled as separate functions: one persistent kernel
// holds every task type, and keeping them apart keeps register allocation
// per task type instead of over their union.
#define TASKFN DEV

// Order-preserving 32-bit image of an fp32 value (+0.0 and -0.0 map to the
// same key, so they compare equal).
DEV uint32_t mono_key(float v) {
  uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
DEV float mono_value(uint32_t m) {
  return __uint_as_float((m & 0x80000000u) ? (m & 0x7fffffffu) : ~m);
}

// The error code passes through an empty asm so that the compare-and-swap
// operands are formed where the error is raised, not once before the
// persistent loop (where they would occupy registers across every task).
DEV void set_error(const Params& p, int code) {
  asm volatile("" : "+v"(code));
  cas_relaxed(p.ctrl + CW_ERROR * kCtrlStride, 0, code);
}

// Thread 0 appends one trace record for a scheduler phase (see trace_mark).
DEV void trace_step(const Params& p, int phase, int worker, uint64_t t0, uint64_t t1) {
  if (p.trace == nullptr || tidx() != 0) return;
  asm volatile("" : "+s"(phase));
  const int i = add_relaxed(p.ctrl + CW_TRACE * kCtrlStride, 1);
  if (i < p.trace_cap) {
    uint64_t* r = p.trace + (size_t)i * 4;
    r[0] = t0;
    r[1] = t0;
    r[2] = t1;
    r[3] = (uint64_t)(uint32_t)make_task(TK_BUILD, phase) | ((uint64_t)(worker & 0xffff) << 32) |
           ((uint64_t)xcc_id() << 48);
  }
}

// Slices of the DOWN split-K: slice ks covers UP column tiles
// [ks*n/s, (ks+1)*n/s).
DEV int slice_lo(int ks, int n, int s) { return ks * n / s; }
DEV int slice_of(int tile, int n, int s) {
  int ks = 0;
  while (ks + 1 < s && slice_lo(ks + 1, n, s) <= tile) ++ks;
  return ks;
}

// GEMM tile used for expert tasks: bf16 runs the multi-stage LDS ring
// (tile2.hpp); fp32 runs the register-staged tile (tile.hpp).
// Ring depth: as many 64-deep K stages as fit in 144 KB of LDS (bytes in
// flight set a streaming task's rate), at most 7.
constexpr int tile2_stages(int bm, int nb) {
  return (147456 / (bm * 128 + nb * 16384)) > 7 ? 7 : (147456 / (bm * 128 + nb * 16384));
}
template <typename Elem, int BM, int NB>
struct GemmSel {
  using T = Tile<Elem, BM, NB>;
};
// Row tiles of at most 64 rows stream their weight panels (non-temporal
// loads): they are mostly the single tiles of lightly loaded experts, whose
// panels no other tile reads, and the hint keeps those streams from
// displacing the panels and rows that the larger tiles reuse.
template <int BM, int NB>
struct GemmSel<bf16_t, BM, NB> {
  using T = Tile2<BM, NB, tile2_stages(BM, NB), 32, false, (BM <= 64)>;
};
// 256-row tiles: 32-deep stages with the loads interleaved into the MFMAs
template <int NB>
struct GemmSel<bf16_t, 256, NB> {
  using T = Tile3<NB>;
};

// Router tiles (32 tokens x 128 experts): a 4-stage ring for bf16 when the
// router width is a multiple of 8 (columns past E are padding), so the router
// scratch fits beside it.
template <typename Elem>
struct RouteSel {
  using T = Tile<Elem, 32, 1>;
};
template <>
struct RouteSel<bf16_t> {
  using T = Tile2<32, 1, 4, 32, true>;   // E may be narrower than 128
};

template <typename T>
struct requires_n_valid {
  static constexpr bool value = false;
};
template <typename Elem, int BM, int NB>
struct requires_n_valid<Tile<Elem, BM, NB>> {
  static constexpr bool value = true;
};

template <typename Elem>
struct Stages {
  using TR = ElemTraits<Elem>;
  static constexpr int cmax(int a, int b) { return a > b ? a : b; }
  // LDS of the largest expert tile over every row class and B count
  static constexpr int kSmemTile =
      cmax(cmax(cmax(GemmSel<Elem, 32, 1>::T::LDS_BYTES, GemmSel<Elem, 64, 1>::T::LDS_BYTES),
                cmax(GemmSel<Elem, 128, 1>::T::LDS_BYTES, GemmSel<Elem, 32, 2>::T::LDS_BYTES)),
           cmax(GemmSel<Elem, 64, 2>::T::LDS_BYTES, GemmSel<Elem, 128, 2>::T::LDS_BYTES));
  // Router scratch after the router tile's own two stages.
  static constexpr int kRouteTile =
      Tile<Elem, 32, 1>::LDS_BYTES > RouteSel<Elem>::T::LDS_BYTES
          ? Tile<Elem, 32, 1>::LDS_BYTES
          : RouteSel<Elem>::T::LDS_BYTES;
  static constexpr int kSmem = kSmemTile;
  // Router LDS: the tile ring, then logits [32][E], histogram [E], bias [E].
  static constexpr int kRouteSmem = kRouteTile + 32 * kMaxE * 4 + 2 * kMaxE * 4;
  static_assert(kRouteSmem <= kSmemTile, "route LDS");
  // build(): its tables; position(): its per-expert tables
  static constexpr int kBuildSmem = 16384;
  static constexpr int kPosSmem = (7 * kMaxE + 4) * 4;
  static_assert(kPosSmem <= kBuildSmem, "position LDS");
  static_assert(kBuildSmem <= kSmemTile, "build LDS");

  // --------------------------------------------------------------- router
  // Top-k with renormalised softmax for `rows` (<= 32) tokens starting at t0,
  // whose fp32 logits sit at L[row * ldl + e] (LDS or global).
  //
  // Token-parallel: a wave takes 8 tokens, 8 lanes per token.  Lane g of a
  // token keeps, in registers, the 8 largest keys among experts g, g+8,
  // g+16, ... (an insertion network, so every lane works on its own token at
  // once); then k merge rounds each take the largest head among the token's
  // 8 lanes (three DPP steps inside the 8-lane group) and pop it.  Selection
  // key = (order-preserving logit image, inverted index): the maximum is the
  // largest logit and, among equal logits, the lowest index.  Round j's
  // winner is kept by lane j of the group, so the weights, the table stores
  // and the histogram update are one instruction per wave.
  static DEV uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
  template <int CTRL>
  static DEV uint64_t dpp_u64(uint64_t x) {
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(x >> 32), CTRL, 0xf, 0xf, false);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, 0xf, 0xf, false);
    return ((uint64_t)hi << 32) | lo;
  }
  template <int CTRL>
  static DEV float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
  }
  // 0xb1: quad_perm [1,0,3,2]; 0x4e: quad_perm [2,3,0,1]; 0x141: row_half_mirror
  // (lane i <-> 7-i inside each 8-lane half row).  Together: every lane of an
  // aligned 8-lane group sees the whole group.
  static DEV uint64_t group8_max(uint64_t x) {
    x = max_u64(x, dpp_u64<0xb1>(x));
    x = max_u64(x, dpp_u64<0x4e>(x));
    return max_u64(x, dpp_u64<0x141>(x));
  }
  static DEV float group8_sum(float x) {
    x += dpp_f32<0xb1>(x);
    x += dpp_f32<0x4e>(x);
    return x + dpp_f32<0x141>(x);
  }

  static DEV void topk(const Params& p, int t0, int rows, const float* L, int ldl,
                       int* hist_s) {
    static_assert(kTB == 32 && kThreads == 256 && kMaxK <= 8, "8 lanes per token");
    const int tid = tidx();
    const int g = tid & 7;                  // lane within the token's group
    const int r = tid >> 3;                 // token row in the tile (0..31)
    const int E = p.E, k = p.k;
    const bool live = r < rows;
    // 1. per lane: the 8 largest keys of its experts, sorted descending
    uint64_t s0 = 0, s1 = 0, s2 = 0, s3 = 0, s4 = 0, s5 = 0, s6 = 0, s7 = 0;
    bool bad = false;
    if (live) {
      for (int e = g; e < E; e += 8) {
        const float v = L[r * ldl + e];
        if (!__builtin_isfinite(v)) bad = true;
        const uint32_t m = __builtin_isfinite(v) ? mono_key(v) : 1u;
        uint64_t x = ((uint64_t)m << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
        auto cs = [&](uint64_t& s) __attribute__((always_inline)) {
          const uint64_t hi = max_u64(s, x);
          x = (s > x) ? x : s;
          s = hi;
        };
        cs(s0); cs(s1); cs(s2); cs(s3); cs(s4); cs(s5); cs(s6); cs(s7);
      }
    }
    if (__any(bad) && (tid & 63) == 0) set_error(p, 7 /* MOE_ERR_NONFINITE */);
    // 2. k merge rounds over the group's heads
    uint64_t mine = 0;       // winner of round g (lanes g < k)
    uint64_t first = 0;      // winner of round 0 (largest logit)
    for (int j = 0; j < k; ++j) {
      const uint64_t w = group8_max(s0);
      if (j == 0) first = w;
      if (g == j) mine = w;
      if (s0 == w) {         // keys are unique: exactly one lane pops
        s0 = s1; s1 = s2; s2 = s3; s3 = s4; s4 = s5; s5 = s6; s6 = s7; s7 = 0;
      }
    }
    // 3. w_j = exp(L_j - L_0) / sum_j' exp(L_j' - L_0)
    const int my_e = (int)(0xffffffffu - (uint32_t)mine);
    const float my_v = mono_value((uint32_t)(mine >> 32));
    const float v0 = mono_value((uint32_t)(first >> 32));
    const float a = (g < k) ? expf(my_v - v0) : 0.f;
    const float s = group8_sum(a);
    if (live && g < k) {
      const int t = t0 + r;
      st_wt(p.idx + (size_t)t * k + g, my_e);
      st_wt(p.w + (size_t)t * k + g, a / s);
      const int el = my_e - p.e_begin;
      if (el >= 0 && el < p.E_loc) atomicAdd(&hist_s[el], 1);
    }
  }

  static DEV void write_hist(const Params& p, int rt, const int* hist_s) {
    for (int e = tidx(); e < p.E_loc; e += kThreads)
      st_wt(p.hist + (size_t)e * p.hist_ld + rt, hist_s[e]);
  }

  // ROUTE(rt, ks): router logits of tokens [32 rt, 32 rt + 32) over K slice
  // ks of rsk.  With rsk == 1 the task also adds the bias, picks the top-k
  // and writes the tile histogram; with rsk > 1 it writes an fp32 partial
  // and the last slice to finish runs route_finish (fixed-order sum, so the
  // logits do not depend on which slice finished last).
  template <typename RT>
  static DEV void route_gemm(const Params& p, int t0, int rows, int k0, int K, float* Ls,
                             float* part, char* smem) {
    const Elem* x = reinterpret_cast<const Elem*>(p.x) + (size_t)t0 * p.d + k0;
    const Elem* wr = reinterpret_cast<const Elem*>(p.wr) + (size_t)k0 * p.E;
    for (int n0 = 0; n0 < p.E; n0 += kBN) {
      typename RT::Args g;
      g.A = x;
      g.lda = p.d;
      g.a_rows = rows;
      g.B[0] = wr + n0;
      g.ldb = p.E;
      if constexpr (requires_n_valid<RT>::value) g.n_valid = min(kBN, p.E - n0);
      else g.b_cols = min(kBN, p.E - n0);
      g.K = K;
      typename RT::Acc acc;
      if constexpr (requires_n_valid<RT>::value) RT::run(g, reinterpret_cast<Elem*>(smem), acc);
      else RT::run(g, smem, acc);
      RT::for_each([&](int row, int col, int fm, int fn, int i) __attribute__((always_inline)) {
        const int e = n0 + col;
        if (e < p.E) {
          const float v = acc[0][fm][fn][i];
          if (part) {
            if (row < rows) st_wt(part + row * p.E + e, v);
          } else {
            Ls[row * p.E + e] = v;
          }
        }
      });
    }
  }

  // Router partials: slice ks of tile rt is a contiguous [32][E] fp32 block
  // at ((rt * rsk + ks) * 32) * E, so one tile's slices form one contiguous
  // range that route_finish pulls into LDS with a single burst of loads.
  static DEV float* route_part_block(const Params& p, int rt, int ks) {
    return p.route_part + ((size_t)rt * p.rsk + ks) * kTB * p.E;
  }

  // Scatter-add combine: router slice ks zeroes its share (rows ks, ks +
  // rsk, ...) of the y rows of its tokens [t0, t0 + rows), which the DOWN
  // tiles then accumulate into (with a fused residual the rows start from
  // the residual instead).
  static DEV void zero_y_rows(const Params& p, int t0, int rows, int ks) {
    for (int r = ks; r < rows; r += p.rsk) {
      float* yr = p.y + (size_t)(t0 + r) * p.d;
      const uint4* rr = p.resid ? reinterpret_cast<const uint4*>(p.resid + (size_t)(t0 + r) * p.d)
                                : nullptr;
      for (int i = tidx(); i < p.d / 4; i += kThreads)
        st_wt16(yr, i * 16, rr ? rr[i] : make_uint4(0, 0, 0, 0));
    }
  }

  static TASKFN void route(const Params& p, int rt, int ks, char* smem, bool scat) {
    const int t0 = rt * kTB;
    const int rows = min(kTB, p.T - t0);
    // the bias load is issued first, so its latency hides under the GEMM
    const float bias_v = (p.rsk == 1 && p.bias && tidx() < p.E) ? p.bias[tidx()] : 0.f;
    if (scat) zero_y_rows(p, t0, rows, ks);
    const int Ks = p.d / p.rsk;
    float* Ls = reinterpret_cast<float*>(smem + kRouteTile);     // [32][E]
    float* part = p.rsk > 1 ? route_part_block(p, rt, ks) : nullptr;
    if (ElemTraits<Elem>::kBf16 && (p.E % 8) == 0)
      route_gemm<typename RouteSel<Elem>::T>(p, t0, rows, ks * Ks, Ks, Ls, part, smem);
    else
      route_gemm<Tile<Elem, 32, 1>>(p, t0, rows, ks * Ks, Ks, Ls, part, smem);
    if (p.rsk == 1) {
      float* bias_s = reinterpret_cast<float*>(smem + kRouteTile + 32 * kMaxE * 4 + kMaxE * 4);
      if (tidx() < p.E) bias_s[tidx()] = bias_v;
      route_topk(p, rt, smem);
    }
  }

  // Sum the K-slice partials of tile rt (contiguous [rsk][32][E] blocks) in
  // slice order, then top-k.
  static TASKFN void route_finish(const Params& p, int rt, char* smem) {
    route_sum_topk(p, rt, route_part_block(p, rt, 0), (size_t)kTB * p.E, smem);
  }

  // ROUTE(g, ks) with 256-token router groups (bf16, E = 128 or 256): the
  // router logits of tokens [256 g, 256 g + 256) over K slice ks of rsk, on
  // the 256-row tile the expert GEMMs use, stored as the fp32 partial
  // route_part[ks][t][e].  A 32-token router task streams the whole of W_r
  // (d x E) for 32 tokens; a group task streams its K slice of W_r once for
  // 256 tokens, an eighth of the router's W_r traffic.  The TK_RFIN tasks of
  // the group's eight 32-token tiles then sum the slices and route.
  static TASKFN void route_wide(const Params& p, int g, int ks, char* smem, bool scat) {
    const int t0 = g * 256;
    const int rows = min(256, p.T - t0);
    if (scat) zero_y_rows(p, t0, rows, ks);
    if constexpr (TR::kBf16) {
      const int Ks = p.d / p.rsk;
      const Elem* x = reinterpret_cast<const Elem*>(p.x) + (size_t)t0 * p.d + (size_t)ks * Ks;
      const Elem* wr = reinterpret_cast<const Elem*>(p.wr) + (size_t)ks * Ks * p.E;
      float* out = p.route_part + ((size_t)ks * p.T + t0) * p.E;
      if (p.E == 256) down_tile<256, 2>(x, p.d, rows, wr, p.E, Ks, out, p.E, smem);
      else down_tile<256, 1>(x, p.d, rows, wr, p.E, Ks, out, p.E, smem);
    }
  }

  // RFIN(rt): logits of tokens [32 rt, 32 rt + 32) = the group's K-slice
  // partials summed in slice order (so the logits do not depend on which
  // slice finished last), then bias and top-k; route_finish does the same
  // for the 32-token router's partials.
  static constexpr int kMaxRouteSlicesWide = 8;
  static TASKFN void route_finish_wide(const Params& p, int rt, char* smem) {
    route_sum_topk(p, rt, p.route_part + (size_t)rt * kTB * p.E, (size_t)p.T * p.E, smem);
  }
  // Burst size of the LDS-staged summation (over the idle router-tile ring,
  // below Ls).
  static constexpr int kSumBurst = kRouteTile < 65536 ? kRouteTile : 65536;
  // Tile rt's logits = sum over ks of the [rows][E] fp32 partial at
  // part0 + ks * stride (floats), in slice order; then bias and top-k.
  // When all slices of the tile fit kSumBurst bytes they are staged in LDS
  // by one burst of direct loads.  Otherwise each thread owns IT float4 items of the tile and reads SL = 16 / IT
  // slices of them per pass, so 16 loads are in flight per thread whatever
  // the router width (IT = 8, 4, 2, 1 for E up to 256, 128, 64, 32).  The
  // loads are unconditional (items past the tile re-read its last item and
  // are never stored): loads under a per-lane condition were each given a
  // wait of their own by the compiler, one memory round trip per load.
  static DEV void route_sum_topk(const Params& p, int rt, const float* part0, size_t stride,
                                 char* smem) {
    const int t0 = rt * kTB;
    const int rows = min(kTB, p.T - t0);
    float* Ls = reinterpret_cast<float*>(smem + kRouteTile);
    float* bias_s = reinterpret_cast<float*>(smem + kRouteTile + 32 * kMaxE * 4 + kMaxE * 4);
    const float bias_v = (p.bias && tidx() < p.E) ? p.bias[tidx()] : 0.f;
    const int tid = tidx();
    const int sb = rows * p.E * 4;                     // bytes of one slice
    const int sreg = (sb + 1023) & ~1023;              // its LDS region: whole 1 KB loads
    if (sreg * p.rsk <= kSumBurst) {
      // every slice of the tile fits one burst of direct global->LDS loads
      // (a single memory round trip; small router widths): stage them over
      // the idle router-tile ring, then add them in slice order.  Lanes past
      // a slice re-load its first bytes into the region's padding.
      const int wave = tid >> 6, lane = tid & 63;
      const int ninst = sreg / 1024;
      for (int j = wave; j < p.rsk * ninst; j += kThreads / 64) {
        const int sl = j / ninst, q = j % ninst;
        int off = q * 1024 + lane * 16;
        if (off >= sb) off = 0;
        dma16(reinterpret_cast<const char*>(part0 + (size_t)sl * stride) + off,
              __builtin_amdgcn_readfirstlane(lds_addr(smem + sl * sreg + q * 1024)));
      }
      wait_vmcnt<0>();
      __syncthreads();
      const float* st = reinterpret_cast<const float*>(smem);
      for (int i = tid; i < rows * p.E; i += kThreads) {
        float v = 0.f;
        for (int ks = 0; ks < p.rsk; ++ks) v += st[ks * (sreg / 4) + i];
        Ls[i] = v;
      }
    } else if (p.E % 4 != 0) {
      // router widths that are not a multiple of 4: one float per item
      const int n = rows * p.E;
      for (int i = tid; i < n; i += kThreads) {
        float a = 0.f;
        for (int ks = 0; ks < p.rsk; ++ks) a += part0[ks * stride + i];
        Ls[i] = a;
      }
    } else if (p.E > 128) {
      sum_slices<8>(p, rows, part0, stride, Ls);
    } else if (p.E > 64) {
      sum_slices<4>(p, rows, part0, stride, Ls);
    } else if (p.E > 32) {
      sum_slices<2>(p, rows, part0, stride, Ls);
    } else {
      sum_slices<1>(p, rows, part0, stride, Ls);
    }
    if (tid < p.E) bias_s[tid] = bias_v;
    __syncthreads();
    route_topk(p, rt, smem);
  }
  template <int IT>
  static DEV void sum_slices(const Params& p, int rows, const float* part0, size_t stride,
                             float* Ls) {
    constexpr int SL = 16 / IT;
    const int n4 = rows * p.E / 4;                     // <= IT * kThreads
    const size_t slice4 = stride / 4;
    const float4* src = reinterpret_cast<const float4*>(part0);
    const int tid = tidx();
    int item[IT];
    float4 acc[IT];
#pragma unroll
    for (int j = 0; j < IT; ++j) {
      item[j] = min(tid + j * kThreads, n4 - 1);
      acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int ks = 0; ks < p.rsk; ks += SL) {
      float4 v[SL][IT];
#pragma unroll
      for (int s = 0; s < SL; ++s)
#pragma unroll
        for (int j = 0; j < IT; ++j)   // slices past rsk re-read the last one (not added)
          v[s][j] = src[(size_t)min(ks + s, p.rsk - 1) * slice4 + item[j]];
#pragma unroll
      for (int s = 0; s < SL; ++s) {
        if (ks + s < p.rsk) {
#pragma unroll
          for (int j = 0; j < IT; ++j) {
            acc[j].x += v[s][j].x; acc[j].y += v[s][j].y;
            acc[j].z += v[s][j].z; acc[j].w += v[s][j].w;
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < IT; ++j) {
      const int i = tid + j * kThreads;
      if (i < n4) *reinterpret_cast<float4*>(Ls + 4 * i) = acc[j];
    }
  }

  // Bias, exported logits, top-k and the tile histogram from Ls (the bias
  // already staged in LDS).
  static DEV void route_topk(const Params& p, int rt, char* smem) {
    const int t0 = rt * kTB;
    const int rows = min(kTB, p.T - t0);
    float* Ls = reinterpret_cast<float*>(smem + kRouteTile);
    int* hist_s = reinterpret_cast<int*>(smem + kRouteTile + 32 * kMaxE * 4);
    const float* bias_s = reinterpret_cast<const float*>(hist_s + kMaxE);
    for (int e = tidx(); e < p.E_loc; e += kThreads) hist_s[e] = 0;
    __syncthreads();
    // element i = r * E + c; the thread's column advances by 256 mod E per
    // pass (no integer division per element)
    {
      const int E = p.E;
      const int step = kThreads % E;
      int c = tidx() % E;
      for (int i = tidx(); i < rows * E; i += kThreads) {
        const float v = Ls[i] + bias_s[c];
        Ls[i] = v;
        p.logits[(size_t)t0 * E + i] = v;
        c += step;
        if (c >= E) c -= E;
      }
    }
    __syncthreads();
    topk(p, t0, rows, Ls, p.E, hist_s);
    __syncthreads();
    write_hist(p, rt, hist_s);
  }

  // Routing from given logits (checking path): top-k + histogram only.
  static TASKFN void topk_from_logits(const Params& p, int rt, char* smem) {
    const int t0 = rt * kTB;
    const int rows = min(kTB, p.T - t0);
    int* hist_s = reinterpret_cast<int*>(smem);
    for (int e = tidx(); e < p.E_loc; e += kThreads) hist_s[e] = 0;
    __syncthreads();
    topk(p, t0, rows, p.logits + (size_t)t0 * p.E, p.E, hist_s);
    __syncthreads();
    write_hist(p, rt, hist_s);
  }

  // ---------------------------------------------------------------- build
  // Workgroup-wide exclusive prefix sum of one int per thread; returns the
  // thread's exclusive prefix, *total receives the sum.  s_w: 4 ints of LDS.
  static DEV int block_exscan(int v, int* s_w, int* total) {
    const int lane = tidx() & 63, wave = tidx() >> 6;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = wave_up(inc, o);
      if (lane >= o) inc += u;
    }
    if (lane == 63) s_w[wave] = inc;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int s = s_w[w];
      base += (w < wave) ? s : 0;
      tot += s;
    }
    __syncthreads();
    *total = tot;
    return base + inc - v;
  }

  // Workgroup-wide float sum in a fixed order (deterministic).
  static DEV float block_sum(float v, float* s_w) {
    const int lane = tidx() & 63, wave = tidx() >> 6;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += wave_xor(v, o);
    if (lane == 0) s_w[wave] = v;
    __syncthreads();
    const float t = (s_w[0] + s_w[1]) + (s_w[2] + s_w[3]);
    __syncthreads();
    return t;
  }

  // Runs once, after every ROUTE tile: counts, offsets, per-tile position
  // bases, expert order (most loaded first), the row-tile table, dependency
  // counters, the permute list and -- the cost model -- the worker split.
  // The pages run this "once routing completes", when every layer's
  // communication and computation volumes are known (Weave abstract).
  // Global memory costs about a microsecond per round trip, so every step
  // issues its loads together and spreads its stores over all threads; the
  // scans and reductions run in LDS and registers.
  // Writes tables and control words (not yet published).
  static TASKFN void build(const Params& p, char* smem, int worker = 0) {
    uint64_t t_step = rtc();
    auto mark = [&](int step) __attribute__((always_inline)) {
      if (p.flags & 0x2 /* trace */) {
        const uint64_t t = rtc();
        trace_step(p, kPhaseBuildStep + step, worker, t_step, t);
        t_step = t;
      }
    };
    int* s_cnt = reinterpret_cast<int*>(smem);            // [256] count of expert e
    int* s_off = s_cnt + 256;                             // [257] offset of expert e
    int* s_ord = s_off + 257;                             // [256] expert of rank r
    int* s_bt = s_ord + 256;                    // [kMaxBands][257] tile base of (band, rank)
    int* s_bp = s_bt + kMaxBands * 257;         // [kMaxBands][257] permute base of (band, rank)
    int* s_w = s_bp + kMaxBands * 257;          // [8] scan / reduction scratch
    float* s_wf = reinterpret_cast<float*>(s_w + 4);
    const int tid = tidx();
    const int El = p.E_loc;
    // 1. per-expert counts: the row sums of the [El][n_rt] tile histogram,
    //    tpe consecutive threads per expert, every load of a thread issued
    //    before any is used (a memory round trip or two in all).  The
    //    per-tile bases inside an expert's segment are prefix sums of the
    //    same rows, which each position task takes for its own tile.
    int run = 0;
    {
      int tpe = 64;
      while (tpe > 1 && tpe * El > kThreads) tpe >>= 1;
      const int e = tid / tpe, sub = tid % tpe;
      const int nq = (p.n_rt + 3) / 4;                   // int4 per row (hist_ld % 4 == 0)
      int sum = 0;
      if (e < El) {
        const int4* row = reinterpret_cast<const int4*>(p.hist + (size_t)e * p.hist_ld);
        for (int q0 = sub; q0 < nq; q0 += 16 * tpe) {
          int4 v[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int q = q0 + u * tpe;
            if (q < nq) v[u] = row[q];
          }
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int q = q0 + u * tpe, r = 4 * q;
            if (q < nq)    // columns past n_rt are padding and never written
              sum += v[u].x + (r + 1 < p.n_rt ? v[u].y : 0) + (r + 2 < p.n_rt ? v[u].z : 0) +
                     (r + 3 < p.n_rt ? v[u].w : 0);
          }
        }
      }
      for (int o = 1; o < tpe; o <<= 1) sum += wave_xor_i(sum, o);
      if (e < El && sub == 0) s_cnt[e] = sum;
      __syncthreads();
      if (tid < El) run = s_cnt[tid];
      __syncthreads();
    }
    // 2. offsets (exclusive scan) and expert order by descending count
    if (tid < El) s_cnt[tid] = run;
    else if (tid < ((El + 7) & ~7)) s_cnt[tid] = -1;   // padding: never outranks an expert
    int total = 0;
    const int off = block_exscan(tid < El ? run : 0, s_w, &total);
    if (tid < El) {
      s_off[tid] = off;
      st_wt(p.counts + tid, run);
      st_wt(p.offsets + tid, off);
    }
    if (tid == 0) {
      s_off[El] = total;
      st_wt(p.offsets + El, total);
    }
    __syncthreads();
    if (tid < El) {
      const int c = run;
      int rank = 0;
      // eight counts per pass (two 16-byte LDS reads, the same address in
      // every lane); the padding up to a multiple of 8 holds -1
      for (int e0 = 0; e0 < El; e0 += 8) {
        const int4 a = *reinterpret_cast<const int4*>(s_cnt + e0);
        const int4 b = *reinterpret_cast<const int4*>(s_cnt + e0 + 4);
        const int ce[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int u = 0; u < 8; ++u) rank += (ce[u] > c) || (ce[u] == c && e0 + u < tid);
      }
      s_ord[rank] = tid;
      st_wt(p.eorder + rank, tid);
    }
    __syncthreads();
    mark(1);
    // 3. row tiles (th = 128 or 256 rows; the last one of an expert takes
    //    the smallest class that holds it) and permute chunks, then the
    //    table, filled by every thread in parallel (one tile per thread per
    //    pass).  Tile order (the temporal schedule of the expert work): the
    //    tiles are dealt into `bands` token bands -- tile m of an expert with
    //    nt tiles goes to band b = the b with lo(nt, b) <= m < lo(nt, b + 1),
    //    lo(nt, b) = ceil(nt b / bands) -- since an expert's rows are sorted
    //    by token, band b holds roughly the b-th quarter (for 4 bands) of
    //    every expert's tokens.  Bands run in order, experts most loaded
    //    first inside a band (longest work first), an expert's tiles
    //    consecutive.  Every expert with a single tile lands in band 0, so
    //    after band b every token tile of the first (b + 1) / bands of the
    //    tokens has all its rows, and its combine overlaps the later bands'
    //    expert GEMMs instead of waiting for the last expert; within a band an
    //    expert's weight panels are still streamed once for all its tiles
    //    there.  bands = 1: plain expert-major order.
    const float esz = TR::kBf16 ? 2.f : 4.f;
    const int NB = p.bands;
    auto lo_of = [&](int nt_, int b) { return (nt_ * b + NB - 1) / NB; };
    int nt = 0, c_r = 0;
    float cost = 0.f;
    if (tid < El) {
      c_r = s_cnt[s_ord[tid]];
      nt = (c_r + p.th - 1) / p.th;
      if (nt > 0) {
        const int last = c_r - p.th * (nt - 1);
        // one worker's time for a tile: its MFMA work (padded rows), or its
        // share of HBM bandwidth for the tile's weights
        const float by = 3.f * esz * (float)p.d * (float)p.f;
        auto tile_cost = [&](int bm) {
          const float fl = 6.f * bm * (float)p.d * (float)p.f;
          return fmaxf(fl / p.cm_mfma_rate, by * (float)p.workers / p.cm_hbm_bw);
        };
        cost = (float)(nt - 1) * tile_cost(p.th) + tile_cost(row_class(last));
      }
    }
    int n_mt = 0, n_perm = 0;
    for (int b = 0; b < NB; ++b) {
      // tiles and permute chunks of rank tid in band b
      int bt = 0, bp = 0;
      if (tid < El) {
        const int m0 = lo_of(nt, b), m1 = lo_of(nt, b + 1);
        bt = m1 - m0;
        if (bt > 0 && !p.gather_a) {   // a fused gather has no permute tasks
          const int lastrows = min(p.th, c_r - p.th * (m1 - 1));
          bp = (bt - 1) * p.pch + (lastrows + p.perm_rows - 1) / p.perm_rows;
        }
      }
      int tot_t = 0, tot_p = 0;
      const int ot = block_exscan(bt, s_w, &tot_t);
      const int op = block_exscan(bp, s_w, &tot_p);
      if (tid < El) {
        s_bt[b * 257 + tid] = n_mt + ot;
        s_bp[b * 257 + tid] = n_perm + op;
      }
      if (tid == 0) {
        s_bt[b * 257 + El] = n_mt + tot_t;
        s_bp[b * 257 + El] = n_perm + tot_p;
      }
      n_mt += tot_t;
      n_perm += tot_p;
    }
    const float tot_cost = block_sum(cost, s_wf);
    if (n_mt > p.max_mt || n_perm > p.max_perm) {
      if (tid == 0) set_error(p, 6 /* MOE_ERR_CAPACITY */);
      return;
    }
    __syncthreads();
    for (int mt = tid; mt < n_mt; mt += kThreads) {
      // band: the last one starting at or before mt
      int b = 0;
      while (b + 1 < NB && s_bt[(b + 1) * 257] <= mt) ++b;
      const int* bt_b = s_bt + b * 257;
      // rank: the last one whose base in the band is <= mt (ranks without a
      // tile in this band share the next rank's base, so they never match)
      int lo = 0, hi = El - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (bt_b[mid] <= mt) lo = mid;
        else hi = mid - 1;
      }
      const int r = lo;
      const int e = s_ord[r];
      const int ntr = (s_cnt[e] + p.th - 1) / p.th;
      const int j = mt - bt_b[r];                 // tile j of this rank in the band
      const int m = lo_of(ntr, b) + j;
      const int rows = min(p.th, s_cnt[e] - p.th * m);
      const int bm = row_class(rows);
      static_assert(sizeof(MTile) == 16, "MTile is one 16-byte store");
      st_wt16(p.mtiles, (uint32_t)mt * 16u,
              make_uint4((unsigned)e, (unsigned)(s_off[e] + p.th * m), (unsigned)rows, (unsigned)bm));
      const int npt = p.gather_a ? 0 : (rows + p.perm_rows - 1) / p.perm_rows;
      st_wt(p.cnt_perm + mt, npt);
      for (int ks = 0; ks < p.splitk; ++ks)
        st_wt(p.cnt_down + mt * p.splitk + ks,
              slice_lo(ks + 1, p.n_up_n, p.splitk) - slice_lo(ks, p.n_up_n, p.splitk));
      const int pbase = s_bp[b * 257 + r] + j * p.pch;
      for (int c2 = 0; c2 < npt; ++c2) st_wt(p.perm_list + pbase + c2, make_task(TK_PERM, mt * p.pch + c2));
    }
    mark(3);
    // 4. spatial split (cost model, per layer).  With Wm memory workers the
    //    gather takes t_mem(Wm) = bytes / min(Wm beta, B_hbm) and the expert
    //    tiles t_mfma(Wm) = cost / (W - Wm); the split minimises their
    //    maximum (t_mem falls and t_mfma rises with Wm, so the optimum is
    //    where they cross: found by bisection, then the better neighbour).
    //    Without a split every worker serves one queue: the gather, at the
    //    device's bandwidth, then the tiles, t_none = bytes / min(W beta,
    //    B_hbm) + cost / W.  The split is taken only when it is predicted at
    //    least kSplitMargin faster than that (a split costs the role
    //    hand-over and a second queue); otherwise Wm = 0.
    if (tid == 0) {
      const int W = p.workers;
      int wm_choice = 0;
      if (p.split_policy == 0 /* cost model */ && W >= 2) {
        constexpr float kSplitMargin = 0.03f;
        // (a gather fused into the UP tiles leaves no memory-bound tasks)
        const float bytes = p.gather_a ? 0.f : 2.f * (float)total * (float)p.d * esz;
        auto t_mem = [&](int wm) { return bytes / fminf((float)wm * p.cm_cu_bw, p.cm_hbm_bw); };
        auto t_mfma = [&](int wm) { return tot_cost / (float)(W - wm); };
        int lo = 1, hi = W - 1;        // first wm with t_mem <= t_mfma (hi if none)
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (t_mem(mid) <= t_mfma(mid)) hi = mid;
          else lo = mid + 1;
        }
        int best = lo;
        float t_best = fmaxf(t_mem(lo), t_mfma(lo));
        if (lo > 1 && fmaxf(t_mem(lo - 1), t_mfma(lo - 1)) < t_best) {
          best = lo - 1;
          t_best = fmaxf(t_mem(lo - 1), t_mfma(lo - 1));
        }
        const float t_none = t_mem(W) + tot_cost / (float)W;
        wm_choice = (t_best < (1.f - kSplitMargin) * t_none) ? best : 0;
      } else if (p.split_policy == 1 /* fixed */) {
        wm_choice = max(1, p.fixed_mem > 0 ? min(p.fixed_mem, W - 1) : W / 8);
      }
      int* cw = p.ctrl;
      st_relaxed(cw + CW_NMT * kCtrlStride, n_mt);
      st_relaxed(cw + CW_NPERM * kCtrlStride, n_perm);
      st_relaxed(cw + CW_WMEM * kCtrlStride, wm_choice);
    }
    mark(4);
  }

  // POS(rt): rows of this tile's kept slots, ascending (token, slot) order
  // inside every expert: row = offsets[e] + (rows of expert e in tiles
  // before rt) + rank of the slot among the tile's slots of expert e.
  // One thread per slot (32 tokens x k <= 256 slots).  The rank inside a
  // wave comes from the lanes holding the same expert (nine ballots over
  // the expert id's bits), plus the slots of that expert in earlier waves.
  // The rows before the tile are the prefix of the expert's histogram row,
  // read for the experts present in the tile only.
  // Returns (to every thread) how many distinct expert row tiles hold the
  // tile's kept slots: the combine of these tokens waits for exactly those
  // tiles' DOWN tasks.  An expert's slots here take the consecutive rows
  // [pre, pre + count) of its segment, so they meet the row tiles
  // pre / th .. (pre + count - 1) / th.
  static TASKFN int position(const Params& p, int rt, char* smem) {
    static_assert(kTB * kMaxK <= kThreads, "one thread per slot");
    static_assert(kMaxE <= 256, "expert id + 1 in nine bits");
    const int t0 = rt * kTB;
    const int rows = min(kTB, p.T - t0);
    const int k = p.k;
    const int ns = rows * k;
    const int El = p.E_loc;
    int* s_wc = reinterpret_cast<int*>(smem);            // [4][kMaxE] slots of e in wave w
    int* s_pre = s_wc + 4 * kMaxE;                       // [kMaxE] rows of e before the tile
    int* s_off = s_pre + kMaxE;                          // [kMaxE] segment offset of e
    int* s_list = s_off + kMaxE;                         // [kMaxE] experts present in the tile
    int* s_w = s_list + kMaxE;                           // [4] scan scratch
    const int i = tidx();
    const int wave = i >> 6, lane = i & 63;
    int e = -1;
    float w = 0.f;
    if (i < ns) {
      e = p.idx[(size_t)t0 * k + i] - p.e_begin;
      w = p.w[(size_t)t0 * k + i];
      if (e >= El || e < 0) e = -1;
    }
    const int eoff_i = i < El ? p.offsets[i] : 0;      // in flight with the slot loads
    for (int j = i; j < 5 * kMaxE; j += kThreads) s_wc[j] = 0;   // s_wc and s_pre
    __syncthreads();
    // lanes of this wave holding the same expert (lanes past the tile's
    // slots hold -1 and match only each other and non-local slots)
    const int key = e + 1;
    uint64_t same = ~0ull;
#pragma unroll
    for (int b = 0; b < 9; ++b) {
      const uint64_t bal = __ballot((key >> b) & 1);
      same &= ((key >> b) & 1) ? bal : ~bal;
    }
    const uint64_t below = (1ull << lane) - 1ull;
    const int rank_w = __popcll(same & below);
    if (e >= 0 && rank_w == 0) s_wc[wave * kMaxE + e] = __popcll(same);
    if (i < El) s_off[i] = eoff_i;
    __syncthreads();
    // experts present: a compact list, then their histogram prefixes
    int cnt = 0;
    if (i < El) cnt = s_wc[i] + s_wc[kMaxE + i] + s_wc[2 * kMaxE + i] + s_wc[3 * kMaxE + i];
    int n_pres = 0;
    const int li = block_exscan(cnt > 0 ? 1 : 0, s_w, &n_pres);
    if (cnt > 0) s_list[li] = i;
    __syncthreads();
    const int nq = (rt + 3) / 4;                          // int4 of a row prefix
    const int npairs = n_pres * nq;
    for (int j0 = i; j0 < npairs; j0 += 8 * kThreads) {
      int4 v[8];
      int ee[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u * kThreads;
        ee[u] = j < npairs ? s_list[j / nq] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u * kThreads;
        if (j < npairs)
          v[u] = *reinterpret_cast<const int4*>(p.hist + (size_t)ee[u] * p.hist_ld + 4 * (j % nq));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u * kThreads;
        if (j < npairs) {
          const int r = 4 * (j % nq);    // columns rt and later do not count
          const int s = v[u].x + (r + 1 < rt ? v[u].y : 0) + (r + 2 < rt ? v[u].z : 0) +
                        (r + 3 < rt ? v[u].w : 0);
          if (s) atomicAdd(s_pre + ee[u], s);
        }
      }
    }
    __syncthreads();
    if (i < ns) {
      if (e < 0) {
        st_wt(p.slot_pos + (size_t)t0 * k + i, -1);
      } else {
        int rank = rank_w;
        for (int v2 = 0; v2 < wave; ++v2) rank += s_wc[v2 * kMaxE + e];
        const int pos = s_off[e] + s_pre[e] + rank;
        st_wt(p.perm + pos, t0 + i / k);
        st_wt(p.rw + pos, w);
        st_wt(p.slot_pos + (size_t)t0 * k + i, pos);
      }
    }
    // distinct row tiles, summed over the experts present
    int nd_e = 0;
    if (cnt > 0) {
      const int pre = s_pre[i];
      nd_e = (pre + cnt - 1) / p.th - pre / p.th + 1;
    }
    int nd = 0;
    block_exscan(nd_e, s_w, &nd);
    return uniform(nd);
  }

  // PERM(mt, c): Xp[r] = x[perm[r]] for rows chunk c of tile mt (16-byte
  // coalesced copies; the local stand-in for expert-parallel dispatch).
  // The chunk's token ids go to LDS first, so every row load of a batch is
  // issued together (one round trip per 64 KB batch).
  // A row-tile record, every field in scalar registers (the record is the
  // same for the whole workgroup; derived addresses then stay uniform).
  static DEV MTile load_mtile(const Params& p, int mt) {
    const MTile t = p.mtiles[mt];
    return MTile{uniform(t.e), uniform(t.row0), uniform(t.rows), uniform(t.bm)};
  }

  static TASKFN void permute(const Params& p, int mt, int c) {
    __shared__ int s_tok[128];
    const MTile t = load_mtile(p, mt);
    const int r0 = t.row0 + c * p.perm_rows;
    const int r1 = min(t.row0 + t.rows, r0 + p.perm_rows);
    if (tidx() < r1 - r0) s_tok[tidx()] = p.perm[r0 + tidx()];
    __syncthreads();
    const int cpr = p.d * (int)sizeof(Elem) / 16;           // 16-byte chunks per row
    const int total = (r1 - r0) * cpr;
    const uint4* x = reinterpret_cast<const uint4*>(p.x);
    char* xp = reinterpret_cast<char*>(p.Xp);
    const size_t row_bytes = (size_t)cpr * 16;
    // 16 loads in flight per thread (64 KB per workgroup): a gather is a
    // latency-bound copy, so bytes in flight set its rate.
    // (the token of every load is read from LDS first, with one wait, so no
    // load waits on an LDS read of its own)
    constexpr int U = 16;
    for (int i0 = tidx(); i0 < total; i0 += U * kThreads) {
      int tok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ii = i0 + u * kThreads;
        tok[u] = ii < total ? s_tok[ii / cpr] : 0;
      }
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ii = i0 + u * kThreads;
        if (ii < total) v[u] = x[(size_t)tok[u] * cpr + ii % cpr];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ii = i0 + u * kThreads;
        if (ii < total)
          st_wt16(uniform_ptr(xp + (size_t)r0 * row_bytes),
                  (uint32_t)((ii / cpr) * row_bytes + (ii % cpr) * 16), v[u]);
      }
    }
    __syncthreads();
  }

  // ------------------------------------------------------------- GEMM tasks
  // Height class of an expert row tile holding `rows` rows.
  static DEV int row_class(int rows) {
    return rows <= 32 ? 32 : rows <= 64 ? 64 : rows <= 128 ? 128 : 256;
  }

  // UP tile: H[rows, n0:n0+128] = silu(A Wg) * (A Wu), rounded to Elem.
  // a_idx: row gather (tile row m reads A row a_idx[m]), or nullptr.
  template <int BM>
  static DEV void up_tile(const Elem* A, int lda, int rows, const Elem* wg, const Elem* wu,
                          int ldb, int K, Elem* Hout, int ldh, char* smem, const int* a_idx) {
    using TL = typename GemmSel<Elem, BM, 2>::T;
    static_assert(TL::LDS_BYTES <= kSmemTile, "UP tile fits the tile LDS");
    typename TL::Args g;
    g.A = A;
    g.lda = lda;
    g.a_rows = rows;
    g.a_idx = a_idx;
    g.B[0] = wg;
    g.B[1] = wu;
    g.ldb = ldb;
    g.K = K;
    if constexpr (!TR::kBf16) g.n_valid = kBN;
    typename TL::Acc acc;
    if constexpr (TR::kBf16) TL::run(g, smem, acc);
    else TL::run(g, reinterpret_cast<Elem*>(smem), acc);
    // stage the tile in LDS, then write whole rows
    constexpr int SLD = kBN + 16 / (int)sizeof(Elem);
    Elem* st = reinterpret_cast<Elem*>(smem);
    TL::for_each([&](int row, int col, int fm, int fn, int i) __attribute__((always_inline)) {
      const float gv = acc[0][fm][fn][i];
      const float uv = acc[1][fm][fn][i];
      const float h = gv / (1.0f + __expf(-gv)) * uv;
      st[row * SLD + col] = TR::from_f(h);
    });
    __syncthreads();
    constexpr int CPR = kBN * (int)sizeof(Elem) / 16;
    for (int i = tidx(); i < rows * CPR; i += kThreads) {
      const int r = i / CPR, c = i % CPR;
      st_wt16(Hout, (uint32_t)(r * ldh * (int)sizeof(Elem) + c * 16),
              *reinterpret_cast<const uint4*>(st + r * SLD + c * (16 / (int)sizeof(Elem))));
    }
    __syncthreads();
  }

  // DOWN tile: Out[r, 0:128] = (A Wd)[r, :] for the valid rows r < rows,
  // fp32, staged through LDS and written as whole 16-byte row chunks
  // (write-through: a combine task on another XCD reads them).  The weighted
  // sum over a token's experts is the combine task's job, so no output
  // element is ever written twice and no atomics are needed.
  // NB = 2: two adjacent 128-column blocks of Wd share the A tile (a
  // 256-column task), written as two consecutive column blocks of Out.
  // scatter (small layers): instead, out[tok(r), cols] += wt(r) * (A Wd)[r, :]
  // with fp32 atomics -- the weighted scatter-add combine, fused into the
  // DOWN epilogue; tok / wt of the tile's rows come from the LDS table
  // down_rows() filled before the tile (so nothing extra stays live across
  // the K loop).
  template <int BM, int NB>
  static DEV void down_tile(const Elem* A, int lda, int rows, const Elem* wd, int ldb, int K,
                            float* out, int ldo, char* smem, bool scatter = false,
                            bool stream = false) {
    using TL = typename GemmSel<Elem, BM, NB>::T;
    static_assert(TL::LDS_BYTES <= kSmemTile, "DOWN tile fits the tile LDS");
    typename TL::Args g;
    g.A = A;
    g.lda = lda;
    g.a_rows = rows;
#pragma unroll
    for (int m = 0; m < NB; ++m) g.B[m] = wd + m * kBN;
    g.ldb = ldb;
    g.K = K;
    if constexpr (!TR::kBf16) g.n_valid = kBN;
    typename TL::Acc acc;
    if constexpr (TR::kBf16) TL::run(g, smem, acc);
    else TL::run(g, reinterpret_cast<Elem*>(smem), acc);
    // stage one [BM][128] fp32 block at a time (rows padded by 4 floats
    // against bank conflicts)
    constexpr int SLD = kBN + 4;
    static_assert(BM * SLD * 4 <= kSmemTile, "DOWN staging fits the tile LDS");
    float* st = reinterpret_cast<float*>(smem);
    constexpr int CPR = kBN * 4 / 16;
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      TL::for_each([&](int row, int col, int fm, int fn, int i) __attribute__((always_inline)) {
        st[row * SLD + col] = acc[m][fm][fn][i];
      });
      __syncthreads();
      if (scatter) {
        // one column per thread: each atomic instruction covers 64
        // consecutive floats of one token row
        const int* s_tok = down_rows_tok();
        const float* s_wt = down_rows_wt();
        for (int i = tidx(); i < rows * kBN; i += kThreads) {
          const int r = i / kBN, c = i % kBN;
          unsafeAtomicAdd(out + (size_t)s_tok[r] * ldo + m * kBN + c, s_wt[r] * st[r * SLD + c]);
        }
      } else if (stream) {
        for (int i = tidx(); i < rows * CPR; i += kThreads) {
          const int r = i / CPR, c = i % CPR;
          st_wt16_stream(uniform_ptr(out + m * kBN), (uint32_t)(r * ldo * 4 + c * 16),
                         *reinterpret_cast<const uint4*>(st + r * SLD + c * 4));
        }
      } else {
        for (int i = tidx(); i < rows * CPR; i += kThreads) {
          const int r = i / CPR, c = i % CPR;
          st_wt16(uniform_ptr(out + m * kBN), (uint32_t)(r * ldo * 4 + c * 16),
                  *reinterpret_cast<const uint4*>(st + r * SLD + c * 4));
        }
      }
      __syncthreads();
    }
  }

  // Dispatch on the row class (and, for bf16, the 256-row class and the
  // 256-column DOWN task).
  template <typename F>
  static DEV void by_class(int bm, F&& f) {
    if (bm == 32) f(std::integral_constant<int, 32>{});
    else if (bm == 64) f(std::integral_constant<int, 64>{});
    else if (bm == 128 || !TR::kBf16) f(std::integral_constant<int, 128>{});
    else if constexpr (TR::kBf16) f(std::integral_constant<int, 256>{});
  }
  // LDS table of the scatter epilogue: token and weight of each tile row.
  static DEV int* down_rows_tok() {
    __shared__ int s_tok[256];
    return s_tok;
  }
  static DEV float* down_rows_wt() {
    __shared__ float s_wt[256];
    return s_wt;
  }
  // Fill it: tok == nullptr means tokens row_tok0 + r with weight 1.
  static DEV void down_rows(int rows, const int* tok, const float* wt, int row_tok0) {
    const int r = tidx();
    if (r < rows) {
      down_rows_tok()[r] = tok ? tok[r] : row_tok0 + r;
      down_rows_wt()[r] = tok ? wt[r] : 1.0f;
    }
  }

  static DEV void down_any(int bm, int nb, const Elem* A, int lda, int rows, const Elem* wd,
                           int ldb, int K, float* out, int ldo, char* smem, bool scatter,
                           bool stream = false) {
    by_class(bm, [&](auto c) __attribute__((always_inline)) {
      constexpr int BM = decltype(c)::value;
      if constexpr (TR::kBf16) {
        if (nb == 2) {
          down_tile<BM, 2>(A, lda, rows, wd, ldb, K, out, ldo, smem, scatter, stream);
          return;
        }
      }
      down_tile<BM, 1>(A, lda, rows, wd, ldb, K, out, ldo, smem, scatter, stream);
    });
  }
  static DEV void up_any(int bm, const Elem* A, int lda, int rows, const Elem* wg, const Elem* wu,
                         int ldb, int K, Elem* Hout, int ldh, char* smem,
                         const int* a_idx = nullptr) {
    by_class(bm, [&](auto c) __attribute__((always_inline)) {
      up_tile<decltype(c)::value>(A, lda, rows, wg, wu, ldb, K, Hout, ldh, smem, a_idx);
    });
  }

  // UP(mt, n).  With the gather fused (p.gather_a) the tile reads its rows
  // straight from x through the permutation (row r of the expert-contiguous
  // order is token perm[r]), so no permuted copy Xp is written or read;
  // otherwise from Xp, which the permute tasks filled.
  static TASKFN void up(const Params& p, int mt, int n, char* smem) {
    const MTile t = load_mtile(p, mt);
    const Elem* A = p.gather_a ? reinterpret_cast<const Elem*>(p.x)
                               : reinterpret_cast<const Elem*>(p.Xp) + (size_t)t.row0 * p.d;
    const int* a_idx = p.gather_a ? p.perm + t.row0 : nullptr;
    const size_t eo = (size_t)t.e * p.d * p.f + (size_t)n * kBN;
    const Elem* wg = reinterpret_cast<const Elem*>(p.wg) + eo;
    const Elem* wu = reinterpret_cast<const Elem*>(p.wu) + eo;
    Elem* H = reinterpret_cast<Elem*>(p.H) + (size_t)t.row0 * p.f + (size_t)n * kBN;
    up_any(t.bm, A, p.d, t.rows, wg, wu, p.f, p.d, H, p.f, smem, a_idx);
  }

  static TASKFN void down(const Params& p, int mt, int n, int ks, char* smem, bool scat) {
    const MTile t = load_mtile(p, mt);
    const int k_lo = slice_lo(ks, p.n_up_n, p.splitk) * kBN;
    const int K = slice_lo(ks + 1, p.n_up_n, p.splitk) * kBN - k_lo;
    const Elem* A = reinterpret_cast<const Elem*>(p.H) + (size_t)t.row0 * p.f + k_lo;
    const int n0 = n * kBN * p.down_nb;
    const Elem* wd = reinterpret_cast<const Elem*>(p.wd) + (size_t)t.e * p.f * p.d +
                     (size_t)k_lo * p.d + n0;
    if (scat) {
      down_rows(t.rows, p.perm + t.row0, p.rw + t.row0, 0);   // read after the K loop's barriers
      down_any(t.bm, p.down_nb, A, p.f, t.rows, wd, p.d, K, p.y + n0, p.d, smem, true);
      return;
    }
    float* out = o_slice(p, ks) + (size_t)t.row0 * p.d + n0;
    down_any(t.bm, p.down_nb, A, p.f, t.rows, wd, p.d, K, out, p.d, smem, false, p.o_stream != 0);
  }

  // DOWN output rows of K slice ks: [T*k][d] fp32.
  static DEV float* o_slice(const Params& p, int ks) {
    return p.O + (size_t)ks * p.T * p.k * p.d;
  }

  // Shared (always-on) experts: every token, weight 1, input x directly.
  static TASKFN void shared_up(const Params& p, int s, int m, int n, char* smem) {
    const int r0 = m * p.th;
    const int rows = min(p.th, p.T - r0);
    const Elem* A = reinterpret_cast<const Elem*>(p.x) + (size_t)r0 * p.d;
    const size_t so = (size_t)s * p.d * p.fs + (size_t)n * kBN;
    const Elem* wg = reinterpret_cast<const Elem*>(p.sg) + so;
    const Elem* wu = reinterpret_cast<const Elem*>(p.su) + so;
    Elem* H = reinterpret_cast<Elem*>(p.Hs) + ((size_t)s * p.T + r0) * p.fs + (size_t)n * kBN;
    up_any(row_class(rows), A, p.d, rows, wg, wu, p.fs, p.d, H, p.fs, smem);
  }

  static TASKFN void shared_down(const Params& p, int s, int m, int n, char* smem, bool scat) {
    const int r0 = m * p.th;
    const int rows = min(p.th, p.T - r0);
    const int n0 = n * kBN * p.down_nb;
    const Elem* A = reinterpret_cast<const Elem*>(p.Hs) + ((size_t)s * p.T + r0) * p.fs;
    const Elem* wd = reinterpret_cast<const Elem*>(p.sd) + (size_t)s * p.fs * p.d + n0;
    if (scat) {
      down_rows(rows, nullptr, nullptr, r0);
      down_any(row_class(rows), p.down_nb, A, p.fs, rows, wd, p.d, p.fs, p.y + n0, p.d, smem,
               true);
      return;
    }
    float* out = p.Ys + ((size_t)s * p.T + r0) * p.d + n0;
    down_any(row_class(rows), p.down_nb, A, p.fs, rows, wd, p.d, p.fs, out, p.d, smem, false);
  }

  // ------------------------------------------------------------- combine
  // COMB(rt, cc): y[t, cols] = sum_j w[t,j] * (sum_ks O_ks[slot_pos[t,j], cols])
  // over the token's kept slots in slot order, then + sum_s Ys[s][t, cols]
  // over the shared experts, for the 32 tokens of tile rt and the column
  // chunk cc.  The weighted combine of the MoE layer (xxqk.cn/news/665650
  // s1, last stage; it stands in for expert-parallel combine, Weave
  // abstract): a token's output needs every one of its experts, so the task
  // becomes ready only when all DOWN tiles holding its rows have finished.
  // Fixed summation order: y does not depend on the schedule.
  // 16 bytes of combined y at base + byte_off (base uniform over the
  // workgroup): written through to memory when a NORM task (on any XCD)
  // reads them in this launch; otherwise a plain store, left in this XCD's
  // L2 until the kernel's end-of-launch release writes it back.
  static DEV void st_y16(const Params& p, float* base, uint32_t byte_off, uint4 v) {
    if (p.fuse_norm) {
      st_wt16(base, byte_off, v);
    } else {
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(base) + byte_off) = v;
    }
  }

  static TASKFN void combine(const Params& p, int rt, int cc, char* smem) {
    const int t0 = rt * kTB;
    const int rows = min(kTB, p.T - t0);
    const int k = p.k;
    int* s_pos = reinterpret_cast<int*>(smem);               // [32 * k]
    float* s_w = reinterpret_cast<float*>(s_pos + kTB * kMaxK);
    for (int i = tidx(); i < rows * k; i += kThreads) {
      s_pos[i] = p.slot_pos[(size_t)t0 * k + i];
      s_w[i] = p.w[(size_t)t0 * k + i];
    }
    __syncthreads();
    const int c4 = p.comb_cols / 4;                      // float4 per row chunk
    const int col0 = cc * p.comb_cols;
    const size_t slice = (size_t)p.T * k * p.d;
    const int n = rows * c4;
    // A combine task is a latency-bound gather and the persistent kernel runs
    // one workgroup per CU, so each thread keeps many loads in flight: CU
    // (token, float4) items per pass.  Every slot row index of the pass is
    // read from LDS first (one wait), so no load waits on an LDS read of its
    // own; then the first K slice of every kept slot of all items is issued
    // before any is used, then each further K slice as one burst, then the
    // sums; the shared experts' rows and the residual follow as one more
    // burst (the expert rows' registers are free by then).  Each O row is
    // read once, with the non-temporal hint.
    constexpr int CU = 2;
    for (int i0 = tidx(); i0 < n; i0 += CU * kThreads) {
      int pos[CU][kMaxK];
      float wt[CU][kMaxK];
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const int i = i0 + u * kThreads;
        const int r = i / c4;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
          const bool ok = i < n && j < k;
          pos[u][j] = ok ? s_pos[r * k + j] : -1;
          wt[u][j] = ok ? s_w[r * k + j] : 0.f;
        }
      }
      float4 v[CU][kMaxK];
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const int i = i0 + u * kThreads;
        const int col = col0 + (i % c4) * 4;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
          v[u][j] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (pos[u][j] >= 0)
            v[u][j] = ld_stream4(p.O + (size_t)pos[u][j] * p.d + col);
        }
      }
      // further K slices (only layers with a DOWN split-K and combine tasks)
      for (int ks = 1; ks < p.splitk; ++ks) {
#pragma unroll
        for (int u = 0; u < CU; ++u) {
          const int i = i0 + u * kThreads;
          const int col = col0 + (i % c4) * 4;
#pragma unroll
          for (int j = 0; j < kMaxK; ++j) {
            if (pos[u][j] >= 0) {
              const float4 b = ld_stream4(p.O + ks * slice + (size_t)pos[u][j] * p.d + col);
              v[u][j].x += b.x; v[u][j].y += b.y; v[u][j].z += b.z; v[u][j].w += b.w;
            }
          }
        }
      }
      // weighted sum over the token's kept slots, in slot order
      float4 acc[CU];
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
          if (pos[u][j] >= 0) {
            const float wj = wt[u][j];
            acc[u].x += wj * v[u][j].x;
            acc[u].y += wj * v[u][j].y;
            acc[u].z += wj * v[u][j].z;
            acc[u].w += wj * v[u][j].w;
          }
        }
      }
      // shared experts (weight 1), then the residual (h = residual + MoE(x))
      if (p.n_shared > 0 || p.resid) {
        float4 ex[CU][5];
#pragma unroll
        for (int u = 0; u < CU; ++u) {
          const int i = i0 + u * kThreads;
          const int r = i / c4, col = col0 + (i % c4) * 4;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            ex[u][s] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (i < n && s < p.n_shared)
              ex[u][s] = *reinterpret_cast<const float4*>(p.Ys + ((size_t)s * p.T + t0 + r) * p.d + col);
          }
          ex[u][4] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (i < n && p.resid)
            ex[u][4] = *reinterpret_cast<const float4*>(p.resid + (size_t)(t0 + r) * p.d + col);
        }
#pragma unroll
        for (int u = 0; u < CU; ++u) {
#pragma unroll
          for (int s = 0; s < 5; ++s) {
            acc[u].x += ex[u][s].x; acc[u].y += ex[u][s].y; acc[u].z += ex[u][s].z; acc[u].w += ex[u][s].w;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const int i = i0 + u * kThreads;
        if (i >= n) continue;
        const int r = i / c4, col = col0 + (i % c4) * 4;
        st_y16(p, uniform_ptr(p.y + (size_t)t0 * p.d), (uint32_t)((r * p.d + col) * 4),
               make_uint4(__float_as_uint(acc[u].x), __float_as_uint(acc[u].y),
                          __float_as_uint(acc[u].z), __float_as_uint(acc[u].w)));
      }
    }
    __syncthreads();
  }

  // -------------------------------------------------------- block tail
  // NORM(rt): y_norm[t] = y[t] / sqrt(mean_c y[t,c]^2 + eps) * gamma for the
  // 32 tokens of tile rt, y already holding residual + MoE output -- the
  // residual and normalisation stages the blog walk-through keeps inside the
  // big MoE kernel (xxqk.cn/news/665650 section 1), fused so the layer output
  // is not re-read by a separate kernel.  One wave per token in turn; each
  // lane sums the squares of its columns in a fixed order, then a butterfly
  // over the wave (every lane ends with the same bits), so the result does
  // not depend on the schedule.  `coherent`: y was accumulated with atomics
  // (scatter combine), so it is read with device-coherent loads.
  static TASKFN void norm(const Params& p, int rt, bool coherent) {
    if (coherent) norm_rows<true>(p, rt);
    else norm_rows<false>(p, rt);
  }
  template <bool COHERENT>
  static DEV void norm_rows(const Params& p, int rt) {
    const int t0 = rt * kTB;
    const int rows = min(kTB, p.T - t0);
    const int wave = tidx() >> 6, lane = tidx() & 63;
    // one wave per row; a row's float4 chunks in passes of U per lane, the
    // U loads of a pass unconditional (chunks past the row re-read its last
    // chunk and are dropped) and in flight together
    constexpr int U = 8;
    const int n4 = p.d / 4;
    auto load = [&](const float* yr, int c) __attribute__((always_inline)) {
      if constexpr (COHERENT) return ld_coherent4(yr + 4 * c);
      else return *reinterpret_cast<const float4*>(yr + 4 * c);
    };
    for (int r = wave; r < rows; r += kThreads / 64) {
      const float* yr = p.y + (size_t)(t0 + r) * p.d;
      float ss = 0.f;
      for (int c0 = 0; c0 < n4; c0 += 64 * U) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = load(yr, min(c0 + u * 64 + lane, n4 - 1));
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (c0 + u * 64 + lane < n4)
            ss += v[u].x * v[u].x + v[u].y * v[u].y + v[u].z * v[u].z + v[u].w * v[u].w;
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) ss += wave_xor(ss, o);
      const float scale = 1.0f / sqrtf(ss / (float)p.d + p.norm_eps);
      Elem* out = reinterpret_cast<Elem*>(p.y_norm) + (size_t)(t0 + r) * p.d;
      for (int c0 = 0; c0 < n4; c0 += 64 * U) {
        float4 v[U], g[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = min(c0 + u * 64 + lane, n4 - 1);
          v[u] = load(yr, c);
          g[u] = *reinterpret_cast<const float4*>(p.norm_w + 4 * c);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * 64 + lane;
          if (c >= n4) continue;
          const float o0 = v[u].x * scale * g[u].x, o1 = v[u].y * scale * g[u].y;
          const float o2 = v[u].z * scale * g[u].z, o3 = v[u].w * scale * g[u].w;
          if constexpr (TR::kBf16) {
            *reinterpret_cast<uint2*>(out + 4 * c) =
                make_uint2((uint32_t)f2bf(o0) | ((uint32_t)f2bf(o1) << 16),
                           (uint32_t)f2bf(o2) | ((uint32_t)f2bf(o3) << 16));
          } else {
            *reinterpret_cast<float4*>(out + 4 * c) = make_float4(o0, o1, o2, o3);
          }
        }
      }
    }
    __syncthreads();
  }
};

}  // namespace moe
