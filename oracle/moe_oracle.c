/*
 * moe_oracle.c -- plain CPU reference of one Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or run this library.  The GPU path
 * never calls it, includes it or shares code with it.
 *
 * What it computes.  The Weave pages name the stages of an MoE layer kept
 * inside one persistent kernel -- gate/router, top-k expert choice, the
 * per-expert FFN GEMMs, the weighted merge of expert outputs
 * (xxqk.cn/news/665650 section 1, "large kernel" paragraph;
 * m.xxqk.cn/news/657744 section 1.1) -- and say the dynamic scheduler only
 * reorders that work, never changes it (xxqk.cn/news/665650 section 3.1:
 * only the scheduling policy changes between the compared kernels).  No page
 * writes the formulas, so this file takes the standard definitions and fixes
 * every open choice explicitly:
 *
 *   L[t,e]   = (sum_i x[t,i] * Wr[i,e]) + b[e]                      (step 1)
 *   top-k    = the k experts with the largest L, equal values broken
 *              toward the lower expert index; +0.0 and -0.0 are equal (2)
 *   w[t,j]   = exp(L[t,idx_j] - L[t,idx_0]) / sum_j' exp(...)         (3)
 *              (= softmax over all E renormalised over the chosen k)
 *   local    = slots whose expert lies in [e_begin, e_end) are kept,
 *              weights are NOT renormalised again                      (4)
 *   counts, offsets, stable positions in ascending (token, slot) order (5,6)
 *   Xp[r]    = x[perm[r]]                                              (7)
 *   h        = silu(Xp[r] Wg[e]) * (Xp[r] Wu[e]),  silu(z)=z/(1+e^-z)  (8)
 *   O[r]     = h Wd[e]
 *   y[t]     = sum_{kept j, ascending} w[t,j] O[slot_pos[t,j]]
 *              + sum_s SwiGLU_s(x[t])   (shared experts, weight 1)     (9)
 *
 * Arithmetic is IEEE double throughout (inputs are fp32 or bf16 and are
 * widened exactly); the router logits are rounded once to fp32 because the
 * expert choice is defined on fp32 logits.  Every dot product is summed in
 * ascending index order, plainly, with no blocking.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

/* Widen element i of an fp32 or bf16 array to double.  bf16 is the upper 16
 * bits of an fp32, so the widening is exact. */
static double elem(const void* p, int dtype, size_t i) {
  if (dtype == ORC_F32) return (double)((const float*)p)[i];
  uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Step 1: router logits, fp64 sum in ascending i, bias added last, rounded to
 * fp32.  x is [T,d], wr is [d,E], bias is [E] or NULL. */
void oracle_logits(int T, int d, int E, const void* x, int x_dtype,
                   const void* wr, int wr_dtype, const float* bias,
                   float* logits) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      double s = 0.0;
      for (int i = 0; i < d; ++i)
        s += elem(x, x_dtype, (size_t)t * d + i) *
             elem(wr, wr_dtype, (size_t)i * E + e);
      if (bias) s += (double)bias[e];
      logits[(size_t)t * E + e] = (float)s;
    }
  }
}

/* Steps 2-6: expert choice, gate weights, local filter, counts, offsets and
 * stable positions.
 *   idx[T*k], w[T*k]          chosen experts (global ids) and their weights
 *   counts[E_loc], offsets[E_loc+1]
 *   perm[R], rw[R]            token and weight of every kept routed row
 *   slot_pos[T*k]             row of each slot, -1 if filtered out
 * Returns R (number of kept rows), or -1 if a logit is not finite, or -2 on
 * bad arguments. */
int oracle_route(int T, int E, int k, int e_begin, int e_end,
                 const float* logits, int32_t* idx, double* w,
                 int32_t* counts, int32_t* offsets, int32_t* perm,
                 int32_t* slot_pos, double* rw) {
  if (T < 0 || E < 1 || k < 1 || k > E || e_begin < 0 || e_end > E ||
      e_begin >= e_end)
    return -2;
  for (size_t i = 0; i < (size_t)T * E; ++i)
    if (!isfinite(logits[i])) return -1;
  const int E_loc = e_end - e_begin;
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  for (int t = 0; t < T; ++t) {
    const float* L = logits + (size_t)t * E;
    memset(taken, 0, (size_t)E);
    /* Selection sort: the j-th pick is the largest remaining logit; scanning
     * e upward and replacing only on a strictly larger value keeps the lower
     * index on ties, and C's > treats +0.0 and -0.0 as equal. */
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || L[e] > L[best]) best = e;
      }
      taken[best] = 1;
      idx[(size_t)t * k + j] = best;
    }
    double a[256 + 1];
    double* av = (k <= 256) ? a : (double*)malloc(sizeof(double) * (size_t)k);
    const double l0 = (double)L[idx[(size_t)t * k]];
    double s = 0.0;
    for (int j = 0; j < k; ++j) {
      av[j] = exp((double)L[idx[(size_t)t * k + j]] - l0);
      s += av[j];
    }
    for (int j = 0; j < k; ++j) w[(size_t)t * k + j] = av[j] / s;
    if (av != a) free(av);
  }
  free(taken);

  for (int e = 0; e < E_loc; ++e) counts[e] = 0;
  for (size_t i = 0; i < (size_t)T * k; ++i) {
    int e = idx[i];
    if (e >= e_begin && e < e_end) counts[e - e_begin]++;
  }
  offsets[0] = 0;
  for (int e = 0; e < E_loc; ++e) offsets[e + 1] = offsets[e] + counts[e];

  int32_t* cur = (int32_t*)calloc((size_t)E_loc, sizeof(int32_t));
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < k; ++j) {
      size_t s = (size_t)t * k + j;
      int e = idx[s];
      if (e < e_begin || e >= e_end) {
        slot_pos[s] = -1;
        continue;
      }
      int el = e - e_begin;
      int pos = offsets[el] + cur[el]++;
      perm[pos] = t;
      slot_pos[s] = pos;
      rw[pos] = w[s];
    }
  }
  free(cur);
  return offsets[E_loc];
}

/* One SwiGLU expert applied to one input row (step 8):
 *   g = xr Wg, u = xr Wu (ascending i), h = silu(g) u, out = h Wd (ascending
 *   f).  wg, wu are [d,f]; wd is [f,d]; out is [d]; g, u are scratch [f]. */
static void swiglu_row(int d, int f, const void* xrow_base, int x_dtype,
                       size_t x_off, const void* wg, const void* wu,
                       const void* wd, int w_dtype, size_t wgu_off,
                       size_t wd_off, double* g, double* u, double* out) {
  for (int n = 0; n < f; ++n) g[n] = u[n] = 0.0;
  for (int i = 0; i < d; ++i) {
    double xi = elem(xrow_base, x_dtype, x_off + (size_t)i);
    size_t row = wgu_off + (size_t)i * f;
    for (int n = 0; n < f; ++n) {
      g[n] += xi * elem(wg, w_dtype, row + n);
      u[n] += xi * elem(wu, w_dtype, row + n);
    }
  }
  for (int n = 0; n < f; ++n) g[n] = silu(g[n]) * u[n]; /* g now holds h */
  for (int c = 0; c < d; ++c) out[c] = 0.0;
  for (int n = 0; n < f; ++n) {
    double hn = g[n];
    size_t row = wd_off + (size_t)n * d;
    for (int c = 0; c < d; ++c) out[c] += hn * elem(wd, w_dtype, row + c);
  }
}

/* Steps 7-9 for a chosen set of tokens.  Routing (idx, w, slot_pos) comes
 * from oracle_route.  For every requested token t_sel[q] the output row
 * y[q, 0:d] is  sum over kept slots j (ascending) of w[t,j] * O_e(x[t])
 * plus the shared experts.  Expert e's weights sit at index (e - e_begin) of
 * wg/wu/wd.  Reading Xp[slot_pos] = x[perm[slot_pos]] = x[t] (step 7), the
 * gathered row of slot (t,j) is x[t] itself.
 *   x       [T,d]            dtype x_dtype
 *   wg, wu  [E_loc,d,f]      wd [E_loc,f,d]     dtype w_dtype
 *   sg, su  [n_shared,d,fs]  sd [n_shared,fs,d] (may be NULL if n_shared=0)
 *   y       [n_sel,d]        double              */
void oracle_moe_rows(int T, int d, int E, int k, int f, int e_begin,
                     int e_end, int n_shared, int fs, const void* x,
                     int x_dtype, const void* wg, const void* wu,
                     const void* wd, const void* sg, const void* su,
                     const void* sd, int w_dtype, const int32_t* idx,
                     const double* w, const int32_t* slot_pos, int n_sel,
                     const int32_t* t_sel, double* y) {
  (void)T;
  (void)E;
  const int fmax = f > fs ? f : fs;
#pragma omp parallel
  {
    double* g = (double*)malloc(sizeof(double) * (size_t)fmax);
    double* u = (double*)malloc(sizeof(double) * (size_t)fmax);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
    for (int q = 0; q < n_sel; ++q) {
      int t = t_sel[q];
      double* yr = y + (size_t)q * d;
      for (int c = 0; c < d; ++c) yr[c] = 0.0;
      for (int j = 0; j < k; ++j) {
        size_t s = (size_t)t * k + j;
        if (slot_pos[s] < 0) continue; /* filtered out (not local) */
        int el = idx[s] - e_begin;
        swiglu_row(d, f, x, x_dtype, (size_t)t * d, wg, wu, wd, w_dtype,
                   (size_t)el * d * f, (size_t)el * f * d, g, u, o);
        for (int c = 0; c < d; ++c) yr[c] += w[s] * o[c];
      }
      for (int sh = 0; sh < n_shared; ++sh) {
        swiglu_row(d, fs, x, x_dtype, (size_t)t * d, sg, su, sd, w_dtype,
                   (size_t)sh * d * fs, (size_t)sh * fs * d, g, u, o);
        for (int c = 0; c < d; ++c) yr[c] += o[c];
      }
    }
    free(g);
    free(u);
    free(o);
  }
  (void)e_end;
}

/* Steps 7-8 in the per-expert order the pages' stage list implies: every
 * kept row r (expert-contiguous, ascending) gets O[r] = SwiGLU_e(Xp[r]) with
 * Xp[r] = x[perm[r]] gathered explicitly.  Step 9 then combines per token.
 * This is the whole-layer form; oracle_moe_rows is the same arithmetic per
 * token.  O is [R,d] double scratch supplied by the caller; y is [T,d]. */
void oracle_moe_layer(int T, int d, int E, int k, int f, int e_begin,
                      int e_end, int n_shared, int fs, const void* x,
                      int x_dtype, const void* wg, const void* wu,
                      const void* wd, const void* sg, const void* su,
                      const void* sd, int w_dtype, const int32_t* idx,
                      const double* w, const int32_t* offsets,
                      const int32_t* perm, const int32_t* slot_pos, double* O,
                      double* y) {
  (void)E;
  (void)idx;
  const int E_loc = e_end - e_begin;
  const int R = offsets[E_loc];
  const int fmax = f > fs ? f : fs;
  const size_t xsz = (x_dtype == ORC_F32) ? 4 : 2;
  /* Step 7: explicit gather into an expert-contiguous buffer. */
  unsigned char* Xp = (unsigned char*)malloc(xsz * (size_t)(R > 0 ? R : 1) * d);
  for (int r = 0; r < R; ++r)
    memcpy(Xp + xsz * (size_t)r * d,
           (const unsigned char*)x + xsz * (size_t)perm[r] * d, xsz * (size_t)d);
#pragma omp parallel
  {
    double* g = (double*)malloc(sizeof(double) * (size_t)fmax);
    double* u = (double*)malloc(sizeof(double) * (size_t)fmax);
    /* Step 8: expert e owns rows [offsets[e], offsets[e+1]). */
#pragma omp for schedule(dynamic, 1)
    for (int r = 0; r < R; ++r) {
      int el = 0;
      while (offsets[el + 1] <= r) ++el;
      swiglu_row(d, f, Xp, x_dtype, (size_t)r * d, wg, wu, wd, w_dtype,
                 (size_t)el * d * f, (size_t)el * f * d, g, u,
                 O + (size_t)r * d);
    }
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    /* Step 9: weighted combine per token, slots ascending, then shared. */
#pragma omp for schedule(dynamic, 1)
    for (int t = 0; t < T; ++t) {
      double* yr = y + (size_t)t * d;
      for (int c = 0; c < d; ++c) yr[c] = 0.0;
      for (int j = 0; j < k; ++j) {
        int pos = slot_pos[(size_t)t * k + j];
        if (pos < 0) continue;
        double wj = w[(size_t)t * k + j];
        for (int c = 0; c < d; ++c) yr[c] += wj * O[(size_t)pos * d + c];
      }
      for (int sh = 0; sh < n_shared; ++sh) {
        swiglu_row(d, fs, x, x_dtype, (size_t)t * d, sg, su, sd, w_dtype,
                   (size_t)sh * d * fs, (size_t)sh * fs * d, g, u, o);
        for (int c = 0; c < d; ++c) yr[c] += o[c];
      }
    }
    free(o);
    free(g);
    free(u);
  }
  free(Xp);
}

/* Residual add and RMSNorm of the layer output -- the "residual and
 * normalisation" stages the blog walk-through keeps inside the big MoE kernel
 * (xxqk.cn/news/665650 section 1).  No page writes the formula; this is the
 * standard RMSNorm of the pre-norm transformer block, applied to the block
 * output so it is the next block's normalised input:
 *   h[t,c]  = residual[t,c] + y[t,c]
 *   ms[t]   = (1/d) sum_{c ascending} h[t,c]^2
 *   hn[t,c] = h[t,c] / sqrt(ms[t] + eps) * gamma[c]
 * Arithmetic in fp64.  residual [T,d] fp32 (NULL = zero), gamma [d] fp32,
 * y, h, hn [T,d] double. */
void oracle_residual_rmsnorm(int T, int d, const double* y, const float* residual,
                             const float* gamma, double eps, double* h,
                             double* hn) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const double* yr = y + (size_t)t * d;
    double* hr = h + (size_t)t * d;
    double ss = 0.0;
    for (int c = 0; c < d; ++c) {
      hr[c] = (residual ? (double)residual[(size_t)t * d + c] : 0.0) + yr[c];
      ss += hr[c] * hr[c];
    }
    const double r = 1.0 / sqrt(ss / (double)d + eps);
    for (int c = 0; c < d; ++c) hn[(size_t)t * d + c] = hr[c] * r * (double)gamma[c];
  }
}

/* Threads the OpenMP runtime will use (for reporting). */
int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      extern int omp_get_num_threads(void);
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}
