// moe.hip -- host side of the C ABI declared in include/moe.h: descriptor
// validation, workspace carving, and the launches of each scheduling mode.
// All device work lives in sched.hpp / stages.hpp / tile.hpp.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "launch.hpp"
#include "sched.hpp"

using namespace moe;

namespace moe {

// Initial value of control word w (the first int of its 128-byte line; the
// rest of the line is padding).  QA starts with the router tasks in its
// slots, QC with the shared-expert UP tiles; queue totals other than QA's are
// unknown until the builder publishes them.
__host__ __device__ inline int ctrl_init(const Params& p, int w) {
  const int seeded = p.n_route + (p.route_wide ? p.n_rt : 0);   // router (+ finish) tasks
  if (w == CW_TAIL + QA) return seeded;
  if (w == CW_TOTAL + QA) return seeded + p.n_rt;
  if (w == CW_TAIL + QC) return p.n_sup;
  if (w == CW_TOTAL + QM || w == CW_TOTAL + QC || w == CW_TOTAL + QH) return 0x7fffffff;
  if (w >= CW_UTOTAL && w < CW_UTOTAL + kXcds) return 0x7fffffff;
  if (w == CW_LTOTAL) return 0x7fffffff;
  return 0;
}

// Control block reset + queue seeding, launched before every call.  Every
// word of the control block has exactly one writer here (the thread whose
// index it is), which stores the word's initial value directly.
DEV void reset_body(const Params& p, int gid, int stride) {
  const int ncw = CW_COUNT * kCtrlStride;
  for (int i = gid; i < ncw; i += stride)
    p.ctrl[i] = (i % kCtrlStride == 0) ? ctrl_init(p, i / kCtrlStride) : 0;
  const size_t ns = (size_t)kNumQueues * p.q_cap;
  const int n_route = p.n_route;
  const int n_fin = p.route_wide ? p.n_rt : 0;
  for (size_t i = gid; i < ns; i += stride) {
    const size_t q = i / p.q_cap, j = i % p.q_cap;
    int v = 0;
    if (q == QA && j < (size_t)n_route) v = make_task(TK_ROUTE, (int)j) + 1;
    else if (q == QA && j < (size_t)(n_route + n_fin)) v = make_task(TK_RFIN, (int)j - n_route) + 1;
    else if (q == QC && j < (size_t)p.n_sup) v = make_task(TK_SUP, (int)j) + 1;
    p.slots[i] = v;
  }
  // K slices outstanding per router tile (per 256-token group with route_wide)
  const int n_rc = p.route_wide ? p.n_rg : p.n_rt;
  for (int i = gid; i < n_rc; i += stride) p.cnt_route[i] = p.rsk;
  const int nsm = p.n_shared * p.n_smt;
  for (int i = gid; i < nsm; i += stride) p.cnt_sdown[i] = p.n_s_up_n + 1;
  // combine tiles: the shared DOWN tiles over their tokens, plus one unit
  // that the tile's POS task replaces by its routed DOWN tiles
  for (int i = gid; i < p.n_rt; i += stride) p.cnt_comb[i] = 1 + p.n_shared * p.n_down_n;
  // a token tile's NORM task waits for its combine column chunks
  for (int i = gid; i < p.n_rt; i += stride) p.cnt_norm[i] = p.n_cc;
  if (p.flags & (MOE_FLAG_XCD_AFFINITY | MOE_FLAG_LOCAL_QUEUES)) {
    const size_t nu = (size_t)kXcds * p.q_cap;
    for (size_t i = gid; i < nu; i += stride) p.uslots[i] = 0;
  }
}

__global__ __launch_bounds__(kThreads) void k_reset(Params p) {
  reset_body(p, blockIdx.x * kThreads + threadIdx.x, gridDim.x * kThreads);
}

// The same for several layers at once (blockIdx.y = layer; parameter blocks
// in device memory, read through the constant address space).
__global__ __launch_bounds__(kThreads) void k_reset_layers(const Params* layers) {
  ConstParams* lp = (ConstParams*)layers;
  const Params& p = *(const Params*)(lp + blockIdx.y);
  reset_body(p, blockIdx.x * kThreads + threadIdx.x, gridDim.x * kThreads);
}

}  // namespace moe

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxWorkersBound = 4096;  // queue slack for the largest grid
constexpr int kMaxLayers = 1024;        // layers per moe_layers call

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  Params p;          // geometry only (pointers filled by carve)
  int esz;
  size_t off_ctrl, off_slots, off_uslots, off_logits, off_idx, off_w, off_hist, off_counts,
      off_offsets, off_eorder, off_route_part, off_cnt_route, off_perm, off_rw, off_slotpos, off_mtiles, off_cnt_perm,
      off_cnt_down, off_cnt_sdown, off_perm_list, off_cnt_comb, off_cnt_norm, off_xp,
      off_h, off_hs,
      off_o, off_ys, total;
};

int validate(const moe_desc* d) {
  if (!d) return MOE_ERR_ARG;
  if (d->T < 0 || d->d <= 0 || d->E < 1 || d->E > kMaxE || d->k < 1 || d->k > kMaxK ||
      d->k > d->E || d->f <= 0)
    return MOE_ERR_ARG;
  const int e_end = d->e_end > 0 ? d->e_end : d->E;
  if (d->e_begin < 0 || e_end > d->E || d->e_begin >= e_end) return MOE_ERR_ARG;
  if (d->n_shared < 0 || d->n_shared > 4) return MOE_ERR_ARG;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ERR_ARG;
  if (d->mode < MOE_DYNAMIC || d->mode > MOE_MULTI_KERNEL) return MOE_ERR_ARG;
  if (d->split_policy < MOE_SPLIT_COST_MODEL || d->split_policy > MOE_SPLIT_NONE) return MOE_ERR_ARG;
  if (d->split_k < 0 || d->split_k > 8) return MOE_ERR_ARG;
  if (d->d % kBN || d->f % kBN) return MOE_ERR_UNSUPPORTED;
  if (d->n_shared > 0 && (d->f_shared <= 0 || d->f_shared % kBN)) return MOE_ERR_UNSUPPORTED;
  if ((d->flags & MOE_FLAG_TRACE) && (!d->trace || d->trace_cap <= 0)) return MOE_ERR_ARG;
  // the queue ids must fit the payload field
  const long long rows = (long long)d->T * d->k;
  const long long mt = rows / 128 + (e_end - d->e_begin);
  if (mt * (d->d / kBN) * 8 >= (1ll << kKindShift)) return MOE_ERR_UNSUPPORTED;
  if (mt * 128 >= (1ll << kKindShift)) return MOE_ERR_UNSUPPORTED;  // permute payloads
  if (d->row_tile != 0 && d->row_tile != 128 && d->row_tile != 256) return MOE_ERR_ARG;
  if (d->row_tile == 256 && d->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d->combine < MOE_COMBINE_AUTO || d->combine > MOE_COMBINE_TASKS) return MOE_ERR_ARG;
  if (d->bands < 0 || d->bands > kMaxBands) return MOE_ERR_ARG;
  if (d->claim_batch < 0 || d->claim_batch > 8) return MOE_ERR_ARG;
  // local continuation queues take the place of the per-XCD UP queues and
  // of the continuation-priority queue
  if ((d->flags & MOE_FLAG_LOCAL_QUEUES) &&
      (d->flags & (MOE_FLAG_XCD_AFFINITY | MOE_FLAG_CONT_PRIORITY)))
    return MOE_ERR_ARG;
  return MOE_OK;
}

void make_layout(const moe_desc* d, Layout* L) {
  Params& p = L->p;
  memset(&p, 0, sizeof p);
  p.T = d->T;
  p.d = d->d;
  p.E = d->E;
  p.k = d->k;
  p.f = d->f;
  p.e_begin = d->e_begin;
  const int e_end = d->e_end > 0 ? d->e_end : d->E;
  p.E_loc = e_end - d->e_begin;
  p.n_shared = d->n_shared;
  p.fs = d->n_shared > 0 ? d->f_shared : kBN;
  p.dtype = d->dtype;
  L->esz = d->dtype == MOE_BF16 ? 2 : 4;
  // the permute is fused into the UP tiles' row loads (x rows gathered
  // through perm) unless asked for as separate tasks; the bf16 tiles address
  // x with 32-bit per-lane byte offsets
  p.gather_a = !(d->flags & MOE_FLAG_EXPLICIT_PERMUTE) &&
               (d->dtype != MOE_BF16 || (long long)d->T * d->d * 2 + 65536 < (1ll << 32));
  p.n_rt = (d->T + kTB - 1) / kTB;
  p.hist_ld = std::max(4, (p.n_rt + 3) / 4 * 4);
  // Router tasks over 256-token groups on the 256-row tile (bf16, E = 128
  // or 256, at least 8 groups): K slices of a multiple of 32, at most 8,
  // about 256 tasks in all.  Otherwise over 32-token tiles: K slices enough
  // for ~256 router tasks, each slice at least 256 deep and a divisor of
  // d/64.
  p.route_wide = d->dtype == MOE_BF16 && (d->E == 128 || d->E == 256) && d->T >= 2048 &&
                 !(d->flags & MOE_FLAG_NARROW_ROUTER);
  p.n_rg = (d->T + 255) / 256;
  if (p.route_wide) {
    const int ksteps = d->d / 32;
    const int want = std::max(1, (256 + p.n_rg - 1) / p.n_rg);
    p.rsk = 1;
    for (int sl = 1; sl <= std::min(ksteps, Stages<bf16_t>::kMaxRouteSlicesWide); ++sl)
      if (ksteps % sl == 0 && sl <= want) p.rsk = sl;
  } else {
    const int ksteps = d->d / 64;
    const int want = std::max(1, (256 + std::max(p.n_rt, 1) - 1) / std::max(p.n_rt, 1));
    p.rsk = 1;
    for (int sl = 1; sl <= ksteps; ++sl)
      if (ksteps % sl == 0 && sl <= want && d->d / sl >= 256) p.rsk = sl;
  }
  p.n_route = (p.route_wide ? p.n_rg : p.n_rt) * p.rsk;
  // Expert row tiles: 256 rows for large bf16 layers (the 256 x 256 task
  // reads half the LDS bytes per MFMA flop of a 128-row one), 128 otherwise
  // (small layers need many tasks, and their experts hold few rows).
  // DOWN tasks then cover 256 columns when d allows.
  p.th = d->row_tile ? d->row_tile
                     : (d->dtype == MOE_BF16 && (long long)d->T * d->k > 8192 ? 256 : 128);
  p.down_nb = (p.th == 256 && d->d % 256 == 0) ? 2 : 1;
  p.n_up_n = d->f / kBN;
  p.n_down_n = d->d / (kBN * p.down_nb);
  int sk = d->split_k;
  // automatic DOWN split-K: one slice per 3584 of f (measured on the
  // decode-shaped f = 14336: 4 slices shorten the last wave of DOWN tasks,
  // the tail of an HBM-bound layer; 8 add more partial traffic than they save)
  if (sk == 0) sk = std::max(1, std::min(8, d->f / 3584));
  p.splitk = std::min(sk, p.n_up_n);
  p.n_s_up_n = p.fs / kBN;
  p.n_smt = (d->T + p.th - 1) / p.th;
  // rows per permute task: a power of two in [2, 128] moving at most 256 KB,
  // and small enough that a small layer's gather spreads over about two
  // tasks per CU (32 KB minimum per task)
  int pr = 128;
  {
    const long long row_bytes = (long long)d->d * L->esz;
    const long long total = (long long)d->T * d->k * row_bytes;
    const long long target = std::max(32768ll, std::min(262144ll, total / 512));
    while (pr > 2 && (long long)pr * row_bytes > target) pr >>= 1;
  }
  p.perm_rows = pr;
  // row-tile order: token bands (see the builder); 0 = automatic: one band
  // (plain expert-major order, measured fastest on the expert-share layer)
  p.bands = d->bands > 0 ? std::min(d->bands, kMaxBands) : 1;
  p.pch = p.th / pr;
  const long long R = (long long)d->T * d->k;
  p.max_mt = (int)(R / 128 + p.E_loc + 1);
  p.max_perm = (int)((R + pr - 1) / pr + p.max_mt);
  p.n_sup = p.n_shared * p.n_smt * p.n_s_up_n;
  p.n_sdown = p.n_shared * p.n_smt * p.n_down_n;
  // Combine: a layer with at most 4096 routed rows scatter-adds in the DOWN
  // epilogue (no extra stage after the last DOWN tile; measured faster on
  // the decode-shaped and 16-layer stress workloads); larger layers write O
  // rows and sum them per token in combine tasks (fixed order, none of the
  // atomic traffic on y that dominated large layers' DOWN time).
  p.comb_scatter = d->combine == MOE_COMBINE_SCATTER ||
                   (d->combine == MOE_COMBINE_AUTO && (long long)d->T * d->k <= 4096);
  // combine chunks: the widest of 512 / 256 / 128 columns that divides d
  // and still gives about two combine tasks per CU; small-T layers get
  // narrow chunks, so the combine that follows the last DOWN tile spreads
  // over the whole device
  p.comb_cols = 128;
  for (int cols = 512; cols > 128; cols >>= 1)
    if (d->d % cols == 0 && (long long)p.n_rt * (d->d / cols) >= 512) {
      p.comb_cols = cols;
      break;
    }
  p.n_cc = d->d / p.comb_cols;
  // O (the fp32 DOWN rows) larger than the 256 MiB last-level cache cannot
  // stay cached until the combine reads it: the DOWN tiles then write it with
  // streaming stores, so it does not displace the weight panels and A rows
  // that other tiles reuse.
  p.o_stream = !p.comb_scatter &&
               sizeof(float) * (size_t)p.splitk * d->T * d->k * d->d > ((size_t)256 << 20);
  const long long qa = (long long)p.n_route + (long long)p.n_rt * (p.route_wide ? 2 : 1);
  const long long qc = (long long)p.max_mt * (p.n_up_n + p.n_down_n * p.splitk) + p.n_sup +
                       p.n_sdown + p.max_perm + (long long)p.n_rt * p.n_cc;
  p.q_cap = (int)(std::max(qa, qc) + kMaxWorkersBound);

  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + std::max<size_t>(bytes, 1));
    return at;
  };
  const size_t Tk = (size_t)d->T * d->k;
  L->off_ctrl = take(sizeof(int) * CW_COUNT * kCtrlStride);
  L->off_slots = take(sizeof(int) * (size_t)kNumQueues * p.q_cap);
  L->off_uslots = take(sizeof(int) * (size_t)kXcds * p.q_cap);
  L->off_logits = take(sizeof(float) * (size_t)d->T * d->E);
  L->off_route_part = take(p.route_wide ? sizeof(float) * (size_t)p.rsk * d->T * d->E
                           : p.rsk > 1  ? sizeof(float) * (size_t)p.rsk * p.n_rt * kTB * d->E
                                        : 0);
  L->off_cnt_route = take(sizeof(int) * (size_t)std::max(1, p.n_rt));
  L->off_idx = take(sizeof(int) * Tk);
  L->off_w = take(sizeof(float) * Tk);
  L->off_hist = take(sizeof(int) * (size_t)p.E_loc * p.hist_ld);
  L->off_counts = take(sizeof(int) * p.E_loc);
  L->off_offsets = take(sizeof(int) * (p.E_loc + 1));
  L->off_eorder = take(sizeof(int) * p.E_loc);
  L->off_perm = take(sizeof(int) * Tk);
  L->off_rw = take(sizeof(float) * Tk);
  L->off_slotpos = take(sizeof(int) * Tk);
  L->off_mtiles = take(sizeof(MTile) * p.max_mt);
  L->off_cnt_perm = take(sizeof(int) * p.max_mt);
  L->off_cnt_down = take(sizeof(int) * (size_t)p.max_mt * p.splitk);
  L->off_cnt_sdown = take(sizeof(int) * (size_t)std::max(1, p.n_shared * p.n_smt));
  L->off_perm_list = take(sizeof(int) * p.max_perm);
  L->off_cnt_comb = take(sizeof(int) * (size_t)std::max(1, p.n_rt));
  L->off_cnt_norm = take(sizeof(int) * (size_t)std::max(1, p.n_rt));
  L->off_xp = take(p.gather_a ? 0 : (size_t)L->esz * Tk * d->d);
  L->off_h = take((size_t)L->esz * Tk * d->f);
  L->off_hs = take((size_t)L->esz * d->n_shared * d->T * (d->n_shared ? d->f_shared : 0));
  L->off_o = take(sizeof(float) * (size_t)p.splitk * Tk * d->d);
  L->off_ys = take(sizeof(float) * (size_t)d->n_shared * d->T * d->d);
  L->total = o;
}

void carve(Layout* L, void* ws) {
  Params& p = L->p;
  char* b = static_cast<char*>(ws);
  p.ctrl = reinterpret_cast<int*>(b + L->off_ctrl);
  p.slots = reinterpret_cast<int*>(b + L->off_slots);
  p.uslots = reinterpret_cast<int*>(b + L->off_uslots);
  p.logits = reinterpret_cast<float*>(b + L->off_logits);
  p.route_part = reinterpret_cast<float*>(b + L->off_route_part);
  p.cnt_route = reinterpret_cast<int*>(b + L->off_cnt_route);
  p.idx = reinterpret_cast<int*>(b + L->off_idx);
  p.w = reinterpret_cast<float*>(b + L->off_w);
  p.hist = reinterpret_cast<int*>(b + L->off_hist);
  p.counts = reinterpret_cast<int*>(b + L->off_counts);
  p.offsets = reinterpret_cast<int*>(b + L->off_offsets);
  p.eorder = reinterpret_cast<int*>(b + L->off_eorder);
  p.perm = reinterpret_cast<int*>(b + L->off_perm);
  p.rw = reinterpret_cast<float*>(b + L->off_rw);
  p.slot_pos = reinterpret_cast<int*>(b + L->off_slotpos);
  p.mtiles = reinterpret_cast<MTile*>(b + L->off_mtiles);
  p.cnt_perm = reinterpret_cast<int*>(b + L->off_cnt_perm);
  p.cnt_down = reinterpret_cast<int*>(b + L->off_cnt_down);
  p.cnt_sdown = reinterpret_cast<int*>(b + L->off_cnt_sdown);
  p.perm_list = reinterpret_cast<int*>(b + L->off_perm_list);
  p.cnt_comb = reinterpret_cast<int*>(b + L->off_cnt_comb);
  p.cnt_norm = reinterpret_cast<int*>(b + L->off_cnt_norm);
  p.O = reinterpret_cast<float*>(b + L->off_o);
  p.Ys = reinterpret_cast<float*>(b + L->off_ys);
  p.Xp = b + L->off_xp;
  p.H = b + L->off_h;
  p.Hs = b + L->off_hs;
}

// Resident persistent workgroups per CU for each kernel, per device.
struct DevInfo {
  int cus = 0;
  int bpc[2][2] = {{0, 0}, {0, 0}};  // [dtype][dynamic, static]
};
std::mutex g_mu;
DevInfo g_dev[64];

int dev_info(int dev, DevInfo* out) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (dev < 0 || dev >= 64) return MOE_ERR_HIP;
  DevInfo& di = g_dev[dev];
  if (di.cus == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return MOE_ERR_HIP;
    int b = 0;
    if (occupancy_dynamic_f32(&b) != hipSuccess) return MOE_ERR_HIP;
    di.bpc[0][0] = b;
    if (occupancy_static_f32(&b) != hipSuccess) return MOE_ERR_HIP;
    di.bpc[0][1] = b;
    if (occupancy_dynamic_bf16(&b) != hipSuccess) return MOE_ERR_HIP;
    di.bpc[1][0] = b;
    if (occupancy_static_bf16(&b) != hipSuccess) return MOE_ERR_HIP;
    di.bpc[1][1] = b;
    di.cus = cus;
  }
  *out = di;
  return MOE_OK;
}

int workers_for(const moe_desc* d, int* workers, int* cus, int* bpc) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  DevInfo di;
  int rc = dev_info(dev, &di);
  if (rc) return rc;
  const int b = di.bpc[d->dtype == MOE_BF16][d->mode == MOE_STATIC_PARTITION];
  if (b < 1) return MOE_ERR_UNSUPPORTED;
  int w = di.cus * b;
  if (d->max_workers > 0) w = std::min(w, d->max_workers);
  *workers = std::min(w, kMaxWorkersBound);
  if (cus) *cus = di.cus;
  if (bpc) *bpc = b;
  return MOE_OK;
}

#define HIP_OK(x)                          \
  do {                                     \
    if ((x) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

int launch_reset(const Params& p, hipStream_t s) {
  const int reset_blocks = (int)std::min<long long>(
      1024, ((long long)kNumQueues * p.q_cap + kThreads - 1) / kThreads + 1);
  hipLaunchKernelGGL(k_reset, dim3(reset_blocks), dim3(kThreads), 0, s, p);
  HIP_OK(hipGetLastError());
  return MOE_OK;
}

int launch_layer(const moe_desc* d, const Params& p, hipStream_t s) {
  int rc = launch_reset(p, s);
  if (rc) return rc;
  const bool bf16 = d->dtype == MOE_BF16;
  const bool scat = p.comb_scatter != 0;
  hipError_t e;
  if (d->mode == MOE_DYNAMIC)
    e = bf16 ? (scat ? launch_dynamic_bf16_scatter(p, s) : launch_dynamic_bf16_rows(p, s))
             : launch_dynamic_f32(scat, p, s);
  else if (d->mode == MOE_STATIC_PARTITION)
    e = bf16 ? launch_static_bf16(scat, p, s) : launch_static_f32(scat, p, s);
  else
    e = bf16 ? launch_stages_bf16(p, s) : launch_stages_f32(p, s);
  HIP_OK(e);
  return MOE_OK;
}

int copy_routing(const moe_desc* d, const Params& p, const moe_routing* r, hipStream_t s) {
  if (!r) return MOE_OK;
  const size_t Tk = (size_t)d->T * d->k;
  auto cp = [&](void* dst, const void* src, size_t bytes) {
    if (!dst || bytes == 0) return hipSuccess;
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
  };
  HIP_OK(cp(r->logits, p.logits, sizeof(float) * d->T * d->E));
  HIP_OK(cp(r->topk_idx, p.idx, sizeof(int) * Tk));
  HIP_OK(cp(r->topk_w, p.w, sizeof(float) * Tk));
  HIP_OK(cp(r->expert_counts, p.counts, sizeof(int) * p.E_loc));
  HIP_OK(cp(r->offsets, p.offsets, sizeof(int) * (p.E_loc + 1)));
  HIP_OK(cp(r->perm, p.perm, sizeof(int) * Tk));
  HIP_OK(cp(r->slot_pos, p.slot_pos, sizeof(int) * Tk));
  return MOE_OK;
}

// Cost-model constants, measured once on MI355X and frozen (bench.py reports
// the same quantities re-measured from a task trace beside them): the
// sustained per-CU MFMA rate in expert tiles, the bytes/s one worker moves in
// a gather task, and the device HBM bandwidth a streaming tile sustains.
void set_cost_model(const moe_desc* d, Params* p) {
  p->cm_mfma_rate = (d->dtype == MOE_BF16 ? 4.3e12f : 0.3e12f);
  p->cm_cu_bw = 26e9f;
  p->cm_hbm_bw = 6.0e12f;
}

int fill_params(const moe_desc* d, Layout* L, void* ws, size_t ws_bytes) {
  int rc = validate(d);
  if (rc) return rc;
  make_layout(d, L);
  if (!ws || ws_bytes < L->total) return MOE_ERR_WORKSPACE;
  carve(L, ws);
  Params& p = L->p;
  rc = workers_for(d, &p.workers, nullptr, nullptr);
  if (rc) return rc;
  p.mode = d->mode;
  p.split_policy = d->split_policy;
  p.fixed_mem = d->fixed_mem_workers;
  p.flags = d->flags;
  if (!(p.flags & MOE_FLAG_REF_SYNC)) p.flags |= MOE_FLAG_PHASE_SYNC;
  const long long ms = d->timeout_ms > 0 ? d->timeout_ms : 2000;
  p.timeout_ticks = ms * 100000ll;  // 100 MHz constant clock
  if (d->timeout_ticks > 0) p.timeout_ticks = d->timeout_ticks;
  p.claim_batch = d->claim_batch > 0 ? d->claim_batch : 1;
  set_cost_model(d, &p);
  p.trace = (d->flags & MOE_FLAG_TRACE) ? d->trace : nullptr;
  p.trace_cap = d->trace_cap;
  return MOE_OK;
}

int run_layer(const moe_desc* d, const void* x, const moe_weights* w, const float* residual,
              const float* norm_weight, float norm_eps, float* y, void* y_norm,
              const moe_routing* routing, void* workspace, size_t ws_bytes, void* stream) {
  Layout L;
  int rc = fill_params(d, &L, workspace, ws_bytes);
  if (rc) return rc;
  if (d->T == 0) return MOE_OK;
  if (!x || !w || !y || !w->w_router || !w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_ARG;
  if (d->n_shared > 0 && (!w->ws_gate || !w->ws_up || !w->ws_down)) return MOE_ERR_ARG;
  Params& p = L.p;
  p.x = x;
  p.wr = w->w_router;
  p.bias = w->router_bias;
  p.wg = w->w_gate;
  p.wu = w->w_up;
  p.wd = w->w_down;
  p.sg = w->ws_gate;
  p.su = w->ws_up;
  p.sd = w->ws_down;
  p.y = y;
  p.resid = residual;
  p.norm_w = norm_weight;
  p.y_norm = y_norm;
  p.norm_eps = norm_eps;
  p.fuse_norm = y_norm != nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = launch_layer(d, p, s);
  if (rc) return rc;
  rc = copy_routing(d, p, routing, s);
  if (rc) return rc;
  if (d->flags & MOE_FLAG_CHECK) return moe_last_device_error(d, workspace, stream);
  return MOE_OK;
}

// ------------------------------------------- no-allocation entry point
// The workspace of moe_layer_no_alloc: a fixed device array of this library,
// one per GPU the library runs on, held until the process ends.  Host code
// never uses the array's name as an address (it is only a host-side handle):
// its device address comes from hipGetSymbolAddress, once per device, with
// that device current, and is kept per device.
constexpr size_t kScratchBytes = MOE_NO_ALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % kAlign == 0, "scratch size");

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch[64] = {};

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return MOE_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layer_no_alloc(const moe_desc* d, const void* x, const moe_weights* w, float* y,
                       const moe_routing* routing, void* stream) {
  const size_t need = moe_workspace_size(d);
  if (need == 0) return MOE_ERR_ARG;
  if (need > kScratchBytes) return MOE_ERR_TOO_LARGE;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc) return rc;
  return run_layer(d, x, w, nullptr, nullptr, 0.f, y, nullptr, routing, ws, need, stream);
}


size_t moe_workspace_size(const moe_desc* d) {
  if (validate(d) != MOE_OK) return 0;
  Layout L;
  make_layout(d, &L);
  return L.total;
}

int moe_query(const moe_desc* d, moe_info* info) {
  int rc = validate(d);
  if (rc) return rc;
  if (!info) return MOE_ERR_ARG;
  Layout L;
  make_layout(d, &L);
  memset(info, 0, sizeof *info);
  rc = workers_for(d, &info->workers, &info->cus, &info->blocks_per_cu);
  if (rc) return rc;
  info->route_tiles = L.p.n_rt;
  info->up_ntiles = L.p.n_up_n;
  info->down_ntiles = L.p.n_down_n;
  info->split_k = L.p.splitk;
  info->permute_rows = L.p.perm_rows;
  info->max_mtiles = L.p.max_mt;
  info->max_tasks = L.p.q_cap;
  info->route_splits = L.p.rsk;
  info->route_groups = L.p.route_wide ? L.p.n_rg : 0;
  info->combine_chunks = L.p.n_cc;
  info->row_tile = L.p.th;
  info->combine = L.p.comb_scatter ? MOE_COMBINE_SCATTER : MOE_COMBINE_TASKS;
  info->workspace_bytes = L.total;
  set_cost_model(d, &L.p);
  info->cost_mfma_flops_per_cu = L.p.cm_mfma_rate;
  info->cost_gather_bytes_per_worker = L.p.cm_cu_bw;
  info->cost_hbm_bytes = L.p.cm_hbm_bw;
  info->bands = L.p.bands;
  info->gather_fused = L.p.gather_a;
  return MOE_OK;
}

// Several layers: the parameter blocks first, then each layer's workspace.
size_t layers_params_bytes(int n) { return align_up(sizeof(Params) * (size_t)n); }

size_t moe_layers_workspace_size(const moe_desc* d, int n) {
  if (!d || n < 1 || n > kMaxLayers) return 0;
  size_t total = layers_params_bytes(n);
  for (int l = 0; l < n; ++l) {
    const size_t b = moe_workspace_size(d + l);
    if (b == 0) return 0;
    total += align_up(b);
  }
  return total;
}

int moe_layers(const moe_desc* d, int n, const void* const* x, const moe_weights* w,
               float* const* y, const moe_routing* routing, void* workspace, size_t ws_bytes,
               void* stream) {
  if (!d || n < 1 || n > kMaxLayers || !x || !w || !y) return MOE_ERR_ARG;
  const size_t need = moe_layers_workspace_size(d, n);
  if (need == 0) return MOE_ERR_ARG;
  if (!workspace || ws_bytes < need) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(workspace);
  size_t off = layers_params_bytes(n);
  std::vector<Params> ps;
  std::vector<int> which;
  ps.reserve(n);
  which.reserve(n);
  bool one_launch = true;
  for (int l = 0; l < n; ++l) {
    const size_t wl = align_up(moe_workspace_size(d + l));
    Layout L;
    int rc = fill_params(d + l, &L, base + off, wl);
    if (rc) return rc;
    off += wl;
    if (d[l].T == 0) continue;
    const moe_weights* wt = w + l;
    if (!x[l] || !y[l] || !wt->w_router || !wt->w_gate || !wt->w_up || !wt->w_down)
      return MOE_ERR_ARG;
    if (d[l].n_shared > 0 && (!wt->ws_gate || !wt->ws_up || !wt->ws_down)) return MOE_ERR_ARG;
    Params& p = L.p;
    p.x = x[l];
    p.wr = wt->w_router;
    p.bias = wt->router_bias;
    p.wg = wt->w_gate;
    p.wu = wt->w_up;
    p.wd = wt->w_down;
    p.sg = wt->ws_gate;
    p.su = wt->ws_up;
    p.sd = wt->ws_down;
    p.y = y[l];
    if (d[l].mode != MOE_DYNAMIC || d[l].dtype != d[0].dtype) one_launch = false;
    if (!ps.empty() && p.workers != ps[0].workers) one_launch = false;
    ps.push_back(p);
    which.push_back(l);
  }
  if (ps.empty()) return MOE_OK;
  if (!one_launch) {
    // the baselines (and mixed element types) run layer by layer
    for (size_t i = 0; i < ps.size(); ++i) {
      int rc = launch_layer(d + which[i], ps[i], s);
      if (rc) return rc;
    }
  } else {
    // parameter blocks to the device (pageable source: the copy is staged
    // before the call returns), then one persistent launch per run of
    // consecutive layers with the same combine mode
    Params* dev_ps = reinterpret_cast<Params*>(base);
    HIP_OK(hipMemcpyAsync(dev_ps, ps.data(), sizeof(Params) * ps.size(), hipMemcpyHostToDevice, s));
    const bool bf16 = d[which[0]].dtype == MOE_BF16;
    size_t a = 0;
    while (a < ps.size()) {
      size_t b = a + 1;
      while (b < ps.size() && ps[b].comb_scatter == ps[a].comb_scatter) ++b;
      long long qmax = 0;
      for (size_t i = a; i < b; ++i) qmax = std::max<long long>(qmax, (long long)kNumQueues * ps[i].q_cap);
      const int reset_blocks = (int)std::min<long long>(1024, (qmax + kThreads - 1) / kThreads + 1);
      hipLaunchKernelGGL(k_reset_layers, dim3(reset_blocks, (unsigned)(b - a)), dim3(kThreads), 0, s,
                         dev_ps + a);
      HIP_OK(hipGetLastError());
      const bool scat = ps[a].comb_scatter != 0;
      HIP_OK(bf16 ? launch_dynamic_layers_bf16(scat, dev_ps + a, (int)(b - a), ps[a].workers, s)
                  : launch_dynamic_layers_f32(scat, dev_ps + a, (int)(b - a), ps[a].workers, s));
      a = b;
    }
  }
  for (size_t i = 0; i < ps.size(); ++i) {
    if (!routing) break;
    int rc = copy_routing(d + which[i], ps[i], routing + which[i], s);
    if (rc) return rc;
  }
  if (d[0].flags & MOE_FLAG_CHECK) {
    HIP_OK(hipStreamSynchronize(s));
    for (size_t i = 0; i < ps.size(); ++i) {
      int err = 0;
      HIP_OK(hipMemcpy(&err, reinterpret_cast<const char*>(ps[i].ctrl) + sizeof(int) * CW_ERROR * kCtrlStride,
                       sizeof(int), hipMemcpyDeviceToHost));
      if (err) return err;
    }
  }
  return MOE_OK;
}

int moe_layer(const moe_desc* d, const void* x, const moe_weights* w, float* y,
              const moe_routing* routing, void* workspace, size_t ws_bytes, void* stream) {
  return run_layer(d, x, w, nullptr, nullptr, 0.f, y, nullptr, routing, workspace, ws_bytes,
                   stream);
}

int moe_layer_norm(const moe_desc* d, const void* x, const moe_weights* w,
                   const float* residual, const float* norm_weight, float norm_eps, float* y,
                   void* y_norm, const moe_routing* routing, void* workspace, size_t ws_bytes,
                   void* stream) {
  if (!norm_weight || !y_norm || !(norm_eps >= 0.f)) return MOE_ERR_ARG;
  return run_layer(d, x, w, residual, norm_weight, norm_eps, y, y_norm, routing, workspace,
                   ws_bytes, stream);
}

int moe_route_from_logits(const moe_desc* d, const float* logits, const moe_routing* routing,
                          void* workspace, size_t ws_bytes, void* stream) {
  Layout L;
  int rc = fill_params(d, &L, workspace, ws_bytes);
  if (rc) return rc;
  if (d->T == 0) return MOE_OK;
  if (!logits) return MOE_ERR_ARG;
  Params& p = L.p;
  p.route_from_logits = 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIP_OK(hipMemcpyAsync(p.logits, logits, sizeof(float) * d->T * d->E, hipMemcpyDeviceToDevice, s));
  rc = launch_reset(p, s);
  if (rc) return rc;
  HIP_OK(d->dtype == MOE_BF16 ? launch_route_only_bf16(p, s) : launch_route_only_f32(p, s));
  rc = copy_routing(d, p, routing, s);
  if (rc) return rc;
  if (d->flags & MOE_FLAG_CHECK) return moe_last_device_error(d, workspace, stream);
  return MOE_OK;
}

int moe_last_device_error(const moe_desc* d, const void* workspace, void* stream) {
  if (validate(d) != MOE_OK || !workspace) return MOE_ERR_ARG;
  Layout L;
  make_layout(d, &L);
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIP_OK(hipStreamSynchronize(s));
  int err = 0;
  const char* base = static_cast<const char*>(workspace) + L.off_ctrl;
  HIP_OK(hipMemcpy(&err, base + sizeof(int) * CW_ERROR * kCtrlStride, sizeof(int),
                   hipMemcpyDeviceToHost));
  return err;
}

int moe_last_schedule(const moe_desc* d, const void* workspace, void* stream, moe_schedule* out) {
  if (validate(d) != MOE_OK || !workspace || !out) return MOE_ERR_ARG;
  Layout L;
  make_layout(d, &L);
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIP_OK(hipStreamSynchronize(s));
  int cw[CW_COUNT * kCtrlStride];
  HIP_OK(hipMemcpy(cw, static_cast<const char*>(workspace) + L.off_ctrl, sizeof cw,
                   hipMemcpyDeviceToHost));
  out->mem_workers = cw[CW_WMEM * kCtrlStride];
  out->row_tiles = cw[CW_NMT * kCtrlStride];
  out->permute_tasks = cw[CW_NPERM * kCtrlStride];
  out->error = cw[CW_ERROR * kCtrlStride];
  return MOE_OK;
}

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape (d, f and f_shared must be multiples of 128)";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_TIMEOUT: return "device watchdog timeout";
    case MOE_ERR_CAPACITY: return "device table capacity exceeded";
    case MOE_ERR_NONFINITE: return "non-finite router logit";
    case MOE_ERR_TOO_LARGE: return "layer needs more workspace than the library's static scratch";
    default: return "unknown error";
  }
}

}  // extern "C"
