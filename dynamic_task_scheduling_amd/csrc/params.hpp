// params.hpp -- the launch-parameter block (host and device) and the task /
// queue / control-word encodings of the persistent scheduler.
#pragma once
#include <stdint.h>

namespace moe {

// Task kinds.  A task id packs the kind in bits [30:27] and a payload below.
enum TaskKind : int {
  TK_ROUTE = 1,  // payload rt * rsk + ks: router K slice ks of tokens [32 rt, 32 rt + 32);
                 // with 256-token router groups, g * rsk + ks: of tokens [256 g, 256 g + 256)
  TK_POS = 2,    // payload rt: stable positions of those tokens' slots
  TK_PERM = 3,   // payload mt * pch + c: gather rows chunk c of row-tile mt
  TK_UP = 4,     // payload mt * n_up_n + n: gate/up GEMM + SiLU-gate epilogue
  TK_DOWN = 5,   // payload (mt * n_down_n + n) * splitk + ks: DOWN GEMM -> O rows
  TK_SUP = 6,    // payload (s * n_smt + m) * n_s_up_n + n: shared-expert UP
  TK_SDOWN = 7,  // payload (s * n_smt + m) * n_down_n + n: shared-expert DOWN -> Ys rows
  TK_BUILD = 8,  // (trace only) scheduler phases: payload = kPhase* id
  TK_COMB = 9,   // payload rt * n_cc + cc: y rows of tokens [32 rt, 32 rt + 32), column chunk cc
  TK_NORM = 10,  // payload rt: RMSNorm of the (residual-added) y rows of tokens [32 rt, 32 rt + 32)
  TK_RFIN = 11,  // payload rt: sum of the router K slices of tokens [32 rt, 32 rt + 32), then top-k
};
// Trace phase ids (payload of TK_BUILD records).
constexpr int kPhaseBuild = 0;          // the whole post-routing builder
constexpr int kPhasePublish = 1;        // publishing its tables, seeding queues
constexpr int kPhaseBuildStep = 2;      // + s: builder step s (1..4)
constexpr int kPhaseRouteFinish = 0x100;  // + rt: router partial reduction of tile rt
constexpr int kKindShift = 27;
constexpr int kPayloadMask = (1 << kKindShift) - 1;
__host__ __device__ inline int make_task(int kind, int payload) {
  return (kind << kKindShift) | payload;
}
__host__ __device__ inline int task_kind(int id) { return id >> kKindShift; }
__host__ __device__ inline int task_payload(int id) { return id & kPayloadMask; }

// Ready queues.
// Ready queues.  QA: router and position tiles; QM: permute (gather) tasks;
// QC: new expert work (UP tiles, shared-expert UP tiles); QH: continuation
// work (DOWN tiles, shared DOWN tiles, combine and NORM tasks), taken before
// QC so that started row tiles finish first.
enum Queue : int { QA = 0, QM = 1, QC = 2, QH = 3, kNumQueues = 4 };

// Control words; each sits on its own 128-byte line (index * kCtrlStride).
enum CtrlWord : int {
  CW_HEAD = 0,         // + queue
  CW_TAIL = 4,         // + queue
  CW_TOTAL = 8,        // + queue: tasks that will ever enter the queue
  CW_ROUTE_DONE = 12,
  CW_POS_DONE = 13,
  CW_SPLIT_READY = 14, // 1 once the task builder has published its tables
  CW_WMEM = 15,        // memory-bound worker count chosen by the cost model
  CW_ROLE = 16,        // role tickets handed out after the routing phase
  CW_TICKET = 17,      // worker tickets (dynamic worker ids)
  CW_ERROR = 18,       // first device error code
  CW_NMT = 19,         // expert row tiles
  CW_NPERM = 20,       // permute tasks
  CW_BAR_COUNT = 21,   // grid barrier (static mode)
  CW_BAR_GEN = 22,
  CW_TRACE = 23,       // trace cursor
  CW_UHEAD = 24,       // + XCD: per-XCD UP queues (XCD affinity)
  CW_UTAIL = 32,       // + XCD
  CW_UTOTAL = 40,      // + XCD
  CW_LTOTAL = 48,      // local queues: continuation tasks that will be pushed
  CW_LCLAIMED = 49,    // local queues: continuation tasks claimed so far
  CW_COUNT = 50
};
constexpr int kXcds = 8;   // MI355X: 8 XCDs, each with its own L2
constexpr int kMaxBands = 4;  // token bands of the row-tile order
constexpr int kCtrlStride = 32;

struct MTile {
  int e;     // local expert
  int row0;  // first row in the expert-contiguous buffers
  int rows;  // valid rows (<= bm)
  int bm;    // tile height class: 32, 64, 128 or 256
};

struct Params {
  // shape
  int T, d, E, k, f, e_begin, E_loc, n_shared, fs;
  int dtype;
  // derived geometry
  int n_rt;        // router / position tiles of 32 tokens
  int rsk;         // router K slices (divides d / 64)
  int route_wide;  // 1: router tasks are 256-token groups x K slices on the 256-row
                  //    tile, each 32-token tile then summed and routed by a TK_RFIN task
  int n_rg;        // router groups of 256 tokens (route_wide)
  int n_route;     // router GEMM tasks: n_rt * rsk, or n_rg * rsk (route_wide)
  int hist_ld;     // row stride of hist (n_rt rounded up to 4)
  int th;          // expert row-tile height: 128 or 256 rows
  int n_up_n;      // f / 128
  int down_nb;     // 128-column blocks per DOWN task: 1 or 2
  int n_down_n;    // DOWN column tasks = d / (128 * down_nb)
  int splitk;      // DOWN split-K slices
  int n_s_up_n;    // fs / 128
  int n_smt;       // shared-expert row tiles of th tokens
  int perm_rows;   // rows per permute task (divides 128)
  int pch;         // permute chunks per row tile = th / perm_rows
  int max_mt;      // capacity of the row-tile table
  int max_perm;    // capacity of the permute list
  int bands;       // token bands of the row-tile order (1..kMaxBands)
  int n_sup, n_sdown;
  int gather_a;     // 1: UP tiles gather their rows from x through perm (no
                    //    permute tasks, no Xp); 0: permute tasks fill Xp
  int comb_scatter; // 1: DOWN tiles scatter-add w * (H Wd) into y (small layers);
                    // 0: DOWN tiles write O rows, combine tasks sum them
  int o_stream;    // 1: O is larger than the last-level cache, so DOWN tiles
                   //    write it with streaming (non-temporal) stores
  int comb_cols;   // y columns per combine task (divides d)
  int n_cc;        // combine chunks per token tile = d / comb_cols
  int q_cap;       // slots per queue
  // scheduling
  int workers;
  int mode, split_policy, fixed_mem;
  unsigned flags;
  int claim_batch;      // compute-queue slots one claim reserves (1..8)
  long long timeout_ticks;
  float cm_mfma_rate;   // cost model: sustained MFMA flop/s per CU
  float cm_cu_bw;       // cost model: bytes/s one CU moves in a gather
  float cm_hbm_bw;      // cost model: device bytes/s
  // inputs
  const void* x;
  const void* wr;
  const float* bias;
  const void* wg;
  const void* wu;
  const void* wd;
  const void* sg;
  const void* su;
  const void* sd;
  float* y;
  // workspace
  int* ctrl;
  int* slots;      // [kNumQueues][q_cap]
  int* uslots;     // [kXcds][q_cap] per-XCD queues (XCD affinity, local queues)
  float* logits;   // [T][E]
  float* route_part;  // router partial sums (rsk > 1): [n_rt][rsk][32][E], or
                      // [rsk][T][E] with route_wide
  int* cnt_route;  // [n_rt] router slices still running
  int* idx;        // [T][k]
  float* w;        // [T][k]
  int* hist;       // [E_loc][hist_ld]
  int* counts;     // [E_loc]
  int* offsets;    // [E_loc + 1]
  int* eorder;     // [E_loc] local experts by descending count
  int* perm;       // [T*k]
  float* rw;       // [T*k]
  int* slot_pos;   // [T*k]
  MTile* mtiles;   // [max_mt]
  int* cnt_perm;   // [max_mt]
  int* cnt_down;   // [max_mt * splitk]
  int* cnt_sdown;  // [n_shared * n_smt]
  int* perm_list;  // [max_perm]
  int* cnt_comb;   // [n_rt] DOWN / shared-DOWN tiles a combine tile still waits for
  void* Xp;        // [T*k][d]
  void* H;         // [T*k][f]
  void* Hs;        // [n_shared][T][fs]
  float* O;        // [splitk][T*k][d] fp32 DOWN output rows (per K slice)
  float* Ys;       // [n_shared][T][d] fp32 shared-expert DOWN output
  // fused block tail (residual add + RMSNorm of the layer output)
  const float* resid;    // [T][d] fp32 added to y, or null
  const float* norm_w;   // [d] fp32 RMSNorm weight
  void* y_norm;          // [T][d] Elem: RMSNorm(y) * norm_w
  float norm_eps;
  int fuse_norm;         // 1: NORM tasks follow the combine
  int* cnt_norm;         // [n_rt] combine chunks a NORM task still waits for
  uint64_t* trace; // [trace_cap][4]
  int trace_cap;
  int route_from_logits;  // 1: logits are an input, y untouched
};

}  // namespace moe
