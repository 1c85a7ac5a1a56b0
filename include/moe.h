/*
 * moe.h -- C ABI of the MI355X (gfx950) Mixture-of-Experts megakernel library.
 *
 * One call runs a whole MoE layer on one GPU:
 *   router GEMM -> softmax top-k -> stable count/scan/positions of every
 *   (token, expert) slot in expert-contiguous order -> per-expert SwiGLU
 *   GEMM tasks (bf16 MFMA, x rows gathered through the positions in the
 *   tile's loader, fused SiLU-gate epilogue) -> weighted per-token combine of
 *   the experts' output rows (fixed order, no atomics; small layers
 *   scatter-add in the DOWN epilogue instead) -> optionally the residual add
 *   and RMSNorm (moe_layer_norm).
 *
 * The stages are those the Weave pages place inside one persistent MoE
 * kernel (xxqk.cn/news/665650 section 1; m.xxqk.cn/news/657744 section 2.1).
 * The default mode runs them as ONE persistent kernel whose workgroups claim
 * ready tasks from atomic queues (xxqk.cn/news/665650 section 2.1, the
 * TaskQueue / fetch_task scheme), with per-task dependency counters instead
 * of global barriers (same page, section 2.3; m.xxqk.cn/news/657744 section
 * 2.3), and a post-routing cost model that decides whether to split the
 * workers into a memory-bound group (the gather = the local stand-in for
 * expert-parallel dispatch, as separate tasks with MOE_FLAG_EXPLICIT_PERMUTE)
 * and an MFMA-bound group (expert GEMMs), per the spatial and temporal
 * schedulers of the Weave abstract (arxivdaily.com/papers/2609.21483); with
 * the gather fused into the GEMM tiles (the default) there is no memory-bound
 * task to split off.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, row-major, owned by the caller.
 *    The library allocates nothing and keeps no per-call state: everything
 *    it needs lives in the caller's workspace (sized by moe_workspace_size),
 *    so a call can be captured in a HIP graph.
 *  - Calls are asynchronous on `hip_stream` (a hipStream_t, NULL = default
 *    stream).  Argument errors are returned synchronously before anything is
 *    launched.  Errors found on the device (watchdog timeout, non-finite
 *    logit) are written to the workspace; read them with
 *    moe_last_device_error after synchronising, or set MOE_FLAG_CHECK to
 *    have moe_layer synchronise and return them.
 *  - A workspace may be used by one call at a time.
 */
#ifndef DTS_MOE_H
#define DTS_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of x, the expert weights, the router weights and the
 * intermediate buffers.  Accumulation is always fp32; y is always fp32. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Scheduling mode.  Every mode runs the same device tile code and gives the
 * same routing bit for bit; with MOE_COMBINE_TASKS (each output row summed
 * over its experts by one combine task, in slot order) also the same y, bit
 * for bit; with MOE_COMBINE_SCATTER y differs by fp32 summation order.
 *  MOE_DYNAMIC           one persistent kernel, dependency-driven ready
 *                        queues, count-sized worker split (the method).
 *  MOE_STATIC_PARTITION  one persistent kernel, tasks pre-assigned to
 *                        workers round-robin, fixed worker split, a grid
 *                        barrier between stages (the static fused kernel the
 *                        pages compare against, xxqk.cn/news/665650 s3.2).
 *  MOE_MULTI_KERNEL      one ordinary launch per stage on the stream; each
 *                        launch boundary is the only synchronisation
 *                        (xxqk.cn/news/665650 section 1.2). */
typedef enum {
  MOE_DYNAMIC = 0,
  MOE_STATIC_PARTITION = 1,
  MOE_MULTI_KERNEL = 2
} moe_mode;

/* How the persistent kernel sizes the memory-bound worker group.
 *  MOE_SPLIT_COST_MODEL  from the per-expert counts, after routing.
 *  MOE_SPLIT_FIXED       desc.fixed_mem_workers (default: workers / 8).
 *  MOE_SPLIT_NONE        one ready queue shared by every worker. */
typedef enum {
  MOE_SPLIT_COST_MODEL = 0,
  MOE_SPLIT_FIXED = 1,
  MOE_SPLIT_NONE = 2
} moe_split_policy;

/* How the weighted combine of the experts' rows is done.
 *  MOE_COMBINE_AUTO     scatter-add when T * k <= 4096, else tasks.
 *  MOE_COMBINE_SCATTER  each DOWN tile adds w * (H Wd) into y with fp32
 *                       atomics (y zeroed by the router tasks); the last
 *                       bits of y then depend on the order of the atomics.
 *  MOE_COMBINE_TASKS    DOWN tiles write fp32 rows; one combine task per
 *                       32 tokens and column chunk sums a token's experts in
 *                       slot order once all their DOWN tiles are done; y is
 *                       the same bit for bit in every mode and run. */
typedef enum {
  MOE_COMBINE_AUTO = 0,
  MOE_COMBINE_SCATTER = 1,
  MOE_COMBINE_TASKS = 2
} moe_combine;

/* Flags. */
#define MOE_FLAG_CHECK 0x1u      /* synchronise and return device errors   */
#define MOE_FLAG_TRACE 0x2u      /* record per-task timestamps in desc.trace */
#define MOE_FLAG_PHASE_SYNC 0x4u /* static mode: barriers between stages (default on) */
#define MOE_FLAG_REF_SYNC 0x8u   /* static mode: per-task counter waits instead of barriers */
#define MOE_FLAG_NO_STEAL 0x10u  /* dynamic split: compute workers never take permute tasks */
#define MOE_FLAG_XCD_AFFINITY 0x20u /* dynamic: UP tasks of column tile n on XCD n % 8's queue */
#define MOE_FLAG_FIFO 0x40u      /* dynamic: one compute queue in push order (the default;
                                    overrides MOE_FLAG_CONT_PRIORITY)       */
#define MOE_FLAG_CONT_PRIORITY 0x80u /* dynamic: continuation work (DOWN, shared DOWN, combine,
                                        NORM) in its own queue, served first */
#define MOE_FLAG_LOCAL_QUEUES 0x100u /* dynamic: continuation work in the local queue of the
                                        XCD that made it ready; workers take their own XCD's
                                        first, then the global queue, then steal from other
                                        XCDs (xxqk.cn/news/665650 s4.4).  Not combinable
                                        with XCD_AFFINITY or CONT_PRIORITY (MOE_ERR_ARG) */
#define MOE_FLAG_EXPLICIT_PERMUTE 0x400u /* permute (dispatch) as separate memory-bound tasks
                                           writing Xp, the stage the pages schedule on
                                           memory workers; default: the gather is fused
                                           into the UP tiles' row loads (x rows read through
                                           perm), with no Xp and no permute tasks */
#define MOE_FLAG_NARROW_ROUTER 0x800u /* router tasks over 32-token tiles (each streams all
                                         of W_r) even where 256-token router groups
                                         apply (bf16, E = 128 or 256, T >= 2048) */
#define MOE_FLAG_PERTURB 0x200u  /* dynamic: race perturbation for tests -- pseudo-random
                                    sleeps before claims and dependency decrements,
                                    pushed bursts in reverse order (m.xxqk.cn/news/657744
                                    s3.3); changes timing only, never results */

/* Return codes. */
#define MOE_OK 0
#define MOE_ERR_ARG 1         /* NULL pointer, bad shape, k > E, E > 256    */
#define MOE_ERR_WORKSPACE 2   /* workspace NULL or smaller than required    */
#define MOE_ERR_UNSUPPORTED 3 /* d or f not a multiple of 128, etc.         */
#define MOE_ERR_HIP 4         /* a HIP runtime call failed                  */
#define MOE_ERR_TIMEOUT 5     /* device watchdog: a wait exceeded its limit */
#define MOE_ERR_CAPACITY 6    /* a device table overflowed its capacity     */
#define MOE_ERR_NONFINITE 7   /* a router logit was NaN or infinite         */
#define MOE_ERR_TOO_LARGE 8   /* moe_layer_no_alloc: workspace > its scratch  */

/* Size of the static per-device scratch moe_layer_no_alloc works in. */
#define MOE_NO_ALLOC_SCRATCH_BYTES ((size_t)64 << 20)

typedef struct moe_desc {
  int T;              /* tokens (>= 0)                                      */
  int d;              /* model dim, multiple of 128                         */
  int E;              /* router width = global experts, 1..256              */
  int k;              /* experts per token, 1..min(E, 8)                    */
  int f;              /* expert FFN dim, multiple of 128                    */
  int e_begin, e_end; /* local experts [e_begin, e_end); e_end=0 -> E       */
  int n_shared;       /* always-on shared experts (weight 1), 0..4          */
  int f_shared;       /* their FFN dim, multiple of 128                     */
  int dtype;          /* moe_dtype                                          */
  int mode;           /* moe_mode                                           */
  int split_policy;   /* moe_split_policy                                   */
  int fixed_mem_workers; /* for MOE_SPLIT_FIXED; 0 = workers / 8            */
  int split_k;        /* DOWN split-K slices; 0 = automatic                 */
  int max_workers;    /* cap on persistent workgroups; 0 = all resident     */
  unsigned flags;     /* MOE_FLAG_*                                         */
  uint64_t* trace;    /* device buffer for MOE_FLAG_TRACE, or NULL          */
  int trace_cap;      /* records that fit in trace (3 x uint64 each)        */
  int timeout_ms;     /* device watchdog per wait; 0 = 2000 ms              */
  int row_tile;       /* expert row-tile height 128 or 256 (bf16 only);
                         0 = automatic (256 when T*k > 8192 in bf16)        */
  int combine;        /* moe_combine                                        */
  int bands;          /* row-tile order: tiles dealt into this many token
                         bands, run band by band (1 = plain expert-major
                         order); 0 = automatic (1)                          */
  int timeout_ticks;  /* > 0: watchdog limit per wait in ticks of the 100 MHz
                         device clock, overriding timeout_ms (lets a test
                         force the watchdog; every wait then gives up and the
                         call reports MOE_ERR_TIMEOUT)                      */
  int claim_batch;    /* dynamic: compute-queue slots one atomic claim
                         reserves, 1..8 (xxqk.cn/news/665650 s4.2, batched
                         fetch); 0 = 1                                      */
} moe_desc;

/* Weights.  E_loc = e_end - e_begin.  Element type = desc.dtype.
 *   w_router [d, E]         (router_bias [E] fp32, may be NULL)
 *   w_gate   [E_loc, d, f]  SiLU branch;   w_up [E_loc, d, f]  linear branch
 *   w_down   [E_loc, f, d]
 *   ws_gate, ws_up [n_shared, d, f_shared], ws_down [n_shared, f_shared, d]
 *   (NULL when n_shared == 0). */
typedef struct moe_weights {
  const void* w_router;
  const float* router_bias;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const void* ws_gate;
  const void* ws_up;
  const void* ws_down;
} moe_weights;

/* Routing results, for checking (every pointer may be NULL = not wanted).
 *   logits        [T, E]      fp32 router logits (bias included)
 *   topk_idx      [T, k]      chosen global expert ids, best first; equal
 *                             logits break toward the lower id
 *   topk_w        [T, k]      fp32 weights, softmax renormalised over the k
 *   expert_counts [E_loc]     kept rows per local expert
 *   offsets       [E_loc+1]   exclusive prefix of expert_counts
 *   perm          [T*k]       token of each kept row, rows grouped by
 *                             expert, tokens ascending inside an expert
 *                             (first offsets[E_loc] entries valid)
 *   slot_pos      [T, k]      row of each (token, slot), -1 if not local */
typedef struct moe_routing {
  float* logits;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* expert_counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* slot_pos;
} moe_routing;

/* Information about how a descriptor will run (filled by moe_query). */
typedef struct moe_info {
  int workers;          /* persistent workgroups launched                  */
  int cus;              /* compute units on the device                     */
  int blocks_per_cu;    /* resident workgroups per CU for the megakernel   */
  int route_tiles;      /* router / position tiles (32 tokens each)        */
  int up_ntiles;        /* f / 128                                         */
  int down_ntiles;      /* DOWN column tasks: d / 128, or d / 256 with 256-row tiles */
  int split_k;          /* DOWN split-K actually used                      */
  int permute_rows;     /* rows per permute task                           */
  int max_mtiles;       /* capacity of the expert row-tile table           */
  int max_tasks;        /* capacity of the ready queues                    */
  int route_splits;     /* router K slices per router tile                 */
  int combine_chunks;   /* combine tasks per 32-token tile (d / columns)   */
  int row_tile;         /* expert row-tile height (128 or 256)             */
  int combine;          /* MOE_COMBINE_SCATTER or MOE_COMBINE_TASKS        */
  size_t workspace_bytes;
  /* the cost model's frozen constants (measured once on MI355X) */
  float cost_mfma_flops_per_cu;      /* sustained MFMA flop/s of one CU in expert tiles */
  float cost_gather_bytes_per_worker; /* bytes/s one worker moves in a gather task */
  float cost_hbm_bytes;              /* device bytes/s a streaming tile sustains */
  int bands;            /* token bands of the row-tile order               */
  int gather_fused;     /* 1: the UP tiles gather x rows themselves (no
                           permute tasks, no Xp); 0: explicit permute    */
  int route_groups;     /* router tasks over 256-token groups (each group's
                           route_splits K slices, then one finish task per
                           32-token tile); 0: over 32-token router tiles */
} moe_info;

/* Bytes of workspace a call with this descriptor needs (0 on a bad
 * descriptor).  The workspace holds every piece of scheduling state -- queues,
 * dependency counters, task tables -- and the intermediate rows, so the
 * library allocates nothing (the graph-capture and overlap chapter, hncyxsy.com/news/277526,
 * CUDA Graph section: state resident at fixed addresses, nothing allocated
 * inside a captured region).  Caller-owned, any device allocation, 256-byte
 * aligned; reusable across calls with the same descriptor. */
size_t moe_workspace_size(const moe_desc* desc);

/* Fill `info` for this descriptor on the current device: workers, tile and
 * task geometry, and the cost model's frozen constants.  Host only (no
 * launch).  MOE_ERR_ARG on a bad descriptor or NULL info, MOE_ERR_HIP if the
 * device cannot be queried. */
int moe_query(const moe_desc* desc, moe_info* info);

/* Run one MoE layer (the stages the blog walk-through keeps inside one MoE
 * kernel, xxqk.cn/news/665650 section 1 -- gate/router, top-k, dispatch
 * (here: the expert-contiguous gather), expert FFN GEMMs, weighted combine --
 * scheduled as desc.mode says; m.xxqk.cn/news/657744 section 2.1 for the task
 * units):
 *   y[T,d] (fp32, overwritten) = sum over each token's kept top-k experts of
 *   w * SwiGLU_e(x[t]) + sum of the shared experts.
 * x [T,d] in desc.dtype; weights per moe_weights; device pointers.  `routing`
 * may be NULL; otherwise the requested tables are written (the
 * routing(topk_idx, topk_w, expert_counts) check surface).  Asynchronous on
 * hip_stream; argument errors (MOE_ERR_ARG / WORKSPACE / UNSUPPORTED) return
 * before any launch, launch failures MOE_ERR_HIP; device errors go to the
 * workspace (see moe_last_device_error) unless MOE_FLAG_CHECK is set. */
int moe_layer(const moe_desc* desc, const void* x, const moe_weights* weights,
              float* y, const moe_routing* routing, void* workspace,
              size_t workspace_bytes, void* hip_stream);

/* moe_layer with the block tail fused in: the residual add and the
 * normalisation the blog walk-through lists among the big kernel's stages
 * (xxqk.cn/news/665650 section 1), done by tasks of the same persistent
 * kernel as soon as a token tile's rows are complete, instead of a separate
 * kernel re-reading y:
 *   y[t]      = residual[t] + MoE(x)[t]                       (fp32)
 *   y_norm[t] = y[t] / sqrt(mean_c y[t,c]^2 + norm_eps) * norm_weight
 * residual [T,d] fp32 (NULL: no residual), norm_weight [d] fp32, y_norm
 * [T,d] in desc.dtype (bf16 layers: rounded to nearest even).  Every other
 * argument, the ownership and the errors as moe_layer; MOE_ERR_ARG also for a
 * NULL norm_weight or y_norm, or a negative / NaN norm_eps. */
int moe_layer_norm(const moe_desc* desc, const void* x, const moe_weights* weights,
                   const float* residual, const float* norm_weight, float norm_eps,
                   float* y, void* y_norm, const moe_routing* routing, void* workspace,
                   size_t workspace_bytes, void* hip_stream);

/* moe_layer for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * workspace is a fixed device array of this library, MOE_NO_ALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, held until the process ends; nothing is allocated.  A
 * layer whose moe_workspace_size exceeds it gets MOE_ERR_TOO_LARGE before
 * any launch.  Every call on a GPU shares that GPU's scratch (each call
 * re-initialises what must start at zero): calls that overlap in time on one
 * GPU -- e.g. on two streams -- race and must not be issued.  Arguments,
 * results and other errors as moe_layer. */
int moe_layer_no_alloc(const moe_desc* desc, const void* x, const moe_weights* weights,
                       float* y, const moe_routing* routing, void* hip_stream);

/* Bytes of workspace moe_layers needs for these n_layers descriptors (0 on
 * a bad descriptor or n_layers outside 1..1024): the layers' parameter
 * blocks, then each layer's moe_workspace_size, 256-byte aligned. */
size_t moe_layers_workspace_size(const moe_desc* descs, int n_layers);

/* Several independent MoE layers (descs[l], x[l], weights[l], y[l]; arrays of
 * n_layers; routing: NULL or an array of n_layers, each entry as in
 * moe_layer) in ONE persistent launch when every layer uses MOE_DYNAMIC and
 * the same element type: a worker that runs out of layer l's work goes on to
 * layer l + 1's router tiles while others finish layer l, so each layer's
 * routing overlaps the previous layer's expert tail (the multi-layer
 * follow-up of m.xxqk.cn/news/657744 section 6.3, against the per-layer
 * synchronisation windows of xxqk.cn/news/665650 section 3.3).  Layers whose
 * combine mode differs from the previous layer's start a new launch; the
 * baseline modes run layer by layer.  Results equal n calls of moe_layer.
 * The parameter blocks are copied from host memory with hipMemcpyAsync before
 * the launch (so this call is not meant for graph capture).  Errors as
 * moe_layer; with MOE_FLAG_CHECK in descs[0].flags the first layer's device
 * error found is returned. */
int moe_layers(const moe_desc* descs, int n_layers, const void* const* x,
               const moe_weights* weights, float* const* y, const moe_routing* routing,
               void* workspace, size_t workspace_bytes, void* hip_stream);

/* Routing only, from caller-supplied fp32 logits [T, E] (device): top-k,
 * weights, counts, offsets, perm and slot_pos, with the same device code the
 * layer uses (top-k with renormalised weights, xxqk.cn/news/665650 section 1).
 * Lets a checker feed identical logits to this library and to a reference
 * and compare the tables bit for bit.  Errors as moe_layer; a NaN or
 * infinite logit is the device error MOE_ERR_NONFINITE. */
int moe_route_from_logits(const moe_desc* desc, const float* logits,
                          const moe_routing* routing, void* workspace,
                          size_t workspace_bytes, void* hip_stream);

/* Synchronise `hip_stream` and return the device error word of the last
 * call that used `workspace` (MOE_OK if none): the watchdog and capacity
 * checks the persistent scheduler makes instead of hanging (the early-exit
 * and deadlock pitfalls of m.xxqk.cn/news/657744 section 3.3).  MOE_ERR_ARG
 * on a bad descriptor or NULL workspace, MOE_ERR_HIP if the copy fails. */
int moe_last_device_error(const moe_desc* desc, const void* workspace,
                          void* hip_stream);

/* What the scheduler decided in the last call that used a workspace: the
 * memory-bound worker group the post-routing cost model sized (the spatial
 * scheduler of the Weave abstract, arxivdaily.com/papers/2609.21483), and the
 * task counts the builder made from the per-expert counts. */
typedef struct moe_schedule {
  int mem_workers;    /* workers that start on the permute queue (0: no split) */
  int row_tiles;      /* expert row tiles                                   */
  int permute_tasks;  /* gather tasks                                       */
  int error;          /* device error word (MOE_OK if none)                 */
} moe_schedule;

/* Synchronise `hip_stream` and fill `out` from the control block of the last
 * call that used `workspace`.  Returns MOE_ERR_ARG on a bad descriptor or a
 * NULL pointer, MOE_ERR_HIP if a copy fails. */
int moe_last_schedule(const moe_desc* desc, const void* workspace, void* hip_stream,
                      moe_schedule* out);

/* Human-readable text for a return code. */
const char* moe_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* DTS_MOE_H */
