/*
 * moe.h — C ABI of libmoe.so, the MI355X (gfx950) forward pass of a sparse
 * Mixture-of-Experts layer.
 *
 * Sources (web pages; cited by title and section):
 *   [SMoE]   "Sparse Mixture-of-Experts", bigdataschool.ru wiki.
 *   [HF-MoE] "Что такое Mixture of Experts (MoE) в трансформерах: архитектура и
 *            параллелизм", aglamov.biz.
 *   [GW]     "Архитектура MoE в больших языковых моделях — кто такие «эксперты»?",
 *            gerwin.io.
 *
 * The layer, per token t with hidden state x_t ([SMoE] "Роутер и top-k gating",
 * "Expert capacity и capacity factor"; [HF-MoE] "Бэкенд для экспертов"):
 *   logits_t = W_r x_t                       bias-free router linear
 *   S_t      = top-k experts of softmax(logits_t); equal logits go to the lower index
 *   g_tj     = p_t[S_tj] / sum_j' p_t[S_tj']   renormalised gates
 *   capacity C = ceil(capacity_factor * T / E); assignments are filled first come,
 *   first served in token order; overflow assignments are dropped
 *   (variants, chosen in moe_desc: a rank-major fill order, and redirection of
 *   overflow to the token's next ranked expert, [GW] "Как работает MoE: принцип
 *   маршрутизации", load-balancing item 4)
 *   y_t      = [shared expert(x_t)] + sum_{kept j} g_tj * FFN_{S_tj}(x_t)
 *   FFN_e(x) = W_d[e] (silu(W_g[e] x) * (W_u[e] x))   bias-free SwiGLU
 *
 * Conventions for every call below
 *   - Tensor pointers are DEVICE pointers unless stated otherwise; row-major;
 *     allocated and owned by the caller.  The library keeps no pointer after a
 *     call returns and never writes an input.
 *   - Calls only enqueue work on `stream` (NULL = the default stream).  They never
 *     synchronise the device and never allocate or free device memory: scratch
 *     space comes from the caller's workspace `ws` of `ws_bytes` bytes.
 *   - Arguments are validated on the host before any HIP call.  On failure the
 *     call returns a non-zero moe_status, enqueues nothing, and moe_last_error()
 *     describes the problem.  Errors raised by a kernel while it runs surface at
 *     the caller's next synchronisation.
 *   - Every device pointer must be 16-byte aligned.
 *   - Stateless and thread-safe: calls on different streams may run concurrently
 *     as long as their output and workspace buffers do not overlap.
 *   - Element types: MOE_DTYPE_F32 (float) or MOE_DTYPE_BF16 (bfloat16 stored as
 *     16-bit words) for x, all weights, expert outputs and the layer output.
 *     Router logits and gates are always float.  Accumulation is float.
 *   - bf16 layers need d_model and d_ff (and d_ff_shared) to be multiples of 64
 *     (otherwise MOE_ERR_UNSUPPORTED); f32 layers accept any positive size.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_NO_CAPACITY (-1)
#define MOE_MAX_EXPERTS 1024

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,     /* bad argument: NULL/misaligned pointer, size out of range */
  MOE_ERR_UNSUPPORTED = 2, /* valid but not implemented: dtype, shape granularity */
  MOE_ERR_WORKSPACE = 3,   /* ws is NULL or ws_bytes is smaller than required */
  MOE_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum moe_dtype { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype;

/* Order in which the capacity fill visits the assignments (t, j). */
typedef enum moe_fill_order {
  MOE_FILL_TOKEN_MAJOR = 0, /* token t before token t+1, then rank j ([SMoE] "Подводные камни ...") */
  MOE_FILL_RANK_MAJOR = 1   /* every token's rank-0 choice before any rank-1 choice, ... */
} moe_fill_order;

/* What happens to an assignment that finds its expert full. */
typedef enum moe_overflow {
  MOE_OVERFLOW_DROP = 0,   /* dropped ([SMoE] "Expert capacity и capacity factor") */
  MOE_OVERFLOW_REROUTE = 1 /* offered to the token's next ranked expert ([GW] "Как работает MoE:
                              принцип маршрутизации", item 4); see moe_dispatch_reroute */
} moe_overflow;

/* Shape of one MoE layer call. */
typedef struct moe_desc {
  int32_t num_tokens;  /* T >= 0; T == 0 makes every call a no-op returning MOE_OK */
  int32_t d_model;     /* d >= 1 */
  int32_t d_ff;        /* f >= 1: hidden width of each routed expert */
  int32_t num_experts; /* 1 <= E <= MOE_MAX_EXPERTS */
  int32_t top_k;       /* 1 <= k <= E */
  int32_t capacity;    /* C >= 0 rows per expert, or MOE_NO_CAPACITY */
  int32_t d_ff_shared; /* 0: no shared expert; else hidden width of the always-on expert */
  int32_t dtype;       /* moe_dtype */
  int32_t fill_order;  /* moe_fill_order (0 = token-major) */
  int32_t overflow;    /* moe_overflow (0 = drop) */
} moe_desc;

/* Expert weights of one layer (device pointers).  Packed layouts follow the
 * runtime layout of [HF-MoE] "Рефакторинг загрузки весов": gate_up_proj holds,
 * per expert, the gate projection rows (w1) followed by the up projection rows
 * (w3); down_proj holds w2.  Zero-initialise the struct, so that the optional
 * fields at its end are NULL unless set. */
typedef struct moe_weights {
  const void *w_router;         /* [E, d] */
  const void *w_gate_up;        /* [E, 2f, d]: rows 0..f-1 gate, f..2f-1 up */
  const void *w_down;           /* [E, d, f] */
  const void *w_shared_gate_up; /* [2 f_s, d] or NULL when d_ff_shared == 0 */
  const void *w_shared_down;    /* [d, f_s]   or NULL when d_ff_shared == 0 */
  /* Optional, bf16 only, both or neither: w_gate_up and w_down also in the tile-major
   * layout that moe_tile_expert_weights writes (NULL: not given).  The large-tile regime of
   * the routed experts' grouped GEMMs then reads these copies -- one contiguous 16 KB
   * block per weight tile and K step instead of 256 rows of 64 bytes; w_gate_up and
   * w_down stay required (the streaming kernel reads them).  The caller keeps the two
   * forms equal.  Read by moe_forward, moe_forward_expert_shard (the range's experts) and
   * moe_backward (the recomputed gate_up projection). */
  const void *w_gate_up_tiled;
  const void *w_down_tiled;
  /* Optional, bf16 only, both or neither: the shared expert's weights in the same tile-major
   * layout (moe_tile_expert_weights with a descriptor of one expert, d_ff = d_ff_shared,
   * top_k = 1).  Read by moe_forward, moe_forward_expert_shard (with add_shared) and
   * moe_backward when the shared expert takes the large-tile regime (T >= 256). */
  const void *w_shared_gate_up_tiled;
  const void *w_shared_down_tiled;
} moe_weights;

/* Optional routing outputs of moe_forward (device pointers; any may be NULL,
 * in which case the workspace holds that table instead). */
typedef struct moe_routing {
  float *logits;           /* [T, E] */
  int32_t *topk_ids;       /* [T, k] */
  float *topk_gates;       /* [T, k] */
  int32_t *expert_counts;  /* [E]   demand per expert, before capacity */
  int32_t *expert_offsets; /* [E+1] exclusive prefix sum of kept rows per expert */
  int32_t *slot;           /* [T, k] slot inside the expert's buffer, -1 = dropped */
  int32_t *row_token;      /* [R_max] token of each kept row (rows sorted by expert, then slot) */
  int32_t *assigned_ids;   /* [T, k] expert serving each assignment: topk_ids unless redirected */
} moe_routing;

/* ---------------------------------------------------------------- host helpers */

/* Expert capacity ceil(capacity_factor * T / E), evaluated in IEEE double in that
 * order ([SMoE] "Expert capacity и capacity factor").  Returns MOE_NO_CAPACITY
 * when capacity_factor <= 0 or is not finite; returns 0 for T < 0 or E < 1; values
 * above INT32_MAX are clamped to INT32_MAX.  Host only, no device access. */
int32_t moe_capacity(int32_t num_tokens, int32_t num_experts, double capacity_factor);

/* Capacity variant with a top-k factor, ceil(capacity_factor * (k * T) / E) in IEEE
 * double: the batch counted in assignments rather than tokens.  Same special cases
 * as moe_capacity; k < 1 returns 0.  Host only. */
int32_t moe_capacity_topk(int32_t num_tokens, int32_t num_experts, int32_t top_k, double capacity_factor);

/* Upper bound R_max on kept rows: min(T*k, E*C), or T*k without capacity.
 * Returns -1 for an invalid descriptor. */
int64_t moe_max_rows(const moe_desc *desc);

/* Workspace bytes needed by moe_forward for this descriptor (enough for every
 * other call with the same descriptor too).  Returns 0 for an invalid descriptor. */
size_t moe_workspace_size(const moe_desc *desc);

/* Workspace bytes needed by moe_grouped_swiglu_gemm. Returns 0 on invalid input. */
size_t moe_grouped_gemm_workspace_size(int32_t num_groups, int64_t rows_max, int32_t d_ff, int32_t dtype);

const char *moe_status_string(moe_status status);

/* Detail of the last failure in the calling thread ("" if none). */
const char *moe_last_error(void);

/* The ids precondition of moe_dispatch_permute, moe_dispatch_reroute and
 * moe_combine_unpermute, checked on a HOST copy of the ids ([SMoE] "Роутер и top-k
 * gating": each id names one of the E experts): every topk_ids_host[t][j], [T, k] int32,
 * lies in [0, E).  Returns MOE_OK, or MOE_ERR_INVALID with moe_last_error() naming the
 * first entry outside the range.  Host only, no device access.
 * Release builds do not check ids on the device: an id outside [0, E) is treated as no
 * expert (slot -1, not counted, never indexes a table).  The debug build of the library
 * (libmoe_debug.so, compiled with MOE_DEBUG_CHECKS) runs this check inside those three
 * calls on a synchronous copy of the device ids, before it enqueues any work, and returns
 * its MOE_ERR_INVALID. */
moe_status moe_check_topk_ids(const moe_desc *desc, const int32_t *topk_ids_host);

/* 1 in the debug build (MOE_DEBUG_CHECKS: host checks of device-side preconditions, which
 * synchronise the stream), 0 otherwise. */
int32_t moe_debug_checks(void);

/* ---------------------------------------------------------------- hot path */

/* Router linear ([SMoE] "Роутер и top-k gating": logits from a linear layer
 * without bias).
 *   x           [T, d] dtype
 *   w_router    [E, d] dtype
 *   logit_offset [E] float or NULL: added to every token's logits (synthetic skew)
 *   logits      [T, E] float, written.  Accumulated in float. */
moe_status moe_router_logits(const moe_desc *desc, const void *x, const void *w_router,
                             const float *logit_offset, float *logits, hipStream_t stream);

/* Softmax over experts, top-k and renormalised gates ([SMoE] "Роутер и top-k
 * gating").  Selection ranks the logits (softmax is increasing); equal logits go
 * to the lower expert index, and -0.0 equals +0.0.  Logits must be finite or -inf.
 *   logits     [T, E] float
 *   topk_ids   [T, k] int32, written in descending logit order
 *   topk_gates [T, k] float, written: exp(l_j - l_max) / sum over the k selected */
moe_status moe_router_topk(const moe_desc *desc, const float *logits, int32_t *topk_ids,
                           float *topk_gates, hipStream_t stream);

/* Capacity-limited dispatch ([SMoE] "Expert capacity и capacity factor",
 * "Подводные камни collapse экспертов и token dropping"; [HF-MoE] "Бэкенд для
 * экспертов": tokens sorted by expert id before one grouped GEMM).
 * Walking assignments (t, j) in desc->fill_order (token-major: t outer, j inner;
 * rank-major: j outer, t inner), each takes the next free slot of its expert while
 * fewer than C are taken; later ones are dropped.  desc->overflow must be
 * MOE_OVERFLOW_DROP (MOE_ERR_INVALID otherwise; redirection is moe_dispatch_reroute).
 *   topk_ids       [T, k] int32, each in [0, E) (precondition; see moe_check_topk_ids: an id
 *                  outside the range is treated as dropped, slot -1, and not counted)
 *   x              [T, d] dtype, or NULL when x_perm is NULL
 *   expert_counts  [E]   int32, written: demand per expert
 *   expert_offsets [E+1] int32, written: offsets[0] = 0, offsets[e+1] - offsets[e] =
 *                  min(counts[e], C)
 *   slot           [T, k] int32, written: slot in the expert's buffer or -1 if dropped
 *   row_token      [R_max] int32, written for rows < offsets[E]: the row's token; the rows
 *                  of an expert are in slot order (its assignments in fill order)
 *   x_perm         [R_max, d] dtype or NULL: row offsets[e] + slot(t, j) = x[t];
 *                  rows >= offsets[E] are left unspecified
 *   ws             at least moe_workspace_size(desc) bytes */
moe_status moe_dispatch_permute(const moe_desc *desc, const int32_t *topk_ids, const void *x,
                                int32_t *expert_counts, int32_t *expert_offsets, int32_t *slot,
                                int32_t *row_token, void *x_perm, void *ws, size_t ws_bytes,
                                hipStream_t stream);

/* Capacity-limited dispatch with redirection of overflow ([GW] "Как работает MoE:
 * принцип маршрутизации", load-balancing item 4: an assignment beyond an expert's
 * capacity may be sent on to the next most suitable expert instead of dropped).
 * Two passes, both in desc->fill_order:
 *   1. the plain fill of moe_dispatch_permute: kept assignments are exactly those
 *      of the drop policy;
 *   2. the i-th overflowing assignment of token t (i counted in rank order j) is
 *      offered to the expert ranked k + i in t's router order (descending logit,
 *      equal logits to the lower index); offers take the next free slot of that
 *      expert while it has room left after pass 1, otherwise (or if k + i >= E)
 *      they are dropped.  Each expert's rows: its pass-1 rows, then its offers.
 * Gates are not changed: a redirected assignment keeps its gate.  Without capacity
 * nothing overflows and the result is that of moe_dispatch_permute.
 *   logits         [T, E] float (the router's, as given to moe_router_topk)
 *   topk_ids       [T, k] int32 as written by moe_router_topk from those logits
 *   expert_counts  [E]   int32, written: the router's demand per expert (pass 1)
 *   expert_offsets [E+1] int32, written: exclusive prefix of the final kept rows
 *   slot           [T, k] int32, written: slot in the serving expert's buffer, or -1
 *   assigned_ids   [T, k] int32, written: serving expert (topk_ids[t][j] unless
 *                  redirected; for a dropped assignment, topk_ids[t][j])
 *   row_token      [R_max] int32, written for rows < offsets[E]
 *   ws             at least moe_workspace_size(desc) bytes
 * Pass assigned_ids as the ids of moe_combine_unpermute.  desc->overflow is not
 * consulted. */
moe_status moe_dispatch_reroute(const moe_desc *desc, const float *logits, const int32_t *topk_ids,
                                int32_t *expert_counts, int32_t *expert_offsets, int32_t *slot,
                                int32_t *assigned_ids, int32_t *row_token, void *ws, size_t ws_bytes,
                                hipStream_t stream);

/* Grouped SwiGLU expert FFN over rows sorted by group ([HF-MoE] "Бэкенд для
 * экспертов": one grouped GEMM over tokens sorted by expert id; [HF-MoE]
 * "Рефакторинг загрузки весов": packed gate_up / down layouts).
 * For every group g and row r in [group_offsets[g], group_offsets[g+1]):
 *   y_rows[r] = W_d[g] (silu(W_g[g] x_rows[r]) * (W_u[g] x_rows[r]))
 * The hidden activation is rounded to dtype between the two projections.
 *   num_groups      G >= 1 (<= MOE_MAX_EXPERTS)
 *   rows_max        rows available in x_rows / y_rows; group_offsets[G] <= rows_max
 *   group_rows_max  the caller's bound on any one group's rows (a tiling hint: larger
 *                   groups are still computed correctly); >= 1
 *   x_rows          [rows_max, d] dtype
 *   group_offsets   [G+1] int32 DEVICE array, non-decreasing, group_offsets[0] >= 0
 *   w_gate_up       [G, 2f, d] dtype;  w_down [G, d, f] dtype
 *   y_rows          [rows_max, d] dtype, written for rows inside a group
 *   ws              at least moe_grouped_gemm_workspace_size(G, rows_max, f, dtype) */
moe_status moe_grouped_swiglu_gemm(int32_t num_groups, int64_t rows_max, int32_t group_rows_max,
                                   int32_t d_model, int32_t d_ff, int32_t dtype, const void *x_rows,
                                   const int32_t *group_offsets, const void *w_gate_up,
                                   const void *w_down, void *y_rows, void *ws, size_t ws_bytes,
                                   hipStream_t stream);

/* The two halves of moe_grouped_swiglu_gemm as single launches (same contracts; same
 * sources; no workspace):
 *   moe_grouped_gate_up_swiglu: h_rows[r] = silu(W_g[g] a_r) * (W_u[g] a_r), h_rows
 *     [rows_max, f] dtype (rounded to dtype), where a_r = x_rows[r], or, when row_index
 *     is not NULL, a_r = x_rows[row_index[r]] with x_rows holding x_row_count rows (a
 *     row gather: the dispatch's row_token lets the projection read token rows straight
 *     from x, so x_perm need not exist; x_rows must then be < 2 GiB);
 *   moe_grouped_down: y_rows[r] = W_d[g] h_rows[r], y_rows [rows_max, d] dtype. */
moe_status moe_grouped_gate_up_swiglu(int32_t num_groups, int64_t rows_max, int32_t group_rows_max, int32_t d_model,
                                      int32_t d_ff, int32_t dtype, const void *x_rows, const int32_t *row_index,
                                      int64_t x_row_count, const int32_t *group_offsets, const void *w_gate_up,
                                      void *h_rows, hipStream_t stream);
moe_status moe_grouped_down(int32_t num_groups, int64_t rows_max, int32_t group_rows_max, int32_t d_model,
                            int32_t d_ff, int32_t dtype, const void *h_rows, const int32_t *group_offsets,
                            const void *w_down, void *y_rows, hipStream_t stream);

/* Gate-weighted combine back to token order, without atomics ([SMoE] "Роутер и
 * top-k gating": weighted sum of the selected experts' outputs; "Expert capacity и
 * capacity factor": a dropped assignment contributes nothing; [GW] drawbacks item
 * 5: shared expert added with weight 1).
 *   out[t] = shared_out[t] (or 0) + sum_{j: slot[t,j] >= 0} topk_gates[t,j] *
 *            y_perm[expert_offsets[topk_ids[t,j]] + slot[t,j]], summed in float in
 *            order j = 0..k-1, then rounded to dtype.
 *   topk_ids: the expert serving each assignment -- the router's ids, or the
 *   assigned_ids of moe_dispatch_reroute when overflow is redirected; each in [0, E)
 *   (precondition, see moe_check_topk_ids: an id outside the range adds nothing).
 *   y_perm [R_max, d] dtype; shared_out [T, d] dtype or NULL; out [T, d] dtype */
moe_status moe_combine_unpermute(const moe_desc *desc, const void *y_perm, const int32_t *topk_ids,
                                 const float *topk_gates, const int32_t *slot,
                                 const int32_t *expert_offsets, const void *shared_out, void *out,
                                 hipStream_t stream);

/* Switch-style auxiliary load-balancing loss ([SMoE] "Маршрутизация токена и auxiliary
 * loss"): loss = alpha * E * sum_i f_i * P_i, where f_i = expert_counts[i] / (T * k) is
 * the share of the batch's assignments routed to expert i (router choice, before
 * capacity) and P_i the softmax probability of expert i averaged over the T tokens.
 * For k = 1 this is the page's formula; uniform routing gives alpha.
 *   logits        [T, E] float (as written by moe_router_logits)
 *   expert_counts [E] int32 (as written by moe_dispatch_permute)
 *   loss          [1] float, written (device)
 *   ws            at least moe_workspace_size(desc) bytes
 * Float accumulation in fixed orders: bit-reproducible. */
moe_status moe_router_aux_loss(const moe_desc *desc, const float *logits, const int32_t *expert_counts, float alpha,
                               float *loss, void *ws, size_t ws_bytes, hipStream_t stream);

/* The whole layer: router linear, top-k, dispatch, routed grouped SwiGLU FFN, the
 * shared expert if desc->d_ff_shared > 0, and combine.  The dispatch follows
 * desc->fill_order and desc->overflow (moe_dispatch_permute or moe_dispatch_reroute).
 *   x [T, d] dtype, smaller than 2 GiB; logit_offset [E] float or NULL; out [T, d] dtype
 *   routing: NULL, or a struct whose non-NULL fields receive the routing tables
 *   ws: at least moe_workspace_size(desc) bytes
 * Only kernel launches on `stream` (no host synchronisation, allocation or memset): the
 * call can be captured into a HIP graph.  Deterministic: equal inputs give bitwise equal
 * outputs and routing tables. */
moe_status moe_forward(const moe_desc *desc, const moe_weights *weights, const void *x,
                       const float *logit_offset, void *out, moe_routing *routing, void *ws,
                       size_t ws_bytes, hipStream_t stream);

/* Bytes of the fixed scratch array behind moe_forward_noalloc (per GPU). */
#define MOE_NOALLOC_WORKSPACE_BYTES (128u << 20)

/* For callers that cannot allocate device memory -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation: moe_forward with its workspace taken
 * from a fixed array of MOE_NOALLOC_WORKSPACE_BYTES that the library holds on each GPU it
 * runs on (until the process ends), instead of a caller workspace.  No allocation: the
 * call neither allocates nor frees device memory.  Layers whose moe_workspace_size
 * exceeds MOE_NOALLOC_WORKSPACE_BYTES fail with MOE_ERR_WORKSPACE before any launch (e.g.
 * decode steps and Switch-style layers fit; the Mixtral- and DeepSeek-shaped layers do
 * not).  Every call on one GPU uses that GPU's one array: calls that overlap in time on
 * the same GPU (different streams or threads without ordering) race and give undefined
 * results; calls ordered on one stream are fine.  Nothing in the array has to start at
 * zero (every kernel writes what it reads back).  The first call on a device resolves
 * that device's array address with that device current.  Arguments, results and other
 * errors as for moe_forward. */
moe_status moe_forward_noalloc(const moe_desc *desc, const moe_weights *weights, const void *x,
                               const float *logit_offset, void *out, moe_routing *routing,
                               hipStream_t stream);

/* Stages of moe_forward in launch order, as moe_forward_staged marks them. */
typedef enum moe_stage {
  MOE_STAGE_ROUTER = 0,                /* router linear and top-k (the next k ranks too when redirecting) */
  MOE_STAGE_DISPATCH = 1,              /* capacity fill: counts, offsets, slots, row order */
  MOE_STAGE_PACK_ROWS = 2,             /* large-tile regime: gathered x rows copied to the packed tile layout */
  MOE_STAGE_GATE_UP = 3,               /* routed gate_up + SwiGLU grouped GEMM, main launch */
  MOE_STAGE_GATE_UP_TAILS = 4,         /* large-tile regime: the groups' tail rows, streaming launch */
  MOE_STAGE_DOWN = 5,                  /* routed down grouped GEMM, main launch (and its K-split sum) */
  MOE_STAGE_DOWN_TAILS = 6,            /* large-tile regime: tail rows of the down projection */
  MOE_STAGE_SHARED_PACK_ROWS = 7,      /* shared expert: its row offsets (large-tile regime), packed x rows */
  MOE_STAGE_SHARED_GATE_UP = 8,        /* shared expert gate_up + SwiGLU, main launch */
  MOE_STAGE_SHARED_GATE_UP_TAILS = 9,  /* shared expert: tail rows */
  MOE_STAGE_SHARED_DOWN = 10,          /* shared expert down projection, main launch */
  MOE_STAGE_SHARED_DOWN_TAILS = 11,    /* shared expert: tail rows of the down projection */
  MOE_STAGE_COMBINE = 12,              /* gate-weighted combine into out */
  MOE_NUM_STAGES = 13
} moe_stage;

/* moe_forward with HIP events recorded on `stream` between its launches, so that a caller
 * can time each stage of the very launches moe_forward makes (same kernels, arguments and
 * order; the records add only event markers to the stream).
 *   stage_events  host array of MOE_NUM_STAGES + 1 events created by the caller (hipEventCreate,
 *                 timing enabled): stage_events[0] is recorded before the first launch and
 *                 stage_events[s + 1] after the launches of stage s; a stage that launches
 *                 nothing (absent shared expert, streaming regime without tails, ...) ends where
 *                 the previous one ended.  NULL entries: MOE_ERR_INVALID.
 * Other arguments, results and errors as for moe_forward. */
moe_status moe_forward_staged(const moe_desc *desc, const moe_weights *weights, const void *x,
                              const float *logit_offset, void *out, moe_routing *routing, void *ws,
                              size_t ws_bytes, hipStream_t stream, hipEvent_t *stage_events);

/* Weight gradients of moe_backward (device pointers). */
typedef struct moe_grads {
  void *dw_router;         /* [E, d] float */
  void *dw_gate_up;        /* [E, 2f, d] dtype: gate rows then up rows, as w_gate_up */
  void *dw_down;           /* [E, d, f] dtype */
  void *dw_shared_gate_up; /* [2 f_s, d] dtype, or NULL when d_ff_shared == 0 */
  void *dw_shared_down;    /* [d, f_s]   dtype, or NULL when d_ff_shared == 0 */
} moe_grads;

/* Workspace bytes needed by moe_backward; 0 for an invalid or unsupported descriptor. */
size_t moe_backward_workspace_size(const moe_desc *desc);

/* Backward pass of the layer: gradients of L = sum(dy * out) for the out of moe_forward,
 * with the routing held fixed (top-k choice, slots and drops are piecewise constant;
 * [HF-MoE] "Обучение MoE с помощью Transformers": in training the expert projections
 * run as grouped GEMMs too).  Per kept row of expert e with gate g:
 *   dH' = dy W_d[e];  dg = dH' . H;  [dG dU] from g dH' through SwiGLU;
 *   dx += [dG dU] W_gu[e];  dW_d[e] += (g dy) (x) H;  dW_gu[e] += [dG dU] (x) x;
 * gates (softmax over the selected logits): dl_j = g_j (dg_j - sum g dg), dW_r = dl^T x,
 * dx += dl W_r; the shared expert likewise with g = 1 for every token.  Experts without
 * kept rows get zero gradients.  bf16 layers only (MOE_ERR_UNSUPPORTED otherwise).
 *   x, dy      [T, d] dtype (the forward's input; the loss gradient w.r.t. out)
 *   routing    the tables moe_forward wrote for x: topk_ids, topk_gates, expert_offsets,
 *              slot, row_token (and assigned_ids when desc->overflow redirects) are read
 *   dx         [T, d] dtype, written
 *   grads      written in full (see moe_grads)
 *   ws         at least moe_backward_workspace_size(desc) bytes
 * Accumulation in float; every sum in a fixed order (bit-reproducible).  Only kernel
 * launches on `stream` (capturable into a HIP graph). */
moe_status moe_backward(const moe_desc *desc, const moe_weights *weights, const void *x, const moe_routing *routing,
                        const void *dy, void *dx, moe_grads *grads, void *ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of the tile-major copy of num_experts experts' gate_up (which = 0) or down
 * (which = 1) weights for desc's shapes: per expert, ceil(f / 128) gate_up tiles (128 gate
 * rows and their 128 up rows each) or ceil(d / 256) down tiles (256 rows each), times K/32
 * steps (K = d for gate_up, f for down), times 16 KB.  0 for an invalid descriptor, a
 * dtype other than bf16, num_experts < 1 or another `which`.  Host only. */
size_t moe_tiled_weights_bytes(const moe_desc *desc, int32_t num_experts, int32_t which);

/* Writes the tile-major copies of num_experts experts' routed weights: a one-time
 * preparation of the runtime layout at weight-loading time ([HF-MoE] "Рефакторинг
 * загрузки весов": checkpoint weights are converted once, on load, into the layout the
 * runtime computes with).  Tile nt, K step kt of expert e is the 16 KB block
 * (e * tiles + nt) * K/32 + kt: the tile's 256 weight rows by 32 values, 64 bytes per row,
 * 16-byte chunk c of row r stored at chunk position c ^ ((r >> 2) & 3), rows past the
 * matrix zero.  gate_up tile nt holds gate rows 128 nt .. 128 nt + 127 followed by the
 * matching up rows (f apart); down tile nt holds rows 256 nt .. 256 nt + 255.  Inputs as in
 * moe_weights ([num_experts, 2f, d] and [num_experts, d, f]); outputs sized by
 * moe_tiled_weights_bytes, 16-byte aligned, not overlapping the inputs.  bf16 only
 * (MOE_ERR_UNSUPPORTED otherwise).  Only kernel launches on `stream`. */
moe_status moe_tile_expert_weights(const moe_desc *desc, int32_t num_experts, const void *w_gate_up,
                                   const void *w_down, void *w_gate_up_tiled, void *w_down_tiled,
                                   hipStream_t stream);

/* One rank's share of expert parallelism ([HF-MoE] "Параллелизм экспертов
 * (Expert Parallelism)": each device holds a contiguous subset of the experts,
 * computes them, and partial outputs are summed across devices with an all-reduce;
 * global expert indices map to local ones and the other experts are masked).
 * Routing, capacity and dispatch run over all E experts, so slots and drops are those
 * of the whole layer; only experts [expert_begin, expert_end) run their FFN, with
 * weights->w_gate_up / w_down holding just those experts ([expert_end - expert_begin,
 * ...], local index 0 = expert_begin); the router weights are the full [E, d].
 *   out_partial[t] = (add_shared ? shared(x_t) : 0)
 *                    + sum over kept j with expert in range of g_tj * FFN_e(x_t)
 * Summing the partials of a partition of [0, E) (shared expert added by exactly one
 * range) gives moe_forward's output up to float summation order.  Other arguments as
 * for moe_forward; 0 <= expert_begin <= expert_end <= E. */
moe_status moe_forward_expert_shard(const moe_desc *desc, const moe_weights *weights, int32_t expert_begin,
                                    int32_t expert_end, int32_t add_shared, const void *x, const float *logit_offset,
                                    void *out_partial, moe_routing *routing, void *ws, size_t ws_bytes,
                                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
