// C ABI of libmoe.so: host-side validation, workspace layout and the launch order of
// the forward pass.  Declarations and contracts are in include/moe.h.
#include "moe.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MOE_TRY_HIP(expr, what)                             \
  do {                                                      \
    moe_status st_ = hip_status((expr), (what));            \
    if (st_ != MOE_OK) return st_;                          \
  } while (0)
#define MOE_TRY(expr)                 \
  do {                                \
    moe_status st_ = (expr);          \
    if (st_ != MOE_OK) return st_;    \
  } while (0)

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_ptr(const void *p, const char *name) {
  if (!p) return fail(MOE_ERR_INVALID, "%s is NULL", name);
  if (!aligned16(p)) return fail(MOE_ERR_INVALID, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

moe_status check_opt_ptr(const void *p, const char *name) { return p ? check_ptr(p, name) : MOE_OK; }

// Optional tile-major copies of a pair of weight matrices: both or neither, bf16 only.
moe_status check_tiled_pair(const void *gu, const void *dn, int32_t dtype, const char *gu_name, const char *dn_name) {
  if (!gu && !dn) return MOE_OK;
  if (!gu || !dn) return fail(MOE_ERR_INVALID, "%s and %s: give both or neither", gu_name, dn_name);
  if (dtype != MOE_DTYPE_BF16) return fail(MOE_ERR_UNSUPPORTED, "tile-major weights are bf16 only");
  MOE_TRY(check_ptr(gu, gu_name));
  return check_ptr(dn, dn_name);
}

moe_status check_tiled(const moe_weights &w, int32_t dtype) {
  return check_tiled_pair(w.w_gate_up_tiled, w.w_down_tiled, dtype, "w_gate_up_tiled", "w_down_tiled");
}

moe_status check_shared_tiled(const moe_weights &w, int32_t dtype) {
  return check_tiled_pair(w.w_shared_gate_up_tiled, w.w_shared_down_tiled, dtype, "w_shared_gate_up_tiled",
                          "w_shared_down_tiled");
}

size_t elem_bytes(int32_t dtype) { return dtype == MOE_DTYPE_BF16 ? 2 : 4; }

moe_status check_dtype_dims(int32_t dtype, int64_t d, int64_t f, int64_t fs) {
  if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16) return fail(MOE_ERR_UNSUPPORTED, "dtype %d", (int)dtype);
  if (dtype == MOE_DTYPE_BF16) {
    if (d % 64 || f % 64 || fs % 64)
      return fail(MOE_ERR_UNSUPPORTED, "bf16 layers need d_model, d_ff and d_ff_shared to be multiples of 64 "
                                       "(got %lld, %lld, %lld)", (long long)d, (long long)f, (long long)fs);
    // one expert's weights are addressed through 32-bit buffer offsets
    if (2 * std::max(f, fs) * d * 2 >= ((int64_t)1 << 31))
      return fail(MOE_ERR_UNSUPPORTED, "one expert's gate_up weights must be smaller than 2 GiB");
  }
  return MOE_OK;
}

moe_status check_desc(const moe_desc *desc) {
  if (!desc) return fail(MOE_ERR_INVALID, "desc is NULL");
  const moe_desc &D = *desc;
  if (D.num_tokens < 0) return fail(MOE_ERR_INVALID, "num_tokens %d < 0", D.num_tokens);
  if (D.d_model < 1 || D.d_ff < 1) return fail(MOE_ERR_INVALID, "d_model and d_ff must be >= 1");
  if (D.num_experts < 1 || D.num_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_INVALID, "num_experts %d outside [1, %d]", D.num_experts, MOE_MAX_EXPERTS);
  if (D.top_k < 1 || D.top_k > D.num_experts)
    return fail(MOE_ERR_INVALID, "top_k %d outside [1, num_experts=%d]", D.top_k, D.num_experts);
  if (D.capacity < 0 && D.capacity != MOE_NO_CAPACITY)
    return fail(MOE_ERR_INVALID, "capacity %d: must be >= 0 or MOE_NO_CAPACITY", D.capacity);
  if (D.d_ff_shared < 0) return fail(MOE_ERR_INVALID, "d_ff_shared %d < 0", D.d_ff_shared);
  if (D.fill_order != MOE_FILL_TOKEN_MAJOR && D.fill_order != MOE_FILL_RANK_MAJOR)
    return fail(MOE_ERR_INVALID, "fill_order %d is not a moe_fill_order", D.fill_order);
  if (D.overflow != MOE_OVERFLOW_DROP && D.overflow != MOE_OVERFLOW_REROUTE)
    return fail(MOE_ERR_INVALID, "overflow %d is not a moe_overflow", D.overflow);
  if ((int64_t)D.num_tokens * D.top_k > INT32_MAX)
    return fail(MOE_ERR_INVALID, "num_tokens * top_k exceeds INT32_MAX");
  if ((int64_t)D.num_tokens * D.d_model * (int64_t)elem_bytes(D.dtype) >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "x must be smaller than 2 GiB (32-bit row gather offsets)");
  return check_dtype_dims(D.dtype, D.d_model, D.d_ff, D.d_ff_shared);
}

// The ids precondition of the dispatch and combine calls, on a host copy: every entry in
// [0, E).  Names the first entry outside the range.
moe_status check_ids_host(const moe_desc &D, const int32_t *ids) {
  const int64_t n = (int64_t)D.num_tokens * D.top_k;
  for (int64_t q = 0; q < n; ++q)
    if (ids[q] < 0 || ids[q] >= D.num_experts)
      return fail(MOE_ERR_INVALID, "topk_ids[%lld][%d] = %d is outside [0, %d)", (long long)(q / D.top_k),
                  (int)(q % D.top_k), (int)ids[q], D.num_experts);
  return MOE_OK;
}

#ifdef MOE_DEBUG_CHECKS
// Debug builds: the same check on a synchronous copy of the device ids, before any launch.
moe_status debug_check_ids(const moe_desc &D, const int32_t *ids_dev, hipStream_t s) {
  std::vector<int32_t> h((size_t)D.num_tokens * D.top_k);
  if (h.empty()) return MOE_OK;
  MOE_TRY_HIP(hipMemcpyAsync(h.data(), ids_dev, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s),
              "debug check: copy topk_ids to the host");
  MOE_TRY_HIP(hipStreamSynchronize(s), "debug check: synchronise");
  return check_ids_host(D, h.data());
}
#define MOE_DEBUG_CHECK_IDS(D, ids, s) MOE_TRY(debug_check_ids((D), (ids), (s)))
#else
#define MOE_DEBUG_CHECK_IDS(D, ids, s) ((void)0)
#endif

int64_t max_rows(const moe_desc &D) {
  const int64_t tk = (int64_t)D.num_tokens * D.top_k;
  if (D.capacity == MOE_NO_CAPACITY) return tk;
  return std::min<int64_t>(tk, (int64_t)D.num_experts * D.capacity);
}

// Workspace of float partials for K splits of the down projection: layers of few
// experts (large groups, large-tile regime), where one rank's share of expert
// parallelism can leave a handful of tiles.
size_t down_split_bytes(const moe_desc &D) {
  if (D.dtype != MOE_DTYPE_BF16 || D.num_experts > 16) return 0;
  return (size_t)4 * max_rows(D) * D.d_model * 4;
}

// Largest number of rows any one expert can hold: min(T, C).
int32_t group_rows_bound(const moe_desc &D) {
  if (D.capacity == MOE_NO_CAPACITY) return D.num_tokens;
  return std::min(D.num_tokens, D.capacity);
}

constexpr size_t kAlign = 256;
size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

// Workspace layout of moe_forward; every region starts on a 256-byte boundary.
struct Layout {
  size_t logits, ids, gates, counts, offsets, slot, row_token, spare, assigned, hist, x_packed, hidden, hidden_tail,
      y_perm, sh_x_packed, sh_hidden, sh_hidden_tail, sh_out, sh_offsets, router_part, down_split, total;
};

// Whether copying the x rows into the packed tile layout pays in the large-tile regime: each
// row is re-read by every weight tile of the gate_up projection (ceil(f / 128) of them), and
// the copy costs a read and a write of the rows.  With f >= 4096 (>= 32 tiles) it wins (the
// 14336-wide Mixtral-style experts: a 28 us copy, gate_up 5% faster); a 2048-wide shared
// expert over 16384 tokens of width 7168 measured a 112 us copy that saved its gate_up
// projection 13 us.
bool pack_rows_wins(int64_t f) { return f >= 4096; }

// Whether the routed experts may take the large-tile regime (an expert can hold 256 rows)
// with packed operands below 2 GiB.
bool packable(const moe_desc &D) {
  if (D.dtype != MOE_DTYPE_BF16 || group_rows_bound(D) < 256) return false;
  const int64_t R = max_rows(D);
  return moe::packed_rows_bytes(R, D.num_experts, D.d_model) < ((int64_t)1 << 31) &&
         moe::packed_rows_bytes(R, D.num_experts, D.d_ff) < ((int64_t)1 << 31);
}

// Whether the shared expert (one group of all T rows) takes the large-tile regime with its
// x rows and H in the packed tile layout, below 2 GiB each.
bool shared_packable(const moe_desc &D) {
  if (D.dtype != MOE_DTYPE_BF16 || D.d_ff_shared == 0 || D.num_tokens < 256) return false;
  return moe::packed_rows_bytes(D.num_tokens, 1, D.d_model) < ((int64_t)1 << 31) &&
         moe::packed_rows_bytes(D.num_tokens, 1, D.d_ff_shared) < ((int64_t)1 << 31);
}

bool rerouting(const moe_desc &D) { return D.overflow == MOE_OVERFLOW_REROUTE && D.capacity != MOE_NO_CAPACITY; }

Layout layout(const moe_desc &D) {
  Layout L{};
  const size_t T = D.num_tokens, E = D.num_experts, k = D.top_k, d = D.d_model, f = D.d_ff, fs = D.d_ff_shared;
  const size_t R = (size_t)max_rows(D), s = elem_bytes(D.dtype);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  L.logits = take(T * E * 4);
  L.ids = take(T * k * 4);
  L.gates = take(T * k * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.slot = take(T * k * 4);
  L.row_token = take(R * 4);
  // redirection of overflow: the experts ranked k .. 2k-1 per token, the serving experts
  L.spare = take(D.overflow == MOE_OVERFLOW_REROUTE ? T * k * 4 : 0);
  L.assigned = take(D.overflow == MOE_OVERFLOW_REROUTE ? T * k * 4 : 0);
  L.hist = take(std::max(moe::dispatch_workspace_bytes((int)T, (int)k, (int)E, D.overflow == MOE_OVERFLOW_REROUTE),
                         moe::aux_loss_workspace_bytes((int)T, (int)E)));
  // packed tile layouts of the gathered x rows and of H when a group can reach the
  // large-tile regime (any expert range holds all of a group's rows)
  const bool pack = packable(D);
  L.x_packed = take(pack && pack_rows_wins(f) ? (size_t)moe::packed_rows_bytes((int64_t)R, (int)E, (int)d) : 0);
  L.hidden = take(std::max(R * f * s, pack ? (size_t)moe::packed_rows_bytes((int64_t)R, (int)E, (int)f) : (size_t)0));
  // H of the groups' tail rows (streaming kernel, row-major at the rows' own positions)
  // when H itself is packed
  L.hidden_tail = take(pack ? R * f * s : 0);
  L.y_perm = take(R * d * s);
  // the shared expert in the large-tile regime: H packed, x rows packed when that pays, a row-major H for
  // its tail rows
  const bool sh_pack = shared_packable(D);
  L.sh_x_packed = take(sh_pack && pack_rows_wins(fs) ? (size_t)moe::packed_rows_bytes((int64_t)T, 1, (int)d) : 0);
  L.sh_hidden = take(std::max(fs ? T * fs * s : 0,
                              sh_pack ? (size_t)moe::packed_rows_bytes((int64_t)T, 1, (int)fs) : (size_t)0));
  L.sh_hidden_tail = take(sh_pack ? T * fs * s : 0);
  L.sh_out = take(fs ? T * d * s : 0);
  L.sh_offsets = take(fs ? 2 * 4 : 0);
  L.router_part = take(D.dtype == MOE_DTYPE_BF16 ? moe::router_partials_bytes((int)T, (int)d, (int)E) : 0);
  L.down_split = take(down_split_bytes(D));
  L.total = o;
  return L;
}

template <typename P>
P *at(void *ws, size_t off) {
  return reinterpret_cast<P *>(static_cast<uint8_t *>(ws) + off);
}

moe::GroupedGemmArgs projection_args(int32_t G, int64_t rows_max, int32_t group_rows_max, int32_t d, int32_t f,
                                     const void *in, const int32_t *offsets, const void *w, void *out, bool gate_up,
                                     const int32_t *row_index = nullptr, int64_t in_rows = 0) {
  moe::GroupedGemmArgs a{};
  a.A = in;
  a.row_index = row_index;
  a.a_rows = in_rows;
  a.offsets = offsets;
  a.num_groups = G;
  a.group_rows_max = group_rows_max;
  a.rows_max = rows_max;
  a.W = w;
  a.w_group_stride = gate_up ? (int64_t)2 * f * d : (int64_t)d * f;
  a.n_out = gate_up ? f : d;
  a.K = gate_up ? d : f;
  a.out = out;
  a.swiglu = gate_up;
  return a;
}

moe_status run_projection(const moe::GroupedGemmArgs &a, int32_t dtype, hipStream_t s, const char *what) {
  return hip_status(dtype == MOE_DTYPE_BF16 ? moe::launch_grouped_gemm_bf16(a, s) : moe::launch_grouped_gemm_f32(a, s),
                    what);
}

moe_status check_projection(int32_t G, int64_t rows_max, int32_t group_rows_max, int32_t d, int32_t f, int32_t dtype) {
  if (G < 1 || G > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID, "num_groups %d outside [1, %d]", G, MOE_MAX_EXPERTS);
  if (rows_max < 0 || rows_max > INT32_MAX) return fail(MOE_ERR_INVALID, "rows_max %lld", (long long)rows_max);
  if (group_rows_max < 1) return fail(MOE_ERR_INVALID, "group_rows_max %d < 1", group_rows_max);
  if (d < 1 || f < 1) return fail(MOE_ERR_INVALID, "d_model and d_ff must be >= 1");
  return check_dtype_dims(dtype, d, f, 0);
}

// Events of moe_forward_staged: ev[0] before the first launch, ev[s + 1] after the launches of
// stage s (moe_stage order).  A stage that launches nothing ends where the previous one did.
struct StageMarks {
  hipEvent_t *ev = nullptr;
  hipStream_t stream = nullptr;
  int next = 0;  // first stage whose end is not yet recorded
  hipError_t err = hipSuccess;
  void start() {
    if (ev && err == hipSuccess) err = hipEventRecord(ev[0], stream);
  }
  void end(int stage) {
    if (!ev) return;
    for (; next <= stage; ++next)
      if (err == hipSuccess) err = hipEventRecord(ev[next + 1], stream);
  }
};

void mark_end(StageMarks *m, int stage) {
  if (m) m->end(stage);
}

// The stages of one grouped FFN (routed experts or the shared expert) as moe_stage values.
struct FfnStages {
  int pack, gate_up, gate_up_tails, down, down_tails;
};
constexpr FfnStages kRoutedStages{MOE_STAGE_PACK_ROWS, MOE_STAGE_GATE_UP, MOE_STAGE_GATE_UP_TAILS, MOE_STAGE_DOWN,
                                  MOE_STAGE_DOWN_TAILS};
constexpr FfnStages kSharedStages{MOE_STAGE_SHARED_PACK_ROWS, MOE_STAGE_SHARED_GATE_UP,
                                  MOE_STAGE_SHARED_GATE_UP_TAILS, MOE_STAGE_SHARED_DOWN,
                                  MOE_STAGE_SHARED_DOWN_TAILS};

struct AfterMain {
  StageMarks *marks;
  int stage;
  static void call(void *ctx) {
    auto *a = static_cast<AfterMain *>(ctx);
    mark_end(a->marks, a->stage);
  }
};

moe_status run_grouped_ffn(int32_t G, int64_t rows_max, int32_t group_rows_max, int32_t d, int32_t f, int32_t dtype,
                           const void *x_rows, const int32_t *offsets, const void *w_gate_up, const void *w_down,
                           void *y_rows, void *hidden, hipStream_t s, const int32_t *row_index = nullptr,
                           int64_t x_row_count = 0, float *split_ws = nullptr, void *x_packed = nullptr,
                           void *hidden_tail = nullptr, const void *w_gate_up_tiled = nullptr,
                           const void *w_down_tiled = nullptr, StageMarks *marks = nullptr,
                           const FfnStages &st = kRoutedStages) {
  AfterMain gu_main{marks, st.gate_up}, dn_main{marks, st.down};
  if (hidden_tail && dtype == MOE_DTYPE_BF16 && moe::grouped_gemm_big_regime(rows_max, G, group_rows_max)) {
    // Large-tile regime: the gate_up projection writes H in the packed tile layout, so that
    // every stage of the down projection loads one contiguous 16 KB block; with x_packed the
    // gathered rows of x are first copied into that layout too (see pack_rows_wins).  The
    // groups' tail rows (left to the streaming kernel) use x and a row-major H instead.
    // one tail choice for both projections and the packing: they number the same tiles
    const int tail = moe::big_tails(G, std::min(d, f));
    const int64_t xb = moe::packed_rows_bytes(rows_max, G, d), hb = moe::packed_rows_bytes(rows_max, G, f);
    const bool pack_x = x_packed != nullptr;
    if (pack_x)
      MOE_TRY_HIP(moe::launch_pack_rows(x_rows, row_index, offsets, G, rows_max, d, x_packed, s, tail), "pack x rows");
    mark_end(marks, st.pack);
    moe::GroupedGemmArgs gu = pack_x ? projection_args(G, rows_max, group_rows_max, d, f, x_packed, offsets, w_gate_up,
                                                       hidden, true, nullptr, xb)
                                     : projection_args(G, rows_max, group_rows_max, d, f, x_rows, offsets, w_gate_up,
                                                       hidden, true, row_index, x_row_count);
    gu.a_packed = pack_x;
    gu.out_packed = true;
    gu.tail = tail;
    gu.tail_A = x_rows;
    gu.tail_row_index = row_index;
    gu.tail_a_rows = row_index ? x_row_count : rows_max;
    gu.tail_out = hidden_tail;
    gu.W_packed = w_gate_up_tiled;
    gu.after_main = AfterMain::call;
    gu.after_main_ctx = &gu_main;
    MOE_TRY(run_projection(gu, dtype, s, "gate_up grouped GEMM"));
    mark_end(marks, st.gate_up_tails);
    moe::GroupedGemmArgs down = projection_args(G, rows_max, group_rows_max, d, f, hidden, offsets, w_down, y_rows,
                                                false, nullptr, hb);
    down.a_packed = true;
    down.tail = tail;
    down.tail_A = hidden_tail;
    down.tail_a_rows = rows_max;
    down.split_ws = split_ws;
    down.W_packed = w_down_tiled;
    down.after_main = AfterMain::call;
    down.after_main_ctx = &dn_main;
    MOE_TRY(run_projection(down, dtype, s, "down grouped GEMM"));
    mark_end(marks, st.down_tails);
    return MOE_OK;
  }
  mark_end(marks, st.pack);  // no row packing in this regime
  moe::GroupedGemmArgs gu = projection_args(G, rows_max, group_rows_max, d, f, x_rows, offsets, w_gate_up, hidden,
                                            true, row_index, x_row_count);
  gu.after_main = AfterMain::call;
  gu.after_main_ctx = &gu_main;
  MOE_TRY(run_projection(gu, dtype, s, "gate_up grouped GEMM"));
  mark_end(marks, st.gate_up_tails);
  moe::GroupedGemmArgs down = projection_args(G, rows_max, group_rows_max, d, f, hidden, offsets, w_down, y_rows, false);
  down.split_ws = split_ws;  // lets the large-tile kernel cut few tiles along K
  down.after_main = AfterMain::call;
  down.after_main_ctx = &dn_main;
  MOE_TRY(run_projection(down, dtype, s, "down grouped GEMM"));
  mark_end(marks, st.down_tails);
  return MOE_OK;
}


}  // namespace

namespace moe {
// Failure with a message, for entry points defined in other files of the library.
moe_status api_fail(moe_status st, const char *what, const char *detail) { return fail(st, "%s: %s", what, detail); }
}  // namespace moe

extern "C" {

int32_t moe_capacity(int32_t num_tokens, int32_t num_experts, double capacity_factor) {
  if (!(capacity_factor > 0.0) || !std::isfinite(capacity_factor)) return MOE_NO_CAPACITY;
  if (num_tokens < 0 || num_experts < 1) return 0;
  const double c = std::ceil(capacity_factor * (double)num_tokens / (double)num_experts);
  if (c >= (double)INT32_MAX) return INT32_MAX;
  return (int32_t)c;
}

int32_t moe_capacity_topk(int32_t num_tokens, int32_t num_experts, int32_t top_k, double capacity_factor) {
  if (!(capacity_factor > 0.0) || !std::isfinite(capacity_factor)) return MOE_NO_CAPACITY;
  if (num_tokens < 0 || num_experts < 1 || top_k < 1) return 0;
  const double c = std::ceil(capacity_factor * ((double)top_k * (double)num_tokens) / (double)num_experts);
  if (c >= (double)INT32_MAX) return INT32_MAX;
  return (int32_t)c;
}

int64_t moe_max_rows(const moe_desc *desc) {
  if (check_desc(desc) != MOE_OK) return -1;
  return max_rows(*desc);
}

size_t moe_workspace_size(const moe_desc *desc) {
  if (check_desc(desc) != MOE_OK) return 0;
  return layout(*desc).total;
}

size_t moe_grouped_gemm_workspace_size(int32_t num_groups, int64_t rows_max, int32_t d_ff, int32_t dtype) {
  if (num_groups < 1 || num_groups > MOE_MAX_EXPERTS || rows_max < 0 || d_ff < 1) return 0;
  if (dtype != MOE_DTYPE_F32 && dtype != MOE_DTYPE_BF16) return 0;
  return align_up((size_t)std::max<int64_t>(rows_max, 1) * d_ff * elem_bytes(dtype));
}

const char *moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: unsupported dtype or shape";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime error";
  }
  return "unknown moe_status";
}

const char *moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_check_topk_ids(const moe_desc *desc, const int32_t *topk_ids_host) {
  MOE_TRY(check_desc(desc));
  if (desc->num_tokens == 0) return ok();
  if (!topk_ids_host) return fail(MOE_ERR_INVALID, "topk_ids_host is NULL");
  MOE_TRY(check_ids_host(*desc, topk_ids_host));
  return ok();
}

int32_t moe_debug_checks(void) {
#ifdef MOE_DEBUG_CHECKS
  return 1;
#else
  return 0;
#endif
}

moe_status moe_router_logits(const moe_desc *desc, const void *x, const void *w_router, const float *logit_offset,
                             float *logits, hipStream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc &D = *desc;
  if (D.num_tokens == 0) return ok();
  MOE_TRY(check_ptr(x, "x"));
  MOE_TRY(check_ptr(w_router, "w_router"));
  MOE_TRY(check_opt_ptr(logit_offset, "logit_offset"));
  MOE_TRY(check_ptr(logits, "logits"));
  if (D.dtype == MOE_DTYPE_BF16)
    MOE_TRY_HIP(moe::launch_router_logits_bf16(x, w_router, logit_offset, logits, D.num_tokens, D.d_model,
                                               D.num_experts, stream), "router logits");
  else
    MOE_TRY_HIP(moe::launch_router_logits_f32(static_cast<const float *>(x), static_cast<const float *>(w_router),
                                              logit_offset, logits, D.num_tokens, D.d_model, D.num_experts, stream),
                "router logits");
  return ok();
}

moe_status moe_router_topk(const moe_desc *desc, const float *logits, int32_t *topk_ids, float *topk_gates,
                           hipStream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc &D = *desc;
  if (D.num_tokens == 0) return ok();
  MOE_TRY(check_ptr(logits, "logits"));
  MOE_TRY(check_ptr(topk_ids, "topk_ids"));
  MOE_TRY(check_ptr(topk_gates, "topk_gates"));
  MOE_TRY_HIP(moe::launch_router_topk(logits, D.num_tokens, D.num_experts, D.top_k, topk_ids, topk_gates, stream),
              "router top-k");
  return ok();
}

moe_status moe_dispatch_permute(const moe_desc *desc, const int32_t *topk_ids, const void *x, int32_t *expert_counts,
                                int32_t *expert_offsets, int32_t *slot, int32_t *row_token, void *x_perm, void *ws,
                                size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc &D = *desc;
  MOE_TRY(check_ptr(expert_offsets, "expert_offsets"));
  MOE_TRY(check_ptr(expert_counts, "expert_counts"));
  if (D.num_tokens == 0) return ok();
  MOE_TRY(check_ptr(topk_ids, "topk_ids"));
  MOE_TRY(check_ptr(slot, "slot"));
  MOE_TRY(check_ptr(row_token, "row_token"));
  MOE_TRY(check_opt_ptr(x_perm, "x_perm"));
  if (x_perm) MOE_TRY(check_ptr(x, "x"));
  if (D.overflow != MOE_OVERFLOW_DROP)
    return fail(MOE_ERR_INVALID, "moe_dispatch_permute drops overflow; redirection is moe_dispatch_reroute");
  const size_t need = moe::dispatch_workspace_bytes(D.num_tokens, D.top_k, D.num_experts, false);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "dispatch needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : (size_t)0);
  MOE_TRY(check_ptr(ws, "ws"));
  MOE_DEBUG_CHECK_IDS(D, topk_ids, stream);
  MOE_TRY_HIP(moe::launch_dispatch(topk_ids, D.num_tokens, D.top_k, D.num_experts, D.capacity,
                                   D.fill_order == MOE_FILL_RANK_MAJOR, expert_counts, expert_offsets, slot, row_token,
                                   static_cast<int32_t *>(ws), stream),
              "dispatch");
  if (x_perm)
    MOE_TRY_HIP(moe::launch_gather_rows(x, row_token, expert_offsets + D.num_experts, max_rows(D), D.d_model,
                                        (int)elem_bytes(D.dtype), x_perm, stream),
                "gather rows");
  return ok();
}

moe_status moe_dispatch_reroute(const moe_desc *desc, const float *logits, const int32_t *topk_ids,
                                int32_t *expert_counts, int32_t *expert_offsets, int32_t *slot, int32_t *assigned_ids,
                                int32_t *row_token, void *ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc &D = *desc;
  MOE_TRY(check_ptr(expert_offsets, "expert_offsets"));
  MOE_TRY(check_ptr(expert_counts, "expert_counts"));
  if (D.num_tokens == 0) return ok();
  MOE_TRY(check_ptr(logits, "logits"));
  MOE_TRY(check_ptr(topk_ids, "topk_ids"));
  MOE_TRY(check_ptr(slot, "slot"));
  MOE_TRY(check_ptr(assigned_ids, "assigned_ids"));
  MOE_TRY(check_ptr(row_token, "row_token"));
  const int T = D.num_tokens, k = D.top_k, E = D.num_experts;
  const size_t spare_bytes = align_up((size_t)T * k * 4);
  const size_t need = spare_bytes + moe::dispatch_workspace_bytes(T, k, E, true);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "dispatch with redirection needs %zu workspace bytes, got %zu", need,
                ws ? ws_bytes : (size_t)0);
  MOE_TRY(check_ptr(ws, "ws"));
  MOE_DEBUG_CHECK_IDS(D, topk_ids, stream);
  const bool rank_major = D.fill_order == MOE_FILL_RANK_MAJOR;
  if (D.capacity == MOE_NO_CAPACITY) {  // nothing overflows
    MOE_TRY_HIP(moe::launch_dispatch(topk_ids, T, k, E, D.capacity, rank_major, expert_counts, expert_offsets, slot,
                                     row_token, static_cast<int32_t *>(ws), stream),
                "dispatch");
    MOE_TRY_HIP(hipMemcpyAsync(assigned_ids, topk_ids, (size_t)T * k * 4, hipMemcpyDeviceToDevice, stream),
                "assigned ids");
    return ok();
  }
  int32_t *spare = static_cast<int32_t *>(ws);
  MOE_TRY_HIP(moe::launch_router_topk(logits, T, E, k, nullptr, nullptr, stream, spare), "next-ranked experts");
  MOE_TRY_HIP(moe::launch_dispatch_reroute(topk_ids, spare, T, k, E, D.capacity, rank_major, expert_counts,
                                           expert_offsets, slot, assigned_ids, row_token,
                                           at<int32_t>(ws, spare_bytes), stream),
              "dispatch with redirection");
  return ok();
}

moe_status moe_grouped_swiglu_gemm(int32_t num_groups, int64_t rows_max, int32_t group_rows_max, int32_t d_model,
                                   int32_t d_ff, int32_t dtype, const void *x_rows, const int32_t *group_offsets,
                                   const void *w_gate_up, const void *w_down, void *y_rows, void *ws, size_t ws_bytes,
                                   hipStream_t stream) {
  MOE_TRY(check_projection(num_groups, rows_max, group_rows_max, d_model, d_ff, dtype));
  if (rows_max == 0) return ok();
  MOE_TRY(check_ptr(x_rows, "x_rows"));
  MOE_TRY(check_ptr(group_offsets, "group_offsets"));
  MOE_TRY(check_ptr(w_gate_up, "w_gate_up"));
  MOE_TRY(check_ptr(w_down, "w_down"));
  MOE_TRY(check_ptr(y_rows, "y_rows"));
  const size_t need = moe_grouped_gemm_workspace_size(num_groups, rows_max, d_ff, dtype);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "grouped GEMM needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : (size_t)0);
  MOE_TRY(check_ptr(ws, "ws"));
  MOE_TRY(run_grouped_ffn(num_groups, rows_max, std::min<int64_t>(group_rows_max, rows_max), d_model, d_ff, dtype,
                          x_rows, group_offsets, w_gate_up, w_down, y_rows, ws, stream));
  return ok();
}

moe_status moe_grouped_gate_up_swiglu(int32_t num_groups, int64_t rows_max, int32_t group_rows_max, int32_t d_model,
                                      int32_t d_ff, int32_t dtype, const void *x_rows, const int32_t *row_index,
                                      int64_t x_row_count, const int32_t *group_offsets, const void *w_gate_up,
                                      void *h_rows, hipStream_t stream) {
  MOE_TRY(check_projection(num_groups, rows_max, group_rows_max, d_model, d_ff, dtype));
  if (rows_max == 0) return ok();
  MOE_TRY(check_ptr(x_rows, "x_rows"));
  MOE_TRY(check_opt_ptr(row_index, "row_index"));
  if (row_index) {
    if (x_row_count < 1) return fail(MOE_ERR_INVALID, "x_row_count %lld < 1 with a row_index", (long long)x_row_count);
    if (x_row_count * d_model * (int64_t)elem_bytes(dtype) >= ((int64_t)1 << 31))
      return fail(MOE_ERR_UNSUPPORTED, "gathered activations must be smaller than 2 GiB");
  }
  MOE_TRY(check_ptr(group_offsets, "group_offsets"));
  MOE_TRY(check_ptr(w_gate_up, "w_gate_up"));
  MOE_TRY(check_ptr(h_rows, "h_rows"));
  MOE_TRY(run_projection(projection_args(num_groups, rows_max, (int32_t)std::min<int64_t>(group_rows_max, rows_max),
                                         d_model, d_ff, x_rows, group_offsets, w_gate_up, h_rows, true, row_index,
                                         x_row_count),
                         dtype, stream, "gate_up grouped GEMM"));
  return ok();
}

moe_status moe_grouped_down(int32_t num_groups, int64_t rows_max, int32_t group_rows_max, int32_t d_model,
                            int32_t d_ff, int32_t dtype, const void *h_rows, const int32_t *group_offsets,
                            const void *w_down, void *y_rows, hipStream_t stream) {
  MOE_TRY(check_projection(num_groups, rows_max, group_rows_max, d_model, d_ff, dtype));
  if (rows_max == 0) return ok();
  MOE_TRY(check_ptr(h_rows, "h_rows"));
  MOE_TRY(check_ptr(group_offsets, "group_offsets"));
  MOE_TRY(check_ptr(w_down, "w_down"));
  MOE_TRY(check_ptr(y_rows, "y_rows"));
  MOE_TRY(run_projection(projection_args(num_groups, rows_max, (int32_t)std::min<int64_t>(group_rows_max, rows_max),
                                         d_model, d_ff, h_rows, group_offsets, w_down, y_rows, false),
                         dtype, stream, "down grouped GEMM"));
  return ok();
}

moe_status moe_combine_unpermute(const moe_desc *desc, const void *y_perm, const int32_t *topk_ids,
                                 const float *topk_gates, const int32_t *slot, const int32_t *expert_offsets,
                                 const void *shared_out, void *out, hipStream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc &D = *desc;
  if (D.num_tokens == 0) return ok();
  MOE_TRY(check_opt_ptr(y_perm, "y_perm"));
  if (!y_perm && max_rows(D) > 0) return fail(MOE_ERR_INVALID, "y_perm is NULL");
  MOE_TRY(check_ptr(topk_ids, "topk_ids"));
  MOE_TRY(check_ptr(topk_gates, "topk_gates"));
  MOE_TRY(check_ptr(slot, "slot"));
  MOE_TRY(check_ptr(expert_offsets, "expert_offsets"));
  MOE_TRY(check_opt_ptr(shared_out, "shared_out"));
  MOE_TRY(check_ptr(out, "out"));
  MOE_DEBUG_CHECK_IDS(D, topk_ids, stream);
  // ids outside [0, E) add nothing (with a slot >= 0 they would index past expert_offsets)
  MOE_TRY_HIP(moe::launch_combine(y_perm, topk_ids, topk_gates, slot, expert_offsets, shared_out, out, D.num_tokens,
                                  D.d_model, D.top_k, D.dtype == MOE_DTYPE_BF16, stream, 0, D.num_experts),
              "combine");
  return ok();
}

moe_status moe_router_aux_loss(const moe_desc *desc, const float *logits, const int32_t *expert_counts, float alpha,
                               float *loss, void *ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc &D = *desc;
  if (D.num_tokens == 0) return ok();
  MOE_TRY(check_ptr(logits, "logits"));
  MOE_TRY(check_ptr(expert_counts, "expert_counts"));
  MOE_TRY(check_ptr(loss, "loss"));
  const size_t need = moe::aux_loss_workspace_bytes(D.num_tokens, D.num_experts);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "aux loss needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : (size_t)0);
  MOE_TRY(check_ptr(ws, "ws"));
  MOE_TRY_HIP(moe::launch_aux_loss(logits, expert_counts, D.num_tokens, D.num_experts, D.top_k, alpha, loss,
                                   static_cast<float *>(ws), stream),
              "aux loss");
  return ok();
}

}  // extern "C"

namespace {

// The layer for experts [e_begin, e_end) of the routing: routing, capacity and dispatch
// over all experts (so slots are those of the whole layer), the FFN of the range's
// experts with its weights (index 0 = expert e_begin), and the combine of their
// contributions, plus the shared expert when add_shared.
moe_status forward_range(const moe_desc &D, const moe_weights *weights, const void *x, const float *logit_offset,
                         void *out, moe_routing *routing, void *ws, size_t ws_bytes, hipStream_t stream,
                         int32_t e_begin, int32_t e_end, bool add_shared, StageMarks *marks = nullptr) {
  if (!weights) return fail(MOE_ERR_INVALID, "weights is NULL");
  if (D.num_tokens == 0) return ok();
  MOE_TRY(check_ptr(x, "x"));
  MOE_TRY(check_ptr(out, "out"));
  MOE_TRY(check_ptr(weights->w_router, "w_router"));
  const bool any_local = e_end > e_begin;
  if (any_local) {
    MOE_TRY(check_ptr(weights->w_gate_up, "w_gate_up"));
    MOE_TRY(check_ptr(weights->w_down, "w_down"));
    MOE_TRY(check_tiled(*weights, D.dtype));
  }
  MOE_TRY(check_opt_ptr(logit_offset, "logit_offset"));
  if (D.d_ff_shared > 0 && add_shared) {
    MOE_TRY(check_ptr(weights->w_shared_gate_up, "w_shared_gate_up"));
    MOE_TRY(check_ptr(weights->w_shared_down, "w_shared_down"));
    MOE_TRY(check_shared_tiled(*weights, D.dtype));
  }
  moe_routing R{};
  if (routing) {
    R = *routing;
    MOE_TRY(check_opt_ptr(R.logits, "routing.logits"));
    MOE_TRY(check_opt_ptr(R.topk_ids, "routing.topk_ids"));
    MOE_TRY(check_opt_ptr(R.topk_gates, "routing.topk_gates"));
    MOE_TRY(check_opt_ptr(R.expert_counts, "routing.expert_counts"));
    MOE_TRY(check_opt_ptr(R.expert_offsets, "routing.expert_offsets"));
    MOE_TRY(check_opt_ptr(R.slot, "routing.slot"));
    MOE_TRY(check_opt_ptr(R.row_token, "routing.row_token"));
    MOE_TRY(check_opt_ptr(R.assigned_ids, "routing.assigned_ids"));
  }
  const Layout L = layout(D);
  if (!ws || ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "moe_forward needs %zu workspace bytes, got %zu", L.total, ws ? ws_bytes : (size_t)0);
  MOE_TRY(check_ptr(ws, "ws"));

  float *logits = R.logits ? R.logits : at<float>(ws, L.logits);
  int32_t *ids = R.topk_ids ? R.topk_ids : at<int32_t>(ws, L.ids);
  float *gates = R.topk_gates ? R.topk_gates : at<float>(ws, L.gates);
  int32_t *counts = R.expert_counts ? R.expert_counts : at<int32_t>(ws, L.counts);
  int32_t *offsets = R.expert_offsets ? R.expert_offsets : at<int32_t>(ws, L.offsets);
  int32_t *slot = R.slot ? R.slot : at<int32_t>(ws, L.slot);
  int32_t *row_token = R.row_token ? R.row_token : at<int32_t>(ws, L.row_token);
  const int T = D.num_tokens, E = D.num_experts, k = D.top_k, d = D.d_model, f = D.d_ff, fs = D.d_ff_shared;
  const bool bf = D.dtype == MOE_DTYPE_BF16;
  const int64_t rmax = max_rows(D);
  void *y_perm = at<void>(ws, L.y_perm);

  if (marks) marks->start();
  if (!bf)
    MOE_TRY_HIP(moe::launch_router_logits_f32(static_cast<const float *>(x),
                                              static_cast<const float *>(weights->w_router), logit_offset, logits, T,
                                              d, E, stream),
                "router logits");
  // router linear + top-k (+ the next k ranks when redirecting overflow)
  auto router = [&](int32_t *spare) -> moe_status {
    if (bf)
      return hip_status(moe::launch_router_bf16(x, weights->w_router, logit_offset, logits, T, d, E, k, ids, gates,
                                                spare, at<float>(ws, L.router_part), stream),
                        "router");
    return hip_status(moe::launch_router_topk(logits, T, E, k, ids, gates, stream, spare), "router top-k");
  };
  const bool rank_major = D.fill_order == MOE_FILL_RANK_MAJOR;
  const int32_t *serving = ids;  // expert of each assignment, as the combine reads it
  if (rerouting(D)) {
    int32_t *spare = at<int32_t>(ws, L.spare);
    int32_t *assigned = R.assigned_ids ? R.assigned_ids : at<int32_t>(ws, L.assigned);
    MOE_TRY(router(spare));
    mark_end(marks, MOE_STAGE_ROUTER);
    MOE_TRY_HIP(moe::launch_dispatch_reroute(ids, spare, T, k, E, D.capacity, rank_major, counts, offsets, slot,
                                             assigned, row_token, at<int32_t>(ws, L.hist), stream),
                "dispatch with redirection");
    serving = assigned;
  } else {
    MOE_TRY(router(nullptr));
    mark_end(marks, MOE_STAGE_ROUTER);
    MOE_TRY_HIP(moe::launch_dispatch(ids, T, k, E, D.capacity, rank_major, counts, offsets, slot, row_token,
                                     at<int32_t>(ws, L.hist), stream),
                "dispatch");
    if (R.assigned_ids)
      MOE_TRY_HIP(hipMemcpyAsync(R.assigned_ids, ids, (size_t)T * k * 4, hipMemcpyDeviceToDevice, stream),
                  "assigned ids");
  }
  mark_end(marks, MOE_STAGE_DISPATCH);
  if (rmax > 0 && any_local) {
    // the gate_up projection gathers each expert's token rows from x through row_token,
    // so the permuted copy of x is never materialised; a range of experts is the slice
    // [e_begin, e_end] of the offsets (rows stay in the whole layer's row space)
    MOE_TRY(run_grouped_ffn(e_end - e_begin, rmax, std::max(1, group_rows_bound(D)), d, f, D.dtype, x,
                            offsets + e_begin, weights->w_gate_up, weights->w_down, y_perm, at<void>(ws, L.hidden),
                            stream, row_token, T, down_split_bytes(D) ? at<float>(ws, L.down_split) : nullptr,
                            packable(D) && pack_rows_wins(f) ? at<void>(ws, L.x_packed) : nullptr,
                            packable(D) ? at<void>(ws, L.hidden_tail) : nullptr, weights->w_gate_up_tiled,
                            weights->w_down_tiled, marks, kRoutedStages));
  }
  const void *shared = nullptr;
  if (fs > 0 && add_shared) {
    int32_t *sh_off = at<int32_t>(ws, L.sh_offsets);
    MOE_TRY_HIP(moe::launch_fill_i32(sh_off, 2, 0, T, stream), "shared offsets");
    const bool sp = shared_packable(D);
    MOE_TRY(run_grouped_ffn(1, T, T, d, fs, D.dtype, x, sh_off, weights->w_shared_gate_up, weights->w_shared_down,
                            at<void>(ws, L.sh_out), at<void>(ws, L.sh_hidden), stream, nullptr, 0, nullptr,
                            sp && pack_rows_wins(fs) ? at<void>(ws, L.sh_x_packed) : nullptr,
                            sp ? at<void>(ws, L.sh_hidden_tail) : nullptr,
                            weights->w_shared_gate_up_tiled, weights->w_shared_down_tiled, marks,
                            kSharedStages));
    shared = at<void>(ws, L.sh_out);
  }
  mark_end(marks, MOE_STAGE_SHARED_DOWN_TAILS);
  MOE_TRY_HIP(moe::launch_combine(y_perm, serving, gates, slot, offsets, shared, out, T, d, k, bf, stream, e_begin,
                                  any_local ? e_end : e_begin),
              "combine");
  mark_end(marks, MOE_STAGE_COMBINE);
  if (marks && marks->err != hipSuccess) return hip_status(marks->err, "stage event record");
  return ok();
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_desc *desc, const moe_weights *weights, const void *x, const float *logit_offset,
                       void *out, moe_routing *routing, void *ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_desc(desc));
  return forward_range(*desc, weights, x, logit_offset, out, routing, ws, ws_bytes, stream, 0, desc->num_experts,
                       true);
}

moe_status moe_forward_staged(const moe_desc *desc, const moe_weights *weights, const void *x,
                              const float *logit_offset, void *out, moe_routing *routing, void *ws, size_t ws_bytes,
                              hipStream_t stream, hipEvent_t *stage_events) {
  MOE_TRY(check_desc(desc));
  if (!stage_events) return fail(MOE_ERR_INVALID, "stage_events is NULL");
  for (int i = 0; i <= MOE_NUM_STAGES; ++i)
    if (!stage_events[i]) return fail(MOE_ERR_INVALID, "stage_events[%d] is NULL", i);
  StageMarks marks;
  marks.ev = stage_events;
  marks.stream = stream;
  if (desc->num_tokens == 0) {  // nothing to launch: every stage is empty
    marks.start();
    marks.end(MOE_NUM_STAGES - 1);
    if (marks.err != hipSuccess) return hip_status(marks.err, "stage event record");
  }
  return forward_range(*desc, weights, x, logit_offset, out, routing, ws, ws_bytes, stream, 0, desc->num_experts,
                       true, &marks);
}

size_t moe_tiled_weights_bytes(const moe_desc *desc, int32_t num_experts, int32_t which) {
  if (check_desc(desc) != MOE_OK || desc->dtype != MOE_DTYPE_BF16 || num_experts < 1 || (which != 0 && which != 1))
    return 0;
  const moe_desc &D = *desc;
  return which == 0 ? (size_t)moe::packed_weights_bytes(num_experts, D.d_ff, D.d_model, true)
                    : (size_t)moe::packed_weights_bytes(num_experts, D.d_model, D.d_ff, false);
}

moe_status moe_tile_expert_weights(const moe_desc *desc, int32_t num_experts, const void *w_gate_up,
                                   const void *w_down, void *w_gate_up_tiled, void *w_down_tiled,
                                   hipStream_t stream) {
  MOE_TRY(check_desc(desc));
  const moe_desc &D = *desc;
  if (D.dtype != MOE_DTYPE_BF16) return fail(MOE_ERR_UNSUPPORTED, "tile-major weights are bf16 only");
  if (num_experts < 1 || num_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_INVALID, "num_experts %d outside [1, %d]", num_experts, MOE_MAX_EXPERTS);
  MOE_TRY(check_ptr(w_gate_up, "w_gate_up"));
  MOE_TRY(check_ptr(w_down, "w_down"));
  MOE_TRY(check_ptr(w_gate_up_tiled, "w_gate_up_tiled"));
  MOE_TRY(check_ptr(w_down_tiled, "w_down_tiled"));
  const int d = D.d_model, f = D.d_ff;
  MOE_TRY_HIP(moe::launch_pack_weights(w_gate_up, num_experts, (int64_t)2 * f * d, f, d, true, w_gate_up_tiled,
                                       stream),
              "tile gate_up weights");
  MOE_TRY_HIP(moe::launch_pack_weights(w_down, num_experts, (int64_t)d * f, d, f, false, w_down_tiled, stream),
              "tile down weights");
  return ok();
}

moe_status moe_forward_expert_shard(const moe_desc *desc, const moe_weights *weights, int32_t expert_begin,
                                    int32_t expert_end, int32_t add_shared, const void *x, const float *logit_offset,
                                    void *out_partial, moe_routing *routing, void *ws, size_t ws_bytes,
                                    hipStream_t stream) {
  MOE_TRY(check_desc(desc));
  if (expert_begin < 0 || expert_end < expert_begin || expert_end > desc->num_experts)
    return fail(MOE_ERR_INVALID, "expert range [%d, %d) outside [0, %d]", expert_begin, expert_end,
                desc->num_experts);
  return forward_range(*desc, weights, x, logit_offset, out_partial, routing, ws, ws_bytes, stream, expert_begin,
                       expert_end, add_shared != 0);
}

}  // extern "C"

// ---------------------------------------------------------------------------- backward

namespace {

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

struct BwdLayout {
  size_t dhp, dgu, hg, dxr, poff, dyT, dguT, xT, row_gate, dpart, dl, dl16, dlT, wr_part, dxrt, tpoff, sh_off, dhs,
      dgus, hs, dxs, dyTT, dgusT, total;
  int64_t Rpad, Tpad, Epad;
  bool long_k, shared_long;
  // many rows per expert: dW_gu is formed as its transpose x^T [dG dU] when x (d columns)
  // is the smaller operand to transpose than [dG dU] (2f columns)
  bool x_first;
};

BwdLayout bwd_layout(const moe_desc &D) {
  BwdLayout L{};
  const int64_t T = D.num_tokens, E = D.num_experts, d = D.d_model, f = D.d_ff, fs = D.d_ff_shared;
  const int64_t R = max_rows(D);
  L.Rpad = round_up(R + 32 * E, 8);  // each group padded to a multiple of 32 rows
  L.Tpad = round_up(T, 32);
  L.Epad = round_up(E, 64);
  size_t o = 0;
  auto take = [&](int64_t bytes) {
    const size_t at = o;
    o += align_up((size_t)std::max<int64_t>(bytes, 0));
    return at;
  };
  const int64_t s = 2;
  L.dhp = take(R * f * s);
  L.dgu = take(R * 2 * f * s);
  L.hg = take(R * f * s);
  L.dxr = take(R * d * s);
  L.poff = take((E + 1) * 4);
  // weight gradients: operands read K-major from the row-major activations (x and dy rows
  // gathered to [R, d]); when experts hold many rows the first operand is transposed instead
  // (padded groups), since the matrix cores then need the LDS read path for themselves
  L.long_k = R / E >= 256 && d >= 256 && f >= 256;
  L.x_first = L.long_k && d < 2 * f;
  L.dyT = take(L.long_k ? d * L.Rpad * s : R * d * s);  // transposed, or gathered rows
  L.dguT = take(L.long_k && !L.x_first ? 2 * f * L.Rpad * s : 0);
  L.xT = take(L.x_first ? d * L.Rpad * s : R * d * s);  // transposed, or gathered rows
  L.row_gate = take(R * 4);
  L.dpart = take(R * (f / 16) * 4);  // gate gradients: dH' . H per row and 16-column block
  L.dl = take(T * E * 4);
  L.dl16 = take(T * L.Epad * s);
  L.dlT = take(L.Epad * L.Tpad * s);
  const int64_t wr_split = moe::wgrad_big_f32_splits((int)E, (int)d, L.Tpad);
  L.wr_part = take(wr_split > 1 ? wr_split * E * d * 4 : 0);
  L.dxrt = take(T * d * s);
  L.tpoff = take(2 * 4);
  L.sh_off = take(2 * 4);
  L.dhs = take(fs ? T * fs * s : 0);
  L.dgus = take(fs ? T * 2 * fs * s : 0);
  L.hs = take(fs ? T * fs * s : 0);
  L.dxs = take(fs ? T * d * s : 0);
  L.shared_long = T >= 256 && d >= 256 && fs >= 256;
  // shared weight gradients with many rows: the smaller of each product's two operands is
  // transposed (dy or g H for dW_sd, [dG dU] or x for dW_sgu)
  L.dyTT = take(fs && L.shared_long ? std::min(d, fs) * L.Tpad * s : 0);
  L.dgusT = take(fs && L.shared_long ? std::min(2 * fs, d) * L.Tpad * s : 0);
  L.total = o;
  return L;
}

moe_status check_bwd_desc(const moe_desc *desc) {
  MOE_TRY(check_desc(desc));
  const moe_desc &D = *desc;
  if (D.dtype != MOE_DTYPE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the backward pass is implemented for bf16 layers");
  const BwdLayout L = bwd_layout(D);
  const int64_t f2 = 2 * (int64_t)std::max(D.d_ff, D.d_ff_shared);
  // operands of the weight-gradient GEMM are addressed through 32-bit buffer offsets
  if (f2 * std::max<int64_t>(L.Rpad, L.Tpad) * 2 >= ((int64_t)1 << 31) ||
      (int64_t)D.d_model * std::max<int64_t>(L.Rpad, L.Tpad) * 2 >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "the backward pass needs its transposed activations to stay below 2 GiB");
  return MOE_OK;
}

// w_stride: elements from one group's weight matrix to the next, and at least the size of
// one matrix (the kernels bound their weight reads by it).
moe::GroupedGemmArgs gemm_args(int32_t G, int64_t rows_max, int32_t group_rows_max, const void *A,
                               const int32_t *row_index, int64_t a_rows, const int32_t *offsets, const void *W,
                               int64_t w_stride, int32_t n_out, int32_t K, void *out, bool out_f32 = false) {
  moe::GroupedGemmArgs a{};
  a.A = A;
  a.row_index = row_index;
  a.a_rows = a_rows;
  a.offsets = offsets;
  a.num_groups = G;
  a.group_rows_max = std::max(1, group_rows_max);
  a.rows_max = rows_max;
  a.W = W;
  a.w_group_stride = w_stride;
  a.n_out = n_out;
  a.K = K;
  a.out = out;
  a.swiglu = false;
  a.out_f32 = out_f32;
  return a;
}

}  // namespace

extern "C" {

size_t moe_backward_workspace_size(const moe_desc *desc) {
  if (check_bwd_desc(desc) != MOE_OK) return 0;
  return bwd_layout(*desc).total;
}

moe_status moe_backward(const moe_desc *desc, const moe_weights *weights, const void *x, const moe_routing *routing,
                        const void *dy, void *dx, moe_grads *grads, void *ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_bwd_desc(desc));
  const moe_desc &D = *desc;
  if (!weights) return fail(MOE_ERR_INVALID, "weights is NULL");
  if (!routing) return fail(MOE_ERR_INVALID, "routing is NULL: pass the tables moe_forward wrote");
  if (!grads) return fail(MOE_ERR_INVALID, "grads is NULL");
  if (D.num_tokens == 0) return ok();
  const int T = D.num_tokens, E = D.num_experts, k = D.top_k, d = D.d_model, f = D.d_ff, fs = D.d_ff_shared;
  MOE_TRY(check_ptr(x, "x"));
  MOE_TRY(check_ptr(dy, "dy"));
  MOE_TRY(check_ptr(dx, "dx"));
  MOE_TRY(check_ptr(weights->w_router, "w_router"));
  MOE_TRY(check_ptr(weights->w_gate_up, "w_gate_up"));
  MOE_TRY(check_ptr(weights->w_down, "w_down"));
  MOE_TRY(check_tiled(*weights, D.dtype));
  MOE_TRY(check_ptr(routing->topk_ids, "routing.topk_ids"));
  MOE_TRY(check_ptr(routing->topk_gates, "routing.topk_gates"));
  MOE_TRY(check_ptr(routing->expert_offsets, "routing.expert_offsets"));
  MOE_TRY(check_ptr(routing->slot, "routing.slot"));
  MOE_TRY(check_ptr(routing->row_token, "routing.row_token"));
  if (rerouting(D)) MOE_TRY(check_ptr(routing->assigned_ids, "routing.assigned_ids"));
  MOE_TRY(check_ptr(grads->dw_router, "grads.dw_router"));
  MOE_TRY(check_ptr(grads->dw_gate_up, "grads.dw_gate_up"));
  MOE_TRY(check_ptr(grads->dw_down, "grads.dw_down"));
  if (fs > 0) {
    MOE_TRY(check_ptr(weights->w_shared_gate_up, "w_shared_gate_up"));
    MOE_TRY(check_ptr(weights->w_shared_down, "w_shared_down"));
    MOE_TRY(check_shared_tiled(*weights, D.dtype));
    MOE_TRY(check_ptr(grads->dw_shared_gate_up, "grads.dw_shared_gate_up"));
    MOE_TRY(check_ptr(grads->dw_shared_down, "grads.dw_shared_down"));
  }
  const BwdLayout L = bwd_layout(D);
  if (!ws || ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "moe_backward needs %zu workspace bytes, got %zu", L.total,
                ws ? ws_bytes : (size_t)0);
  MOE_TRY(check_ptr(ws, "ws"));

  const int32_t *ids = routing->topk_ids, *offsets = routing->expert_offsets, *slot = routing->slot,
                *row_token = routing->row_token;
  const int32_t *serving = rerouting(D) ? routing->assigned_ids : ids;
  const float *gates = routing->topk_gates;
  const int64_t R = max_rows(D);
  const int32_t grb = std::max(1, group_rows_bound(D));
  const int32_t *rows_dev = offsets + E;  // kept rows, on the device
  auto W = [&](size_t off) { return at<void>(ws, off); };
  const int64_t s = 2;
  auto hcall = [&](hipError_t e, const char *what) { return hip_status(e, what); };
  auto gemm = [&](const moe::GroupedGemmArgs &a, const char *what) {
    return hcall(moe::launch_grouped_gemm_bf16(a, stream), what);
  };
  int32_t *poff = at<int32_t>(ws, L.poff), *tpoff = at<int32_t>(ws, L.tpoff), *sh_off = at<int32_t>(ws, L.sh_off);
  MOE_TRY(hcall(moe::launch_fill_i32(tpoff, 2, 0, (int32_t)L.Tpad, stream), "offsets"));
  MOE_TRY(hcall(moe::launch_fill_i32(sh_off, 2, 0, T, stream), "offsets"));

  // ---- routed experts
  if (R > 0) {
    if (L.long_k) MOE_TRY(hcall(moe::launch_pad_offsets(offsets, E, poff, stream), "padded offsets"));
    // dH' = dy W_d: W_d [d, f] per expert is K-major for this product
    auto h = gemm_args(E, R, grb, dy, row_token, T, offsets, weights->w_down, (int64_t)d * f, f, d, W(L.dhp));
    h.w_kn = true;
    MOE_TRY(gemm(h, "dH' grouped GEMM"));
    // G | U of every kept row recomputed from x, and the SwiGLU backward formed from them
    // in the same kernel: dG | dU, g H and the gate gradients' block partials
    MOE_TRY(hcall(moe::launch_row_gate(serving, slot, offsets, gates, (int64_t)T * k, at<float>(ws, L.row_gate),
                                       stream),
                  "row gates"));
    auto r = gemm_args(E, R, grb, x, row_token, T, offsets, weights->w_gate_up, (int64_t)2 * f * d, f, d, W(L.dgu));
    r.swiglu = true;
    r.bwd_dhp = W(L.dhp);
    r.bwd_row_gate = at<float>(ws, L.row_gate);
    r.bwd_hg = W(L.hg);
    r.bwd_dpart = at<float>(ws, L.dpart);
    r.W_packed = weights->w_gate_up_tiled;  // read by the large-tile regime
    MOE_TRY(gemm(r, "gate_up recompute + SwiGLU backward"));
    // dx rows = [dG dU] W_gu (W_gu [2f, d] per expert is K-major for this product)
    auto a = gemm_args(E, R, grb, W(L.dgu), nullptr, 0, offsets, weights->w_gate_up, (int64_t)2 * f * d, d, 2 * f,
                       W(L.dxr));
    a.w_kn = true;
    MOE_TRY(gemm(a, "dx grouped GEMM"));
    // weight gradients, grouped over each expert's rows
    if (L.long_k) {
      // many rows per expert (matrix-core bound): the first operand transposed (padded
      // groups), the second K-major straight from the row-major activations (x rows
      // gathered into expert order)
      MOE_TRY(hcall(moe::launch_transpose_bf16(dy, 0, R, d, 1, row_token, offsets, poff, E, L.Rpad, W(L.dyT), L.Rpad,
                                             0, stream),
                  "dy transpose"));
      MOE_TRY(hcall(moe::launch_wgrad_big_kn(W(L.dyT), L.Rpad, poff, W(L.hg), R, offsets, E, d, f, grads->dw_down,
                                           stream),
                  "dW_down"));
      if (L.x_first) {
        // dW_gu^T = x^T [dG dU]: x transposed like dy, [dG dU] read K-major as written,
        // the product stored transposed
        MOE_TRY(hcall(moe::launch_transpose_bf16(x, 0, R, d, 1, row_token, offsets, poff, E, L.Rpad, W(L.xT),
                                               L.Rpad, 0, stream),
                      "x transpose"));
        MOE_TRY(hcall(moe::launch_wgrad_big_kn(W(L.xT), L.Rpad, poff, W(L.dgu), R, offsets, E, d, 2 * f,
                                             grads->dw_gate_up, stream, true),
                      "dW_gate_up"));
      } else {
        MOE_TRY(hcall(moe::launch_transpose_bf16(W(L.dgu), 0, R, 2 * f, 1, nullptr, offsets, poff, E, L.Rpad,
                                               W(L.dguT), L.Rpad, 0, stream),
                      "dGU transpose"));
        MOE_TRY(hcall(moe::launch_gather_rows(x, row_token, rows_dev, R, d, 2, W(L.xT), stream), "x gather"));
        MOE_TRY(hcall(moe::launch_wgrad_big_kn(W(L.dguT), L.Rpad, poff, W(L.xT), R, offsets, E, 2 * f, d,
                                             grads->dw_gate_up, stream),
                      "dW_gate_up"));
      }
    } else {
      // few rows per expert (write bound): both operands K-major straight from the
      // row-major activations (dy and x rows gathered into expert order), no transposes
      MOE_TRY(hcall(moe::launch_gather_rows(dy, row_token, rows_dev, R, d, 2, W(L.dyT), stream), "dy gather"));
      MOE_TRY(hcall(moe::launch_gather_rows(x, row_token, rows_dev, R, d, 2, W(L.xT), stream), "x gather"));
      MOE_TRY(hcall(moe::launch_wgrad_kn(W(L.dyT), R, W(L.hg), R, offsets, E, d, f, grads->dw_down, stream),
                  "dW_down"));
      MOE_TRY(hcall(moe::launch_wgrad_kn(W(L.dgu), R, W(L.xT), R, offsets, E, 2 * f, d, grads->dw_gate_up, stream),
                  "dW_gate_up"));
    }
  } else {
    MOE_TRY(hcall(moe::launch_fill_u32(grads->dw_down, (int64_t)E * d * f * s / 4, 0u, stream), "zero"));
    MOE_TRY(hcall(moe::launch_fill_u32(grads->dw_gate_up, (int64_t)E * 2 * f * d * s / 4, 0u, stream), "zero"));
  }

  // ---- router: dl from the gate gradients; dW_r = dl^T x, dx += dl W_r
  MOE_TRY(hcall(moe::launch_gates_bwd(ids, gates, at<float>(ws, L.dpart), f / 16, serving, slot, offsets, T, E, k,
                                      (int)L.Epad, at<float>(ws, L.dl), W(L.dl16), stream),
              "gate backward"));
  MOE_TRY(hcall(moe::launch_transpose_bf16(W(L.dl16), 0, T, (int)L.Epad, 1, nullptr, nullptr, nullptr, 0, L.Tpad,
                                         W(L.dlT), L.Tpad, 0, stream),
              "dl transpose"));
  // dW_r = dl^T x over the tokens: dl transposed (small), x read K-major as it is
  MOE_TRY(hcall(moe::launch_wgrad_big_kn_f32(W(L.dlT), L.Tpad, tpoff, x, T, sh_off, E, d, L.Tpad,
                                            at<float>(ws, L.wr_part), static_cast<float *>(grads->dw_router), stream),
              "dW_router"));
  {
    // dl W_r: W_r [E, d] is K-major for this product; the contraction runs over Epad, rows
    // past E read as zeros (and dl16's padding columns are zero)
    auto a = gemm_args(1, T, T, W(L.dl16), nullptr, 0, sh_off, weights->w_router, (int64_t)E * d, d, (int32_t)L.Epad,
                       W(L.dxrt));
    a.w_kn = true;
    MOE_TRY(gemm(a, "router dx"));
  }

  // ---- shared expert (weight 1, every token)
  const void *dxs = nullptr;
  if (fs > 0) {
    {
      auto a = gemm_args(1, T, T, dy, nullptr, 0, sh_off, weights->w_shared_down, (int64_t)d * fs, fs, d, W(L.dhs));
      a.w_kn = true;  // W_sd [d, f_s] is K-major for dy W_sd
      MOE_TRY(gemm(a, "shared dH'"));
    }
    {
      // recompute and SwiGLU backward in one kernel (g = 1, no gate gradient)
      auto r = gemm_args(1, T, T, x, nullptr, 0, sh_off, weights->w_shared_gate_up, (int64_t)2 * fs * d, fs, d,
                         W(L.dgus));
      r.swiglu = true;
      r.bwd_dhp = W(L.dhs);
      r.bwd_hg = W(L.hs);
      r.W_packed = weights->w_shared_gate_up_tiled;  // read by the large-tile regime
      MOE_TRY(gemm(r, "shared gate_up recompute + SwiGLU backward"));
    }
    {
      auto a = gemm_args(1, T, T, W(L.dgus), nullptr, 0, sh_off, weights->w_shared_gate_up, (int64_t)2 * fs * d, d,
                         2 * fs, W(L.dxs));
      a.w_kn = true;  // W_sgu [2 f_s, d] is K-major for [dG dU] W_sgu
      MOE_TRY(gemm(a, "shared dx"));
    }
    if (L.shared_long) {
      // each product transposes its smaller operand; the other form is stored transposed
      auto tr = [&](const void *src, int cols, void *dst, const char *what) {
        return hcall(moe::launch_transpose_bf16(src, 0, T, cols, 1, nullptr, nullptr, nullptr, 0, L.Tpad, dst, L.Tpad,
                                                0, stream),
                     what);
      };
      if (fs < d) {  // dW_sd^T = (g H)^T dy
        MOE_TRY(tr(W(L.hs), fs, W(L.dyTT), "shared H transpose"));
        MOE_TRY(hcall(moe::launch_wgrad_big_kn(W(L.dyTT), L.Tpad, tpoff, dy, T, sh_off, 1, fs, d,
                                             grads->dw_shared_down, stream, true),
                      "dW_shared_down"));
      } else {
        MOE_TRY(tr(dy, d, W(L.dyTT), "dy transpose"));
        MOE_TRY(hcall(moe::launch_wgrad_big_kn(W(L.dyTT), L.Tpad, tpoff, W(L.hs), T, sh_off, 1, d, fs,
                                             grads->dw_shared_down, stream),
                      "dW_shared_down"));
      }
      if (d < 2 * fs) {  // dW_sgu^T = x^T [dG dU]
        MOE_TRY(tr(x, d, W(L.dgusT), "x transpose"));
        MOE_TRY(hcall(moe::launch_wgrad_big_kn(W(L.dgusT), L.Tpad, tpoff, W(L.dgus), T, sh_off, 1, d, 2 * fs,
                                             grads->dw_shared_gate_up, stream, true),
                      "dW_shared_gate_up"));
      } else {
        MOE_TRY(tr(W(L.dgus), 2 * fs, W(L.dgusT), "shared dGU transpose"));
        MOE_TRY(hcall(moe::launch_wgrad_big_kn(W(L.dgusT), L.Tpad, tpoff, x, T, sh_off, 1, 2 * fs, d,
                                             grads->dw_shared_gate_up, stream),
                      "dW_shared_gate_up"));
      }
    } else {
      MOE_TRY(hcall(moe::launch_wgrad_kn(dy, T, W(L.hs), T, sh_off, 1, d, fs, grads->dw_shared_down, stream),
                  "dW_shared_down"));
      MOE_TRY(hcall(moe::launch_wgrad_kn(W(L.dgus), T, x, T, sh_off, 1, 2 * fs, d, grads->dw_shared_gate_up, stream),
                  "dW_shared_gate_up"));
    }
    dxs = W(L.dxs);
  }

  // ---- dx: the expert rows of each token, the router term and the shared expert's
  MOE_TRY(hcall(moe::launch_dx_gather(W(L.dxr), R, serving, slot, offsets, T, d, k, W(L.dxrt), dxs, dx, stream), "dx"));
  return ok();
}

}  // extern "C"
