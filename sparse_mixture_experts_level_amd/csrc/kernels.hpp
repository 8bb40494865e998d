// Host-side launchers of the gfx950 kernels (defined in the .hip files).  Each
// launcher only enqueues work on `stream` and returns the launch status; argument
// validation happens in api.cpp before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---- router (router.hip)
hipError_t launch_router_logits_bf16(const void *x, const void *w_router, const float *offset, float *logits,
                                     int T, int d, int E, hipStream_t s);
hipError_t launch_router_logits_f32(const float *x, const float *w_router, const float *offset, float *logits,
                                    int T, int d, int E, hipStream_t s);
// Router linear and top-k in one call for bf16 layers; with few tokens the linear is
// split over d into router_splits() parts whose partial sums (router_partials_bytes()
// of workspace) the top-k kernel adds in order.
int router_splits(int T, int d, int E);
// The router linear as a large-tile GEMM (gemm_big.hip) for many tokens and experts: its
// split count along d (0: not used for this shape) and launch (float partials [S][T][E]).
int router_gemm_splits(int T, int d, int E);
hipError_t launch_router_gemm(const void *x, const void *w_router, int T, int d, int E, float *partials,
                              hipStream_t s);
size_t router_partials_bytes(int T, int d, int E);
hipError_t launch_router_bf16(const void *x, const void *w_router, const float *offset, float *logits, int T, int d,
                              int E, int k, int32_t *ids, float *gates, int32_t *spare, float *partials,
                              hipStream_t s);
// ids / gates may be NULL (not written).  With `spare`, also writes the experts ranked
// k .. 2k-1 per token into spare [T, k] (-1 where the rank is >= E).
hipError_t launch_router_topk(const float *logits, int T, int E, int k, int32_t *ids, float *gates, hipStream_t s,
                              int32_t *spare = nullptr);

// ---- dispatch (dispatch.hip)
// Assignments are walked in fill order: token-major (position p = t * k + j) or, with
// rank_major, rank-major (p = j * T + t).  Blocks own contiguous position ranges.
struct DispatchPlan {
  int64_t per_block;  // positions per block, a multiple of 256
  int num_blocks;
};
DispatchPlan dispatch_plan(int T, int k);
// Workspace of launch_dispatch, or of launch_dispatch_reroute when reroute is set.
size_t dispatch_workspace_bytes(int T, int k, int E, bool reroute);
hipError_t launch_dispatch(const int32_t *ids, int T, int k, int E, int cap /* <0: none */, bool rank_major,
                           int32_t *counts, int32_t *offsets, int32_t *slot, int32_t *row_token, int32_t *ws,
                           hipStream_t s);
// Two-pass fill: the plain fill, then every overflowing assignment is offered to the
// token's next ranked expert (spare [T, k] from launch_router_topk: the i-th overflow of
// a token takes spare[t][i]) and kept if that expert has room left; assigned [T, k]
// receives the serving expert of each assignment.  cap >= 0.
hipError_t launch_dispatch_reroute(const int32_t *ids, const int32_t *spare, int T, int k, int E, int cap,
                                   bool rank_major, int32_t *counts, int32_t *offsets, int32_t *slot,
                                   int32_t *assigned, int32_t *row_token, int32_t *ws, hipStream_t s);
hipError_t launch_gather_rows(const void *x, const int32_t *row_token, const int32_t *offsets_end, int64_t rows_max,
                              int d, int elem_bytes, void *x_perm, hipStream_t s);

// ---- grouped expert GEMMs (gemm_stream.hip, gemm_f32.hip)
// Problem: for group g, rows [offsets[g], offsets[g+1]) of A [rows, K] times the
// group's weight W_g [N_w, K] (K contiguous).  With swiglu, N_w = 2 * n_out and
// out[r, n] = silu(A_r . W_g[n]) * (A_r . W_g[n_out + n]); otherwise N_w = n_out and
// out[r, n] = A_r . W_g[n].  `w_group_stride` is in elements.
struct GroupedGemmArgs {
  const void *A;
  // Optional row gather: with row_index set, row r of a group is A[row_index[r]] and A
  // holds a_rows rows; otherwise rows are contiguous in A.
  const int32_t *row_index;
  int64_t a_rows;
  const int32_t *offsets;
  int num_groups;
  int group_rows_max;  // tiling hint
  int64_t rows_max;    // bound on the total rows over all groups
  const void *W;
  int64_t w_group_stride;
  int n_out;
  int K;
  void *out;
  bool swiglu;
  bool out_f32 = false;  // float output instead of the element type (bf16 kernels, no SwiGLU)
  // Workspace for float partial sums when the large-tile kernel cuts few tiles along K
  // (4 * rows_max * n_out floats); NULL: no K split.
  float *split_ws = nullptr;
  // Weights stored K-major: group g's matrix is [K, n_out] (row stride n_out) instead of
  // [n_out, K] -- the layout the backward pass multiplies by (dy W_d, dGU W_gu).  No SwiGLU.
  bool w_kn = false;
  // Large-tile regime only: A in the packed tile layout (launch_pack_rows; a_rows then
  // bounds the packed buffer in bytes, row_index unused), and/or the SwiGLU output written
  // in that layout for a following large-tile GEMM over the same groups (out sized
  // packed_rows_bytes(rows_max, num_groups, n_out)).
  bool a_packed = false;
  bool out_packed = false;
  // SwiGLU backward epilogue (with swiglu, bf16, plain row layout): instead of H, the
  // kernel forms from the float G, U of each row and bwd_dhp = dH' (bf16 [rows, n_out],
  // rows in group order) out = [dG | dU] (bf16 [rows, 2 n_out]), bwd_hg = g H (bf16
  // [rows, n_out]) and, when bwd_dpart is set, the dot products dH' . H of each row over
  // each 16-column block (float [rows, n_out / 16]); g = bwd_row_gate[row], or 1 when NULL.
  const void *bwd_dhp = nullptr;
  const float *bwd_row_gate = nullptr;
  void *bwd_hg = nullptr;
  float *bwd_dpart = nullptr;
  // Tails, large-tile regime: with tail = kBigTailRows a group's last partial 256-row tile
  // of at most that many rows is left to a streaming launch over the same groups
  // (re-reading that group's weights then costs less than a nearly empty tile); 0: every
  // row in large tiles; -1: chosen by the launch (big_tails()).  With a packed A or output
  // the tail launch reads tail_A instead (row-major; rows through tail_row_index when
  // given, tail_a_rows rows) and writes tail_out (row-major, rows in group order).
  int tail = -1;
  const void *tail_A = nullptr;
  const int32_t *tail_row_index = nullptr;
  int64_t tail_a_rows = 0;
  void *tail_out = nullptr;
  // Streaming kernel: compute only each group's tail rows (set by the large-tile launch).
  bool tails_only = false;
  // The same weights in the packed tile layout (launch_pack_weights), or NULL: the
  // large-tile kernel then reads them with the packed activations or the SwiGLU backward
  // epilogue; the streaming kernel (tails included) reads W.
  const void *W_packed = nullptr;
  // Called on the host after the large-tile launch (and its K-split sum) is enqueued,
  // before the tail launch: lets the caller mark the stream between the two.
  void (*after_main)(void *ctx) = nullptr;
  void *after_main_ctx = nullptr;
};

// Large-tile row tiles and the tail rows left to the streaming kernel.
constexpr int kBigTileRows = 256, kBigTailRows = 128;
// The tail threshold for a large-tile launch over G groups with n_out output columns: the
// streaming tail launch (one workgroup per group and 64 columns) must fill the GPU.
inline int big_tails(int G, int n_out) { return (int64_t)G * ((n_out + 63) / 64) >= 512 ? kBigTailRows : 0; }

// Device-side form of the SwiGLU backward outputs (kernel argument).
struct SwigluBwdOut {
  const uint16_t *dhp;  // bf16
  const float *row_gate;
  uint16_t *hg;        // bf16
  float *dpart;
};
hipError_t launch_grouped_gemm_bf16(const GroupedGemmArgs &a, hipStream_t s);
// Packed tile layout of grouped rows for the large-tile GEMM's A operand: per 256-row tile
// of a group (numbered over all groups in order) and 32-wide K step, a 16 KB block laid out
// as the GEMM's LDS stage; rows gathered through row_index when given.
int64_t packed_rows_bytes(int64_t rows_max, int G, int K);
// Packed tile layout of G groups' row-major weights ([rows, K] each, group stride wstride
// elements) for the large-tile kernel's B operand: per group, weight tile (256 rows: with
// SwiGLU 128 gate rows and the matching up rows, n_out apart) and 32-wide K step, one 16 KB
// block laid out as the kernel's LDS stage; rows past n_out zero.  K a multiple of 32.
int64_t packed_weights_bytes(int G, int n_out, int K, bool swiglu);
hipError_t launch_pack_weights(const void *W, int G, int64_t wstride, int n_out, int K, bool swiglu, void *out,
                               hipStream_t s);
hipError_t launch_pack_rows(const void *src, const int32_t *row_index, const int32_t *offsets, int G, int64_t rows_max,
                            int K, void *out, hipStream_t s, int tail = 0);
// Whether launch_grouped_gemm_bf16 takes the large-tile kernel (many rows per group)
// rather than the streaming one; either reads weights in both layouts (w_kn).
bool grouped_gemm_big_regime(int64_t rows_max, int num_groups, int group_rows_max);
hipError_t launch_grouped_gemm_stream_bf16(const GroupedGemmArgs &a, hipStream_t s);
hipError_t launch_grouped_gemm_big_bf16(const GroupedGemmArgs &a, int64_t rows_total_max, hipStream_t s);
hipError_t launch_grouped_gemm_f32(const GroupedGemmArgs &a, hipStream_t s);

// ---- combine (combine.hip)
hipError_t launch_combine(const void *y_perm, const int32_t *ids, const float *gates, const int32_t *slot,
                          const int32_t *offsets, const void *shared, void *out, int T, int d, int k, bool bf16,
                          hipStream_t s, int e_begin = 0, int e_end = 1 << 30);

// ---- auxiliary load-balancing loss (aux_loss.hip)
size_t aux_loss_workspace_bytes(int T, int E);
hipError_t launch_aux_loss(const float *logits, const int32_t *counts, int T, int E, int k, float alpha, float *loss,
                           float *partial_ws, hipStream_t s);

// ---- small utilities (combine.hip)
hipError_t launch_fill_i32(int32_t *p, int n, int32_t v0, int32_t step, hipStream_t s);

// ---- backward (backward.hip); bf16 activations and weights
// Plain: out[b][c][p] = in[b][p][c] for p < P, zero for p >= rows (row stride out_ld).
// Grouped (group offsets off / poff, G groups): position p of group g holds row off[g] +
// (p - poff[g]) inside the group's rows (through row_index when given), zero in its
// padding, written group-major: group g's [cols, K_g] block at poff[g] * cols, row stride
// K_g = poff[g+1] - poff[g].
hipError_t launch_transpose_bf16(const void *in, int64_t in_stride_b, int64_t rows, int cols, int batch,
                                 const int32_t *row_index, const int32_t *off, const int32_t *poff, int G, int64_t P,
                                 void *out, int64_t out_ld, int64_t out_stride_b, hipStream_t s);
// poff[g] = sum over g' < g of ceil32(off[g'+1] - off[g']), poff[G] = total
hipError_t launch_pad_offsets(const int32_t *off, int G, int32_t *poff, hipStream_t s);
hipError_t launch_fill_u32(void *p, int64_t n_words, uint32_t v, hipStream_t s);
// dl (float [T, E]) and dl16 (bf16 [T, Epad]) from the gate gradients: dg of each kept
// assignment is the sum of the nb block partials [rows, nb] of its row in dpart.
hipError_t launch_gates_bwd(const int32_t *ids, const float *gates, const float *dpart, int nb, const int32_t *serving,
                            const int32_t *slot, const int32_t *offsets, int T, int E, int k, int Epad, float *dl,
                            void *dl16, hipStream_t s);
// row_gate[offsets[serving[i]] + slot[i]] = gates[i] for every kept assignment i < n.
hipError_t launch_row_gate(const int32_t *serving, const int32_t *slot, const int32_t *offsets, const float *gates,
                           int64_t n, float *row_gate, hipStream_t s);
// dx[t] = sum over kept j of dxr[row(t, j)], then extra[t] and extra2[t] when given (float,
// in that order); dxr holds `rows` rows.
hipError_t launch_dx_gather(const void *dxr, int64_t rows, const int32_t *serving, const int32_t *slot,
                            const int32_t *offsets, int T, int d, int k, const void *extra, const void *extra2, void *dx,
                            hipStream_t s);
// out[g][m][n] = sum over rows r in [off[g], off[g+1]) of A[r][m] B[r][n] from row-major
// (K-major) A [a_rows, M] and B [b_rows, N], bf16 out; 128 x 128 tiles for short row
// ranges, no transposes.  M, N multiples of 8; operands below 2 GiB.
hipError_t launch_wgrad_kn(const void *A, int64_t a_rows, const void *B, int64_t b_rows, const int32_t *off, int G,
                           int M, int N, void *out, hipStream_t s);
// out[i] = sum over s < S of part[s * n + i], in slice order (float, n a multiple of 4).
hipError_t launch_ksplit_sum(const float *part, int S, int64_t n, float *out, hipStream_t s);
// out[m][n] = sum over k < K of AT[m][k] B[k][n] in float for one group: AT [M, K] with row
// stride K = poff[1] - poff[0] (a multiple of 32), B [b_rows, N] row-major with rows off_b[0]
// .. off_b[1] - 1; the large-tile weight-gradient form cut along K into
// wgrad_big_f32_splits(M, N, K) slices, their partials in part (that many * M * N floats)
// added in order.  N a multiple of 8.
int wgrad_big_f32_splits(int M, int N, int64_t K);
hipError_t launch_wgrad_big_kn_f32(const void *AT, int64_t lda, const int32_t *poff, const void *B, int64_t b_rows,
                                   const int32_t *off_b, int M, int N, int64_t K, float *part, float *out,
                                   hipStream_t s);
// out[g][m][n] = sum over k < K_g of AT_g[m][k] B[off_b[g] + k][n]: AT group-major transposed
// (group g's [M, K_g] block at poff[g] * M, K_g = poff[g+1] - poff[g] a multiple of 32, zero
// padding), B [b_rows, N] row-major (K-major, unpadded; k past the group's rows reads zero);
// 256 x 256 tiles.  With `transposed` each out[g] is stored as [N, M] (out[g][n][m]).
hipError_t launch_wgrad_big_kn(const void *AT, int64_t lda, const int32_t *poff, const void *B, int64_t b_rows,
                               const int32_t *off_b, int G, int M, int N, void *out, hipStream_t s,
                               bool transposed = false);
}  // namespace moe
