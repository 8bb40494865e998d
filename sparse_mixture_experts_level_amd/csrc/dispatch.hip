// Capacity-limited dispatch of the sparse MoE layer on gfx950 ("Sparse
// Mixture-of-Experts", bigdataschool.ru wiki, sections "Expert capacity и capacity
// factor" and "Подводные камни collapse экспертов и token dropping": first come,
// first served in token order, overflow dropped; the packed runtime path sorts
// tokens by expert id before one grouped GEMM, "Что такое Mixture of Experts (MoE)
// в трансформерах", aglamov.biz, section "Бэкенд для экспертов").
//
// The sequential fill gives assignment (t, j) with expert e the slot
//   slot(t, j) = #{ assignments (t', j') before (t, j) in token-major order with expert e }
// and keeps it iff slot < C.  That count is a stable counting sort by expert, done
// here in parallel and exactly:
//   1. dispatch_count:  per token block, a histogram of expert ids (LDS counters);
//   2. dispatch_assign: each block sums the histograms of the blocks before it (its
//      base per expert), the totals give the per-expert kept counts and their
//      exclusive prefix (offsets); inside the block, elements are ranked in order in
//      chunks of 256 (wavefront ballots match equal experts within a wave, per-wave
//      counts in LDS carry the rank across waves);
//   3. gather_rows:     copies x[row_token[r]] into row r of x_perm with 16-byte
//      coalesced vector moves.
// Only order-independent counter increments use atomics, so every output is
// bit-identical from run to run.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int DP_THREADS = 256;
constexpr int DP_MAX_BLOCKS = 64;

__global__ __launch_bounds__(DP_THREADS) void dispatch_count_kernel(const int32_t *__restrict__ ids, int T, int k,
                                                                    int E, int tokens_per_block,
                                                                    int32_t *__restrict__ hist) {
  __shared__ int32_t s_hist[MOE_MAX_EXPERTS_DEV];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += DP_THREADS) s_hist[e] = 0;
  __syncthreads();
  const int64_t q0 = (int64_t)b * tokens_per_block * k;
  const int64_t q1 = min((int64_t)(b + 1) * tokens_per_block, (int64_t)T) * k;
  for (int64_t q = q0 + threadIdx.x; q < q1; q += DP_THREADS) atomicAdd(&s_hist[ids[q]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += DP_THREADS) hist[(size_t)b * E + e] = s_hist[e];
}

// Block-wide exclusive scan of n <= MOE_MAX_EXPERTS_DEV values held in s[] (in place);
// returns the total.  Deterministic: fixed-shape tree over fixed partitions.
__device__ int block_exclusive_scan(int32_t *s, int n, int32_t *s_part) {
  constexpr int PER = (MOE_MAX_EXPERTS_DEV + DP_THREADS - 1) / DP_THREADS;
  const int tid = threadIdx.x;
  int vals[PER];
  int local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid * PER + i;
    vals[i] = e < n ? s[e] : 0;
    local += vals[i];
  }
  s_part[tid] = local;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 256 partial sums
  for (int off = 1; off < DP_THREADS; off <<= 1) {
    const int v = tid >= off ? s_part[tid - off] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  const int total = s_part[DP_THREADS - 1];
  int run = tid ? s_part[tid - 1] : 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid * PER + i;
    if (e < n) s[e] = run;
    run += vals[i];
  }
  __syncthreads();
  return total;
}

// Lanes of the calling wavefront whose value equals this lane's (only lanes with
// `active` set take part); nbits = bits needed for the largest value.
__device__ __forceinline__ uint64_t match_any(int v, bool active, int nbits) {
  uint64_t m = __ballot(active);
  for (int bit = 0; bit < nbits; ++bit) {
    const uint64_t b = __ballot(active && ((v >> bit) & 1));
    m &= ((v >> bit) & 1) ? b : ~b;
  }
  return active ? m : 0ull;
}

__global__ __launch_bounds__(DP_THREADS) void dispatch_assign_kernel(
    const int32_t *__restrict__ ids, int T, int k, int E, int cap, int tokens_per_block, int num_blocks,
    const int32_t *__restrict__ hist, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ slot, int32_t *__restrict__ row_token) {
  constexpr int NW = DP_THREADS / 64;
  __shared__ int32_t s_base[MOE_MAX_EXPERTS_DEV];  // running slot per expert for this block
  __shared__ int32_t s_off[MOE_MAX_EXPERTS_DEV];   // kept counts, then their exclusive prefix
  __shared__ int32_t s_part[DP_THREADS];
  __shared__ int32_t s_wcnt[NW][MOE_MAX_EXPERTS_DEV];  // per-wave count of an expert in the chunk
  __shared__ int32_t s_wtag[NW][MOE_MAX_EXPERTS_DEV];  // chunk index the count belongs to
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int e = tid; e < E; e += DP_THREADS) {
    int before = 0, total = 0;
    for (int bb0 = 0; bb0 < num_blocks; bb0 += 16) {  // 16 independent loads in flight
      int h[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) h[i] = bb0 + i < num_blocks ? hist[(size_t)(bb0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        before += bb0 + i < b ? h[i] : 0;
        total += h[i];
      }
    }
    s_base[e] = before;
    s_off[e] = cap < 0 ? total : min(total, cap);
    if (b == 0) counts[e] = total;
#pragma unroll
    for (int w = 0; w < NW; ++w) s_wtag[w][e] = -1;
  }
  __syncthreads();
  const int kept_total = block_exclusive_scan(s_off, E, s_part);
  if (b == 0) {
    for (int e = tid; e < E; e += DP_THREADS) offsets[e] = s_off[e];
    if (tid == 0) offsets[E] = kept_total;
  }
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;

  // Elements of the block in token-major order, 256 per chunk: the rank of an element
  // among earlier elements of the chunk with the same expert is the count in earlier
  // waves plus the count of lower lanes of its own wave.
  const int64_t q0 = (int64_t)b * tokens_per_block * k;
  const int64_t q1 = min((int64_t)(b + 1) * tokens_per_block, (int64_t)T) * k;
  int chunk = 0;
  for (int64_t c0 = q0; c0 < q1; c0 += DP_THREADS, ++chunk) {
    const int64_t q = c0 + tid;
    const bool valid = q < q1;
    const int e = valid ? ids[q] : 0;
    const uint64_t m = match_any(e, valid, nbits);
    const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
    const bool leader = valid && in_wave == 0;
    if (leader) {
      s_wcnt[wave][e] = __popcll(m);
      s_wtag[wave][e] = chunk;
    }
    __syncthreads();
    if (valid) {
      int rank = in_wave;
      for (int w = 0; w < wave; ++w) rank += s_wtag[w][e] == chunk ? s_wcnt[w][e] : 0;
      const int sl = s_base[e] + rank;
      if (cap < 0 || sl < cap) {
        slot[q] = sl;
        row_token[s_off[e] + sl] = int32_t(q / k);
      } else {
        slot[q] = -1;
      }
    }
    __syncthreads();
    if (leader) atomicAdd(&s_base[e], __popcll(m));  // order-independent: adds this chunk's count
    __syncthreads();
  }
}

// One wavefront per row: 16-byte moves, rows at or beyond offsets[E] are skipped.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t *__restrict__ x,
                                                          const int32_t *__restrict__ row_token,
                                                          const int32_t *__restrict__ offsets_end, int64_t rows_max,
                                                          int row_bytes, uint8_t *__restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows_max || r >= *offsets_end) return;
  const uint8_t *src = x + (size_t)row_token[r] * row_bytes;
  uint8_t *dst = x_perm + (size_t)r * row_bytes;
  if ((row_bytes & 15) == 0) {
    for (int c = lane * 16; c < row_bytes; c += 64 * 16) stg16(dst + c, ldg16(src + c));
  } else {  // float rows whose width is not a multiple of 4 elements: 4-byte moves
    for (int c = lane * 4; c < row_bytes; c += 64 * 4)
      *reinterpret_cast<uint32_t *>(dst + c) = *reinterpret_cast<const uint32_t *>(src + c);
  }
}

}  // namespace

DispatchPlan dispatch_plan(int T) {
  DispatchPlan p;
  int tpb = (T + DP_MAX_BLOCKS - 1) / DP_MAX_BLOCKS;
  tpb = max(64, ((tpb + 63) / 64) * 64);
  p.tokens_per_block = tpb;
  p.num_blocks = (T + tpb - 1) / tpb;
  return p;
}

size_t dispatch_workspace_bytes(int T, int E) {
  const DispatchPlan p = dispatch_plan(T);
  return (size_t)p.num_blocks * E * sizeof(int32_t);
}

hipError_t launch_dispatch(const int32_t *ids, int T, int k, int E, int cap, int32_t *counts, int32_t *offsets,
                           int32_t *slot, int32_t *row_token, int32_t *hist_ws, hipStream_t s) {
  const DispatchPlan p = dispatch_plan(T);
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(p.num_blocks), dim3(DP_THREADS), 0, s, ids, T, k, E,
                     p.tokens_per_block, hist_ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dispatch_assign_kernel, dim3(p.num_blocks), dim3(DP_THREADS), 0, s, ids, T, k, E, cap,
                     p.tokens_per_block, p.num_blocks, hist_ws, counts, offsets, slot, row_token);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void *x, const int32_t *row_token, const int32_t *offsets_end, int64_t rows_max,
                              int d, int elem_bytes, void *x_perm, hipStream_t s) {
  if (rows_max <= 0) return hipSuccess;
  const int64_t grid = (rows_max + 3) / 4;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const uint8_t *>(x),
                     row_token, offsets_end, rows_max, d * elem_bytes, static_cast<uint8_t *>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
