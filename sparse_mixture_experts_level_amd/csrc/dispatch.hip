// Capacity-limited dispatch of the sparse MoE layer on gfx950 ("Sparse
// Mixture-of-Experts", bigdataschool.ru wiki, sections "Expert capacity и capacity
// factor" and "Подводные камни collapse экспертов и token dropping": first come,
// first served in token order, overflow dropped; the packed runtime path sorts
// tokens by expert id before one grouped GEMM, "Что такое Mixture of Experts (MoE)
// в трансформерах", aglamov.biz, section "Бэкенд для экспертов").
//
// The sequential fill gives assignment (t, j) with expert e the slot
//   slot(t, j) = #{ assignments before (t, j) in fill order with expert e }
// and keeps it iff slot < C.  The fill order is token-major (t, then j) or, as a
// variant, rank-major (j, then t).  That count is a stable counting sort by expert,
// done here in parallel and exactly:
//   1. dispatch_count:  per block of fill positions, a histogram of expert ids;
//   2. dispatch_assign: each block sums the histograms of the blocks before it (its
//      base per expert), the totals give the per-expert kept counts and their
//      exclusive prefix (offsets); inside the block, elements are ranked in order in
//      chunks of 256 (wavefront ballots match equal experts within a wave, per-wave
//      counts in LDS carry the rank across waves);
//   3. gather_rows:     copies x[row_token[r]] into row r of x_perm with 16-byte
//      coalesced vector moves (only when a caller asks for the permuted copy).
// Redirection of overflow to the next most suitable expert ("Архитектура MoE в
// больших языковых моделях", gerwin.io, section "Как работает MoE: принцип
// маршрутизации", load-balancing item 4) runs the same counting sort a second time:
// after the plain fill, each overflowing assignment is offered to the token's next
// ranked expert and the offers are filled, in fill order, into the room the experts
// have left.
// Only order-independent counter increments use atomics, so every output is
// bit-identical from run to run.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int DP_THREADS = 256;
constexpr int DP_MAX_BLOCKS = 64;

// Index into the [T, k] tables of fill position p.
__device__ __forceinline__ int64_t fill_q(int64_t p, int T, int k, bool rank_major) {
  if (!rank_major) return p;
  const int64_t j = p / T;
  return (p - j * T) * k + j;
}

// Histogram of the experts of this block's positions; entries outside [0, E) are skipped
// (negative ones mark "no expert"; larger ones break the caller's precondition and are
// treated as dropped rather than indexing past the tables).
__global__ __launch_bounds__(DP_THREADS) void dispatch_count_kernel(const int32_t *__restrict__ ids, int T, int k,
                                                                    int E, int64_t per_block, int rank_major,
                                                                    int32_t *__restrict__ hist) {
  __shared__ int32_t s_hist[MOE_MAX_EXPERTS_DEV];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += DP_THREADS) s_hist[e] = 0;
  __syncthreads();
  const int64_t n = (int64_t)T * k;
  const int64_t p0 = (int64_t)b * per_block, p1 = min(p0 + per_block, n);
  for (int64_t p = p0 + threadIdx.x; p < p1; p += DP_THREADS) {
    const int e = ids[fill_q(p, T, k, rank_major != 0)];
    if (e >= 0 && e < E) atomicAdd(&s_hist[e], 1);
  }
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

// Sum over blocks of hist[.][e]: all blocks (total) and the blocks before b (before).
__device__ __forceinline__ void hist_sums(const int32_t *__restrict__ hist, int num_blocks, int E, int e, int b,
                                          int &before, int &total) {
  before = 0;
  total = 0;
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
}

constexpr int DP_NW = DP_THREADS / 64;

struct RankLds {
  int32_t wcnt[DP_NW][MOE_MAX_EXPERTS_DEV];  // per-wave count of an expert in the chunk
  int32_t wtag[DP_NW][MOE_MAX_EXPERTS_DEV];  // chunk index the count belongs to
};

// Walks the block's positions [p0, p1) in order, 256 per chunk, and calls
// on_rank(q, e, s_run[e] + rank) for every element whose expert e = sel[q] is in [0, E),
// where rank counts the earlier elements of the walk with the same expert (earlier
// waves of the chunk plus lower lanes of the own wave), and on_skip(q) for every other
// element.  s_run[e] then advances by the chunk's count.  s_run and the tags must be set
// up by the caller (tags to -1).
template <class F, class G>
__device__ __forceinline__ void rank_walk(const int32_t *__restrict__ sel, int T, int k, int E, bool rank_major,
                                          int64_t p0, int64_t p1, int nbits, RankLds &L, int32_t *s_run, F on_rank,
                                          G on_skip) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int chunk = 0;
  for (int64_t c0 = p0; c0 < p1; c0 += DP_THREADS, ++chunk) {
    const int64_t p = c0 + tid;
    const int64_t q = p < p1 ? fill_q(p, T, k, rank_major) : 0;
    const int ev = p < p1 ? sel[q] : -1;
    const bool valid = ev >= 0 && ev < E;
    if (p < p1 && !valid) on_skip(q);
    const int e = valid ? ev : 0;
    const uint64_t m = match_any(e, valid, nbits);
    const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
    const bool leader = valid && in_wave == 0;
    if (leader) {
      L.wcnt[wave][e] = __popcll(m);
      L.wtag[wave][e] = chunk;
    }
    __syncthreads();
    if (valid) {
      int rank = in_wave;
      for (int w = 0; w < wave; ++w) rank += L.wtag[w][e] == chunk ? L.wcnt[w][e] : 0;
      on_rank(q, e, s_run[e] + rank);
    }
    __syncthreads();
    if (leader) atomicAdd(&s_run[e], __popcll(m));  // order-independent: adds this chunk's count
    __syncthreads();
  }
}

__device__ __forceinline__ int bits_for(int E) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  return nbits;
}

// Plain fill (WRITE_ROWS) or the first pass of the two-pass fill (slots only).
template <bool WRITE_ROWS>
__global__ __launch_bounds__(DP_THREADS) void dispatch_assign_kernel(
    const int32_t *__restrict__ ids, int T, int k, int E, int cap, int64_t per_block, int num_blocks, int rank_major,
    const int32_t *__restrict__ hist, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ slot, int32_t *__restrict__ row_token) {
  __shared__ int32_t s_base[MOE_MAX_EXPERTS_DEV];  // running slot per expert for this block
  __shared__ int32_t s_off[MOE_MAX_EXPERTS_DEV];   // kept counts, then their exclusive prefix
  __shared__ int32_t s_part[DP_THREADS];
  __shared__ RankLds L;
  const int b = blockIdx.x, tid = threadIdx.x;

  for (int e = tid; e < E; e += DP_THREADS) {
    int before, total;
    hist_sums(hist, num_blocks, E, e, b, before, total);
    s_base[e] = before;
    s_off[e] = cap < 0 ? total : min(total, cap);
    if (b == 0) counts[e] = total;
#pragma unroll
    for (int w = 0; w < DP_NW; ++w) L.wtag[w][e] = -1;
  }
  __syncthreads();
  if constexpr (WRITE_ROWS) {
    const int kept_total = block_exclusive_scan(s_off, E, s_part);
    if (b == 0) {
      for (int e = tid; e < E; e += DP_THREADS) offsets[e] = s_off[e];
      if (tid == 0) offsets[E] = kept_total;
    }
  }
  const int64_t n = (int64_t)T * k;
  const int64_t p0 = (int64_t)b * per_block, p1 = min(p0 + per_block, n);
  rank_walk(
      ids, T, k, E, rank_major != 0, p0, p1, bits_for(E), L, s_base,
      [&](int64_t q, int e, int sl) {
        if (cap < 0 || sl < cap) {
          slot[q] = sl;
          if constexpr (WRITE_ROWS) row_token[s_off[e] + sl] = int32_t(q / k);
        } else {
          slot[q] = -1;
        }
      },
      [&](int64_t q) { slot[q] = -1; });  // an id outside [0, E): no expert, dropped
}

// The plain fill when one block holds every position (few assignments, e.g. a decode
// step): the histogram, the kept counts' prefix and the ranks in one launch.
__global__ __launch_bounds__(DP_THREADS) void dispatch_single_kernel(const int32_t *__restrict__ ids, int T, int k,
                                                                     int E, int cap, int rank_major,
                                                                     int32_t *__restrict__ counts,
                                                                     int32_t *__restrict__ offsets,
                                                                     int32_t *__restrict__ slot,
                                                                     int32_t *__restrict__ row_token) {
  __shared__ int32_t s_base[MOE_MAX_EXPERTS_DEV];  // running slot per expert
  __shared__ int32_t s_off[MOE_MAX_EXPERTS_DEV];   // demand, then kept counts, then their exclusive prefix
  __shared__ int32_t s_part[DP_THREADS];
  __shared__ RankLds L;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += DP_THREADS) {
    s_base[e] = 0;
    s_off[e] = 0;
#pragma unroll
    for (int w = 0; w < DP_NW; ++w) L.wtag[w][e] = -1;
  }
  __syncthreads();
  const int64_t n = (int64_t)T * k;
  for (int64_t p = tid; p < n; p += DP_THREADS) {
    const int e = ids[fill_q(p, T, k, rank_major != 0)];
    if (e >= 0 && e < E) atomicAdd(&s_off[e], 1);  // order-independent count
  }
  __syncthreads();
  for (int e = tid; e < E; e += DP_THREADS) {
    const int total = s_off[e];
    counts[e] = total;
    s_off[e] = cap < 0 ? total : min(total, cap);
  }
  __syncthreads();
  const int kept_total = block_exclusive_scan(s_off, E, s_part);
  for (int e = tid; e < E; e += DP_THREADS) offsets[e] = s_off[e];
  if (tid == 0) offsets[E] = kept_total;
  rank_walk(
      ids, T, k, E, rank_major != 0, 0, n, bits_for(E), L, s_base,
      [&](int64_t q, int e, int sl) {
        if (cap < 0 || sl < cap) {
          slot[q] = sl;
          row_token[s_off[e] + sl] = int32_t(q / k);
        } else {
          slot[q] = -1;
        }
      },
      [&](int64_t q) { slot[q] = -1; });
}

// Offers of the two-pass fill: the i-th overflowing assignment of token t (in rank
// order j) is offered to spare[t][i], the expert ranked k + i (-1: none).
__global__ __launch_bounds__(256) void reroute_offer_kernel(const int32_t *__restrict__ slot,
                                                            const int32_t *__restrict__ spare, int T, int k,
                                                            int32_t *__restrict__ offer) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  int i = 0;
  for (int j = 0; j < k; ++j) {
    const size_t q = (size_t)t * k + j;
    if (slot[q] < 0) {
      offer[q] = spare[(size_t)t * k + i];
      ++i;
    } else {
      offer[q] = -1;
    }
  }
}

// Second pass: offers take the next free slot of their expert after the first pass's
// kept rows while the expert has room; then every kept row (first pass or offer) is
// written to row_token at the final offsets, and assigned[] gets the serving expert.
__global__ __launch_bounds__(DP_THREADS) void reroute_assign_kernel(
    const int32_t *__restrict__ ids, const int32_t *__restrict__ offer, int T, int k, int E, int cap,
    int64_t per_block, int num_blocks, int rank_major, const int32_t *__restrict__ hist0,
    const int32_t *__restrict__ hist1, int32_t *__restrict__ offsets, int32_t *__restrict__ slot,
    int32_t *__restrict__ assigned, int32_t *__restrict__ row_token) {
  __shared__ int32_t s_base[MOE_MAX_EXPERTS_DEV];  // next slot for this block's offers
  __shared__ int32_t s_off[MOE_MAX_EXPERTS_DEV];   // final kept counts, then their exclusive prefix
  __shared__ int32_t s_part[DP_THREADS];
  __shared__ RankLds L;
  const int b = blockIdx.x, tid = threadIdx.x;

  for (int e = tid; e < E; e += DP_THREADS) {
    int b0, t0, b1, t1;
    hist_sums(hist0, num_blocks, E, e, b, b0, t0);
    hist_sums(hist1, num_blocks, E, e, b, b1, t1);
    const int kept0 = min(t0, cap);
    s_base[e] = kept0 + b1;
    s_off[e] = kept0 + min(t1, cap - kept0);
#pragma unroll
    for (int w = 0; w < DP_NW; ++w) L.wtag[w][e] = -1;
  }
  __syncthreads();
  const int kept_total = block_exclusive_scan(s_off, E, s_part);
  if (b == 0) {
    for (int e = tid; e < E; e += DP_THREADS) offsets[e] = s_off[e];
    if (tid == 0) offsets[E] = kept_total;
  }
  const int64_t n = (int64_t)T * k;
  const int64_t p0 = (int64_t)b * per_block, p1 = min(p0 + per_block, n);
  rank_walk(
      offer, T, k, E, rank_major != 0, p0, p1, bits_for(E), L, s_base,
      [&](int64_t q, int e, int sl) {
        if (sl < cap) {
          slot[q] = sl;
          assigned[q] = e;
          row_token[s_off[e] + sl] = int32_t(q / k);
        } else {
          assigned[q] = ids[q];
        }
      },
      [](int64_t) {});  // no offer: handled below
  // assignments without an offer: kept by the first pass, or dropped with nothing to offer
  for (int64_t p = p0 + tid; p < p1; p += DP_THREADS) {
    const int64_t q = fill_q(p, T, k, rank_major != 0);
    const int o = offer[q];
    if (o >= 0 && o < E) continue;
    const int e = ids[q];
    assigned[q] = e;
    const int sl = slot[q];
    if (sl >= 0) row_token[s_off[e] + sl] = int32_t(q / k);
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

DispatchPlan dispatch_plan(int T, int k) {
  DispatchPlan p;
  const int64_t n = (int64_t)T * k;
  int64_t per = (n + DP_MAX_BLOCKS - 1) / DP_MAX_BLOCKS;
  per = std::max<int64_t>(DP_THREADS, (per + DP_THREADS - 1) / DP_THREADS * DP_THREADS);
  p.per_block = per;
  p.num_blocks = (int)((n + per - 1) / per);
  return p;
}

size_t dispatch_workspace_bytes(int T, int k, int E, bool reroute) {
  const DispatchPlan p = dispatch_plan(T, k);
  const size_t hist = (size_t)p.num_blocks * E * sizeof(int32_t);
  if (!reroute) return hist;
  return 2 * hist + (size_t)T * k * sizeof(int32_t);  // hist0, hist1, offers
}

hipError_t launch_dispatch(const int32_t *ids, int T, int k, int E, int cap, bool rank_major, int32_t *counts,
                           int32_t *offsets, int32_t *slot, int32_t *row_token, int32_t *ws, hipStream_t s) {
  const DispatchPlan p = dispatch_plan(T, k);
  if (p.num_blocks < 1) return hipSuccess;
  if (p.num_blocks == 1) {  // every position in one block: a single launch
    hipLaunchKernelGGL(dispatch_single_kernel, dim3(1), dim3(DP_THREADS), 0, s, ids, T, k, E, cap, (int)rank_major,
                       counts, offsets, slot, row_token);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(p.num_blocks), dim3(DP_THREADS), 0, s, ids, T, k, E, p.per_block,
                     (int)rank_major, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dispatch_assign_kernel<true>, dim3(p.num_blocks), dim3(DP_THREADS), 0, s, ids, T, k, E, cap,
                     p.per_block, p.num_blocks, (int)rank_major, ws, counts, offsets, slot, row_token);
  return hipGetLastError();
}

hipError_t launch_dispatch_reroute(const int32_t *ids, const int32_t *spare, int T, int k, int E, int cap,
                                   bool rank_major, int32_t *counts, int32_t *offsets, int32_t *slot,
                                   int32_t *assigned, int32_t *row_token, int32_t *ws, hipStream_t s) {
  const DispatchPlan p = dispatch_plan(T, k);
  if (p.num_blocks < 1) return hipSuccess;
  int32_t *hist0 = ws, *hist1 = ws + (size_t)p.num_blocks * E, *offer = ws + 2 * (size_t)p.num_blocks * E;
  const int rm = (int)rank_major;
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(p.num_blocks), dim3(DP_THREADS), 0, s, ids, T, k, E, p.per_block, rm,
                     hist0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dispatch_assign_kernel<false>, dim3(p.num_blocks), dim3(DP_THREADS), 0, s, ids, T, k, E, cap,
                     p.per_block, p.num_blocks, rm, hist0, counts, offsets, slot, row_token);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(reroute_offer_kernel, dim3((T + 255) / 256), dim3(256), 0, s, slot, spare, T, k, offer);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(p.num_blocks), dim3(DP_THREADS), 0, s, offer, T, k, E, p.per_block,
                     rm, hist1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(reroute_assign_kernel, dim3(p.num_blocks), dim3(DP_THREADS), 0, s, ids, offer, T, k, E, cap,
                     p.per_block, p.num_blocks, rm, hist0, hist1, offsets, slot, assigned, row_token);
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
