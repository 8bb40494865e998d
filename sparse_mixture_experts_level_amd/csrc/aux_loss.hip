// Switch-style auxiliary load-balancing loss as a by-product of routing
// ("Sparse Mixture-of-Experts", bigdataschool.ru wiki, section "Маршрутизация
// токена и auxiliary loss": alpha times the number of experts times the sum over
// experts of f_i * P_i, with f_i the share of the batch routed to expert i and P_i
// the router probability of expert i averaged over the batch).
//
// f_i comes from the dispatch's per-expert demand counts (kept or dropped), divided
// by the T * k assignments; P_i needs the full softmax of every token.  Two launches,
// both with fixed summation orders (bit-reproducible):
//   1. aux_colsum_kernel: per block of tokens, the column sums of the softmax
//      probabilities (one wavefront per token, lanes over experts; the waves' partial
//      sums are added in wave order);
//   2. aux_finish_kernel: one block adds the block partials in block order and forms
//      alpha * E * sum_i f_i * P_i, reducing over experts in a fixed tree.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int AX_TOK = 256;   // tokens per block
constexpr int AX_WAVES = 4;

template <int VPL>
__global__ __launch_bounds__(256) void aux_colsum_kernel(const float *__restrict__ logits, int T, int E,
                                                         float *__restrict__ partial) {
  __shared__ float s_part[AX_WAVES][MOE_MAX_EXPERTS_DEV];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * AX_TOK;
  const int t1 = min(T, t0 + AX_TOK);
  float acc[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) acc[v] = 0.f;
  for (int t = t0 + wave; t < t1; t += AX_WAVES) {
    const float *row = logits + (size_t)t * E;
    float l[VPL];
    float m = -INFINITY;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lane + 64 * v;
      l[v] = e < E ? row[e] : -INFINITY;
      m = fmaxf(m, l[v]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float z[VPL], s = 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      z[v] = (lane + 64 * v) < E ? expf(l[v] - m) : 0.f;
      s += z[v];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
    const float inv = 1.0f / s;
#pragma unroll
    for (int v = 0; v < VPL; ++v) acc[v] += z[v] * inv;
  }
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = lane + 64 * v;
    if (e < E) s_part[wave][e] = acc[v];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < AX_WAVES; ++w) sum += s_part[w][e];
    partial[(size_t)blockIdx.x * E + e] = sum;
  }
}

__global__ __launch_bounds__(256) void aux_finish_kernel(const float *__restrict__ partial, int nblocks,
                                                         const int32_t *__restrict__ counts, int T, int E, int k,
                                                         float alpha, float *__restrict__ loss) {
  __shared__ float s_term[256];
  const int tid = threadIdx.x;
  float term = 0.f;
  for (int e = tid; e < E; e += 256) {
    float p = 0.f;
    for (int b = 0; b < nblocks; ++b) p += partial[(size_t)b * E + e];
    const float P = p / (float)T;
    const float f = (float)counts[e] / ((float)T * (float)k);
    term += f * P;
  }
  s_term[tid] = term;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if (tid < o) s_term[tid] += s_term[tid + o];
    __syncthreads();
  }
  if (tid == 0) loss[0] = alpha * (float)E * s_term[0];
}

}  // namespace

size_t aux_loss_workspace_bytes(int T, int E) {
  return (size_t)((T + AX_TOK - 1) / AX_TOK) * E * sizeof(float);
}

hipError_t launch_aux_loss(const float *logits, const int32_t *counts, int T, int E, int k, float alpha, float *loss,
                           float *partial_ws, hipStream_t s) {
  const int nblocks = (T + AX_TOK - 1) / AX_TOK;
  const int vpl = (E + 63) / 64;
#define AX_CASE(V)                                                                                             \
  case V:                                                                                                      \
    hipLaunchKernelGGL(aux_colsum_kernel<V>, dim3(nblocks), dim3(256), 0, s, logits, T, E, partial_ws); \
    break;
  switch (vpl <= 1 ? 1 : vpl <= 2 ? 2 : vpl <= 4 ? 4 : vpl <= 8 ? 8 : 16) {
    AX_CASE(1)
    AX_CASE(2)
    AX_CASE(4)
    AX_CASE(8)
    AX_CASE(16)
  }
#undef AX_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(aux_finish_kernel, dim3(1), dim3(256), 0, s, partial_ws, nblocks, counts, T, E, k, alpha, loss);
  return hipGetLastError();
}

}  // namespace moe
