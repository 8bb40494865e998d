// Gate-weighted combine back to token order ("Sparse Mixture-of-Experts",
// bigdataschool.ru wiki, section "Роутер и top-k gating": the layer output is the
// sum of the selected experts' outputs weighted by the renormalised router
// probabilities; section "Expert capacity и capacity factor": a dropped assignment
// adds nothing).  Each token gathers its kept rows -- no atomics, so the sum order
// (shared expert first, then j = 0..k-1) is fixed and the result deterministic.
// Contributions can be restricted to experts [e_begin, e_end) -- one rank's share of
// expert parallelism.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int CB_TOK = 4;  // tokens per workgroup, one wavefront each
constexpr int CB_U = 4;    // 16-byte vectors per lane per pass

// One wavefront per token.  Lanes j < k fetch assignment j's slot, expert and gate in
// parallel and resolve its row; the wave then streams the row vectors, each lane
// summing its columns over j in order.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void *__restrict__ y_perm, const int32_t *__restrict__ ids,
                                                      const float *__restrict__ gates,
                                                      const int32_t *__restrict__ slot,
                                                      const int32_t *__restrict__ offsets,
                                                      const void *__restrict__ shared, void *__restrict__ out, int T,
                                                      int d, int k, int e_begin, int e_end) {
  constexpr int VEC = BF16 ? 8 : 4;  // elements per 16-byte vector
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * CB_TOK + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nvec = d / VEC;
  const size_t es = BF16 ? 2 : 4;
  const uint8_t *yb = static_cast<const uint8_t *>(y_perm);
  for (int v0 = 0; v0 < nvec; v0 += 64 * CB_U) {
    float acc[CB_U][VEC];
#pragma unroll
    for (int u = 0; u < CB_U; ++u) {
      const int c = v0 + lane + 64 * u;
#pragma unroll
      for (int i = 0; i < VEC; ++i) acc[u][i] = 0.f;
      if (shared && c < nvec) {
        const u32x4 q = ldg16(static_cast<const uint8_t *>(shared) + ((size_t)t * d + (size_t)c * VEC) * es);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (BF16) {
            acc[u][2 * i] = __uint_as_float(q[i] << 16);
            acc[u][2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
          } else {
            acc[u][i] = __uint_as_float(q[i]);
          }
        }
      }
    }
    for (int j0 = 0; j0 < k; j0 += 64) {
      // lane j holds assignment j0 + j: its row (or -1) and gate
      int64_t my_row = -1;
      float my_gate = 0.f;
      if (j0 + lane < k) {
        const size_t q = (size_t)t * k + j0 + lane;
        const int sl = slot[q];
        const int e = ids[q];
        my_gate = gates[q];
        if (sl >= 0 && e >= e_begin && e < e_end) my_row = (int64_t)offsets[e] + sl;
      }
      const int kn = min(64, k - j0);
      for (int j = 0; j < kn; ++j) {
        const int64_t row = __shfl(my_row, j, 64);
        const float gj = __shfl(my_gate, j, 64);
        if (row < 0) continue;
        const uint8_t *yr = yb + (size_t)row * d * es;
#pragma unroll
        for (int u = 0; u < CB_U; ++u) {
          const int c = v0 + lane + 64 * u;
          if (c >= nvec) continue;
          const u32x4 q = ldg16(yr + (size_t)c * VEC * es);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (BF16) {
              acc[u][2 * i] = fmaf(gj, __uint_as_float(q[i] << 16), acc[u][2 * i]);
              acc[u][2 * i + 1] = fmaf(gj, __uint_as_float(q[i] & 0xffff0000u), acc[u][2 * i + 1]);
            } else {
              acc[u][i] = fmaf(gj, __uint_as_float(q[i]), acc[u][i]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < CB_U; ++u) {
      const int c = v0 + lane + 64 * u;
      if (c >= nvec) continue;
      u32x4 q;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (BF16) {
          q[i] = pack_bf16x2(acc[u][2 * i], acc[u][2 * i + 1]);
        } else {
          q[i] = __float_as_uint(acc[u][i]);
        }
      }
      stg16(static_cast<uint8_t *>(out) + ((size_t)t * d + (size_t)c * VEC) * es, q);
    }
  }
}

// Scalar fallback for float rows whose width is not a multiple of 4 elements.
__global__ __launch_bounds__(256) void combine_f32_scalar_kernel(const float *__restrict__ y_perm,
                                                                 const int32_t *__restrict__ ids,
                                                                 const float *__restrict__ gates,
                                                                 const int32_t *__restrict__ slot,
                                                                 const int32_t *__restrict__ offsets,
                                                                 const float *__restrict__ shared,
                                                                 float *__restrict__ out, int d, int k, int e_begin,
                                                                 int e_end) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x; c < d; c += 256) {
    float acc = shared ? shared[(size_t)t * d + c] : 0.f;
    for (int j = 0; j < k; ++j) {
      const size_t q = (size_t)t * k + j;
      const int sl = slot[q];
      const int e = ids[q];
      if (sl < 0 || e < e_begin || e >= e_end) continue;
      acc = fmaf(gates[q], y_perm[((size_t)offsets[e] + sl) * d + c], acc);
    }
    out[(size_t)t * d + c] = acc;
  }
}

__global__ void fill_i32_kernel(int32_t *p, int n, int32_t v0, int32_t step) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v0 + i * step;
}

}  // namespace

hipError_t launch_combine(const void *y_perm, const int32_t *ids, const float *gates, const int32_t *slot,
                          const int32_t *offsets, const void *shared, void *out, int T, int d, int k, bool bf16,
                          hipStream_t s, int e_begin, int e_end) {
  const int vec = bf16 ? 8 : 4;
  if (d % vec == 0) {
    const int grid = (T + CB_TOK - 1) / CB_TOK;
    if (bf16)
      hipLaunchKernelGGL(combine_kernel<true>, dim3(grid), dim3(256), 0, s, y_perm, ids, gates, slot, offsets, shared,
                         out, T, d, k, e_begin, e_end);
    else
      hipLaunchKernelGGL(combine_kernel<false>, dim3(grid), dim3(256), 0, s, y_perm, ids, gates, slot, offsets, shared,
                         out, T, d, k, e_begin, e_end);
  } else {
    if (bf16) return hipErrorInvalidValue;  // bf16 rows are validated to be multiples of 64
    hipLaunchKernelGGL(combine_f32_scalar_kernel, dim3(T), dim3(256), 0, s, static_cast<const float *>(y_perm), ids,
                       gates, slot, offsets, static_cast<const float *>(shared), static_cast<float *>(out), d, k,
                       e_begin, e_end);
  }
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int n, int32_t v0, int32_t step, hipStream_t s) {
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v0, step);
  return hipGetLastError();
}

}  // namespace moe
