// Gate-weighted combine back to token order ("Sparse Mixture-of-Experts",
// bigdataschool.ru wiki, section "Роутер и top-k gating": the layer output is the
// sum of the selected experts' outputs weighted by the renormalised router
// probabilities; section "Expert capacity и capacity factor": a dropped assignment
// adds nothing).  Each token gathers its kept rows -- no atomics, so the sum order
// (shared expert first, then j = 0..k-1) is fixed and the result deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int CB_KMAX = 64;  // assignments per token staged in LDS per pass

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void *__restrict__ y_perm, const int32_t *__restrict__ ids,
                                                      const float *__restrict__ gates,
                                                      const int32_t *__restrict__ slot,
                                                      const int32_t *__restrict__ offsets,
                                                      const void *__restrict__ shared, void *__restrict__ out, int d,
                                                      int k) {
  constexpr int VEC = BF16 ? 8 : 4;  // elements per 16-byte vector
  __shared__ int64_t s_row[CB_KMAX];
  __shared__ float s_gate[CB_KMAX];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int nvec = d / VEC;
  // chunks of up to CB_KMAX assignments; acc lives in registers across chunks
  constexpr int MAXV = 8;  // vectors per thread kept in registers: d <= 256*MAXV*VEC
  float acc[MAXV][VEC];
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    const int c = tid + 256 * v;
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[v][i] = 0.f;
    if (shared && c < nvec) {
      if constexpr (BF16) {
        const u32x4 q = ldg16(static_cast<const bf16_t *>(shared) + (size_t)t * d + c * VEC);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[v][2 * i] = __uint_as_float(q[i] << 16);
          acc[v][2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
        }
      } else {
        const u32x4 q = ldg16(static_cast<const float *>(shared) + (size_t)t * d + c * VEC);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[v][i] = __uint_as_float(q[i]);
      }
    }
  }
  for (int j0 = 0; j0 < k; j0 += CB_KMAX) {
    const int kn = min(CB_KMAX, k - j0);
    __syncthreads();
    if (tid < kn) {
      const size_t q = (size_t)t * k + j0 + tid;
      const int sl = slot[q];
      s_row[tid] = sl >= 0 ? (int64_t)offsets[ids[q]] + sl : -1;
      s_gate[tid] = gates[q];
    }
    __syncthreads();
    for (int j = 0; j < kn; ++j) {
      const int64_t row = s_row[j];
      if (row < 0) continue;
      const float gj = s_gate[j];
#pragma unroll
      for (int v = 0; v < MAXV; ++v) {
        const int c = tid + 256 * v;
        if (c >= nvec) continue;
        if constexpr (BF16) {
          const u32x4 q = ldg16(static_cast<const bf16_t *>(y_perm) + (size_t)row * d + c * VEC);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[v][2 * i] = fmaf(gj, __uint_as_float(q[i] << 16), acc[v][2 * i]);
            acc[v][2 * i + 1] = fmaf(gj, __uint_as_float(q[i] & 0xffff0000u), acc[v][2 * i + 1]);
          }
        } else {
          const u32x4 q = ldg16(static_cast<const float *>(y_perm) + (size_t)row * d + c * VEC);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[v][i] = fmaf(gj, __uint_as_float(q[i]), acc[v][i]);
        }
      }
    }
  }
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    const int c = tid + 256 * v;
    if (c >= nvec) continue;
    u32x4 q;
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = pack_bf16x2(acc[v][2 * i], acc[v][2 * i + 1]);
      stg16(static_cast<bf16_t *>(out) + (size_t)t * d + c * VEC, q);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = __float_as_uint(acc[v][i]);
      stg16(static_cast<float *>(out) + (size_t)t * d + c * VEC, q);
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
                                                                 float *__restrict__ out, int d, int k) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x; c < d; c += 256) {
    float acc = shared ? shared[(size_t)t * d + c] : 0.f;
    for (int j = 0; j < k; ++j) {
      const size_t q = (size_t)t * k + j;
      const int sl = slot[q];
      if (sl < 0) continue;
      acc = fmaf(gates[q], y_perm[((size_t)offsets[ids[q]] + sl) * d + c], acc);
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
                          hipStream_t s) {
  const int vec = bf16 ? 8 : 4;
  if (d % vec == 0 && d <= 256 * 8 * vec) {
    if (bf16)
      hipLaunchKernelGGL(combine_kernel<true>, dim3(T), dim3(256), 0, s, y_perm, ids, gates, slot, offsets, shared,
                         out, d, k);
    else
      hipLaunchKernelGGL(combine_kernel<false>, dim3(T), dim3(256), 0, s, y_perm, ids, gates, slot, offsets, shared,
                         out, d, k);
  } else {
    if (bf16) return hipErrorInvalidValue;  // bf16 rows are validated to be multiples of 64
    hipLaunchKernelGGL(combine_f32_scalar_kernel, dim3(T), dim3(256), 0, s, static_cast<const float *>(y_perm), ids,
                       gates, slot, offsets, static_cast<const float *>(shared), static_cast<float *>(out), d, k);
  }
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int n, int32_t v0, int32_t step, hipStream_t s) {
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v0, step);
  return hipGetLastError();
}

}  // namespace moe
