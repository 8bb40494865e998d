// Grouped expert GEMM in float32 for float layers (vector ALU FMA; gfx950 has no
// fast fp32 matrix path that keeps full fp32 products and sums).  Same problem as
// the bf16 kernels: for each group, its rows of A times the group's weight rows,
// with the SwiGLU product fused into the epilogue when requested.  Any sizes.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int FT = 64;   // rows and output columns per tile
constexpr int FK = 16;   // K per LDS stage

template <bool SWIGLU>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(const float *__restrict__ A,
                                                               const int32_t *__restrict__ row_index,
                                                               const int32_t *__restrict__ offsets,
                                                               const float *__restrict__ W, int64_t wstride,
                                                               int n_out, int K, float *__restrict__ out,
                                                               int n_tiles) {
  __shared__ float sA[FK][FT + 1];
  __shared__ float sG[FK][FT + 1];
  __shared__ float sU[SWIGLU ? FK : 1][FT + 1];
  const int g = blockIdx.x / n_tiles, nt = blockIdx.x % n_tiles;
  const int row_begin = offsets[g], row_end = offsets[g + 1];
  if (row_begin >= row_end) return;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int n0 = nt * FT;
  const float *Wg = W + (size_t)g * wstride;

  for (int m0 = row_begin; m0 < row_end; m0 += FT) {
    const int rows = min(FT, row_end - m0);
    float ag[4][4] = {}, au[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += FK) {
      for (int idx = tid; idx < FT * FK; idx += 256) {
        const int r = idx / FK, kk = idx % FK;
        const bool kin = k0 + kk < K;
        const size_t arow = row_index ? (size_t)(r < rows ? row_index[m0 + r] : 0) : (size_t)(m0 + r);
        sA[kk][r] = (r < rows && kin) ? A[arow * K + k0 + kk] : 0.f;
        const int n = n0 + r;
        sG[kk][r] = (n < n_out && kin) ? Wg[(size_t)n * K + k0 + kk] : 0.f;
        if constexpr (SWIGLU) sU[kk][r] = (n < n_out && kin) ? Wg[(size_t)(n_out + n) * K + k0 + kk] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < FK; ++kk) {
        float a[4], w[4], u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] = sA[kk][ty * 4 + i];
          w[i] = sG[kk][tx * 4 + i];
          if constexpr (SWIGLU) u[i] = sU[kk][tx * 4 + i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            ag[i][j] = fmaf(a[i], w[j], ag[i][j]);
            if constexpr (SWIGLU) au[i][j] = fmaf(a[i], u[j], au[i][j]);
          }
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = ty * 4 + i;
      if (r >= rows) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + tx * 4 + j;
        if (n >= n_out) continue;
        float v = ag[i][j];
        if constexpr (SWIGLU) v = (v / (1.0f + expf(-v))) * au[i][j];
        out[(size_t)(m0 + r) * n_out + n] = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_grouped_gemm_f32(const GroupedGemmArgs &a, hipStream_t s) {
  const int n_tiles = (a.n_out + FT - 1) / FT;
  const int64_t grid = (int64_t)a.num_groups * n_tiles;
  if (a.swiglu)
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s,
                       static_cast<const float *>(a.A), a.row_index, a.offsets, static_cast<const float *>(a.W),
                       a.w_group_stride,
                       a.n_out, a.K, static_cast<float *>(a.out), n_tiles);
  else
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s,
                       static_cast<const float *>(a.A), a.row_index, a.offsets, static_cast<const float *>(a.W),
                       a.w_group_stride,
                       a.n_out, a.K, static_cast<float *>(a.out), n_tiles);
  return hipGetLastError();
}

}  // namespace moe
