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

constexpr int CB_TOK = 4;  // wavefronts per workgroup

// One wavefront per (token, column segment of 64 * U 16-byte vectors).  Lanes j < k
// fetch assignment j's slot, expert and gate in parallel and resolve its row; the wave
// then loads JU rows' vectors at a time (more loads in flight) and each lane sums its
// columns over j in order, so the result does not depend on the segmentation.  Every
// byte is read or written once, so loads and stores are marked non-temporal (DeepSeek-shaped
// layer: 147 -> 130 us).
template <bool BF16, int U, int JU>
__global__ __launch_bounds__(256) void combine_kernel(const void *__restrict__ y_perm, const int32_t *__restrict__ ids,
                                                      const float *__restrict__ gates,
                                                      const int32_t *__restrict__ slot,
                                                      const int32_t *__restrict__ offsets,
                                                      const void *__restrict__ shared, void *__restrict__ out, int T,
                                                      int d, int k, int e_begin, int e_end, int nseg) {
  constexpr int VEC = BF16 ? 8 : 4;  // elements per 16-byte vector
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * CB_TOK + (threadIdx.x >> 6);
  const int t = (int)(gw / nseg);
  if (t >= T) return;
  const int v0 = (int)(gw - (int64_t)t * nseg) * 64 * U;
  const int nvec = d / VEC;
  const size_t es = BF16 ? 2 : 4;
  const uint8_t *yb = static_cast<const uint8_t *>(y_perm);
  auto unpack = [&](const u32x4 &q, float *o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (BF16) {
        o[2 * i] = __uint_as_float(q[i] << 16);
        o[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
      } else {
        o[i] = __uint_as_float(q[i]);
      }
    }
  };
  // Lane j < k: assignment j's slot, expert and gate (the first 64), loaded before the
  // shared expert's row so that the two are in flight together: the wave's chain of
  // dependent loads is then slots and shared row, the experts' first rows, the rows
  // (DeepSeek-shaped layer: 94 -> 88 us).  Staging all first rows in LDS per workgroup
  // instead, to drop the middle link, measured 90-92 us (a barrier per workgroup).
  auto fetch = [&](int j0, int &sl, int &e, float &gt) {
    sl = -1;
    e = 0;
    gt = 0.f;
    if (j0 + lane < k) {
      const size_t q = (size_t)t * k + j0 + lane;
      sl = slot[q];
      e = ids[q];
      gt = gates[q];
    }
  };
  int f_sl, f_e;
  float f_g;
  fetch(0, f_sl, f_e, f_g);
  u32x4 shq[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = v0 + lane + 64 * u;
    shq[u] = (shared && c < nvec) ? ldg16_nt(static_cast<const uint8_t *>(shared) + ((size_t)t * d + (size_t)c * VEC) * es)
                                  : u32x4{0u, 0u, 0u, 0u};
  }
  float acc[U][VEC];
#pragma unroll
  for (int u = 0; u < U; ++u) unpack(shq[u], acc[u]);
  for (int j0 = 0; j0 < k; j0 += 64) {
    // lane j holds assignment j0 + j: its row (or -1) and gate
    if (j0 > 0) fetch(j0, f_sl, f_e, f_g);
    int64_t my_row = -1;
    const float my_gate = f_g;
    if (f_sl >= 0 && f_e >= e_begin && f_e < e_end) my_row = (int64_t)offsets[f_e] + f_sl;
    const int kn = min(64, k - j0);
    for (int j1 = 0; j1 < kn; j1 += JU) {
      u32x4 q[JU][U];
      float gj[JU];
      bool live[JU];
#pragma unroll
      for (int jj = 0; jj < JU; ++jj) {
        const int j = j1 + jj;
        const int64_t row = __shfl(my_row, j < kn ? j : 0, 64);
        gj[jj] = __shfl(my_gate, j < kn ? j : 0, 64);
        live[jj] = j < kn && row >= 0;
        const uint8_t *yr = yb + (size_t)(live[jj] ? row : 0) * d * es;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = v0 + lane + 64 * u;
          q[jj][u] = (live[jj] && c < nvec) ? ldg16_nt(yr + (size_t)c * VEC * es) : u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int jj = 0; jj < JU; ++jj) {
        if (!live[jj]) continue;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float v[VEC];
          unpack(q[jj][u], v);
#pragma unroll
          for (int i = 0; i < VEC; ++i) acc[u][i] = fmaf(gj[jj], v[i], acc[u][i]);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
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
    stg16_nt(static_cast<uint8_t *>(out) + ((size_t)t * d + (size_t)c * VEC) * es, q);
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
    // Two vectors per lane when there are tokens enough to fill the GPU, else one vector
    // per lane and more wavefronts per token; rows fetched two at a time when a token has
    // several.  Each wavefront waits through a chain of dependent loads (slot and expert
    // with the shared row, then the expert's offset, then the rows), so the kernel lives on
    // many resident wavefronts: four vectors per lane and four rows at a time (more
    // registers, fewer wavefronts) took 131 us against 95 us on the DeepSeek-shaped layer.
    const int nvec = d / vec;
    const bool wide = (int64_t)T * ((nvec + 127) / 128) >= 4096;
    const int U = wide && nvec >= 128 ? 2 : 1;
    const int nseg = (nvec + 64 * U - 1) / (64 * U);
    const int64_t grid = ((int64_t)T * nseg + CB_TOK - 1) / CB_TOK;
#define CB_LAUNCH(B, UU, J)                                                                                        \
  hipLaunchKernelGGL((combine_kernel<B, UU, J>), dim3((unsigned)grid), dim3(256), 0, s, y_perm, ids, gates, slot,     \
                     offsets, shared, out, T, d, k, e_begin, e_end, nseg)
#define CB_U(B, J)                      \
  do {                                  \
    if (U == 2) CB_LAUNCH(B, 2, J);     \
    else CB_LAUNCH(B, 1, J);            \
  } while (0)
    if (bf16) {
      if (k == 1) CB_U(true, 1); else CB_U(true, 2);
    } else {
      if (k == 1) CB_U(false, 1); else CB_U(false, 2);
    }
#undef CB_U
#undef CB_LAUNCH
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
