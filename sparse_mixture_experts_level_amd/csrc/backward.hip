// Backward pass of the sparse MoE layer on gfx950: the kernels besides the grouped
// GEMMs.  The training setting is the one of "Что такое Mixture of Experts (MoE) в
// трансформерах", aglamov.biz, section "Обучение MoE с помощью Transformers" (the
// expert projections run as grouped GEMMs in training too); the gradient itself is
// the chain rule through the forward with the routing held fixed:
//   per kept row r = (t, j) of expert e, with G = x W_g^T, U = x W_u^T, H = silu(G) U:
//     dH'_r = dy_t W_d[e]                 (unweighted; a grouped GEMM)
//     dg_tj = dH'_r . H_r                 (= dy_t . y_r)
//     dH = g_tj dH';  dG = dH U silu'(G);  dU = dH silu(G)
//     dx_t += [dG dU] W_gu[e]             (a grouped GEMM)
//     dW_d[e] += (g dy_t) (x) H_r,  dW_gu[e] += [dG dU] (x) x_t   (grouped over rows)
//   gates g = softmax over the selected logits:
//     dl_tj = g_tj (dg_tj - sum_j' g_tj' dg_tj'),   dW_r = dl^T x,   dx += dl W_r
// Every kernel here is deterministic: no atomics, fixed summation orders.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int TR = 64;  // transpose tile

// Plain: out[b][c][p] = in[b][p][c] for p < P and c < cols (bf16), zero for p >= rows,
// row stride out_ld.  Grouped (off / poff, G groups; batch 1): position p of group g
// (poff[g] <= p < poff[g+1]) holds row off[g] + (p - poff[g]) while that row belongs to the
// group (through row_index when given), zero in the group's padding, and the output is
// group-major -- group g's [cols, K_g] block (K_g = poff[g+1] - poff[g]) at element
// poff[g] * cols, row stride K_g -- so that each group's operand of the weight-gradient
// GEMM is one contiguous block; positions past poff[G] are not written.  64 x 64 tiles
// through LDS, 16-byte loads and stores; cols and P multiples of 8, group sizes multiples
// of 8.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16_t *__restrict__ in, int64_t in_stride_b,
                                                             int64_t rows, int cols,
                                                             const int32_t *__restrict__ row_index,
                                                             const int32_t *__restrict__ off,
                                                             const int32_t *__restrict__ poff, int G, int64_t P,
                                                             bf16_t *__restrict__ out, int64_t out_ld,
                                                             int64_t out_stride_b) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[TR][TR + 8];
  const int b = blockIdx.z;
  const int64_t p0 = (int64_t)blockIdx.x * TR;
  const int c0 = blockIdx.y * TR;
  const bf16_t *src = in + (size_t)b * in_stride_b;
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int v = tid + 256 * j;
    const int pl = v >> 3, cv = (v & 7) * 8;
    const int64_t p = p0 + pl;
    int64_t r = -1;
    if (p < P) {
      if (!off) {
        r = p < rows ? p : -1;
      } else if (p < poff[G]) {
        int lo = 0, hi = G;  // largest g with poff[g] <= p
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (poff[mid] <= p) lo = mid; else hi = mid;
        }
        const int64_t local = p - poff[lo];
        if (local < off[lo + 1] - off[lo]) r = off[lo] + local;
      }
    }
    u32x4 val = {0u, 0u, 0u, 0u};
    if (r >= 0 && c0 + cv < cols) {
      const int64_t sr = row_index ? (int64_t)row_index[r] : r;
      val = ldg16(src + (size_t)sr * cols + c0 + cv);
    }
    *reinterpret_cast<u32x4 *>(&tile[pl][cv]) = val;
  }
  __syncthreads();
  bf16_t *dst = out + (size_t)b * out_stride_b;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int v = tid + 256 * j;
    const int cl = v >> 3, pv = (v & 7) * 8;
    const int64_t p = p0 + pv;
    if (c0 + cl >= cols || p >= P) continue;
    int64_t o_idx;
    if (!off) {
      o_idx = (int64_t)(c0 + cl) * out_ld + p;
    } else {
      if (p >= poff[G]) continue;
      int lo = 0, hi = G;  // largest g with poff[g] <= p
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (poff[mid] <= p) lo = mid; else hi = mid;
      }
      const int64_t kg = poff[lo + 1] - poff[lo];
      o_idx = (int64_t)poff[lo] * cols + (int64_t)(c0 + cl) * kg + (p - poff[lo]);
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = uint32_t(tile[pv + 2 * q][cl]) | (uint32_t(tile[pv + 2 * q + 1][cl]) << 16);
    stg16(dst + o_idx, o);
  }
}

// poff[g] = sum over g' < g of the group's rows rounded up to 32 (the K chunk of the
// weight-gradient GEMM), poff[G] = total.  One block.
__global__ __launch_bounds__(256) void pad_offsets_kernel(const int32_t *__restrict__ off, int G,
                                                          int32_t *__restrict__ poff) {
  __shared__ int32_t s[MOE_MAX_EXPERTS_DEV + 1];
  for (int g = threadIdx.x; g < G; g += 256) s[g] = (off[g + 1] - off[g] + 31) / 32 * 32;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int g = 0; g < G; ++g) {
      const int v = s[g];
      poff[g] = run;
      run += v;
    }
    poff[G] = run;
  }
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *__restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

// Gradient of the renormalised gates with respect to the logits, one wavefront per token:
// dl[t][ids_j] = g_j (dg_j - sum_j' g_j' dg_j'), zero elsewhere; written as float [T, E]
// and as bf16 [T, Epad] (zero padded).  dg_j = dL/dg_j is the sum of the nb block dot
// products dH' . H of the assignment's row in dpart (0 when dropped), added lane-strided
// and then in a fixed butterfly: the same value in every lane.
__global__ __launch_bounds__(256) void gates_bwd_kernel(const int32_t *__restrict__ ids,
                                                        const float *__restrict__ gates,
                                                        const float *__restrict__ dpart, int nb,
                                                        const int32_t *__restrict__ serving,
                                                        const int32_t *__restrict__ slot,
                                                        const int32_t *__restrict__ offsets, int T, int E, int k,
                                                        int Epad, float *__restrict__ dl,
                                                        bf16_t *__restrict__ dl16) {
  constexpr int QMAX = (MOE_MAX_EXPERTS_DEV + 63) / 64;  // experts per lane
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  // each lane keeps g_j and dg_j of the selected experts among its own (lane + 64 q)
  float my_g[QMAX], my_dg[QMAX];
  bool my_sel[QMAX];
#pragma unroll
  for (int q = 0; q < QMAX; ++q) {
    my_g[q] = 0.0f;
    my_dg[q] = 0.0f;
    my_sel[q] = false;
  }
  float s = 0.0f;
  for (int j = 0; j < k; ++j) {
    const size_t tj = (size_t)t * k + j;
    const int sl = slot[tj];
    float dg = 0.0f;
    if (sl >= 0) {
      const float *p = dpart + ((size_t)offsets[serving[tj]] + sl) * nb;
      for (int b = lane; b < nb; b += 64) dg += p[b];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) dg += __shfl_xor(dg, o, 64);
    }
    const float g = gates[tj];
    s += g * dg;  // same order in every lane
    const int e = ids[tj];
    if ((e & 63) == lane) {
#pragma unroll
      for (int q = 0; q < QMAX; ++q)
        if (q == (e >> 6)) {
          my_g[q] = g;
          my_dg[q] = dg;
          my_sel[q] = true;
        }
    }
  }
#pragma unroll
  for (int q = 0; q < QMAX; ++q) {
    const int e = lane + 64 * q;
    if (e >= Epad) break;
    const float v = my_sel[q] ? my_g[q] * (my_dg[q] - s) : 0.0f;
    if (e < E) dl[(size_t)t * E + e] = v;
    dl16[(size_t)t * Epad + e] = f32_to_bf16(v);
  }
}

// g of every kept row: row offsets[e] + slot of assignment i (expert e = serving[i])
// takes gates[i]; each kept row has exactly one assignment.
__global__ __launch_bounds__(256) void row_gate_kernel(const int32_t *__restrict__ serving,
                                                       const int32_t *__restrict__ slot,
                                                       const int32_t *__restrict__ offsets,
                                                       const float *__restrict__ gates, int64_t n,
                                                       float *__restrict__ row_gate) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int sl = slot[i];
    if (sl >= 0) row_gate[offsets[serving[i]] + sl] = gates[i];
  }
}

// dx[t] = sum over kept j of dxr[row(t, j)] (+ extra[t]) (+ extra2[t]), float sums in
// a fixed order, one wavefront per token, 16-byte vectors.
__global__ __launch_bounds__(256) void dx_gather_kernel(const bf16_t *__restrict__ dxr,
                                                        const int32_t *__restrict__ serving,
                                                        const int32_t *__restrict__ slot,
                                                        const int32_t *__restrict__ offsets, int T, int d, int k,
                                                        const bf16_t *__restrict__ extra,
                                                        const bf16_t *__restrict__ extra2, bf16_t *__restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  for (int c = lane * 8; c < d; c += 64 * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto add = [&](const bf16_t *p) {
      const u32x4 v = ldg16(p);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_to_f32(bf16_t(v[q]));
        acc[2 * q + 1] += bf16_to_f32(bf16_t(v[q] >> 16));
      }
    };
    for (int j = 0; j < k; ++j) {
      const int sl = slot[(size_t)t * k + j];
      if (sl >= 0) add(dxr + ((size_t)offsets[serving[(size_t)t * k + j]] + sl) * d + c);
    }
    if (extra) add(extra + (size_t)t * d + c);
    if (extra2) add(extra2 + (size_t)t * d + c);
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    stg16(dx + (size_t)t * d + c, o);
  }
}

// The same sum for k <= KB with every load unconditional: the token's kept rows are
// resolved once, then each 16-byte column step issues all KB + 2 loads at once -- dropped
// assignments (j < k), j >= k and absent terms read zeros through range-checked buffer
// loads -- and adds them in the same order (zeros change nothing).
template <int KB>
__global__ __launch_bounds__(256) void dx_gather_wide_kernel(const bf16_t *__restrict__ dxr, int64_t rows,
                                                             const int32_t *__restrict__ serving,
                                                             const int32_t *__restrict__ slot,
                                                             const int32_t *__restrict__ offsets, int T, int d, int k,
                                                             const bf16_t *__restrict__ extra,
                                                             const bf16_t *__restrict__ extra2,
                                                             bf16_t *__restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint32_t dbytes = (uint32_t)d * 2u;
  const rsrc_t rres = make_rsrc(dxr, (uint32_t)(rows * dbytes));
  const rsrc_t eres = make_rsrc(extra, extra ? (uint32_t)T * dbytes : 0u);
  const rsrc_t e2res = make_rsrc(extra2, extra2 ? (uint32_t)T * dbytes : 0u);
  uint32_t roff[KB];
#pragma unroll
  for (int j = 0; j < KB; ++j) {
    roff[j] = kOob;
    if (j < k) {
      const int sl = slot[(size_t)t * k + j];
      if (sl >= 0) roff[j] = (uint32_t)(offsets[serving[(size_t)t * k + j]] + sl) * dbytes;
    }
  }
  const uint32_t toff = (uint32_t)t * dbytes;
  for (int c = lane * 8; c < d; c += 64 * 8) {
    u32x4 v[KB + 2];
#pragma unroll
    for (int j = 0; j < KB; ++j) v[j] = buf_ld16(rres, roff[j] + (uint32_t)c * 2u);
    v[KB] = buf_ld16(eres, toff + (uint32_t)c * 2u);
    v[KB + 1] = buf_ld16(e2res, toff + (uint32_t)c * 2u);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KB + 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_to_f32(bf16_t(v[j][q]));
        acc[2 * q + 1] += bf16_to_f32(bf16_t(v[j][q] >> 16));
      }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    stg16(dx + (size_t)t * d + c, o);
  }
}

// The weight-gradient product straight from row-major activations, for short row
// ranges (write bound): for group g with rows off[g] .. off[g+1] - 1,
//   out[g][m][n] = sum over those rows r of A[r][m] * B[r][n]   (bf16 out),
// A [a_rows, M] and B [b_rows, N] row-major -- the contraction runs over rows, so both
// operands are K-major and need no transpose.  128 x 128 output tile per workgroup, 4
// waves of 64 x 64 (2 x 2 blocks of the 32x32x16 MFMA).  Each 32-row chunk of both
// operand tiles moves into LDS as 256-byte rows (direct-to-LDS loads, 16-byte chunk c of
// row r stored at c ^ 4 (r mod 4)), and the MFMA fragments come from LDS transpose reads
// (two per fragment, as in the large-tile kernel's K-major mode).  Two chunks in flight;
// rows past the group read zeros; the tile is staged through LDS and written as 16-byte
// runs.  M and N multiples of 8; an empty group writes zeros.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void wgrad_kn_kernel(const bf16_t *__restrict__ A, int64_t a_rows,
                                                       const bf16_t *__restrict__ B, int64_t b_rows,
                                                       const int32_t *__restrict__ off, int M, int N, int m_tiles,
                                                       int n_tiles, bf16_t *__restrict__ out) {
  constexpr int CH = 32 * 256;  // bytes of one operand's 32-row chunk
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[CH], sA1[CH], sB0[CH], sB1[CH];
  const int per_g = m_tiles * n_tiles;
  const int tile = blockIdx.x;
  const int g = tile / per_g;
  const int rem = tile - g * per_g;
  const int mt = rem / n_tiles, nt = rem - mt * n_tiles;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, lh = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int kb = off[g], kg = off[g + 1] - kb;
  const int nk = (kg + 31) / 32;
  const rsrc_t ares = make_rsrc(A, (uint32_t)min<int64_t>(a_rows * M * 2, 0x7fffffffLL));
  const rsrc_t bres = make_rsrc(B, (uint32_t)min<int64_t>(b_rows * N * 2, 0x7fffffffLL));
  // load instruction q = 2 wave + p brings rows 4 q .. 4 q + 3 of a chunk; lane i: row
  // 4 q + i / 16, stored slot i % 16 holding logical chunk (i % 16) ^ 4 (row % 4)
  int krow[2];
  uint32_t ao[2], bo[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int kr = 4 * (2 * wave + p) + (lane >> 4);
    const int cs = ((lane & 15) ^ (4 * (kr & 3))) << 3;
    krow[p] = kr;
    const int m = mt * 128 + cs, n = nt * 128 + cs;
    ao[p] = m < M ? ((uint32_t)(kb + kr) * (uint32_t)M + (uint32_t)m) * 2u : kOob;
    bo[p] = n < N ? ((uint32_t)(kb + kr) * (uint32_t)N + (uint32_t)n) * 2u : kOob;
  }
  auto issue = [&](int c, uint8_t *la, uint8_t *lb) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const bool ok = c < nk && c * 32 + krow[p] < kg;  // rows past the group: zeros
      const uint32_t ra = (uint32_t)c * 32u * (uint32_t)M * 2u, rb = (uint32_t)c * 32u * (uint32_t)N * 2u;
      buf_ld16_lds(ares, ok && ao[p] != kOob ? ao[p] + ra : kOob, la + (2 * wave + p) * 1024);
      buf_ld16_lds(bres, ok && bo[p] != kOob ? bo[p] + rb : kOob, lb + (2 * wave + p) * 1024);
    }
  };
  // 32x32x16 fragment of the 32 columns nb .. nb + 31 (k = 16 kk + 8 (lane >> 5) .. + 7
  // for column nb + (lane & 31)) from a [32 rows][128 columns] chunk: in a 16-lane group
  // lane 4a + c receives element c of the 8-byte chunks addressed by lanes a, a + 4, a + 8,
  // a + 12, so lane s of group G addresses row k0 + s / 4, columns nb + 16 (G & 1) +
  // 4 (s % 4) .. + 3, with k0 = 16 kk + 8 (G >> 1) (+ 4 for the second read).
  auto frag = [&](const uint8_t *t, int kk, int nb) -> u32x4 {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int G = lane >> 4, sl = lane & 15;
    const int col = nb + (G & 1) * 16 + 4 * (sl & 3);
    u32x4 o;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = kk * 16 + (G >> 1) * 8 + 4 * h + (sl >> 2);
      const uint8_t *q = t + r * 256 + (((col >> 3) ^ (4 * (r & 3))) << 4) + (col & 7) * 2;
      const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)q);
      o[2 * h] = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
      o[2 * h + 1] = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
    }
    return o;
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  auto compute = [&](const uint8_t *la, const uint8_t *lb) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = frag(la, kk, wm * 64 + i * 32);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = frag(lb, kk, wn * 64 + j * 32);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(fb[j], fa[i], acc[i][j]);
    }
  };
  // two stages: chunk c in stage c % 2; this wave's loads of chunk c are complete once
  // at most the next chunk's four loads remain, then one barrier makes every wave's
  // pieces visible; a second barrier keeps the stage until all waves have read it
  if (nk > 0) issue(0, sA0, sB0);
  for (int c0 = 0; c0 < nk; c0 += 2) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int c = c0 + st;
      if (c >= nk) break;
      uint8_t *la = st ? sA1 : sA0, *lb = st ? sB1 : sB0;
      uint8_t *na = st ? sA0 : sA1, *nb = st ? sB0 : sB1;
      if (c + 1 < nk) {
        issue(c + 1, na, nb);
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __builtin_amdgcn_s_barrier();
      compute(la, lb);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // epilogue: acc[i][j] element r holds row mt * 128 + wm * 64 + i * 32 + (lane & 31),
  // column nt * 128 + wn * 64 + j * 32 + 8 (r / 4) + 4 (lane / 32) + r % 4; each wave
  // stages its 64 x 64 (8 KB) in one of the four chunk buffers, 128-byte rows, chunk c
  // of row r at c ^ ((r >> 1) & 7)
  uint8_t *stage = wave == 0 ? sA0 : wave == 1 ? sA1 : wave == 2 ? sB0 : sB1;
  const int m0 = mt * 128 + wm * 64, n0 = nt * 128 + wn * 64;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = i * 32 + lr;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint2 v;
        v.x = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
        v.y = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        *reinterpret_cast<uint2 *>(stage + row * 128 + (((j * 4 + q) ^ ((row >> 1) & 7)) << 4) + lh * 8) = v;
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const size_t obase = (size_t)g * M * N;
  const int c = lane & 7, n = n0 + c * 8;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int row = it * 8 + (lane >> 3), m = m0 + row;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + row * 128 + ((c ^ ((row >> 1) & 7)) << 4));
    if (m < M && n < N) stg16(out + obase + (size_t)m * N + n, v);
  }
}

// out[i] = sum over s < S of part[s * n + i], in order (float, n a multiple of 4).
__global__ __launch_bounds__(256) void ksplit_sum_kernel(const float *__restrict__ part, int S, int64_t n,
                                                         float *__restrict__ out) {
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += (int64_t)gridDim.x * 1024) {
    f32x4 acc = *reinterpret_cast<const f32x4 *>(part + i);
    for (int s = 1; s < S; ++s) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(part + (int64_t)s * n + i);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += v[q];
    }
    *reinterpret_cast<f32x4 *>(out + i) = acc;
  }
}

}  // namespace

hipError_t launch_ksplit_sum(const float *part, int S, int64_t n, float *out, hipStream_t s) {
  if (n % 4) return hipErrorInvalidValue;
  const int64_t blocks = std::min<int64_t>((n / 4 + 255) / 256, 2048);
  hipLaunchKernelGGL(ksplit_sum_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, s, part, S, n, out);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const void *in, int64_t in_stride_b, int64_t rows, int cols, int batch,
                                 const int32_t *row_index, const int32_t *off, const int32_t *poff, int G, int64_t P,
                                 void *out, int64_t out_ld, int64_t out_stride_b, hipStream_t s) {
  if (P <= 0 || cols <= 0 || batch <= 0) return hipSuccess;
  dim3 grid((unsigned)((P + TR - 1) / TR), (unsigned)((cols + TR - 1) / TR), (unsigned)batch);
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, s, static_cast<const bf16_t *>(in), in_stride_b, rows,
                     cols, row_index, off, poff, G, P, static_cast<bf16_t *>(out), out_ld, out_stride_b);
  return hipGetLastError();
}

hipError_t launch_pad_offsets(const int32_t *off, int G, int32_t *poff, hipStream_t s) {
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(256), 0, s, off, G, poff);
  return hipGetLastError();
}

hipError_t launch_fill_u32(void *p, int64_t n_words, uint32_t v, hipStream_t s) {
  if (n_words <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n_words + 255) / 256, 8192);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint32_t *>(p), n_words, v);
  return hipGetLastError();
}

hipError_t launch_gates_bwd(const int32_t *ids, const float *gates, const float *dpart, int nb, const int32_t *serving,
                            const int32_t *slot, const int32_t *offsets, int T, int E, int k, int Epad, float *dl,
                            void *dl16, hipStream_t s) {
  if (Epad > MOE_MAX_EXPERTS_DEV + 63) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gates_bwd_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, ids, gates, dpart, nb, serving,
                     slot, offsets, T, E, k, Epad, dl, static_cast<bf16_t *>(dl16));
  return hipGetLastError();
}

hipError_t launch_row_gate(const int32_t *serving, const int32_t *slot, const int32_t *offsets, const float *gates,
                           int64_t n, float *row_gate, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(row_gate_kernel, dim3((unsigned)blocks), dim3(256), 0, s, serving, slot, offsets, gates, n,
                     row_gate);
  return hipGetLastError();
}

hipError_t launch_dx_gather(const void *dxr, int64_t rows, const int32_t *serving, const int32_t *slot,
                            const int32_t *offsets, int T, int d, int k, const void *extra, const void *extra2, void *dx,
                            hipStream_t s) {
  const bool wide = k <= 8 && (rows + 1) * d * 2 < ((int64_t)1 << 31) && ((int64_t)T + 1) * d * 2 < ((int64_t)1 << 31);
  if (wide) {
    const bf16_t *r = static_cast<const bf16_t *>(dxr), *e = static_cast<const bf16_t *>(extra),
                 *e2 = static_cast<const bf16_t *>(extra2);
    bf16_t *o = static_cast<bf16_t *>(dx);
    const dim3 grid((unsigned)((T + 3) / 4));
    if (k <= 1)
      hipLaunchKernelGGL(dx_gather_wide_kernel<1>, grid, dim3(256), 0, s, r, rows, serving, slot, offsets, T, d, k, e, e2, o);
    else if (k <= 2)
      hipLaunchKernelGGL(dx_gather_wide_kernel<2>, grid, dim3(256), 0, s, r, rows, serving, slot, offsets, T, d, k, e, e2, o);
    else if (k <= 4)
      hipLaunchKernelGGL(dx_gather_wide_kernel<4>, grid, dim3(256), 0, s, r, rows, serving, slot, offsets, T, d, k, e, e2, o);
    else
      hipLaunchKernelGGL(dx_gather_wide_kernel<8>, grid, dim3(256), 0, s, r, rows, serving, slot, offsets, T, d, k, e, e2, o);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(dx_gather_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s,
                     static_cast<const bf16_t *>(dxr), serving, slot, offsets, T, d, k,
                     static_cast<const bf16_t *>(extra), static_cast<const bf16_t *>(extra2), static_cast<bf16_t *>(dx));
  return hipGetLastError();
}

hipError_t launch_wgrad_kn(const void *A, int64_t a_rows, const void *B, int64_t b_rows, const int32_t *off, int G,
                           int M, int N, void *out, hipStream_t s) {
  if (N % 8 || M % 8) return hipErrorInvalidValue;  // whole 16-byte chunks of columns
  if (a_rows * M * 2 >= ((int64_t)1 << 31) || b_rows * N * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int m_tiles = (M + 127) / 128, n_tiles = (N + 127) / 128;
  const int64_t grid = (int64_t)G * m_tiles * n_tiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wgrad_kn_kernel, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const bf16_t *>(A), a_rows,
                     static_cast<const bf16_t *>(B), b_rows, off, M, N, m_tiles, n_tiles, static_cast<bf16_t *>(out));
  return hipGetLastError();
}

}  // namespace moe
