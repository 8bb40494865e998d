// Router of the sparse MoE layer on gfx950: bias-free linear (logits), then softmax,
// top-k and renormalised gates ("Sparse Mixture-of-Experts", bigdataschool.ru wiki,
// section "Роутер и top-k gating").
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// ------------------------------------------------------------------ logits, bf16
//
// logits[T, E] = x[T, d] . W_r[E, d]^T (+ offset), bf16 MFMA with float accumulate.
// A workgroup owns 64 tokens (16 per wave) and every expert, in chunks of up to 256
// experts.  The router weight chunk for 64 values of d is staged in LDS (double
// buffered) and shared by the four waves; each wave streams its own 16 token rows
// straight from HBM into MFMA operand registers.  Loads run four chunks ahead
// through range-checked buffer loads (rows past T or E read as zeros).
namespace {

constexpr int RT_TOK = 64;   // tokens per workgroup
constexpr int RT_KC = 64;    // d values per LDS stage (8 x 16-byte chunks per row)
constexpr int RT_EMAX = 256; // experts per pass

// Split over d (few tokens, long rows): workgroup (blockIdx.x, blockIdx.y) covers the
// chunks [y * cps, (y + 1) * cps) of d and writes its partial sums (without the offset)
// to partials[y][T][E]; the top-k kernel adds the splits in order.
template <int NSUB>  // 16-expert subtiles per pass
__global__ __launch_bounds__(256) void router_logits_bf16_kernel(const bf16_t *__restrict__ x,
                                                                 const bf16_t *__restrict__ w,
                                                                 const float *__restrict__ offset,
                                                                 float *__restrict__ logits, int T, int d, int E,
                                                                 int e_base, int cps, float *__restrict__ partials) {
  constexpr int EC = NSUB * 16;
  constexpr int P = 4;  // chunks in flight
  constexpr int PER_T = (EC * 8 + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][EC * RT_KC * 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tb = blockIdx.x * RT_TOK;
  const int t0 = tb + wave * 16;
  const uint32_t dbytes = (uint32_t)d * 2u;
  // token rows past T and expert rows past E read as zeros (range-checked buffer loads)
  const rsrc_t xres = make_rsrc(x + (size_t)tb * d, (uint32_t)min(RT_TOK, T - tb) * dbytes);
  const rsrc_t wres = make_rsrc(w + (size_t)e_base * d, (uint32_t)min(EC, E - e_base) * dbytes);
  const uint32_t xoff = (uint32_t)(wave * 16 + (lane & 15)) * dbytes + (uint32_t)(lane >> 4) * 16u;
  uint32_t woff[PER_T];
#pragma unroll
  for (int r = 0; r < PER_T; ++r) {
    const int q = tid + 256 * r;
    woff[r] = q < EC * 8 ? (uint32_t)(q >> 3) * dbytes + (uint32_t)(q & 7) * 16u : kOob;
  }
  struct Slot {
    u32x4 a[2];
    u32x4 w[PER_T];
  };
  Slot slot[P];
  const int kb = partials ? blockIdx.y * cps : 0;
  const int nk = partials ? min(cps, d / RT_KC - kb) : d / RT_KC;  // chunks of this workgroup
  auto issue = [&](Slot &sl, int it) {
    const bool ok = it < nk;
    const uint32_t kc = (uint32_t)(kb + it) * (RT_KC * 2);
    sl.a[0] = buf_ld16(xres, ok ? xoff + kc : kOob);
    sl.a[1] = buf_ld16(xres, ok ? xoff + 64u + kc : kOob);
#pragma unroll
    for (int r = 0; r < PER_T; ++r) sl.w[r] = buf_ld16(wres, ok ? woff[r] + kc : kOob);
  };
  auto stage = [&](const Slot &sl, int buf) {
#pragma unroll
    for (int r = 0; r < PER_T; ++r) {
      const int q = tid + 256 * r;
      if ((EC * 8) % 256 == 0 || q < EC * 8) {
        const int row = q >> 3, c = q & 7;
        *reinterpret_cast<u32x4 *>(&lds[buf][(row * 8 + (c ^ (row & 7))) * 16]) = sl.w[r];
      }
    }
  };

  f32x4 acc[NSUB];
#pragma unroll
  for (int n = 0; n < NSUB; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < P - 1; ++s) issue(slot[s], s);
  stage(slot[0], 0);
  __syncthreads();
  // one chunk: issue chunk it + P - 1 into the slot chunk it - 1 used, multiply chunk it,
  // stage chunk it + 1's router weights in the other LDS buffer
  auto step = [&](int it, int s) {
    issue(slot[(s + P - 1) % P], it + P - 1);
    const int buf = it & 1;
#pragma unroll
    for (int n = 0; n < NSUB; ++n) {
      const int row = n * 16 + (lane & 15);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c = ks * 4 + (lane >> 4);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(&lds[buf][(row * 8 + (c ^ (row & 7))) * 16]);
        acc[n] = mfma16(slot[s].a[ks], b, acc[n]);
      }
    }
    if (it + 1 < nk) stage(slot[(s + 1) % P], (it + 1) & 1);
    __syncthreads();
  };
  // Main loop, P chunks per trip with no exit inside a trip, so the loads in flight stay in
  // flight across its back edge (with an exit the compiler drained them at every trip).
  int c0 = 0;
  for (; c0 + P <= nk; c0 += P) {
#pragma unroll
    for (int s = 0; s < P; ++s) step(c0 + s, s);
  }
#pragma unroll
  for (int s = 0; s < P - 1; ++s)
    if (c0 + s < nk) step(c0 + s, s);

  // C layout of the 16x16 MFMA: lane holds column (lane & 15), rows 4*(lane>>4) + i.
#pragma unroll
  for (int n = 0; n < NSUB; ++n) {
    const int e = e_base + n * 16 + (lane & 15);
    if (e >= E) continue;
    const float off = offset && !partials ? offset[e] : 0.f;
    float *dst = partials ? partials + (size_t)blockIdx.y * T * E : logits;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + (lane >> 4) * 4 + i;
      if (t < T) dst[(size_t)t * E + e] = acc[n][i] + off;
    }
  }
}

__global__ __launch_bounds__(256) void router_logits_f32_kernel(const float *__restrict__ x,
                                                                const float *__restrict__ w,
                                                                const float *__restrict__ offset,
                                                                float *__restrict__ logits, int T, int d, int E) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * E) return;
  const int t = int(i / E), e = int(i % E);
  const float *xr = x + (size_t)t * d;
  const float *wr = w + (size_t)e * d;
  float s = 0.f;
  for (int j = 0; j < d; ++j) s = fmaf(xr[j], wr[j], s);
  logits[i] = s + (offset ? offset[e] : 0.f);
}

// ------------------------------------------------------------------ top-k
//
// One wavefront per token.  Each lane holds VPL logits (expert = lane + 64 * v).
// A key orders (logit desc, expert asc): the logit's bits mapped to an unsigned
// order (with -0.0 folded onto +0.0) in the high word, (0xffff - expert) in the low
// word; k rounds of a wavefront max-reduction pick the experts in descending order.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (uint64_t(ord) << 32) | uint32_t(0xffff - e);
}

__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t ord = uint32_t(key >> 32);
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
  return __uint_as_float(u);
}

// One step of the wavefront maximum: each lane takes the larger of its value and the value
// of the lane that DPP control CTRL names (rows outside ROW_MASK keep theirs).  DPP moves
// run in the vector ALU, without the LDS round trip of a lane shuffle.  The moved value
// of a row outside ROW_MASK is 0, the identity of the unsigned maximum, which lets the
// compiler fold the move into the maximum (one v_max_u32 with a DPP source per step instead
// of two copies and a maximum).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, false);
  return o > v ? o : v;
}

// Maximum of a value over the 64 lanes (every lane active), returned to every lane: within
// each quad (lane ^ 1, lane ^ 2), across the quads of each 8-lane half row (half-row
// mirror), across the halves of each 16-lane row (row mirror), then row 0 into row 1 and
// row 2 into row 3 (broadcast of lane 15) and rows 0-1 into rows 2-3 (broadcast of lane
// 31); lane 63 then holds the maximum of all lanes.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step<0xb1>(v);       // quad_perm [1, 0, 3, 2]
  v = dpp_max_step<0x4e>(v);       // quad_perm [2, 3, 0, 1]
  v = dpp_max_step<0x141>(v);      // row_half_mirror
  v = dpp_max_step<0x140>(v);      // row_mirror
  v = dpp_max_step<0x142, 0xa>(v); // row_bcast:15 into rows 1 and 3
  v = dpp_max_step<0x143, 0xc>(v); // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

constexpr int TK_WAVES = 4;

// Selection for token t from the keys of its logits (lane holds experts lane + 64 v).
// Each lane first sorts its VPL keys (descending), so its first key is its candidate.  A
// round takes the largest candidate of the wavefront: the maximum of the candidates' high
// words (the logit order) over the lanes; when several lanes hold that maximum (equal
// logits), the maximum of their low words (the smallest expert) decides.  That is the
// maximum of the whole 64-bit keys, found with 32-bit lane reductions.  The winning lane
// then drops its candidate (its next key moves up; 0 ranks below every real key).
// Every lane follows the k rounds identically (same winner, same running sum of
// exp(l_j - l_max) in the same order); lane (j mod 64) keeps winner j in register
// slot j / 64 and writes it at the end.  No LDS and no barriers.  With `spare`, the
// selection goes on for k more rounds (the experts ranked k .. 2k-1, used to redirect
// overflowing assignments) without gates.
template <int VPL>
__device__ __forceinline__ void topk_select(uint64_t (&key)[VPL], int E, int k, int64_t t, int lane,
                                            int32_t *__restrict__ ids, float *__restrict__ gates,
                                            int32_t *__restrict__ spare) {
  // odd-even transposition sort of the lane's keys, descending
#pragma unroll
  for (int p = 0; p < VPL; ++p)
#pragma unroll
    for (int i = p & 1; i + 1 < VPL; i += 2) {
      const uint64_t hi = key[i] > key[i + 1] ? key[i] : key[i + 1];
      const uint64_t lo = key[i] > key[i + 1] ? key[i + 1] : key[i];
      key[i] = hi;
      key[i + 1] = lo;
    }
  int my_id[VPL], my_sp[VPL];
  float my_z[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    my_id[v] = 0;
    my_sp[v] = -1;
    my_z[v] = 0.f;
  }
  float m = 0.f, sum = 0.f;
  const int rounds = spare ? min(2 * k, E) : k;
  for (int j = 0; j < rounds; ++j) {
    const uint32_t hv = uint32_t(key[0] >> 32), lv = uint32_t(key[0]);
    const uint32_t hmax = wave_max_u32(hv);
    const uint64_t tie = __ballot(hv == hmax);
    uint32_t lmax;
    if (__popcll(tie) == 1) {
      lmax = (uint32_t)__builtin_amdgcn_readlane((int)lv, __ffsll((unsigned long long)tie) - 1);
    } else {
      lmax = wave_max_u32(hv == hmax ? lv : 0u);
    }
    const uint64_t best = (uint64_t(hmax) << 32) | lmax;
    const int e = 0xffff - int(lmax & 0xffffu);
    // the winning lane drops its candidate (keys are distinct: exactly one lane matches)
    const bool win = key[0] == best;
#pragma unroll
    for (int v = 0; v + 1 < VPL; ++v) key[v] = win ? key[v + 1] : key[v];
    key[VPL - 1] = win ? 0ull : key[VPL - 1];
    if (j < k) {
      const float val = key_value(best);
      if (j == 0) m = val;
      const float z = expf(val - m);
      sum += z;
      if ((j & 63) == lane) {
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          if (v == (j >> 6)) {
            my_id[v] = e;
            my_z[v] = z;
          }
      }
    } else {
      const int i = j - k;
      if ((i & 63) == lane) {
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          if (v == (i >> 6)) my_sp[v] = e;
      }
    }
  }
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int j = v * 64 + lane;
    if (j < k) {
      if (ids) ids[t * k + j] = my_id[v];
      if (gates) gates[t * k + j] = my_z[v] / sum;
      if (spare) spare[t * k + j] = my_sp[v];
    }
  }
}

// One wavefront per token: the token's logits (with `partials`, S <= SMAX splits of the
// router linear, first formed as the splits' sum in order s = 0..S-1 plus the offset, and
// written to `logits`), then topk_select.  Every load of a group of up to four splits is
// issued before the first is used (addresses clamped into the arrays, values past E or S
// discarded), so a wave waits for memory once per group rather than once per load.
template <int VPL, int SMAX>  // SMAX = 0: read the logits
__global__ __launch_bounds__(256) void router_topk_kernel(float *__restrict__ logits, int T, int E, int k,
                                                          int32_t *__restrict__ ids, float *__restrict__ gates,
                                                          int32_t *__restrict__ spare,
                                                          const float *__restrict__ partials, int S,
                                                          const float *__restrict__ offset) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * TK_WAVES + wave;
  if (t >= T) return;
  float *row = logits + (size_t)t * E;
  int ec[VPL];  // this lane's experts, clamped into [0, E)
#pragma unroll
  for (int v = 0; v < VPL; ++v) ec[v] = min(lane + 64 * v, E - 1);
  float val[VPL];
  if constexpr (SMAX == 0) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) val[v] = row[ec[v]];
  } else {
    constexpr int G = SMAX < 4 ? SMAX : 4;  // splits loaded together
    float off[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      val[v] = 0.f;
      off[v] = offset ? offset[ec[v]] : 0.f;
    }
#pragma unroll
    for (int s0 = 0; s0 < SMAX; s0 += G) {
      float part[G][VPL];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const size_t sp = (size_t)min(s0 + g, S - 1);
#pragma unroll
        for (int v = 0; v < VPL; ++v) part[g][v] = partials[(sp * T + t) * E + ec[v]];
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int v = 0; v < VPL; ++v)
          if (s0 + g < S) val[v] += part[g][v];
    }
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      if (offset) val[v] += off[v];
      if (lane + 64 * v < E) row[lane + 64 * v] = val[v];
    }
  }
  uint64_t key[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) key[v] = lane + 64 * v < E ? topk_key(val[v], lane + 64 * v) : 0ull;  // 0 ranks below every real key
  topk_select<VPL>(key, E, k, t, lane, ids, gates, spare);
}

// ------------------------------------------------------------------ fused, few experts
//
// Router linear and top-k in one kernel for E <= 16 and many tokens: a workgroup owns
// 16 tokens and all experts; its four waves split d (wave w: the w-th quarter of the
// 64-wide chunks), each streaming its 16 token rows and the expert rows of its quarter
// straight from memory into MFMA operand registers, chunks P ahead.  The four partial
// [16 x E] accumulators meet in LDS and are added in wave order (plus the offset);
// each wave then writes the logits of four tokens and selects their experts.
template <int NSUB>  // 16-expert subtiles
__global__ __launch_bounds__(256) void router_fused_kernel(const bf16_t *__restrict__ x, const bf16_t *__restrict__ w,
                                                           const float *__restrict__ offset,
                                                           float *__restrict__ logits, int T, int d, int E, int k,
                                                           int32_t *__restrict__ ids, float *__restrict__ gates,
                                                           int32_t *__restrict__ spare) {
  constexpr int P = 4;  // chunks in flight
  constexpr int EC = NSUB * 16;
  __shared__ float red[4][16][EC + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * 16;
  const uint32_t dbytes = (uint32_t)d * 2u;
  // token rows past T and expert rows past E read as zeros (range-checked buffer loads)
  const rsrc_t xres = make_rsrc(x + (size_t)t0 * d, (uint32_t)min(16, T - t0) * dbytes);
  const rsrc_t wres = make_rsrc(w, (uint32_t)E * dbytes);
  const int nc = d / RT_KC;
  const int c_lo = wave * nc / 4, c_hi = (wave + 1) * nc / 4;
  // 16x16x32 operands: lane holds row (lane & 15), k = 8 (lane >> 4) .. + 7 of a 32-wide step
  const uint32_t xoff = (uint32_t)(lane & 15) * dbytes + (uint32_t)(lane >> 4) * 16u;
  uint32_t woff[NSUB];
#pragma unroll
  for (int n = 0; n < NSUB; ++n) woff[n] = (uint32_t)(n * 16 + (lane & 15)) * dbytes + (uint32_t)(lane >> 4) * 16u;
  u32x4 sa[P][2], sw[P][NSUB][2];
  auto issue = [&](int sl, int c) {
    const uint32_t kc = c < c_hi ? (uint32_t)c * (RT_KC * 2) : kOob;  // past the quarter: zeros
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      sa[sl][s] = buf_ld16(xres, xoff + kc + s * 64u);
#pragma unroll
      for (int n = 0; n < NSUB; ++n) sw[sl][n][s] = buf_ld16(wres, woff[n] + kc + s * 64u);
    }
  };
  f32x4 acc[NSUB];
#pragma unroll
  for (int n = 0; n < NSUB; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < P - 1; ++s) issue(s, c_lo + s);
  // Main loop, P chunks per trip, while every chunk it issues lies inside the wave's range:
  // no exit inside the trip, so the loads stay in flight across its back edge.
  int c0 = c_lo;
  for (; c0 + 2 * P - 2 < c_hi; c0 += P) {
#pragma unroll
    for (int s = 0; s < P; ++s) {
      issue((s + P - 1) % P, c0 + s + P - 1);
#pragma unroll
      for (int n = 0; n < NSUB; ++n)
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[n] = mfma16(sa[s][h], sw[s][n][h], acc[n]);
    }
  }
  // the last chunks (fewer than 2P - 1)
#pragma unroll
  for (int s = 0; s < 2 * P - 1; ++s) {
    const int c = c0 + s;
    if (c >= c_hi) break;
    if (c + P - 1 < c_hi) issue((s + P - 1) % P, c + P - 1);
#pragma unroll
    for (int n = 0; n < NSUB; ++n)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[n] = mfma16(sa[s % P][h], sw[s % P][n][h], acc[n]);
  }
  // C layout: lane holds expert n * 16 + (lane & 15), tokens 4 (lane >> 4) + i
#pragma unroll
  for (int n = 0; n < NSUB; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * (lane >> 4) + i][n * 16 + (lane & 15)] = acc[n][i];
  __syncthreads();
  for (int q = 0; q < 4; ++q) {
    const int tt = wave * 4 + q;
    const int64_t t = (int64_t)t0 + tt;
    if (t >= T) break;  // wave-uniform
    uint64_t key[1];
    float val = 0.f;
    if (lane < E) {
      val = red[0][tt][lane] + red[1][tt][lane] + red[2][tt][lane] + red[3][tt][lane];
      if (offset) val += offset[lane];
      if (logits) logits[t * E + lane] = val;
    }
    key[0] = lane < E ? topk_key(val, lane) : 0ull;
    topk_select<1>(key, E, k, t, lane, ids, gates, spare);
  }
}

}  // namespace

namespace {

hipError_t router_logits_bf16(const void *x, const void *w_router, const float *offset, float *logits, int T, int d,
                              int E, int splits, float *partials, hipStream_t s) {
  const int grid = (T + RT_TOK - 1) / RT_TOK;
  const int nk = d / RT_KC;
  const int cps = (nk + splits - 1) / splits;
  for (int e0 = 0; e0 < E; e0 += RT_EMAX) {
    const int ec = min(RT_EMAX, E - e0);
    const int nsub = (ec + 15) / 16;
    const bf16_t *xp = static_cast<const bf16_t *>(x);
    const bf16_t *wp = static_cast<const bf16_t *>(w_router);
#define RT_CASE(N)                                                                                      \
  case N:                                                                                               \
    hipLaunchKernelGGL(router_logits_bf16_kernel<N>, dim3(grid, splits), dim3(256), 0, s, xp, wp, offset,    \
                       logits, T, d, E, e0, cps, partials);                                             \
    break;
    switch (nsub <= 1 ? 1 : nsub <= 2 ? 2 : nsub <= 4 ? 4 : nsub <= 8 ? 8 : 16) {
      RT_CASE(1)
      RT_CASE(2)
      RT_CASE(4)
      RT_CASE(8)
      RT_CASE(16)
    }
#undef RT_CASE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t router_topk(float *logits, int T, int E, int k, int32_t *ids, float *gates, int32_t *spare,
                       const float *partials, int S, const float *offset, hipStream_t s) {
  if (partials && (S < 1 || S > 8)) return hipErrorInvalidValue;
  const int grid = (T + TK_WAVES - 1) / TK_WAVES;
  const int vpl = (E + 63) / 64;
  const int smax = !partials ? 0 : S <= 1 ? 1 : S <= 2 ? 2 : S <= 4 ? 4 : 8;
#define TK_LAUNCH(V, SM)                                                                                       \
  hipLaunchKernelGGL((router_topk_kernel<V, SM>), dim3(grid), dim3(256), 0, s, logits, T, E, k, ids, gates,   \
                     spare, partials, S, offset)
#define TK_CASE(V)                  \
  case V:                           \
    switch (smax) {                 \
      case 0: TK_LAUNCH(V, 0); break; \
      case 1: TK_LAUNCH(V, 1); break; \
      case 2: TK_LAUNCH(V, 2); break; \
      case 4: TK_LAUNCH(V, 4); break; \
      default: TK_LAUNCH(V, 8); break; \
    }                               \
    break;
  switch (vpl <= 1 ? 1 : vpl <= 2 ? 2 : vpl <= 4 ? 4 : vpl <= 8 ? 8 : 16) {
    TK_CASE(1)
    TK_CASE(2)
    TK_CASE(4)
    TK_CASE(8)
    TK_CASE(16)
  }
#undef TK_CASE
#undef TK_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_logits_bf16(const void *x, const void *w_router, const float *offset, float *logits, int T,
                                     int d, int E, hipStream_t s) {
  return router_logits_bf16(x, w_router, offset, logits, T, d, E, 1, nullptr, s);
}

// The fused kernel (router linear and top-k in one launch, 16 tokens per workgroup) when
// the router weights, which every workgroup reads from L2, are no larger than its token
// rows (E <= 16) and there are enough tokens to fill the GPU.  With more experts the
// weight re-reads cost more than the launch saves (64 experts, 8192 tokens: 18.7 µs
// against 14.8 µs for the split linear and the top-k kernel).
bool router_fused(int T, int E) { return E <= 16 && (int64_t)T >= 16 * 256; }

// Splits of d for the router linear: enough workgroups to fill the GPU when the tokens
// are few, at least two chunks of 64 per split, at most 8 splits and 64 MiB of partials.
int router_splits(int T, int d, int E) {
  if (router_fused(T, E)) return 1;
  const int64_t base = (int64_t)((T + RT_TOK - 1) / RT_TOK) * ((E + RT_EMAX - 1) / RT_EMAX);
  int S = base >= 256 ? 1 : (int)std::min<int64_t>(8, 256 / std::max<int64_t>(base, 1));
  S = std::max(1, std::min(S, (d / RT_KC) / 2));
  while (S > 1 && (int64_t)S * T * E * 4 > ((int64_t)64 << 20)) S /= 2;
  return S;
}

size_t router_partials_bytes(int T, int d, int E) {
  const int G = router_gemm_splits(T, d, E);
  if (G > 0) return (size_t)G * T * E * 4;
  const int S = router_splits(T, d, E);
  return S > 1 ? (size_t)S * T * E * 4 : 0;
}

hipError_t launch_router_bf16(const void *x, const void *w_router, const float *offset, float *logits, int T, int d,
                              int E, int k, int32_t *ids, float *gates, int32_t *spare, float *partials,
                              hipStream_t s) {
  if (router_fused(T, E)) {
    const int grid = (T + 15) / 16;
    const bf16_t *xp = static_cast<const bf16_t *>(x), *wp = static_cast<const bf16_t *>(w_router);
    hipLaunchKernelGGL(router_fused_kernel<1>, dim3(grid), dim3(256), 0, s, xp, wp, offset, logits, T, d, E, k, ids,
                       gates, spare);
    return hipGetLastError();
  }
  if (const int G = router_gemm_splits(T, d, E)) {
    // many tokens and experts: the large-tile GEMM, its float partials added (with the
    // offset) by the top-k kernel
    hipError_t e = launch_router_gemm(x, w_router, T, d, E, partials, s);
    if (e != hipSuccess) return e;
    return router_topk(logits, T, E, k, ids, gates, spare, partials, G, offset, s);
  }
  const int S = router_splits(T, d, E);
  if (S == 1) {
    hipError_t e = router_logits_bf16(x, w_router, offset, logits, T, d, E, 1, nullptr, s);
    if (e != hipSuccess) return e;
    return router_topk(logits, T, E, k, ids, gates, spare, nullptr, 1, nullptr, s);
  }
  hipError_t e = router_logits_bf16(x, w_router, offset, logits, T, d, E, S, partials, s);
  if (e != hipSuccess) return e;
  return router_topk(logits, T, E, k, ids, gates, spare, partials, S, offset, s);
}

hipError_t launch_router_logits_f32(const float *x, const float *w_router, const float *offset, float *logits, int T,
                                    int d, int E, hipStream_t s) {
  const int64_t n = (int64_t)T * E;
  const int grid = int((n + 255) / 256);
  hipLaunchKernelGGL(router_logits_f32_kernel, dim3(grid), dim3(256), 0, s, x, w_router, offset, logits, T, d, E);
  return hipGetLastError();
}

hipError_t launch_router_topk(const float *logits, int T, int E, int k, int32_t *ids, float *gates, hipStream_t s,
                              int32_t *spare) {
  return router_topk(const_cast<float *>(logits), T, E, k, ids, gates, spare, nullptr, 1, nullptr, s);
}

}  // namespace moe
