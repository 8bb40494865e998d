// Grouped expert GEMM for experts with many rows (compute bound), bf16 on gfx950.
//
// Same problem as the weight-streaming kernel -- per group, its rows of A times the
// group's weight rows, SwiGLU fused for the gate/up projection -- but sized for
// groups of hundreds to thousands of rows, where the contraction is dense enough to
// be bound by the matrix cores ("Что такое Mixture of Experts (MoE) в
// трансформерах", aglamov.biz, section "Бэкенд для экспертов": one grouped GEMM over
// tokens sorted by expert).
//
// Block tile: 256 rows x 256 weight rows, K in steps of 64.  Four wavefronts in a
// 2 x 2 arrangement each own 128 x 128 of the tile as 4 x 4 blocks of the 32x32x16
// bf16 MFMA (256 float accumulators per lane).  Both operand tiles are staged
// through LDS (two buffers of 64 KB), XOR-swizzled by row so the 32-row column reads
// of the MFMA operand layout hit distinct banks; global loads for the next K step
// are issued before the current step's MFMAs.  For SwiGLU the 256 weight rows are
// 128 gate rows and the 128 matching up rows, and each wave owns 64 output columns
// of both, so gate and up accumulators of a column sit in the same lane.
//
// Tiles: each group contributes ceil(rows / 256) row tiles times the column tiles.
// A block finds its group from the offsets (one wavefront scan), and walks the
// group's tiles with the larger operand outermost, so the smaller one is reused
// from cache.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int BG_BM = 256, BG_BN = 256, BG_BK = 64;
constexpr int BG_THREADS = 256;
constexpr int BG_CHUNKS = BG_BM * BG_BK * 2 / 16 / BG_THREADS;  // 16-byte pieces per thread per operand = 8

// LDS offset (bytes) of row r, 16-byte chunk c of a [256][64] bf16 tile.
template <int SW>
__device__ __forceinline__ uint32_t lds_off(int r, int c) {
  const int pc = SW == 0 ? (c ^ (r & 7)) : (c ^ ((r >> 1) & 7));
  return (uint32_t)(r * 8 + pc) * 16u;
}

// Exclusive prefix of ceil(rows_g / BM) over groups, evaluated by one wavefront; returns
// for tile index `m_lin` its group (or -1 past the end), the group's first m tile and
// the number of its m tiles.
__device__ __forceinline__ void find_group(const int32_t *offsets, int G, int m_lin, int &g_out, int &mt_first,
                                           int &mt_count) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  g_out = -1;
  mt_first = 0;
  mt_count = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    const int g = g0 + lane;
    int mt = 0;
    if (g < G) mt = (offsets[g + 1] - offsets[g] + BG_BM - 1) / BG_BM;
    int incl = mt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const uint64_t hit = __ballot(g < G && base + incl > m_lin);
    if (hit) {
      const int l = __ffsll((unsigned long long)hit) - 1;
      g_out = g0 + l;
      const int excl = __shfl(incl - mt, l, 64);
      mt_first = base + excl;
      mt_count = __shfl(mt, l, 64);
      return;
    }
    base += __shfl(incl, 63, 64);
  }
}

template <bool SWIGLU, int SW>
__global__ __launch_bounds__(BG_THREADS, 1) void grouped_gemm_big_kernel(const bf16_t *__restrict__ A,
                                                                         const int32_t *__restrict__ offsets, int G,
                                                                         const bf16_t *__restrict__ W,
                                                                         int64_t wstride, int n_out, int K,
                                                                         bf16_t *__restrict__ out, int n_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BG_BM * BG_BK * 2];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BG_BN * BG_BK * 2];

  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int m_lin = lin / n_tiles;  // rank of this block's tile among all groups' m tiles (n tile folded below)
  int g, mt_first, mt_count;
  // Blocks are numbered group-major: the tiles of group g occupy [mt_first * n_tiles,
  // (mt_first + mt_count) * n_tiles).  Within a group the order is chosen below.
  find_group(offsets, G, m_lin, g, mt_first, mt_count);
  // the scan's results are equal in every lane: keep them (and all that derives from
  // them, like the buffer resources) in scalar registers
  g = __builtin_amdgcn_readfirstlane(g);
  mt_first = __builtin_amdgcn_readfirstlane(mt_first);
  mt_count = __builtin_amdgcn_readfirstlane(mt_count);
  if (g < 0) return;
  const int local = lin - mt_first * n_tiles;  // 0 .. mt_count * n_tiles - 1
  const int row_begin = offsets[g], row_end = offsets[g + 1];
  const int64_t a_bytes = (int64_t)(row_end - row_begin) * K;
  const int64_t b_bytes = (int64_t)(SWIGLU ? 2 : 1) * n_out * K;
  int mt, nt;
  if (a_bytes <= b_bytes) {  // weights larger: weight tile outermost, row tiles reuse it
    nt = local / mt_count;
    mt = local - nt * mt_count;
  } else {
    mt = local / n_tiles;
    nt = local - mt * n_tiles;
  }
  const int m0 = row_begin + mt * BG_BM;
  const int rows = min(BG_BM, row_end - m0);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t kbytes = (uint32_t)K * 2u;
  const int n0 = nt * (SWIGLU ? BG_BN / 2 : BG_BN);  // first output column of the tile

  const rsrc_t ares = make_rsrc(A + (size_t)m0 * K, (uint32_t)rows * kbytes);
  const rsrc_t wres = make_rsrc(W + (size_t)g * wstride, (uint32_t)(wstride * 2));

  // Per-thread global offsets (k = 0) and LDS offsets of its 8 A and 8 B pieces.
  uint32_t agoff[BG_CHUNKS], bgoff[BG_CHUNKS], loff[BG_CHUNKS];
#pragma unroll
  for (int i = 0; i < BG_CHUNKS; ++i) {
    const int q = tid + BG_THREADS * i;
    const int r = q >> 3, c = q & 7;
    agoff[i] = (uint32_t)r * kbytes + (uint32_t)c * 16u;
    int wr;  // weight row held in tile row r
    if (SWIGLU) {
      const int col = n0 + (r & 127);
      wr = col < n_out ? (r < 128 ? col : n_out + col) : -1;
    } else {
      wr = n0 + r < n_out ? n0 + r : -1;
    }
    bgoff[i] = wr >= 0 ? (uint32_t)wr * kbytes + (uint32_t)c * 16u : kOob;
    loff[i] = lds_off<SW>(r, c);
  }

  u32x4 ra[BG_CHUNKS], rb[BG_CHUNKS];
  auto gload = [&](int kt) {
    const uint32_t kc = (uint32_t)kt * (BG_BK * 2);
#pragma unroll
    for (int i = 0; i < BG_CHUNKS; ++i) {
      ra[i] = buf_ld16(ares, agoff[i] + kc);
      rb[i] = buf_ld16(wres, bgoff[i] == kOob ? kOob : bgoff[i] + kc);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < BG_CHUNKS; ++i) {
      *reinterpret_cast<u32x4 *>(&sA[buf][loff[i]]) = ra[i];
      *reinterpret_cast<u32x4 *>(&sB[buf][loff[i]]) = rb[i];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // rows of the operand tiles this lane reads for its MFMA blocks
  int arow[4], brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    arow[i] = wm * 128 + i * 32 + (lane & 31);
    brow[i] = SWIGLU ? (i < 2 ? wn * 64 + i * 32 : 128 + wn * 64 + (i - 2) * 32) + (lane & 31)
                     : wn * 128 + i * 32 + (lane & 31);
  }

  const int nk = K / BG_BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      u32x4 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *reinterpret_cast<const u32x4 *>(&sA[buf][lds_off<SW>(arow[i], c)]);
        bfr[i] = *reinterpret_cast<const u32x4 *>(&sB[buf][lds_off<SW>(brow[i], c)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  32x32 MFMA layout: lane holds column (lane & 31) and rows
  // 8*(r/4) + 4*(lane/32) + (r%4), r = 0..15.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < (SWIGLU ? 2 : 4); ++j) {
      const int col = n0 + (SWIGLU ? wn * 64 : wn * 128) + j * 32 + (lane & 31);
      if (col >= n_out) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 128 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row >= rows) continue;
        float v;
        if constexpr (SWIGLU) {
          v = silu_f32(acc[i][j][r]) * acc[i][j + 2][r];
        } else {
          v = acc[i][j][r];
        }
        out[(size_t)(m0 + row) * n_out + col] = f32_to_bf16(v);
      }
    }
  }
}

}  // namespace

// Upper bound of the total row tiles: sum_g ceil(rows_g / 256) <= ceil(rows / 256) + G.
hipError_t launch_grouped_gemm_big_bf16(const GroupedGemmArgs &a, int64_t rows_total_max, hipStream_t s) {
  const int cols = a.swiglu ? BG_BN / 2 : BG_BN;
  const int n_tiles = (a.n_out + cols - 1) / cols;
  const int64_t m_tiles = (rows_total_max + BG_BM - 1) / BG_BM + a.num_groups;
  const int64_t grid = m_tiles * n_tiles;
  if (a.swiglu)
    hipLaunchKernelGGL((grouped_gemm_big_kernel<true, 0>), dim3((unsigned)grid), dim3(BG_THREADS), 0, s,
                       static_cast<const bf16_t *>(a.A), a.offsets, a.num_groups, static_cast<const bf16_t *>(a.W),
                       a.w_group_stride, a.n_out, a.K, static_cast<bf16_t *>(a.out), n_tiles);
  else
    hipLaunchKernelGGL((grouped_gemm_big_kernel<false, 0>), dim3((unsigned)grid), dim3(BG_THREADS), 0, s,
                       static_cast<const bf16_t *>(a.A), a.offsets, a.num_groups, static_cast<const bf16_t *>(a.W),
                       a.w_group_stride, a.n_out, a.K, static_cast<bf16_t *>(a.out), n_tiles);
  return hipGetLastError();
}

}  // namespace moe
