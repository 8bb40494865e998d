// Grouped expert GEMM for few rows per expert (weight streaming), bf16 on gfx950.
//
// The expert FFN is a dense contraction per expert over that expert's rows (tokens
// sorted by expert id, one grouped GEMM for all experts: "Что такое Mixture of
// Experts (MoE) в трансформерах", aglamov.biz, section "Бэкенд для экспертов").
// When an expert holds at most a few hundred rows, every weight byte is used by few
// MFMAs and the kernel is bound by HBM: the design goal is that each weight byte
// crosses HBM exactly once, with enough loads in flight to saturate it.
//
// Workgroup = 4 wavefronts = one (expert, column tile).  Each wave owns NSUB
// 16-column output subtiles; with SwiGLU it loads the matching gate rows and up
// rows (W rows n and n + n_out) so both accumulators of a column sit in the same
// lane.  Weight rows go straight from HBM into MFMA B-operand registers (16 bytes
// per lane per subtile and 32-wide k step), prefetched two LDS stages ahead.  The
// expert's token rows (A operand, reused by every column tile of the expert) are
// staged through LDS in 64-wide K chunks, XOR-swizzled by row so the 16-lane column
// reads of the MFMA layout spread over distinct banks.  Row blocks of BM rows are
// walked in order, so any group size is computed correctly; 16-row subtiles beyond
// the group's rows skip their MFMAs.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int SG_KC = 64;  // K per pipeline chunk = two 32-wide MFMA k steps

// Loop over K for one block of `rows` <= BM rows starting at m0, specialised on NA,
// the number of 256-thread A load rounds the block needs (ceil(rows * 8 / 256)):
// blocks of few rows issue few A loads and run only the MFMA subtiles they fill.
//
// P chunks are in flight per wave.  Every load is issued unconditionally through a
// buffer resource; chunks past the end of K, token rows past the block's end and
// weight subtiles past n_out get an out-of-range offset and read as zeros without a
// memory access, which keeps the order of outstanding loads static: waiting for
// chunk c never waits for chunks issued after it.
template <int BM, int NSUB, bool SWIGLU, int P, int NA>
__device__ __forceinline__ void stream_block(const rsrc_t wres, const rsrc_t ares, const uint32_t *boff,
                                             const uint32_t *aoff, uint8_t (*ldsA)[BM * SG_KC * 2], int nk, int rows,
                                             int m0, int ncol0, int nvalid, int n_out, bf16_t *__restrict__ out) {
  constexpr int NB = SWIGLU ? 2 * NSUB : NSUB;
  constexpr int MS = (NA * 256 / 8 + 15) / 16 < BM / 16 ? (NA * 256 / 8 + 15) / 16 : BM / 16;
  const int tid = threadIdx.x, lane = tid & 63;
  struct Chunk {
    u32x4 b[2][NB];
    u32x4 a[NA];
  };
  Chunk slot[P];
  // loads of chunk c into a slot; chunks past the end of K get out-of-range offsets
  auto issue = [&](Chunk &ch, int c) {
    // an invalid base is kOob, and kOob + kc stays out of range (kc < 2^31)
    const bool ok = c < nk;
    const uint32_t kc = (uint32_t)c * (SG_KC * 2);
#pragma unroll
    for (int i = 0; i < NA; ++i) ch.a[i] = buf_ld16(ares, ok ? aoff[i] + kc : kOob);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int b = 0; b < NB; ++b) ch.b[s][b] = buf_ld16(wres, ok ? boff[b] + kc + s * 64u : kOob);
  };
  // the same for a chunk known to be inside K: straight-line code, no selects
  auto issue_in = [&](Chunk &ch, int c) {
    const uint32_t kc = (uint32_t)c * (SG_KC * 2);
#pragma unroll
    for (int i = 0; i < NA; ++i) ch.a[i] = buf_ld16(ares, aoff[i] + kc);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int b = 0; b < NB; ++b) ch.b[s][b] = buf_ld16(wres, boff[b] + kc + s * 64u);
  };
  auto stage_a = [&](const Chunk &ch, int buf) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = tid + 256 * i;
      if ((BM * 8) % 256 == 0 || q < BM * 8) {
        const int r = q >> 3, c = q & 7;
        *reinterpret_cast<u32x4 *>(&ldsA[buf][(r * 8 + (c ^ (r & 7))) * 16]) = ch.a[i];
      }
    }
  };
  f32x4 acc[MS][NB];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[i][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Chunk &ch, int buf) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 a[MS];  // all row fragments of this k step first: one LDS wait per step
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        const int r = i * 16 + (lane & 15);
        const int c = s * 4 + (lane >> 4);
        a[i] = *reinterpret_cast<const u32x4 *>(&ldsA[buf][(r * 8 + (c ^ (r & 7))) * 16]);
      }
#pragma unroll
      for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[i][b] = mfma16(a[i], ch.b[s][b], acc[i][b]);
    }
  };

  // prologue: chunks 0 .. P-2 in flight, A of chunk 0 in LDS buffer 0
#pragma unroll
  for (int s = 0; s < P - 1; ++s) issue(slot[s], s);
  stage_a(slot[0], 0);
  __syncthreads();
  // Main loop, P chunks per trip, while every chunk it issues lies inside K: no
  // conditions, so slots, LDS buffers (chunk parity = s & 1, P even) and wait counts are
  // all static.  Step c issues chunk c + P - 1 into the slot chunk c - 1 has finished
  // with, computes chunk c, and stages the A rows of chunk c + 1.
  static_assert(P % 2 == 0, "the LDS buffer of a chunk is its parity");
  int c0 = 0;
  for (; c0 + 2 * P - 2 < nk; c0 += P) {
#pragma unroll
    for (int s = 0; s < P; ++s) {
      issue_in(slot[(s + P - 1) % P], c0 + s + P - 1);
      compute(slot[s], s & 1);
      stage_a(slot[(s + 1) % P], (s + 1) & 1);
      __syncthreads();
    }
  }
  // the last (fewer than 2P - 1) chunks
#pragma unroll
  for (int s = 0; s < 2 * P - 1; ++s) {
    const int c = c0 + s;
    if (c >= nk) break;
    if (c + P - 1 < nk) issue_in(slot[(s + P - 1) % P], c + P - 1);
    compute(slot[s % P], s & 1);
    if (c + 1 < nk) stage_a(slot[(s + 1) % P], (s + 1) & 1);
    __syncthreads();
  }

  // epilogue: C layout of the 16x16 MFMA -- column (lane & 15), rows 4*(lane>>4)+j
#pragma unroll
  for (int i = 0; i < MS; ++i) {
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      if (s >= nvalid) continue;
      const int col = ncol0 + s * 16 + (lane & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = i * 16 + (lane >> 4) * 4 + j;
        if (r >= rows) continue;
        float v;
        if constexpr (SWIGLU) {
          v = silu_f32(acc[i][s][j]) * acc[i][NSUB + s][j];
        } else {
          v = acc[i][s][j];
        }
        out[(size_t)(m0 + r) * n_out + col] = f32_to_bf16(v);
      }
    }
  }
}

// Tiles are taken in block-id order (expert-major, column tile minor); the hardware
// deals consecutive blocks to the 8 XCDs round-robin, which spreads every expert --
// including the few heavily loaded ones -- over all XCDs.
template <int BM, int NSUB, bool SWIGLU, int P>
__global__ __launch_bounds__(256, 2) void grouped_gemm_stream_kernel(const bf16_t *__restrict__ A,
                                                                     const int32_t *__restrict__ row_index,
                                                                     int64_t a_rows,
                                                                     const int32_t *__restrict__ offsets,
                                                                     const bf16_t *__restrict__ W, int64_t wstride,
                                                                     int n_out, int K, bf16_t *__restrict__ out,
                                                                     int n_tiles) {
  constexpr int NB = SWIGLU ? 2 * NSUB : NSUB;  // 16-row weight subtiles per wave
  constexpr int A_PER_T = (BM * 8 + 255) / 256;  // 16-byte A pieces staged per thread per chunk
  __shared__ __attribute__((aligned(16))) uint8_t ldsA[2][BM * SG_KC * 2];

  const int tile = blockIdx.x;
  const int g = tile / n_tiles, nt = tile - g * n_tiles;
  const int row_begin = offsets[g], row_end = offsets[g + 1];
  if (row_begin >= row_end) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncol0 = (nt * 4 + wave) * 16 * NSUB;
  const int nvalid = max(0, min(NSUB, (n_out - ncol0) / 16));  // wave-uniform
  const uint32_t kbytes = (uint32_t)K * 2u;
  const rsrc_t wres = make_rsrc(W + (size_t)g * wstride, (uint32_t)(wstride * 2));

  uint32_t boff[NB];  // byte offset of this lane's 16 bytes in weight subtile b at k = 0
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int sidx = b % NSUB;
    const int r = ncol0 + sidx * 16 + (lane & 15) + (b >= NSUB ? n_out : 0);
    boff[b] = sidx < nvalid ? (uint32_t)r * kbytes + (uint32_t)(lane >> 4) * 16u : kOob;
  }
  const int nk = K / SG_KC;

  for (int m0 = row_begin; m0 < row_end; m0 += BM) {
    const int rows = min(BM, row_end - m0);
    // byte offset of this thread's A pieces at k = 0 (row r, 16-byte column c8); with a
    // row gather the rows come straight from the unpermuted activations
    uint32_t aoff[A_PER_T];
    rsrc_t ares;
    if (row_index) {
      ares = make_rsrc(A, (uint32_t)(a_rows * kbytes));
#pragma unroll
      for (int i = 0; i < A_PER_T; ++i) {
        const int q = tid + 256 * i;
        const int r = q >> 3;
        aoff[i] = (q < BM * 8 && r < rows) ? (uint32_t)row_index[m0 + r] * kbytes + (uint32_t)(q & 7) * 16u : kOob;
      }
    } else {
      ares = make_rsrc(A + (size_t)m0 * K, (uint32_t)rows * kbytes);
#pragma unroll
      for (int i = 0; i < A_PER_T; ++i) {
        const int q = tid + 256 * i;
        aoff[i] = q < BM * 8 ? (uint32_t)(q >> 3) * kbytes + (uint32_t)(q & 7) * 16u : kOob;
      }
    }
    const int na = (rows * 8 + 255) / 256;  // workgroup-uniform
#define SG_BLOCK(N)                                                                                                 \
  if constexpr (N <= A_PER_T) {                                                                                     \
    if (na == N) {                                                                                                  \
      stream_block<BM, NSUB, SWIGLU, P, N>(wres, ares, boff, aoff, ldsA, nk, rows, m0, ncol0, nvalid, n_out, out); \
      continue;                                                                                                     \
    }                                                                                                               \
  }
    SG_BLOCK(1)
    SG_BLOCK(2)
    SG_BLOCK(3)
    SG_BLOCK(4)
#undef SG_BLOCK
  }
}

template <int BM, int NSUB, bool SWIGLU>
hipError_t launch_stream(const GroupedGemmArgs &a, hipStream_t s) {
  constexpr int P = 4;
  const int cols_per_tile = 64 * NSUB;
  const int n_tiles = (a.n_out + cols_per_tile - 1) / cols_per_tile;
  const int64_t grid = (int64_t)a.num_groups * n_tiles;
  hipLaunchKernelGGL((grouped_gemm_stream_kernel<BM, NSUB, SWIGLU, P>), dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const bf16_t *>(a.A), a.row_index, a.a_rows, a.offsets, static_cast<const bf16_t *>(a.W), a.w_group_stride,
                     a.n_out, a.K, static_cast<bf16_t *>(a.out), n_tiles);
  return hipGetLastError();
}

template <bool SWIGLU>
hipError_t launch_stream_bm(const GroupedGemmArgs &a, hipStream_t s) {
  const int r = a.group_rows_max;
  if (r <= 16) return launch_stream<16, 1, SWIGLU>(a, s);
  if (r <= 32) return launch_stream<32, 1, SWIGLU>(a, s);
  if (r <= 64) return launch_stream<64, 1, SWIGLU>(a, s);
  return launch_stream<128, 1, SWIGLU>(a, s);
}

}  // namespace

hipError_t launch_grouped_gemm_stream_bf16(const GroupedGemmArgs &a, hipStream_t s) {
  return a.swiglu ? launch_stream_bm<true>(a, s) : launch_stream_bm<false>(a, s);
}

// Regime choice: the streaming kernel when groups hold few rows on average (each
// weight byte feeds few MFMAs, HBM bound), the 256 x 256 tile kernel when they hold
// many (MFMA bound).  The row bounds are the caller's; either kernel computes any
// group size correctly.
hipError_t launch_grouped_gemm_bf16(const GroupedGemmArgs &a, hipStream_t s) {
  const int64_t avg_rows = a.rows_max / a.num_groups;
  if (avg_rows >= 256 && a.group_rows_max >= 256) return launch_grouped_gemm_big_bf16(a, a.rows_max, s);
  return launch_grouped_gemm_stream_bf16(a, s);
}

}  // namespace moe
