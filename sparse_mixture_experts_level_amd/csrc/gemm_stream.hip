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

constexpr int SG_KC = 64;  // K per LDS stage = two 32-wide MFMA k steps

template <int BM, int NSUB, bool SWIGLU>
__global__ __launch_bounds__(256, 2) void grouped_gemm_stream_kernel(const bf16_t *__restrict__ A,
                                                                     const int32_t *__restrict__ offsets,
                                                                     const bf16_t *__restrict__ W, int64_t wstride,
                                                                     int n_out, int K, bf16_t *__restrict__ out,
                                                                     int n_tiles) {
  constexpr int NB = SWIGLU ? 2 * NSUB : NSUB;  // 16-row weight subtiles per wave
  constexpr int MS = BM / 16;                  // 16-row A subtiles
  constexpr int A_PER_T = (BM * 8 + 255) / 256;  // 16-byte A chunks staged per thread
  __shared__ __attribute__((aligned(16))) uint8_t ldsA[2][BM * SG_KC * 2];

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int g = tile / n_tiles, nt = tile - g * n_tiles;
  const int row_begin = offsets[g], row_end = offsets[g + 1];
  if (row_begin >= row_end) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncol0 = (nt * 4 + wave) * 16 * NSUB;
  const int nvalid = max(0, min(NSUB, (n_out - ncol0) / 16));  // wave-uniform
  const bf16_t *Wg = W + (size_t)g * wstride;
  const int kq = (lane >> 4) * 8;  // this lane's k offset inside a 32-wide step

  const bf16_t *wrow[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int s = b % NSUB;
    const int r = ncol0 + s * 16 + (lane & 15) + (b >= NSUB ? n_out : 0);
    wrow[b] = Wg + (size_t)(s < nvalid ? r : 0) * K + kq;
  }

  const int nk = K / SG_KC;

  for (int m0 = row_begin; m0 < row_end; m0 += BM) {
    const int rows = min(BM, row_end - m0);
    const int msub = (rows + 15) >> 4;

    u32x4 astage[A_PER_T];
    auto loadA = [&](int kc) {
#pragma unroll
      for (int i = 0; i < A_PER_T; ++i) {
        const int q = tid + 256 * i;
        const int r = q >> 3, c = q & 7;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (q < BM * 8 && r < rows) v = ldg16(A + (size_t)(m0 + r) * K + kc + c * 8);
        astage[i] = v;
      }
    };
    auto storeA = [&](int buf) {
#pragma unroll
      for (int i = 0; i < A_PER_T; ++i) {
        const int q = tid + 256 * i;
        if (q < BM * 8) {
          const int r = q >> 3, c = q & 7;
          *reinterpret_cast<u32x4 *>(&ldsA[buf][(r * 8 + (c ^ (r & 7))) * 16]) = astage[i];
        }
      }
    };

    u32x4 bq0[2][NB], bq1[2][NB];  // two prefetch stages x two k steps
    auto loadB = [&](u32x4 (&bq)[2][NB], int kc) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if ((b % NSUB) < nvalid) bq[s][b] = ldg16(wrow[b] + kc + s * 32);
    };

    f32x4 acc[MS][NB];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[i][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const u32x4 (&bq)[2][NB], int buf) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < MS; ++i) {
          if (i < msub) {
            const int r = i * 16 + (lane & 15);
            const int c = s * 4 + (lane >> 4);
            const u32x4 a = *reinterpret_cast<const u32x4 *>(&ldsA[buf][(r * 8 + (c ^ (r & 7))) * 16]);
#pragma unroll
            for (int b = 0; b < NB; ++b)
              if ((b % NSUB) < nvalid) acc[i][b] = mfma16(a, bq[s][b], acc[i][b]);
          }
        }
      }
    };

    // prologue: A stage 0 in LDS, B stages 0 and 1 in flight
    loadA(0);
    loadB(bq0, 0);
    if (nk > 1) loadB(bq1, SG_KC);
    storeA(0);
    __syncthreads();

    for (int it = 0; it < nk; it += 2) {
      // even step: consumes bq0 / LDS buffer 0
      if (it + 1 < nk) loadA((it + 1) * SG_KC);
      compute(bq0, 0);
      if (it + 2 < nk) loadB(bq0, (it + 2) * SG_KC);
      if (it + 1 < nk) storeA(1);
      __syncthreads();
      if (it + 1 >= nk) break;
      // odd step: consumes bq1 / LDS buffer 1
      if (it + 2 < nk) loadA((it + 2) * SG_KC);
      compute(bq1, 1);
      if (it + 3 < nk) loadB(bq1, (it + 3) * SG_KC);
      if (it + 2 < nk) storeA(0);
      __syncthreads();
    }

    // epilogue: C layout of the 16x16 MFMA -- column (lane & 15), rows 4*(lane>>4)+j
#pragma unroll
    for (int i = 0; i < MS; ++i) {
      if (i >= msub) continue;
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
}

template <int BM, int NSUB, bool SWIGLU>
hipError_t launch_stream(const GroupedGemmArgs &a, hipStream_t s) {
  const int cols_per_tile = 64 * NSUB;
  const int n_tiles = (a.n_out + cols_per_tile - 1) / cols_per_tile;
  const int64_t grid = (int64_t)a.num_groups * n_tiles;
  hipLaunchKernelGGL((grouped_gemm_stream_kernel<BM, NSUB, SWIGLU>), dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const bf16_t *>(a.A), a.offsets, static_cast<const bf16_t *>(a.W), a.w_group_stride,
                     a.n_out, a.K, static_cast<bf16_t *>(a.out), n_tiles);
  return hipGetLastError();
}

template <bool SWIGLU>
hipError_t launch_stream_bm(const GroupedGemmArgs &a, hipStream_t s) {
  const int r = a.group_rows_max;
  if (r <= 16) return launch_stream<16, 2, SWIGLU>(a, s);
  if (r <= 32) return launch_stream<32, 2, SWIGLU>(a, s);
  if (r <= 64) return launch_stream<64, 2, SWIGLU>(a, s);
  return launch_stream<128, 2, SWIGLU>(a, s);
}

}  // namespace

hipError_t launch_grouped_gemm_stream_bf16(const GroupedGemmArgs &a, hipStream_t s) {
  return a.swiglu ? launch_stream_bm<true>(a, s) : launch_stream_bm<false>(a, s);
}

hipError_t launch_grouped_gemm_bf16(const GroupedGemmArgs &a, hipStream_t s) {
  return launch_grouped_gemm_stream_bf16(a, s);
}

}  // namespace moe
