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
// lane.  Weight rows come from HBM as whole 128-byte lines (one load instruction: 8 rows
// x 128 bytes of a 64-wide K chunk) marked non-temporal -- each weight byte is read once
// -- into registers, and pass through a small wave-private LDS region into the MFMA
// B-operand layout (16 rows x 64 bytes per 32-wide k step).  Loading the operand layout
// directly splits every line over two instructions; non-temporal loads then fetch each
// line twice, and without the hint the stream reads slower (measured on this GPU: 7.0
// TB/s for whole lines with the hint, 6.25 TB/s for the operand layout without it, 5.3
// TB/s with it).  The expert's token rows (A operand,
// reused by every column tile of the expert) go straight from memory into LDS with
// buffer loads that target LDS (no registers), in 64-wide K chunks, XOR-swizzled by
// row so the 16-lane column reads of the MFMA layout spread over distinct banks.
// Both operands run S - 1 chunks ahead through S register slots / LDS stages (three for
// gate_up, four for the down projection).  bf16 results leave as whole 16-byte pieces.
// Row blocks of BM rows are walked in order, so any group size is computed
// correctly; 16-row subtiles beyond the group's rows skip their MFMAs.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int SG_KC = 64;  // K per pipeline chunk = two 32-wide MFMA k steps

// LDS bytes of one A stage: BM rows of one chunk, and at least the 64 * NW pieces of 16
// bytes that one round of the workgroup's NW waves writes.
template <int BM, int NW>
constexpr int sg_stage_bytes() {
  return (BM * 8 < 64 * NW ? 64 * NW : BM * 8) * 16;
}

// K-major weight tile in LDS: 64 k-rows of 64 columns (8 pieces of 8 columns, 16 bytes
// each); piece p of row r is stored at slot 8 r + (p ^ wt_swz(r)).  The swizzle spreads
// the transpose reads of one instruction -- per 16 lanes, rows r0 .. r0 + 3 of two
// adjacent pieces; the four 16-lane groups 8 rows apart -- over all 64 banks, two groups
// per LDS cycle.
__device__ __forceinline__ int wt_swz(int r) { return (((r >> 1) & 1) | (((r >> 3) & 1) << 1)) << 1; }

// gfx950 LDS transpose read (ds_read_b64_tr_b16), 16-lane groups: lane 4a + c of a group
// receives element c of the 8-byte chunks addressed by lanes a, a + 4, a + 8, a + 12 of
// the group, in that order.  For the 16x16x32 MFMA B operand (lane: column n = lane & 15,
// k = 8 (lane >> 4) .. + 7) a lane addresses k-row k0 + (lane & 15) / 4 and columns
// 4 ((lane & 15) % 4) .. + 3 of its wave's 16, for k0 = 32 s + 8 (lane >> 4) and k0 + 4.
__device__ __forceinline__ u32x4 wt_frag(const uint8_t *tile, int s, int wave, int lane) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const int l16 = lane & 15;
  const int piece = 2 * wave + ((l16 & 3) >> 1), half = (l16 & 1) * 8;
  u32x4 out;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = 32 * s + 8 * (lane >> 4) + 4 * t + (l16 >> 2);
    const uint8_t *p = tile + (r * 8 + (piece ^ wt_swz(r))) * 16 + half;
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)p);
    out[2 * t] = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
    out[2 * t + 1] = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
  }
  return out;
}

// Loop over K for one block of `rows` <= BM rows starting at m0, specialised on NA,
// the number of workgroup-wide rounds of 16-byte A pieces the block needs
// (ceil(rows * 8 / (64 * NW))): blocks of few rows issue few A loads and run only the
// MFMA subtiles they fill.
//
// S register slots / LDS stages; operands run S - 1 chunks ahead.  Step c: wait until
// this thread's loads of chunk c are complete (a fixed number of younger loads may stay
// in flight), barrier (every thread's A pieces of chunk c are in LDS, and every wave is
// done reading the stage about to be refilled), issue chunk c + S - 1 (weights into a
// register slot, A pieces into an LDS stage), compute chunk c.
// Loads are issued unconditionally through buffer resources: token rows past the
// block's end and weight subtiles past n_out get an out-of-range offset and read as
// zeros without a memory access, which keeps the count of loads per step static.
template <int BM, int NSUB, bool SWIGLU, int S, int NW, int NA, typename OutT, bool WT, bool GB>
__device__ __forceinline__ void stream_block(const rsrc_t wres, const rsrc_t ares, const uint32_t *boff,
                                             const uint32_t *aoff, uint8_t *sA0, uint8_t *sA1, uint8_t *sA2,
                                             uint8_t *sA3, uint8_t *const *sW, uint8_t *sWt, uint32_t hrow,
                                             int nk, int rot, int rows, int m0, int ncol0,
                                             int nvalid, int n_out, OutT *__restrict__ out, const SwigluBwdOut &gb) {
  static_assert(S == 3 || S == 4, "three or four stages");
  static_assert(!WT || (NSUB == 1 && NW == 4 && !SWIGLU), "K-major weights: one 64-column tile of four waves");
  static_assert(!GB || (SWIGLU && sizeof(OutT) == 2), "SwiGLU backward: gate and up blocks, bf16 gradients");
  constexpr int NB = SWIGLU ? 2 * NSUB : NSUB;
  constexpr int MS = NA * NW / 2 < BM / 16 ? NA * NW / 2 : BM / 16;  // 16-row subtiles the block can fill
  constexpr int LOADS = NA + 2 * (WT ? 1 : NB);            // loads per thread and chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto stage = [&](int i) -> uint8_t * { return i == 0 ? sA0 : i == 1 ? sA1 : i == 2 ? sA2 : sA3; };
  u32x4 slot[WT ? 1 : S][2][NB];
  // K-major weights: a chunk's 64 x 64 weight tile moves into LDS as rows of 128 bytes,
  // two 1 KB instructions per wave (8 rows each, boff[0] and boff[1]); a chunk advances
  // 64 rows.
  const uint32_t wchunk = (uint32_t)SG_KC * (uint32_t)n_out * 2u;

  auto issue = [&](int sl, int c) {
    int cr = c + rot;  // the chunk of K that step c covers
    if (cr >= nk) cr -= nk;
    const uint32_t kc = (uint32_t)cr * (SG_KC * 2);
    if constexpr (WT) {
#pragma unroll
      for (int p = 0; p < 2; ++p)
        buf_ld16_lds(wres, boff[p] == kOob ? kOob : boff[p] + (uint32_t)c * wchunk, sW[sl] + (wave * 2 + p) * 1024);
    } else if constexpr (!GB) {
      // rows 8 h + lane / 8 of each subtile, 16-byte piece lane % 8 of the chunk's 128 bytes
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int b = 0; b < NB; ++b) slot[sl][h][b] = buf_ld16_nt(wres, boff[b] + kc + (uint32_t)h * hrow);
    } else {
      // the SwiGLU backward's recompute (whose epilogue needs the registers): the MFMA operand
      // layout loaded directly, rows lane % 16, 16-byte piece 4 s + lane / 16
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int b = 0; b < NB; ++b) slot[sl][s][b] = buf_ld16(wres, boff[b] + kc + s * 64u);
    }
    uint8_t *st = stage(sl);
#pragma unroll
    for (int i = 0; i < NA; ++i) buf_ld16_lds(ares, aoff[i] + kc, st + (i * 64 * NW + wave * 64) * 16);
  };
  f32x4 acc[MS][NB];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[i][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 bw[2][NB];  // row-major weights: this step's B fragments (see to_frags)
  auto compute = [&](int sl) {
    const uint8_t *st = stage(sl);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 a[MS];  // all row fragments of this k step first: one LDS wait per step
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        const int r = i * 16 + (lane & 15);
        const int c = s * 4 + (lane >> 4);
        a[i] = *reinterpret_cast<const u32x4 *>(st + (r * 8 + (c ^ (r & 7))) * 16);
      }
      if constexpr (WT) {
        // B fragment (column lane & 15, k = 32 s + 8 (lane >> 4) .. + 7) from the
        // row-major tile with two LDS transpose reads of four k each (wt_frag_addr)
        const u32x4 b = wt_frag(sW[sl], s, wave, lane);
#pragma unroll
        for (int i = 0; i < MS; ++i) acc[i][0] = mfma16(a[i], b, acc[i][0]);
      } else {
#pragma unroll
        for (int i = 0; i < MS; ++i)
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[i][b] = mfma16(a[i], GB ? slot[sl][s][b] : bw[s][b], acc[i][b]);
      }
    }
  };
  // Whole-line weight pieces -> MFMA B fragments through the wave's LDS region: subtile b
  // is 16 rows x 128 bytes, 16-byte piece c of row r stored at piece c ^ (r & 7) (eight
  // consecutive lanes write one row, or read eight rows at one logical piece, on distinct
  // banks).  Fragment of k step s: column lane % 16 (row of the subtile), k = 32 s +
  // 8 (lane / 16) .. + 7, i.e. piece 4 s + lane / 16.  The wave's LDS operations complete
  // in order, so a region is rewritten only after its earlier reads.
  auto to_frags = [&](int sl) {
    if constexpr (!WT && !GB) {
      uint8_t *wl = sWt + wave * (NB * 2048);
      const int wr = lane >> 3;  // row of the subtile written by this lane, minus 8 h
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int r = 8 * h + wr;
          *reinterpret_cast<u32x4 *>(wl + b * 2048 + r * 128 + (((lane & 7) ^ (r & 7)) << 4)) = slot[sl][h][b];
        }
      const int rr = lane & 15;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          bw[s2][b] = *reinterpret_cast<const u32x4 *>(wl + b * 2048 + rr * 128 +
                                                        ((((4 * s2) + (lane >> 4)) ^ (rr & 7)) << 4));
    }
  };
  auto bar = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: chunks 0 .. S-2 in flight (a chunk past K repeats chunk 0: harmless)
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s, s < nk ? s : 0);
  // Main loop, S chunks per trip, while every chunk it issues lies inside K: the loads
  // of chunk c are complete once at most (S - 2) * LOADS younger ones remain.  Bare
  // barrier: a fenced one would also wait for those younger loads.
  int c0 = 0;
  for (; c0 + 2 * S - 2 < nk; c0 += S) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((S - 2) * LOADS) : "memory");
      bar();
      issue((s + S - 1) % S, c0 + s + S - 1);
      to_frags(s);
      compute(s);
    }
  }
  // the last chunks (fewer than 2S - 1): all own loads complete before each barrier
#pragma unroll
  for (int s = 0; s < 2 * S - 1; ++s) {
    const int c = c0 + s;
    if (c >= nk) break;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    bar();
    if (c + S - 1 < nk) issue((s + S - 1) % S, c + S - 1);
    to_frags(s % S);
    compute(s % S);
  }
  // no LDS write may outlive the block, and the next row block refills the stages
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // epilogue: C layout of the 16x16 MFMA -- column (lane & 15), rows 4*(lane>>4)+j
  if constexpr (GB) {
    // SwiGLU backward from the float G, U of each (row, column) and dH' (bf16): with g
    // the row's gate, dG = g dH' U silu'(G), dU = g dH' silu(G), g H, and the dot dH' . H
    // of the row's 16 columns (the wave's subtile), summed over the 16 lanes in a fixed
    // butterfly order.  Staged through the freed A stages, one wave-private region of
    // BM rows x 32 bytes (the wave's 16 columns) per stage: dH' comes in, and dG, dU and
    // g H go out, as 16-byte row pieces (lane: row lane / 2 + 32 it, half lane % 2).
    // Region 0 holds dH' and then g H (each element read and then overwritten by the
    // same lane), region 1 dG, region 2 dU; a wave's LDS accesses complete in order.
    static_assert(NSUB == 1 && S >= 3, "one 16-column subtile per wave, three stages");
    if (nvalid > 0) {  // wave-uniform; every wave reaches the barrier below
      uint8_t *rg0 = sA0 + wave * BM * 32, *rg1 = sA1 + wave * BM * 32, *rg2 = sA2 + wave * BM * 32;
      const int half = lane & 1, col = lane & 15;
      constexpr int PIECES = (MS * 16 + 31) / 32;  // 16-byte row-piece rounds
#pragma unroll
      for (int it = 0; it < PIECES; ++it) {
        const int q = it * 32 + (lane >> 1);
        if (q < rows)
          *reinterpret_cast<u32x4 *>(rg0 + q * 32 + half * 16) =
              ldg16(gb.dhp + (size_t)(m0 + q) * n_out + ncol0 + half * 8);
      }
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < MS; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = i * 16 + (lane >> 4) * 4 + j;
          const bool ok = r < rows;
          bf16_t *e0 = reinterpret_cast<bf16_t *>(rg0 + r * 32 + col * 2);
          const float z = acc[i][0][j], u = acc[i][1][j], d = bf16_to_f32(*e0);
          const float g = gb.row_gate ? (ok ? gb.row_gate[m0 + r] : 0.0f) : 1.0f;
          const float sg = sigmoid_fast(z);
          const float sz = z * sg;                         // silu(z)
          const float H = sz * u;
          float dot = d * H;
          const float dh = g * d;
          const float dsilu = sg * (1.0f + z * (1.0f - sg));  // silu'(z)
          *reinterpret_cast<bf16_t *>(rg1 + r * 32 + col * 2) = f32_to_bf16(dh * u * dsilu);
          *reinterpret_cast<bf16_t *>(rg2 + r * 32 + col * 2) = f32_to_bf16(dh * sz);
          *e0 = f32_to_bf16(g * H);
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) dot += __shfl_xor(dot, o, 64);
          if (gb.dpart && ok && col == 0) gb.dpart[(size_t)(m0 + r) * (n_out / 16) + ncol0 / 16] = dot;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int it = 0; it < PIECES; ++it) {
        const int q = it * 32 + (lane >> 1);
        if (q < rows) {
          const size_t row = (size_t)(m0 + q);
          const int c = ncol0 + half * 8;
          stg16(out + row * 2 * n_out + c, *reinterpret_cast<const u32x4 *>(rg1 + q * 32 + half * 16));
          stg16(out + row * 2 * n_out + n_out + c, *reinterpret_cast<const u32x4 *>(rg2 + q * 32 + half * 16));
          stg16(gb.hg + row * n_out + c, *reinterpret_cast<const u32x4 *>(rg0 + q * 32 + half * 16));
        }
      }
    }
    // the next row block refills the stages: every wave is done with its region
    __syncthreads();
    return;
  }
  if constexpr (sizeof(OutT) == 2 && NSUB == 1) {
    // bf16 output as whole 16-byte pieces, non-temporal: each wave writes its 16 columns of
    // the block's rows into its 32-byte slice of a [rows][NW x 32 bytes] image in the freed
    // first stage, then the workgroup stores the image row by row, NW x 2 lanes per row.  The
    // stores cost the weight stream far more than their bytes: the DeepSeek-shaped down
    // projection took 1.09 ms with them and 0.94 ms with none; written as full non-temporal
    // pieces, 1.05 ms (and the Switch-shaped gate_up 198 -> 182 us).
    constexpr int RBO = NW * 32;  // bytes of one image row
    constexpr int PPR = RBO / 16;  // 16-byte pieces per row
    if (nvalid > 0) {
#pragma unroll
      for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = i * 16 + (lane >> 4) * 4 + j;
          if (r >= rows) continue;
          float v;
          if constexpr (SWIGLU)
            v = silu_f32(acc[i][0][j]) * acc[i][1][j];
          else
            v = acc[i][0][j];
          *reinterpret_cast<bf16_t *>(sA0 + r * RBO + wave * 32 + (lane & 15) * 2) = f32_to_bf16(v);
        }
    }
    __syncthreads();
    const int col0 = ncol0 - wave * 16;  // the workgroup's first column
    for (int q = tid; q < rows * PPR; q += 64 * NW) {
      const int r = q / PPR, c = q - r * PPR;
      if (col0 + c * 8 < n_out)
        stg16_nt(out + (size_t)(m0 + r) * n_out + col0 + c * 8, *reinterpret_cast<const u32x4 *>(sA0 + r * RBO + c * 16));
    }
    __syncthreads();  // the next row block refills the stages
  } else {
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
          store_out(out + (size_t)(m0 + r) * n_out + col, v);
        }
      }
    }
  }
}

// Tiles are taken in block-id order (expert-major, column tile minor); the hardware
// deals consecutive blocks to the 8 XCDs round-robin, which spreads every expert --
// including the few heavily loaded ones -- over all XCDs.  NW waves per workgroup
// share the staged A rows: wider workgroups load each token row fewer times.
template <int BM, int NSUB, bool SWIGLU, int S, int NW, typename OutT, bool WT = false, bool GB = false>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void grouped_gemm_stream_kernel(const bf16_t *__restrict__ A,
                                                                     const int32_t *__restrict__ row_index,
                                                                     int64_t a_rows,
                                                                     const int32_t *__restrict__ offsets,
                                                                     const bf16_t *__restrict__ W, int64_t wstride,
                                                                     int n_out, int K, OutT *__restrict__ out,
                                                                     int n_tiles, const SwigluBwdOut gb, int tail) {
  constexpr int NB = SWIGLU ? 2 * NSUB : NSUB;  // 16-row weight subtiles per wave
  constexpr int NT = 64 * NW;                     // threads
  constexpr int A_PER_T = (BM * 8 + NT - 1) / NT;  // 16-byte A pieces per thread and chunk
  constexpr int STAGE = sg_stage_bytes<BM, NW>();
  // one LDS array per stage, so that waiting for the loads into one stage never waits
  // for the loads into another
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[STAGE], sA1[STAGE], sA2[STAGE], sA3[S > 3 ? STAGE : 16];
  // K-major weights: one 8 KB weight tile per stage
  constexpr int WSTAGE = WT ? SG_KC * 64 * 2 : 16;
  __shared__ __attribute__((aligned(1024))) uint8_t sW0[WSTAGE], sW1[WSTAGE], sW2[WSTAGE],
      sW3[S > 3 ? WSTAGE : 16];
  uint8_t *const sW[4] = {sW0, sW1, sW2, sW3};
  // row-major weights: each wave's region for turning whole-line pieces into MFMA fragments
  __shared__ __attribute__((aligned(1024))) uint8_t sWt[WT || GB ? 16 : NW * NB * 2048];

  const int tile = blockIdx.x;
  int g = tile / n_tiles;
  const int nt = tile - g * n_tiles;
  if (tail > 0 && gridDim.x <= 64u * (unsigned)n_tiles) {
    // Only the groups whose last partial large tile is a tail (0 < rows mod 256 <= tail)
    // have work: workgroup `tile` takes column tile nt of the (tile / n_tiles)-th of them,
    // so the live workgroups are the first ones dispatched and spread over the CUs.  Mapped
    // to their own groups, they sat among the exiting workgroups of the other groups and
    // shared CUs: the down projection's tails of a Mixtral-shaped layer (five of eight
    // groups) took 139 us that way and 121 us compacted.  The scan reads G + 1 offsets, so
    // it is kept to launches of at most 64 groups.
    const int G = (int)(gridDim.x / (unsigned)n_tiles);
    int want = g;
    g = -1;
    for (int i = 0, lo = offsets[0]; i < G; ++i) {
      const int hi = offsets[i + 1];
      const int r = (hi - lo) % kBigTileRows;
      if (r > 0 && r <= tail && want-- == 0) {
        g = i;
        break;
      }
      lo = hi;
    }
    if (g < 0) return;
  }
  int row_begin = offsets[g];
  const int row_end = offsets[g + 1];
  if (tail > 0) {  // only the rows past the group's last full large tile, when at most `tail`
    const int rem = (row_end - row_begin) % kBigTileRows;
    if (rem > tail) return;
    row_begin = row_end - rem;
  }
  if (row_begin >= row_end) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ncol0 = (nt * NW + wave) * 16 * NSUB;
  const int nvalid = max(0, min(NSUB, (n_out - ncol0) / 16));  // wave-uniform
  const uint32_t kbytes = (uint32_t)K * 2u;
  const rsrc_t wres = make_rsrc(W + (size_t)g * wstride, (uint32_t)(wstride * 2));

  uint32_t boff[NB < 2 ? 2 : NB];
  if constexpr (WT) {
    // this lane's piece of weight-tile instruction q = 2 wave + p at k = 0: k-row
    // 8 q + lane / 8, piece (lane % 8) ^ wt_swz(row), columns nt * 64 + 8 piece .. + 7
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = (wave * 2 + p) * 8 + (lane >> 3);
      const int col = nt * 64 + ((lane & 7) ^ wt_swz(r)) * 8;
      boff[p] = col < n_out ? ((uint32_t)r * (uint32_t)n_out + (uint32_t)col) * 2u : kOob;
    }
  } else {
    // byte offset of this lane's 16 bytes in weight subtile b at k = 0 (rows 0 .. 7 of it)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int sidx = b % NSUB;
      if constexpr (GB) {  // MFMA operand layout: row lane % 16, piece lane / 16
        const int r = ncol0 + sidx * 16 + (lane & 15) + (b >= NSUB ? n_out : 0);
        boff[b] = sidx < nvalid ? (uint32_t)r * kbytes + (uint32_t)(lane >> 4) * 16u : kOob;
      } else {  // whole lines: row lane / 8 (+ 8 h, hrow bytes further), piece lane % 8
        const int r = ncol0 + sidx * 16 + (lane >> 3) + (b >= NSUB ? n_out : 0);
        boff[b] = sidx < nvalid ? (uint32_t)r * kbytes + (uint32_t)(lane & 7) * 16u : kOob;
      }
    }
  }
  const int nk = K / SG_KC;
  // Rows a multiple of 4 KB long (K a multiple of 2048): each workgroup walks the K chunks
  // from its own starting chunk (block id mod the chunk count), wrapping around, so that at
  // any moment the workgroups read different offsets of their rows.  At a common offset,
  // rows that far apart land every concurrent request on the same few memory channels: a
  // plain read of 8 KB rows in this pattern measured 6.1 TB/s in step against 7.1 TB/s
  // rotated (4 KB rows: 6.8 against 7.1).  Other row lengths keep the common order, in which
  // the workgroups of one expert share each chunk of its token rows through L2 (rotating the
  // 14 KB rows of a 7168-wide layer cost its gate_up 4%).  The sum over K runs in the
  // workgroup's order: each output still has one fixed order.
  const int rot = (WT || GB || (kbytes & 4095u)) ? 0 : (int)(blockIdx.x % (unsigned)nk);

  for (int m0 = row_begin; m0 < row_end; m0 += BM) {
    const int rows = min(BM, row_end - m0);
    // A piece q = i * NT + tid lands in LDS at q * 16: row q / 8, stored 16-byte column
    // q % 8, which holds logical column (q % 8) ^ (row % 8).  Its source: that row of the
    // block (gathered from the unpermuted activations through row_index when given).
    uint32_t aoff[A_PER_T];
    rsrc_t ares = row_index ? make_rsrc(A, (uint32_t)(a_rows * kbytes)) : make_rsrc(A + (size_t)m0 * K,
                                                                                     (uint32_t)rows * kbytes);
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int q = tid + NT * i;
      const int r = q >> 3, c = (q & 7) ^ (r & 7);
      uint32_t o = kOob;
      if (r < rows) {
        const uint32_t row = row_index ? (uint32_t)row_index[m0 + r] : (uint32_t)r;
        o = row * kbytes + (uint32_t)c * 16u;
      }
      aoff[i] = o;
    }
    const int na = (rows * 8 + NT - 1) / NT;  // workgroup-uniform
#define SG_BLOCK(N)                                                                                              \
  if constexpr (N <= A_PER_T) {                                                                                  \
    if (na == N) {                                                                                               \
      stream_block<BM, NSUB, SWIGLU, S, NW, N, OutT, WT, GB>(wres, ares, boff, aoff, sA0, sA1, sA2, sA3, sW, sWt,     \
                                                         8u * kbytes, nk, rot, rows,                               \
                                                         m0, ncol0, nvalid, n_out, out, gb);                      \
      continue;                                                                                                  \
    }                                                                                                            \
  }
    SG_BLOCK(1)
    SG_BLOCK(2)
    SG_BLOCK(3)
    SG_BLOCK(4)
#undef SG_BLOCK
  }
}

template <int BM, int NSUB, bool SWIGLU, int S, int NW = 4, typename OutT = bf16_t, bool WT = false, bool GB = false>
hipError_t launch_stream(const GroupedGemmArgs &a, hipStream_t s) {
  const int cols_per_tile = 16 * NW * NSUB;
  const int n_tiles = (a.n_out + cols_per_tile - 1) / cols_per_tile;
  const int64_t grid = (int64_t)a.num_groups * n_tiles;
  const SwigluBwdOut gb{static_cast<const bf16_t *>(a.bwd_dhp), a.bwd_row_gate, static_cast<bf16_t *>(a.bwd_hg),
                        a.bwd_dpart};
  hipLaunchKernelGGL((grouped_gemm_stream_kernel<BM, NSUB, SWIGLU, S, NW, OutT, WT, GB>), dim3((unsigned)grid), dim3(64 * NW), 0, s,
                     static_cast<const bf16_t *>(a.A), a.row_index, a.a_rows, a.offsets,
                     static_cast<const bf16_t *>(a.W), a.w_group_stride, a.n_out, a.K, static_cast<OutT *>(a.out),
                     n_tiles, gb, a.tails_only ? a.tail : 0);
  return hipGetLastError();
}

// K-major weights (no SwiGLU, bf16 output): weight tiles share LDS with the A stages, so
// 128-row blocks take three stages to keep two workgroups per CU.
hipError_t launch_stream_kn(const GroupedGemmArgs &a, hipStream_t s) {
  if (a.n_out % 64) return hipErrorInvalidValue;  // whole 64-column weight tiles
  const int r = a.group_rows_max;
  if (r <= 16) return launch_stream<16, 1, false, 4, 4, bf16_t, true>(a, s);
  if (r <= 32) return launch_stream<32, 1, false, 4, 4, bf16_t, true>(a, s);
  if (r <= 64) return launch_stream<64, 1, false, 4, 4, bf16_t, true>(a, s);
  return launch_stream<128, 1, false, 3, 4, bf16_t, true>(a, s);
}

template <bool SWIGLU, typename OutT = bf16_t, bool GB = false>
hipError_t launch_stream_bm(const GroupedGemmArgs &a, hipStream_t s) {
  // three stages for gate_up (two weight subtiles per wave keep enough bytes in flight),
  // four for down (one subtile per wave: a deeper pipeline instead)
  constexpr int S = SWIGLU ? 3 : 4;
  const int r = a.group_rows_max;
  if (r <= 16) return launch_stream<16, 1, SWIGLU, S, 4, OutT, false, GB>(a, s);
  if (r <= 32) return launch_stream<32, 1, SWIGLU, S, 4, OutT, false, GB>(a, s);
  if (r <= 64) return launch_stream<64, 1, SWIGLU, S, 4, OutT, false, GB>(a, s);
  return launch_stream<128, 1, SWIGLU, S, 4, OutT, false, GB>(a, s);
}

}  // namespace

hipError_t launch_grouped_gemm_stream_bf16(const GroupedGemmArgs &a, hipStream_t s) {
  if (a.a_packed || a.out_packed) return hipErrorInvalidValue;  // a layout of the large-tile kernel
  if (a.w_kn) return (a.swiglu || a.out_f32) ? hipErrorInvalidValue : launch_stream_kn(a, s);
  if (a.bwd_dhp) return a.swiglu && !a.out_f32 ? launch_stream_bm<true, bf16_t, true>(a, s) : hipErrorInvalidValue;
  if (a.swiglu) return launch_stream_bm<true>(a, s);
  return a.out_f32 ? launch_stream_bm<false, float>(a, s) : launch_stream_bm<false>(a, s);
}

// Regime choice: the streaming kernel when groups hold few rows on average (each
// weight byte feeds few MFMAs, HBM bound), the 256 x 256 tile kernel when they hold
// many (MFMA bound).  The row bounds are the caller's; either kernel computes any
// group size correctly.
bool grouped_gemm_big_regime(int64_t rows_max, int num_groups, int group_rows_max) {
  return num_groups > 0 && rows_max / num_groups >= 256 && group_rows_max >= 256;
}

hipError_t launch_grouped_gemm_bf16(const GroupedGemmArgs &a, hipStream_t s) {
  if (grouped_gemm_big_regime(a.rows_max, a.num_groups, a.group_rows_max))
    return launch_grouped_gemm_big_bf16(a, a.rows_max, s);
  return launch_grouped_gemm_stream_bf16(a, s);
}

}  // namespace moe
