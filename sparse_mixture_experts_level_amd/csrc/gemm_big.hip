// Grouped expert GEMM for experts with many rows (compute bound), bf16 on gfx950.
//
// Same problem as the weight-streaming kernel -- per group, its rows of A times the
// group's weight rows, SwiGLU fused for the gate/up projection -- but sized for
// groups of hundreds to thousands of rows, where the contraction is dense enough to
// be bound by the matrix cores ("Что такое Mixture of Experts (MoE) в
// трансформерах", aglamov.biz, section "Бэкенд для экспертов": one grouped GEMM over
// tokens sorted by expert).
//
// Block tile: 256 rows x 256 weight rows.  Eight wavefronts (two per SIMD) in a
// 2 x 4 arrangement each own 128 x 64 of the tile as 4 x 2 blocks of the 32x32x16
// bf16 MFMA.  For SwiGLU the 256 weight rows are 128 gate rows and the 128 matching
// up rows, and each wave owns 32 output columns of both, so gate and up
// accumulators of a column sit in the same lane.
//
// Tiles: each group contributes ceil(rows / 256) row tiles times the column tiles.
// A block finds its group from the offsets (one wavefront scan).  When the group's
// weights are the larger operand, its tiles are walked weight tile outermost, so the row
// tiles that share a weight tile run together and reuse it from cache; otherwise in bands
// of four row tiles, weight tile outer within a band.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int BG_BM = kBigTileRows, BG_BN = 256;
constexpr int PR_STEPS = 4;  // K steps one row-packing workgroup copies

// Pipeline: K advances in steps of 32.  Operand tiles go from HBM straight into LDS
// (buffer loads with an LDS destination, no registers), into four stages that are
// separate LDS arrays, three steps ahead of the MFMAs (schedule at the main loop).
//
// LDS tile layout: 256 rows of 64 bytes (4 chunks of 16 bytes); chunk c of row r is
// stored at chunk c ^ ((r >> 2) & 3).  An MFMA operand load reads one chunk of 32
// consecutive rows; LDS serves 16 lanes (256 bytes, 64 banks) at a time, and any 16
// consecutive rows then fall on 16 distinct 16-byte bank groups.  One load instruction fills 1 KB = 16 rows; lane p of it
// brings row 16 * blk + p / 4, stored chunk p % 4.

// K splits for a launch with `tiles` output tiles and `steps` 32-wide K steps, for
// launches of fewer tiles than CUs: the split count (at most 4, at least 64 steps per
// split) whose blocks fill the 256 CUs' last round best, the larger one on a tie.
// Evaluated identically by the GEMM and by the reduction that adds the splits.
__host__ __device__ __forceinline__ int big_ksplit(int tiles, int steps, int min_steps = 64) {
  if (tiles <= 0 || tiles >= 256) return 1;
  int best = 1;
  float best_fill = 0.f;
  for (int s = 1; s <= 4; ++s) {
    if (s > 1 && steps / s < min_steps) break;
    const int blocks = tiles * s;
    const float fill = (float)blocks / (float)(((blocks + 255) / 256) * 256);
    if (fill >= best_fill) {
      best_fill = fill;
      best = s;
    }
  }
  return best;
}

// The router linear on this kernel (one group of M rows, no offsets array): splits of at
// least this many 32-wide steps; the router's top-k kernel adds the float partials.
constexpr int kRouterMinSteps = 32;

// Sum of the K splits' float partials in order, rounded to bf16, for the rows below
// offsets[G]; nothing to do when the launch was not split.
__global__ __launch_bounds__(256) void big_split_reduce_kernel(const float *__restrict__ part, int64_t stride,
                                                               const int32_t *__restrict__ offsets, int G,
                                                               int n_tiles, int steps, int n_out,
                                                               bf16_t *__restrict__ out, int tail) {
  const int tiles = __builtin_amdgcn_readfirstlane(total_row_blocks<BG_BM>(offsets, G, tail)) * n_tiles;
  const int ks = big_ksplit(tiles, steps);
  if (ks == 1) return;
  const int64_t rows = offsets[G];
  const int64_t n8 = rows * n_out / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < ks; ++s) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(part + s * stride + i * 8);
      const f32x4 b = *reinterpret_cast<const f32x4 *>(part + s * stride + i * 8 + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[q] += a[q];
        acc[4 + q] += b[q];
      }
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    stg16(out + i * 8, o);
  }
}

// WG: the weight-gradient form, grouped over the contraction instead of the rows: with
// K_g = offsets[g+1] - offsets[g] (a multiple of 32),
//   out[g][m][n] = sum over k < K_g of A_g[m][k] * W[offsets_b[g] + k][n],
// A_g = A + offsets[g] * M, K-contiguous with row stride K_g (group-major transposed
// activations, zero padded; lda bounds the buffer), and W [ldb rows, n_out] K-major (BKN;
// rows past offsets_b[g+1] read zeros); every group M x n_out, written at out + g * M * n_out.
// APK: A is in the packed tile layout (pack_rows_kernel); OPK: the SwiGLU output is
// written in that layout, for a following large-tile GEMM over the same groups.  BPK: the
// weights are in their packed tile layout (pack_weights_kernel; wstride is the packed
// group's size in elements).
template <bool SWIGLU, typename OutT = bf16_t, bool WG = false, bool BKN = false, bool APK = false, bool OPK = false,
          bool GB = false, bool TO = false, bool BPK = false>
__global__ __launch_bounds__(512, 1) void grouped_gemm_big_kernel(const bf16_t *__restrict__ A,
                                                                         const int32_t *__restrict__ row_index,
                                                                         int64_t a_rows,
                                                                         const int32_t *__restrict__ offsets, int G,
                                                                         const bf16_t *__restrict__ W,
                                                                         int64_t wstride, int n_out, int K,
                                                                         OutT *__restrict__ out, int n_tiles,
                                                                         int64_t lda, int64_t ldb, int M,
                                                                         float *__restrict__ split_out,
                                                                         int64_t split_stride,
                                                                         const int32_t *__restrict__ offsets_b,
                                                                         const SwigluBwdOut gb, int tail) {
  // Eight waves (two per SIMD) in a 2 x 4 arrangement, each 128 rows x 64 weight rows.
  constexpr int WN_W = 4;                        // waves along the weight rows
  constexpr int NBUF = 4;                        // LDS stages
  constexpr int BK = 32;                         // K per step
  constexpr int RB = BK * 2;                     // bytes per tile row
  constexpr int NCH = RB / 16;                   // 16-byte chunks per tile row
  constexpr int RPI = 1024 / RB;                 // tile rows per 1 KB load instruction
  constexpr int NW = 8;                          // waves
  constexpr int NI = BG_BN / WN_W / 32;          // 32-wide weight blocks per wave
  constexpr int TILE = BG_BM * BK * 2;           // 16 KB per operand and stage
  constexpr int IPW = TILE / 1024 / NW;          // 1 KB load instructions per wave, operand and stage
  static_assert(!BKN || !SWIGLU, "K-major operands: plain store");
  static_assert(!(APK || OPK) || !WG, "packed operands: the forward form");
  static_assert(!OPK || SWIGLU, "packed output: the SwiGLU projection");
  static_assert(!GB || (SWIGLU && !WG && !APK && !OPK && sizeof(OutT) == 2),
                "SwiGLU backward: the forward form's gate and up blocks, bf16 gradients");
  static_assert(!TO || (WG && sizeof(OutT) == 2), "transposed output: the weight-gradient form, bf16");
  static_assert(!BPK || (!WG && !BKN), "packed weights: the forward form's row-major weights");
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[TILE], sA1[TILE], sA2[TILE], sA3[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[TILE], sB1[TILE], sB2[TILE], sB3[TILE];
  auto bufA = [&](int b) -> uint8_t * { return b == 0 ? sA0 : b == 1 ? sA1 : b == 2 ? sA2 : sA3; };
  auto bufB = [&](int b) -> uint8_t * { return b == 0 ? sB0 : b == 1 ? sB1 : b == 2 ? sB2 : sB3; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN_W, wn = wave % WN_W;
  // Swizzle of a row's 16-byte chunks (64-byte rows): chunk c of row r at
  // c ^ ((r >> 2) & 3), so 16 consecutive rows read at one logical chunk land on 16
  // distinct 16-byte bank groups of a 256-byte LDS cycle, and rows 32 apart keep the
  // same swizzle.
  auto swz = [&](int r) -> int { return (r >> 2) & 3; };
  // This lane's global offsets (k = 0) for its IPW instructions per operand.
  uint32_t agoff[IPW], bgoff[IPW];
  int krow[IPW];  // WG with K-major operands: this lane's k-row within a step, per instruction
  int m0, rows, n0, nk, ks = 0, kbase = 0, kvalid = 0, m_tile = 0, n_tile = 0;
  bool partial = false;
  rsrc_t ares, wres;
  OutT *obase;
  int64_t ostride;
  if constexpr (!WG) {
    // The grid is sized from a bound on the rows; blocks past the real tile count leave,
    // and the real tiles are spread over the XCDs by the remap over their own count (a
    // remap over the whole grid would crowd them onto the first XCDs when the bound is
    // loose).
    // With split_out, few tiles are cut along K as well (big_ksplit()): split ks writes
    // its float partial sums to split_out + ks * split_stride, and a reduction adds them.
    // Tiles of at most `tail` rows (a group's last partial tile) are left to a streaming
    // launch: they do not exist here.
    // Without an offsets array (the router linear): one group of rows [0, M).
    const bool one = offsets == nullptr;
    const int tiles =
        (one ? (M + BG_BM - 1) / BG_BM : __builtin_amdgcn_readfirstlane(total_row_blocks<BG_BM>(offsets, G, tail))) *
        n_tiles;
    const int ksplit = split_out ? big_ksplit(tiles, K / BK, one ? kRouterMinSteps : 64) : 1;
    const int real_blocks = tiles * ksplit;
    if ((int)blockIdx.x >= real_blocks) return;
    const int lin0 = xcd_remap(blockIdx.x, real_blocks);
    ks = lin0 / tiles;
    const int lin = lin0 - ks * tiles;
    const int m_lin = lin / n_tiles;  // rank of this block's tile among all groups' m tiles
    int g, mt_first, mt_count;
    // Blocks are numbered group-major: the tiles of group g occupy [mt_first * n_tiles,
    // (mt_first + mt_count) * n_tiles).  Within a group the order is chosen below.
    if (one) {
      g = 0;
      mt_first = 0;
      mt_count = (M + BG_BM - 1) / BG_BM;
    } else {
      find_row_block<BG_BM>(offsets, G, m_lin, g, mt_first, mt_count, tail);
    }
    // the scan's results are equal in every lane: keep them (and all that derives from
    // them, like the buffer resources) in scalar registers
    g = __builtin_amdgcn_readfirstlane(g);
    mt_first = __builtin_amdgcn_readfirstlane(mt_first);
    mt_count = __builtin_amdgcn_readfirstlane(mt_count);
    if (g < 0) return;
    const int local = lin - mt_first * n_tiles;  // 0 .. mt_count * n_tiles - 1
    const int row_begin = one ? 0 : offsets[g], row_end = one ? M : offsets[g + 1];
    const int64_t a_bytes = (int64_t)(row_end - row_begin) * K;
    const int64_t b_bytes = (int64_t)(SWIGLU ? 2 : 1) * n_out * K;
    int mt, nt;
    if (a_bytes <= b_bytes) {  // weights larger: weight tile outermost, row tiles reuse it
      nt = local / mt_count;
      mt = local - nt * mt_count;
    } else {
      // activations larger (the shared expert: every token one group): bands of four row
      // tiles, weight tile outer within a band, so the 32 tiles an XCD runs at once hold
      // four row tiles and eight weight tiles rather than two and sixteen, fewer operand
      // bytes past its L2 (DeepSeek-shaped shared expert: 760 + 404 -> 745 + 386 us)
      constexpr int BAND = 4;
      const int band = local / (BAND * n_tiles), r = local - band * BAND * n_tiles;
      const int bm = min(BAND, mt_count - band * BAND);  // row tiles in this band
      nt = r / bm;
      mt = band * BAND + (r - nt * bm);
    }
    m0 = row_begin + mt * BG_BM;
    rows = min(BG_BM, row_end - m0);
    m_tile = mt_first + mt;  // rank of this row tile among all groups' row tiles
    n0 = nt * (SWIGLU ? BG_BN / 2 : BG_BN);  // first output column of the tile
    n_tile = nt;
    const uint32_t kbytes = (uint32_t)K * 2u;
    // A rows: contiguous from m0, or gathered from the unpermuted activations by row_index
    if constexpr (APK)  // the tiles' K steps are 16 KB blocks, a_rows bounds the buffer in bytes
      ares = make_rsrc(A, (uint32_t)a_rows);
    else
      ares = row_index ? make_rsrc(A, (uint32_t)(a_rows * kbytes)) : make_rsrc(A + (size_t)m0 * K, (uint32_t)rows * kbytes);
    wres = make_rsrc(W + (size_t)g * wstride, (uint32_t)(wstride * 2));
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int blk = wave * IPW + i;
      const int r = blk * RPI + lane / NCH;
      const int c = (lane % NCH) ^ swz(r);
      if (APK)  // a stage image: instruction blk copies bytes blk * 1 KB .. + 1 KB of the block
        agoff[i] = (uint32_t)blk * 1024u + (uint32_t)lane * 16u;
      else if (row_index)
        agoff[i] = r < rows ? (uint32_t)row_index[m0 + r] * kbytes + (uint32_t)c * 16u : kOob;
      else
        agoff[i] = (uint32_t)r * kbytes + (uint32_t)c * 16u;
      if constexpr (BPK) {
        // packed weights: a stage image, like the packed A
        bgoff[i] = (uint32_t)blk * 1024u + (uint32_t)lane * 16u;
      } else if constexpr (BKN) {
        // K-major weights [K, n_out]: instruction blk brings k-rows 2 blk and 2 blk + 1 of
        // the step, 512 bytes (256 columns) each; lane p of a row stores the row's chunk
        // p ^ (4 (row & 3)) at slot p
        const int kr = 2 * blk + (lane >> 5);
        const int col = n0 + (((lane & 31) ^ (4 * (kr & 3))) << 3);
        bgoff[i] = col < n_out ? ((uint32_t)kr * (uint32_t)n_out + (uint32_t)col) * 2u : kOob;
      } else {
        int wr;  // weight row held in tile row r, -1 past n_out
        if (SWIGLU) {
          const int col = n0 + (r & 127);
          wr = col < n_out ? (r < 128 ? col : n_out + col) : -1;
        } else {
          wr = n0 + r < n_out ? n0 + r : -1;
        }
        bgoff[i] = wr >= 0 ? (uint32_t)wr * kbytes + (uint32_t)c * 16u : kOob;
      }
    }
    const int steps = K / BK, sps = (steps + ksplit - 1) / ksplit;
    kbase = ks * sps;
    nk = max(0, min(sps, steps - kbase));
    partial = ksplit > 1;
    obase = out;
    ostride = n_out;
  } else {
    // With split_out (one group, float), K is the number of K slices: slice ks writes its
    // float partial sums to split_out + ks * split_stride, and a reduction adds them.
    const int m_tiles = (M + BG_BM - 1) / BG_BM;
    const int per_g = m_tiles * n_tiles;
    const int ksplit = split_out ? max(1, K) : 1;
    const int real_blocks = G * per_g * ksplit;
    if ((int)blockIdx.x >= real_blocks) return;
    const int lin0 = xcd_remap(blockIdx.x, real_blocks);
    ks = lin0 / (G * per_g);
    const int lin = lin0 - ks * (G * per_g);
    const int g = lin / per_g, local = lin - g * per_g;
    int mt, nt;
    if (M <= n_out) {  // the B operand larger: its tile outermost
      nt = local / m_tiles;
      mt = local - nt * m_tiles;
    } else {
      mt = local / n_tiles;
      nt = local - mt * n_tiles;
    }
    m0 = mt * BG_BM;
    rows = min(BG_BM, M - m0);
    n0 = nt * BG_BN;
    const int kb = offsets[g];
    const int64_t kg = offsets[g + 1] - kb;
    static_assert(BKN, "the weight-gradient form reads its second operand K-major");
    // A transposed (group g's [M, K_g] block at offsets[g] * M, K_g a multiple of 32, zero
    // padding); W K-major: [ldb rows, n_out] row-major with group g's k-rows
    // offsets_b[g] .. offsets_b[g+1] - 1 (unpadded; k-rows past them read zeros).
    // Instruction blk of W brings k-rows 2 blk and 2 blk + 1 of the step (512 bytes
    // each), chunk p of a row at slot p ^ (4 (row & 3)), as the forward mode's W.
    const int steps = (int)(kg / BK), sps = (steps + ksplit - 1) / ksplit;
    kbase = ks * sps;
    nk = max(0, min(sps, steps - kbase));
    partial = ksplit > 1;
    const int kbb = offsets_b[g];
    kvalid = offsets_b[g + 1] - kbb;
    ares = make_rsrc(A, (uint32_t)(M * lda * 2));
    wres = make_rsrc(W, (uint32_t)(ldb * n_out * 2));
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int blk = wave * IPW + i;
      const int r = blk * RPI + lane / NCH;
      const int c = (lane % NCH) ^ swz(r);
      agoff[i] = r < rows ? (uint32_t)(((int64_t)kb * M + (int64_t)(m0 + r) * kg) * 2) + (uint32_t)c * 16u : kOob;
      const int kr = 2 * blk + (lane >> 5);
      const int cs = ((lane & 31) ^ (4 * (kr & 3))) << 3;
      krow[i] = kr;
      bgoff[i] = n0 + cs < n_out ? ((uint32_t)(kbb + kr) * (uint32_t)n_out + (uint32_t)(n0 + cs)) * 2u : kOob;
    }
    obase = out + (size_t)g * M * n_out;
    ostride = n_out;
  }
  auto issue = [&](int kt, int b) {  // loads of step kt into stage b; steps past K read zeros
    const bool ok = kt < nk;
    const uint32_t kc = (uint32_t)(kbase + kt) * (BK * 2);
    // K-major operands advance BK rows per step; packed weights: block (n_tile, step)
    const uint32_t kcb = BKN ? (uint32_t)(kbase + kt) * (uint32_t)BK * (uint32_t)n_out * 2u
                       : BPK ? ((uint32_t)n_tile * (uint32_t)(K / BK) + (uint32_t)(kbase + kt)) * (uint32_t)TILE
                             : kc;
    // packed A: block (m_tile, step) of the tile-major layout
    const uint32_t kca = APK ? ((uint32_t)m_tile * (uint32_t)(K / BK) + (uint32_t)(kbase + kt)) * (uint32_t)TILE : kc;
    uint8_t *la = bufA(b), *lb = bufB(b);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int blk = wave * IPW + i;
      bool okb = ok;
      if constexpr (BKN && WG) okb = ok && (kbase + kt) * BK + krow[i] < kvalid;  // k-rows past the group: zeros
      buf_ld16_lds(ares, (ok && agoff[i] != kOob) ? agoff[i] + kca : kOob, la + blk * 1024);
      buf_ld16_lds(wres, (okb && bgoff[i] != kOob) ? bgoff[i] + kcb : kOob, lb + blk * 1024);
    }
  };
  // K-major weights: the 32x32x16 MFMA fragment of weight block j (columns nb .. nb + 31 of
  // the tile, k = 16 kk + 8 (lane >> 5) .. + 7 for column nb + (lane & 31)) from the
  // [32 k-rows][256 columns] stage, with two LDS transpose reads of four k each.  In a
  // 16-lane group lane 4a + c receives element c of the 8-byte chunks addressed by lanes
  // a, a + 4, a + 8, a + 12; so lane s of group G addresses k-row k0 + s / 4 and columns
  // nb + 16 (G & 1) + 4 (s % 4) .. + 3, with k0 = 16 kk + 8 (G >> 1) (+ 4 for the second).
  auto kn_frag = [&](const uint8_t *lb, int kk, int nb) -> u32x4 {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int G = lane >> 4, sl = lane & 15;
    const int col = nb + (G & 1) * 16 + 4 * (sl & 3);
    u32x4 out;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r = kk * 16 + (G >> 1) * 8 + 4 * t + (sl >> 2);
      const uint8_t *p = lb + r * 512 + (((col >> 3) ^ (4 * (r & 3))) << 4) + (col & 7) * 2;
      const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)p);
      out[2 * t] = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
      out[2 * t + 1] = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
    }
    return out;
  };

  f32x16 acc[4][NI];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x16{};

  // LDS byte offset of this lane's operand row for MFMA block 0 and chunk c; block i
  // is 32 rows further (same swizzle), a constant distance.
  const int ar0 = wm * 128 + (lane & 31);
  const int br0 = SWIGLU ? wn * (NI / 2) * 32 + (lane & 31) : wn * NI * 32 + (lane & 31);
  auto roff = [&](int r, int c) -> int { return r * RB + ((c ^ swz(r)) << 4); };
  {
    // Ping-pong: the two waves of each SIMD (group 0 = waves 0..3, group 1 = waves
    // 4..7) alternate between a memory phase -- issue the loads of step k + 3, wait
    // for this wave's loads of step k + 1, read step k's operand fragments from LDS --
    // and a compute phase -- the step's MFMAs, at raised priority.  Group 1 runs one
    // barrier behind group 0, so while one group computes the other feeds.
    //   Loads of step k land before any wave reads them: each wave completes its own
    //   loads of step k + 1 in mem(k), before the barrier that precedes every read of
    //   step k + 1.  A stage is refilled (step k + 3 in mem(k)) only after the barrier
    //   that follows both groups' reads of its previous step k - 1.
    // Prefetch distance D = NBUF - 1 steps; a wave in mem(k) issues step k + D and
    // completes its own loads of step k + 1 (at most D - 1 younger steps in flight).
    constexpr int D = NBUF - 1;
    static_assert(IPW == 2 && D == 3, "the waits below count two loads per operand and step, three steps ahead");
    const bool second = wave >= 4;
    u32x4 af[BK / 16][4], bfr[BK / 16][NI];
    auto wait_next = [&]() {
      // the two younger steps' loads (2 operands x 2 instructions each) may stay in flight
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    };
    auto mem = [&](int kt, int b) {
      issue(kt + D, (b + D) % NBUF);
      wait_next();  // this wave's loads of step kt + 1 done
      const uint8_t *la = bufA(b), *lb = bufB(b);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int c = kk * 2 + (lane >> 5);
        const uint8_t *pa = la + roff(ar0, c);
        const uint8_t *pb = lb + roff(br0, c);
#pragma unroll
        for (int i = 0; i < 4; ++i) af[kk][i] = *reinterpret_cast<const u32x4 *>(pa + i * 32 * RB);
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          if constexpr (BKN) {
            bfr[kk][j] = kn_frag(lb, kk, wn * NI * 32 + j * 32);
          } else {
            const int dr = SWIGLU ? (j < NI / 2 ? j * 32 : 128 + (j - NI / 2) * 32) : j * 32;
            bfr[kk][j] = *reinterpret_cast<const u32x4 *>(pb + dr * RB);
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };
    auto comp = [&]() {
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            if constexpr (TO)  // A first: a lane's accumulator holds four consecutive rows
              acc[i][j] = mfma32(af[kk][i], bfr[kk][j], acc[i][j]);
            else
              acc[i][j] = mfma32(bfr[kk][j], af[kk][i], acc[i][j]);
          }
      __builtin_amdgcn_s_setprio(0);
    };
    auto bar = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // prologue: steps 0 .. D-1 issued; step 0 landed for every wave before the first read
#pragma unroll
    for (int b = 0; b < D; ++b) issue(b, b);
    wait_next();
    bar();
    if (second) bar();
    // Whole trips of NBUF steps, then the rest: with an exit inside the trip the compiler
    // lost track, at the loop head, of which stage each in-flight load fills, and waited
    // there for all but the newest step's loads before the first fragment read.
    int k0 = 0;
    for (; k0 + NBUF <= nk; k0 += NBUF) {
#pragma unroll
      for (int b = 0; b < NBUF; ++b) {
        mem(k0 + b, b);
        bar();
        comp();
        bar();
      }
    }
#pragma unroll
    for (int b = 0; b < NBUF - 1; ++b) {
      if (k0 + b >= nk) break;
      mem(k0 + b, b);
      bar();
      comp();
      bar();
    }
    if (!second) bar();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS write may outlive the block
  // every wave's loads have landed and its LDS reads are done: the stages are free
  __syncthreads();

  // Epilogue through LDS.  The weight fragment is the MFMA's first operand, so the
  // 32x32 accumulator of block (i, j) holds, in lane l, tile row i * 32 + (l & 31) and
  // the four consecutive columns j * 32 + 8 * (r / 4) + 4 * (l / 32) + (r % 4), r % 4 =
  // 0..3.  Each wave stages its 128-row part of the tile in its own 16 KB stage array,
  // then stores whole 16-byte column runs, 8 .. 16 lanes per row.
  static_assert(WN_W == 4 && NBUF * TILE >= 4 * 16384, "the epilogue needs 16 KB per wave in the stages");
  // wave w's 16 KB: the w-th 16 KB of the A stages (waves 0-3) or of the B stages (4-7)
  constexpr int PER = TILE / 16384;  // 16 KB regions per stage array
  uint8_t *stage = (wave < 4 ? bufA((wave & 3) / PER) : bufB((wave & 3) / PER)) + ((wave & 3) % PER) * 16384;
  const int lr = lane & 31, lh = lane >> 5;
  if constexpr (GB) {
    // SwiGLU backward from the float G (acc[i][0]) and U (acc[i][1]) of each (row,
    // column): lane l holds row wm * 128 + i * 32 + (l & 31) and, per q = 0..3, the four
    // consecutive columns n0 + wn * 32 + 8 q + 4 (l / 32) .. + 3.  With g the row's gate:
    // dG = g dH' U silu'(G), dU = g dH' silu(G), g H, and the dot dH' . H over each
    // 16-column block (q = 0, 1 and q = 2, 3), added over the lane's eight values in order
    // and then with lane l ^ 32's.  The wave's 128 rows x 32 columns move through its
    // 16 KB of LDS as two 8 KB halves laid out as the forward's H stage (64-byte rows,
    // 16-byte chunk c of row r at c ^ ((r >> 2) & 3)), in and out as 16-byte runs: dH'
    // in to half 0; dU back into half 0 (each 8 bytes read and then overwritten by the
    // same lane) and dG into half 1; both out; then g H, formed again from the registers,
    // into half 0 and out.  A wave's LDS accesses complete in order.
    const int cw = n0 + wn * 32;  // the wave's first column
    uint8_t *h0 = stage, *h1 = stage + 8192;
    auto lds_at = [&](int row, int q) { return row * 64 + ((q ^ ((row >> 2) & 3)) << 4) + lh * 8; };
    // 16-byte run it of the wave's block: row it * 16 + lane / 4, chunk lane % 4
    auto run_row = [&](int it) { return it * 16 + (lane >> 2); };
    auto run_lds = [&](int it) {
      const int row = run_row(it), c = lane & 3;
      return row * 64 + ((c ^ ((row >> 2) & 3)) << 4);
    };
    if (cw < n_out) {  // wave-uniform: whole 32-column blocks (n_out a multiple of 32)
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int rl = wm * 128 + run_row(it);
        if (rl < rows)
          *reinterpret_cast<u32x4 *>(h0 + run_lds(it)) =
              ldg16(gb.dhp + (size_t)(m0 + rl) * n_out + cw + (lane & 3) * 8);
      }
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_wave_barrier();
      float gr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = wm * 128 + i * 32 + lr;
        const bool ok = rl < rows;
        gr[i] = gb.row_gate ? (ok ? gb.row_gate[m0 + rl] : 0.0f) : 1.0f;
        float dot[2] = {0.0f, 0.0f};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int at = lds_at(i * 32 + lr, q);
          const uint2 dv = *reinterpret_cast<const uint2 *>(h0 + at);
          float rg[4], ru[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float z = acc[i][0][4 * q + e], u = acc[i][1][4 * q + e];
            const float d = bf16_to_f32(bf16_t((e < 2 ? dv.x : dv.y) >> (16 * (e & 1))));
            const float sg = sigmoid_fast(z);
            const float sz = z * sg;  // silu(z)
            dot[q >> 1] += d * (sz * u);
            const float dh = gr[i] * d;
            rg[e] = dh * u * (sg * (1.0f + z * (1.0f - sg)));  // silu'(z)
            ru[e] = dh * sz;
          }
          *reinterpret_cast<uint2 *>(h1 + at) = uint2{pack_bf16x2(rg[0], rg[1]), pack_bf16x2(rg[2], rg[3])};
          *reinterpret_cast<uint2 *>(h0 + at) = uint2{pack_bf16x2(ru[0], ru[1]), pack_bf16x2(ru[2], ru[3])};
        }
        // lane l's blocks hold columns 8 q + 4 (l / 32): lane l and l ^ 32 together cover them
        const float d0 = dot[0] + __shfl_xor(dot[0], 32, 64), d1 = dot[1] + __shfl_xor(dot[1], 32, 64);
        if (gb.dpart && ok && lh == 0)
          *reinterpret_cast<float2 *>(gb.dpart + (size_t)(m0 + rl) * (n_out / 16) + cw / 16) = float2{d0, d1};
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int rl = wm * 128 + run_row(it);
        if (rl < rows) {
          bf16_t *o = out + (size_t)(m0 + rl) * 2 * n_out + cw + (lane & 3) * 8;
          stg16(o, *reinterpret_cast<const u32x4 *>(h1 + run_lds(it)));
          stg16(o + n_out, *reinterpret_cast<const u32x4 *>(h0 + run_lds(it)));
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // half 0 read out before g H overwrites it
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float rh[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float z = acc[i][0][4 * q + e], u = acc[i][1][4 * q + e];
            rh[e] = gr[i] * (z * sigmoid_fast(z) * u);
          }
          *reinterpret_cast<uint2 *>(h0 + lds_at(i * 32 + lr, q)) =
              uint2{pack_bf16x2(rh[0], rh[1]), pack_bf16x2(rh[2], rh[3])};
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int rl = wm * 128 + run_row(it);
        if (rl < rows)
          stg16(gb.hg + (size_t)(m0 + rl) * n_out + cw + (lane & 3) * 8,
                *reinterpret_cast<const u32x4 *>(h0 + run_lds(it)));
      }
    }
    return;
  }
  if constexpr (SWIGLU) {
    static_assert(sizeof(OutT) == 2 && NI == 2, "SwiGLU: bf16 output, one gate and one up block per wave");
    // 128 rows x 32 columns of H, 64-byte rows; 16-byte chunk c of row r at c ^ ((r >> 2) & 3)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = i * 32 + lr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint2 v;
        v.x = pack_bf16x2(silu_f32(acc[i][0][4 * q]) * acc[i][1][4 * q],
                          silu_f32(acc[i][0][4 * q + 1]) * acc[i][1][4 * q + 1]);
        v.y = pack_bf16x2(silu_f32(acc[i][0][4 * q + 2]) * acc[i][1][4 * q + 2],
                          silu_f32(acc[i][0][4 * q + 3]) * acc[i][1][4 * q + 3]);
        *reinterpret_cast<uint2 *>(stage + row * 64 + ((q ^ ((row >> 2) & 3)) << 4) + lh * 8) = v;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if constexpr (OPK) {
      // The staged 128 x 32 is exactly one half (rows wm * 128 ..) of block (m_tile, k step
      // (n0 + wn * 32) / 32) of H in the packed layout -- 64-byte rows, chunk c of tile row
      // R at c ^ ((R >> 2) & 3), as a stage of the GEMM that reads H -- so it is copied out
      // whole; rows past the group hold zeros (their A rows read zeros).
      if (n0 + wn * 32 < n_out) {
        bf16_t *blkp = obase + ((size_t)m_tile * (n_out / 32) + (n0 + wn * 32) / 32) * (TILE / 2) + wm * (TILE / 4);
#pragma unroll
        for (int it = 0; it < 8; ++it)
          stg16(blkp + (it * 64 + lane) * 8, *reinterpret_cast<const u32x4 *>(stage + (it * 64 + lane) * 16));
      }
    } else {
      const int gcol = n0 + wn * 32 + (lane & 3) * 8;
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int row = it * 16 + (lane >> 2);
        const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + row * 64 + (((lane & 3) ^ ((row >> 2) & 3)) << 4));
        const int grow = wm * 128 + row;
        if (grow < rows && gcol < n_out) stg16(obase + (size_t)(m0 + grow) * ostride + gcol, v);
      }
    }
  } else {
    const int gcol0 = n0 + wn * 64;
    if (partial || sizeof(OutT) == 4) {
      // float: two passes of 64 rows x 64 columns, 256-byte rows; chunk c of row r at c ^ (r & 15)
      float *fbase = partial ? split_out + (size_t)ks * split_stride : reinterpret_cast<float *>(obase);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int row = ii * 32 + lr;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c = j * 8 + q * 2 + lh;
              const f32x4 v = {acc[2 * p + ii][j][4 * q], acc[2 * p + ii][j][4 * q + 1], acc[2 * p + ii][j][4 * q + 2],
                               acc[2 * p + ii][j][4 * q + 3]};
              *reinterpret_cast<f32x4 *>(stage + row * 256 + ((c ^ (row & 15)) << 4)) = v;
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int c = lane & 15, gcol = gcol0 + c * 4;
#pragma unroll
        for (int it = 0; it < 16; ++it) {
          const int row = it * 4 + (lane >> 4);
          const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + row * 256 + ((c ^ (row & 15)) << 4));
          const int grow = wm * 128 + p * 64 + row;
          if (grow < rows && gcol < n_out) stg16(fbase + (size_t)(m0 + grow) * ostride + gcol, v);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next pass writes
      }
    } else if constexpr (TO) {
      // Transposed bf16 store, out[n][m] with row stride M: with A the MFMA's first operand,
      // block (i, j) holds in lane l column j * 32 + (l & 31) and the four consecutive rows
      // i * 32 + 8 (r / 4) + 4 (l / 32) .. + 3.  The wave's 128 x 64 goes to LDS as 64
      // column-rows of 128 values (256 bytes; 16-byte chunk c of column-row n at c ^ (n & 15))
      // and leaves as 16-byte runs along the rows.
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = j * 32 + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint2 v;
            v.x = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
            v.y = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            *reinterpret_cast<uint2 *>(stage + n * 256 + (((4 * i + q) ^ (n & 15)) << 4) + lh * 8) = v;
          }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int c = lane & 15, grow = wm * 128 + c * 8;  // eight rows per 16-byte run
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int n = it * 4 + (lane >> 4), gn = gcol0 + n;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + n * 256 + ((c ^ (n & 15)) << 4));
        if (grow < rows && gn < n_out) stg16(obase + (size_t)gn * M + m0 + grow, v);
      }
    } else if constexpr (sizeof(OutT) == 2) {
      // bf16: 128 rows x 64 columns, 128-byte rows; chunk c of row r at c ^ ((r >> 1) & 7)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
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
      const int c = lane & 7, gcol = gcol0 + c * 8;
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int row = it * 8 + (lane >> 3);
        const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + row * 128 + ((c ^ ((row >> 1) & 7)) << 4));
        const int grow = wm * 128 + row;
        if (grow < rows && gcol < n_out) stg16(obase + (size_t)(m0 + grow) * ostride + gcol, v);
      }
    }
  }
}

// Packed tile layout of a grouped A operand: for row tile m (the rank of a 256-row tile
// among all groups' row tiles, as the GEMM numbers them) and K step kt, a 16 KB block at
// (m * K / 32 + kt) * 16 KB holding the tile's 256 rows x 32 values as the GEMM's LDS stage
// does -- 64-byte rows, 16-byte chunk c of row r at c ^ ((r >> 2) & 3) -- rows past the
// group zero.  The GEMM then loads each stage as one contiguous 16 KB block instead of 256
// rows of 64 bytes.  Rows gathered through row_index if given.
__global__ __launch_bounds__(256) void pack_rows_kernel(const bf16_t *__restrict__ src,
                                                        const int32_t *__restrict__ row_index,
                                                        const int32_t *__restrict__ offsets, int G, int K,
                                                        bf16_t *__restrict__ out, int tail) {
  // one workgroup per row tile and PR_STEPS consecutive K steps: each row's 256 bytes of them
  // (two whole lines) are read by 16 consecutive threads, every load issued before the stores
  // (Mixtral-shaped x rows: 31 -> 22 us against one workgroup per 64-byte step)
  const int steps = K / 32;
  const int spans = (steps + PR_STEPS - 1) / PR_STEPS;
  const int m_lin = blockIdx.x / spans, kt0 = (blockIdx.x - m_lin * spans) * PR_STEPS;
  int g, first, count;
  find_row_block<BG_BM>(offsets, G, m_lin, g, first, count, tail);
  if (g < 0) return;
  const int m0 = offsets[g] + (m_lin - first) * BG_BM, row_end = offsets[g + 1];
  u32x4 v[PR_STEPS * 4];
#pragma unroll
  for (int i = 0; i < PR_STEPS * 4; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int r = q / (PR_STEPS * 4), cc = q % (PR_STEPS * 4);  // row, 16-byte piece of its span
    v[i] = u32x4{0u, 0u, 0u, 0u};
    if (m0 + r < row_end && kt0 + cc / 4 < steps) {
      const int64_t sr = row_index ? (int64_t)row_index[m0 + r] : (int64_t)(m0 + r);
      v[i] = ldg16(src + sr * K + kt0 * 32 + cc * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < PR_STEPS * 4; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int r = q / (PR_STEPS * 4), cc = q % (PR_STEPS * 4);
    const int kt = kt0 + cc / 4, c = cc % 4;
    if (kt < steps) {
      bf16_t *blk = out + ((size_t)m_lin * steps + kt) * (BG_BM * 32);
      stg16(blk + r * 32 + ((c ^ ((r >> 2) & 3)) << 3), v[i]);
    }
  }
}

// Packed tile layout of grouped row-major weights ([n_rows, K] per group, group stride
// wstride elements) for the forward form's B operand: for group g, weight tile nt and K
// step kt, a 16 KB block at ((g * n_tiles + nt) * K / 32 + kt) * 16 KB holding the tile's
// 256 weight rows x 32 values as the GEMM's LDS stage does (the layout of pack_rows).
// The tile's rows are those the GEMM assigns it: with SwiGLU, gate rows nt * 128 .. + 127
// then the matching up rows (n_out apart); otherwise rows nt * 256 .. + 255; rows past
// n_out zero.
__global__ __launch_bounds__(256) void pack_weights_kernel(const bf16_t *__restrict__ W, int64_t wstride, int n_out,
                                                           int K, int n_tiles, int swiglu,
                                                           bf16_t *__restrict__ out) {
  const int steps = K / 32;
  const int64_t b = blockIdx.x;
  const int64_t gt = b / steps;
  const int kt = (int)(b - gt * steps);
  const int g = (int)(gt / n_tiles), nt = (int)(gt - (int64_t)g * n_tiles);
  bf16_t *blk = out + b * (BG_BN * 32);
  const bf16_t *wg = W + (size_t)g * wstride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int r = q >> 2, c = q & 3;
    int wr;  // weight row held in tile row r, -1 past n_out
    if (swiglu) {
      const int col = nt * (BG_BN / 2) + (r & 127);
      wr = col < n_out ? (r < 128 ? col : n_out + col) : -1;
    } else {
      wr = nt * BG_BN + r < n_out ? nt * BG_BN + r : -1;
    }
    u32x4 v = {0u, 0u, 0u, 0u};
    if (wr >= 0) v = ldg16(wg + (int64_t)wr * K + kt * 32 + c * 8);
    stg16(blk + r * 32 + ((c ^ ((r >> 2) & 3)) << 3), v);
  }
}

}  // namespace

template <bool SWIGLU, typename OutT = bf16_t, bool BKN = false, bool APK = false, bool OPK = false, bool GB = false,
          bool BPK = false>
hipError_t launch_big(const GroupedGemmArgs &a, int64_t rows_total_max, hipStream_t s) {
  if (a.n_out % 8) return hipErrorInvalidValue;  // the epilogue stores runs of 8 columns
  const int cols = SWIGLU ? BG_BN / 2 : BG_BN;
  const int n_tiles = (a.n_out + cols - 1) / cols;
  // packed weights: the group stride of their layout
  const void *W = BPK ? a.W_packed : a.W;
  const int64_t wstride = BPK ? packed_weights_bytes(1, a.n_out, a.K, SWIGLU) / 2 : a.w_group_stride;
  if (BPK && (a.K % 32 || wstride * 2 >= ((int64_t)1 << 32))) return hipErrorInvalidValue;
  const int64_t m_tiles = (rows_total_max + BG_BM - 1) / BG_BM + a.num_groups;
  // K splits only for a plain bf16 store with a workspace for the partials
  float *split = (!SWIGLU && sizeof(OutT) == 2 && a.split_ws && a.row_index == nullptr) ? a.split_ws : nullptr;
  const SwigluBwdOut gb{static_cast<const bf16_t *>(a.bwd_dhp), a.bwd_row_gate, static_cast<bf16_t *>(a.bwd_hg),
                        a.bwd_dpart};
  const int64_t split_stride = rows_total_max * a.n_out;
  const int64_t grid = m_tiles * n_tiles * (split ? 4 : 1);
  hipLaunchKernelGGL((grouped_gemm_big_kernel<SWIGLU, OutT, false, BKN, APK, OPK, GB, false, BPK>), dim3((unsigned)grid),
                     dim3(512), 0, s, static_cast<const bf16_t *>(a.A), a.row_index, a.a_rows, a.offsets, a.num_groups,
                     static_cast<const bf16_t *>(W), wstride, a.n_out, a.K, static_cast<OutT *>(a.out),
                     n_tiles, (int64_t)0, (int64_t)0, 0, split, split_stride, nullptr, gb, a.tail);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  const int64_t blocks = std::min<int64_t>((rows_total_max * a.n_out / 8 + 255) / 256, 4096);
  hipLaunchKernelGGL(big_split_reduce_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, s, split,
                     split_stride, a.offsets, a.num_groups, n_tiles, a.K / 32, a.n_out,
                     static_cast<bf16_t *>(a.out), a.tail);
  return hipGetLastError();
}

// Upper bound of the total row tiles: sum_g ceil(rows_g / 256) <= ceil(rows / 256) + G.
namespace {

hipError_t launch_big_tiles(const GroupedGemmArgs &a, int64_t rows_total_max, hipStream_t s) {
  const bool bp = a.W_packed != nullptr;
  if (bp && a.w_kn) return hipErrorInvalidValue;  // packed weights: the row-major forward form
  if (a.bwd_dhp) {  // the SwiGLU backward epilogue: plain rows in, bf16 gradients out
    if (!a.swiglu || a.out_f32 || a.w_kn || a.a_packed || a.out_packed || a.n_out % 32) return hipErrorInvalidValue;
    return bp ? launch_big<true, bf16_t, false, false, false, true, true>(a, rows_total_max, s)
              : launch_big<true, bf16_t, false, false, false, true>(a, rows_total_max, s);
  }
  if (a.a_packed || a.out_packed) {  // the packed tile layout (pack_rows): SwiGLU in, plain down
    if (a.w_kn || a.out_f32) return hipErrorInvalidValue;
    if (a.swiglu) {
      if (!a.out_packed) return hipErrorInvalidValue;
      if (!a.a_packed)  // row-major (or gathered) A, packed H
        return bp ? launch_big<true, bf16_t, false, false, true, false, true>(a, rows_total_max, s)
                  : launch_big<true, bf16_t, false, false, true>(a, rows_total_max, s);
      return bp ? launch_big<true, bf16_t, false, true, true, false, true>(a, rows_total_max, s)
                : launch_big<true, bf16_t, false, true, true>(a, rows_total_max, s);
    }
    if (!a.a_packed || a.out_packed) return hipErrorInvalidValue;
    return bp ? launch_big<false, bf16_t, false, true, false, false, true>(a, rows_total_max, s)
              : launch_big<false, bf16_t, false, true, false>(a, rows_total_max, s);
  }
  if (bp) return hipErrorInvalidValue;  // packed weights: with the packed activations or the SwiGLU backward
  if (a.w_kn) {  // K-major weights: bf16 output, no SwiGLU
    if (a.swiglu || a.out_f32) return hipErrorInvalidValue;
    return launch_big<false, bf16_t, true>(a, rows_total_max, s);
  }
  if (a.swiglu) return launch_big<true>(a, rows_total_max, s);
  return a.out_f32 ? launch_big<false, float>(a, rows_total_max, s) : launch_big<false>(a, rows_total_max, s);
}

}  // namespace

// The 256-row tiles, then, when tails are on (a.tail, or big_tails() for -1), the groups'
// last partial tiles of at most kBigTailRows rows on the streaming kernel: after the K-split
// reduction, which writes every row.
hipError_t launch_grouped_gemm_big_bf16(const GroupedGemmArgs &a0, int64_t rows_total_max, hipStream_t s) {
  GroupedGemmArgs a = a0;
  if (a.tail < 0) a.tail = big_tails(a.num_groups, a.n_out);
  if (a.tail != 0 && a.tail != kBigTailRows) return hipErrorInvalidValue;
  if (a.tail && ((a.a_packed && !a.tail_A) || (a.out_packed && !a.tail_out))) return hipErrorInvalidValue;
  hipError_t e = launch_big_tiles(a, rows_total_max, s);
  if (e != hipSuccess) return e;
  if (a.after_main) a.after_main(a.after_main_ctx);
  if (!a.tail) return e;
  GroupedGemmArgs t = a;
  t.tails_only = true;
  t.group_rows_max = std::min(a.group_rows_max, kBigTailRows);
  t.split_ws = nullptr;
  if (a.a_packed) {
    t.A = a.tail_A;
    t.row_index = a.tail_row_index;
    t.a_rows = a.tail_a_rows;
    t.a_packed = false;
  }
  if (a.out_packed) {
    t.out = a.tail_out;
    t.out_packed = false;
  }
  return launch_grouped_gemm_stream_bf16(t, s);
}

// The router linear logits = x W_r^T as a GEMM on the large tiles: tokens as rows, the
// router weights [E, d] as the weight rows, split along d so that the launch fills the GPU;
// float partial sums [splits][T][E] (without the offset) for the top-k kernel to add.  Used
// when the tiles of E columns are at least half full and the launch has 192 or more blocks;
// returns 0 otherwise.
int router_gemm_splits(int T, int d, int E) {
  if (E < BG_BN / 2 || E % 8 || T < 1 || d % 32) return 0;  // the epilogue stores runs of 8 columns
  const int tiles = ((T + BG_BM - 1) / BG_BM) * ((E + BG_BN - 1) / BG_BN);
  const int ks = big_ksplit(tiles, d / 32, kRouterMinSteps);
  return tiles * ks >= 192 ? ks : 0;
}

hipError_t launch_router_gemm(const void *x, const void *w_router, int T, int d, int E, float *partials,
                              hipStream_t s) {
  const int ks = router_gemm_splits(T, d, E);
  if (ks < 1) return hipErrorInvalidValue;
  const int n_tiles = (E + BG_BN - 1) / BG_BN;
  const int64_t grid = (int64_t)((T + BG_BM - 1) / BG_BM) * n_tiles * ks;
  // ks == 1: the kernel stores the float sums through `out` (= partials); else its partials
  hipLaunchKernelGGL((grouped_gemm_big_kernel<false, float>), dim3((unsigned)grid), dim3(512), 0, s,
                     static_cast<const bf16_t *>(x), nullptr, (int64_t)0, nullptr, 1,
                     static_cast<const bf16_t *>(w_router), (int64_t)E * d, E, d, partials, n_tiles, (int64_t)0,
                     (int64_t)0, T, ks > 1 ? partials : nullptr, (int64_t)T * E, nullptr, SwigluBwdOut{}, 0);
  return hipGetLastError();
}

int64_t packed_weights_bytes(int G, int n_out, int K, bool swiglu) {
  const int cols = swiglu ? BG_BN / 2 : BG_BN;
  return (int64_t)G * ((n_out + cols - 1) / cols) * (K / 32) * (BG_BN * 32 * 2);
}

hipError_t launch_pack_weights(const void *W, int G, int64_t wstride, int n_out, int K, bool swiglu, void *out,
                               hipStream_t s) {
  if (K % 32 || n_out < 1 || G < 1) return hipErrorInvalidValue;
  const int cols = swiglu ? BG_BN / 2 : BG_BN;
  const int n_tiles = (n_out + cols - 1) / cols;
  const int64_t grid = (int64_t)G * n_tiles * (K / 32);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const bf16_t *>(W), wstride,
                     n_out, K, n_tiles, swiglu ? 1 : 0, static_cast<bf16_t *>(out));
  return hipGetLastError();
}

int64_t packed_rows_bytes(int64_t rows_max, int G, int K) {
  return ((rows_max + BG_BM - 1) / BG_BM + G) * BG_BM * (int64_t)K * 2;
}

hipError_t launch_pack_rows(const void *src, const int32_t *row_index, const int32_t *offsets, int G, int64_t rows_max,
                            int K, void *out, hipStream_t s, int tail) {
  if (K % 32) return hipErrorInvalidValue;
  const int64_t grid = ((rows_max + BG_BM - 1) / BG_BM + G) * ((K / 32 + PR_STEPS - 1) / PR_STEPS);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const bf16_t *>(src), row_index,
                     offsets, G, K, static_cast<bf16_t *>(out), tail);
  return hipGetLastError();
}

// Weight gradients with the second operand K-major: out[g][m][n] = sum over k < K_g of
// AT_g[m][k] B[off_b[g] + k][n], AT_g = AT + poff[g] * M with row stride K_g = poff[g+1] -
// poff[g] (group-major transposed, zero padded to multiples of 32), B [b_rows, N] row-major
// with group g's rows off_b[g] .. off_b[g+1] - 1 (k past them: zero).  M and N multiples of
// 8; an empty group writes zeros.  With `transposed`, out[g] is stored as [N, M] (out[g][n][m]).
hipError_t launch_wgrad_big_kn(const void *AT, int64_t lda, const int32_t *poff, const void *B, int64_t b_rows,
                               const int32_t *off_b, int G, int M, int N, void *out, hipStream_t s, bool transposed) {
  if (N % 8 || M % 8) return hipErrorInvalidValue;
  const int m_tiles = (M + BG_BM - 1) / BG_BM, n_tiles = (N + BG_BN - 1) / BG_BN;
  const int64_t grid = (int64_t)G * m_tiles * n_tiles;
  if (grid <= 0) return hipSuccess;
  if (transposed)
    hipLaunchKernelGGL((grouped_gemm_big_kernel<false, bf16_t, true, true, false, false, false, true>),
                       dim3((unsigned)grid), dim3(512), 0, s, static_cast<const bf16_t *>(AT), nullptr, (int64_t)0, poff,
                       G, static_cast<const bf16_t *>(B), (int64_t)0, N, 0, static_cast<bf16_t *>(out), n_tiles, lda,
                       b_rows, M, nullptr, (int64_t)0, off_b, SwigluBwdOut{}, 0);
  else
    hipLaunchKernelGGL((grouped_gemm_big_kernel<false, bf16_t, true, true>), dim3((unsigned)grid), dim3(512), 0, s,
                       static_cast<const bf16_t *>(AT), nullptr, (int64_t)0, poff, G, static_cast<const bf16_t *>(B),
                       (int64_t)0, N, 0, static_cast<bf16_t *>(out), n_tiles, lda, b_rows, M, nullptr, (int64_t)0,
                       off_b, SwigluBwdOut{}, 0);
  return hipGetLastError();
}

// Number of K slices of the float weight-gradient form with one group (M x N output,
// K rows): enough blocks to fill the GPU, at least 8 steps of 32 per slice.
int wgrad_big_f32_splits(int M, int N, int64_t K) {
  const int tiles = ((M + BG_BM - 1) / BG_BM) * ((N + BG_BN - 1) / BG_BN);
  const int64_t steps = K / 32;
  if (tiles >= 256 || steps < 16) return 1;
  return (int)std::min<int64_t>({64, std::max(1, 256 / tiles), steps / 8});
}

// out[m][n] = sum over k < K of AT[m][k] B[k][n] in float, one group: AT [M, K] with row
// stride K = poff[1] - poff[0] (a multiple of 32, zero padding), B [b_rows, N] row-major
// with rows off_b[0] .. off_b[1] - 1 (k past them: zero).  Cut along K into
// wgrad_big_f32_splits() slices whose float partials (part, slices * M * N floats) are
// added in slice order.  N a multiple of 8.
hipError_t launch_wgrad_big_kn_f32(const void *AT, int64_t lda, const int32_t *poff, const void *B, int64_t b_rows,
                                   const int32_t *off_b, int M, int N, int64_t K, float *part, float *out,
                                   hipStream_t s) {
  if (N % 8) return hipErrorInvalidValue;
  const int S = wgrad_big_f32_splits(M, N, K);
  const int m_tiles = (M + BG_BM - 1) / BG_BM, n_tiles = (N + BG_BN - 1) / BG_BN;
  const int64_t grid = (int64_t)m_tiles * n_tiles * S;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_big_kernel<false, float, true, true>), dim3((unsigned)grid), dim3(512), 0, s,
                     static_cast<const bf16_t *>(AT), nullptr, (int64_t)0, poff, 1, static_cast<const bf16_t *>(B),
                     (int64_t)0, N, S, out, n_tiles, lda, b_rows, M, S > 1 ? part : nullptr, (int64_t)M * N, off_b,
                     SwigluBwdOut{}, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  return launch_ksplit_sum(part, S, (int64_t)M * N, out, s);
}

}  // namespace moe
