// Device-side helpers shared by the gfx950 kernels of libmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bfloat16 storage word
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;   // CDNA wavefront width
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, each with its own L2
#define MOE_MAX_EXPERTS_DEV 1024  // equals MOE_MAX_EXPERTS of the C ABI

__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// Round-to-nearest-even float -> bfloat16 (NaN stays NaN) with gfx950's conversion
// instruction (v_cvt_pk_bf16_f32): bit-identical to adding 0x7fff plus the kept lsb and
// truncating, for every non-NaN float including denormals and ties (checked on the GPU
// over 2^26 inputs).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f)); }

// Store of a float result as the output element type (bf16, rounded to nearest even, or float).
template <typename OutT>
__device__ __forceinline__ void store_out(OutT *p, float v) {
  if constexpr (sizeof(OutT) == 4)
    *p = v;
  else
    *p = f32_to_bf16(v);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// 16-byte vector load/store through the vector memory path.
__device__ __forceinline__ u32x4 ldg16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void stg16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
// The same, marked non-temporal: for data touched once (streamed through, not reused).
__device__ __forceinline__ u32x4 ldg16_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void stg16_nt(void *p, u32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p)); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Raw buffer resources: loads whose byte offset is at or beyond `num_bytes` return
// zeros without touching memory (hardware range check).  kOob is such an offset.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)num_bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// The same load marked non-temporal (cache policy bit nt): for data read once, such as
// streamed expert weights.  A plain read of a 4 GiB buffer measured 6.7 TB/s with it against
// 6.0 TB/s without on this GPU.
constexpr int kCpolNt = 2;
__device__ __forceinline__ u32x4 buf_ld16_nt(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolNt);
}
// 16 bytes per lane from a buffer straight into LDS: lane i's data lands at
// lds_wave_base + 16 * i (lds_wave_base must be equal across the wavefront).
__device__ __forceinline__ void buf_ld16_lds(rsrc_t r, uint32_t off, void *lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_wave_base, 16, off, 0, 0,
                                           0);
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Workgroups are handed to the 8 XCDs round-robin by block id.  This maps the
// block id to a logical tile index so that each XCD works on one contiguous range
// of tiles, which keeps tiles that share operands inside one L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  if (nblocks < kNumXcd) return bid;
  const int xcd = bid % kNumXcd, idx = bid / kNumXcd;
  const int per = nblocks / kNumXcd, rem = nblocks % kNumXcd;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// Groups cut into blocks of BM rows: group g holds row_blocks<BM>(rows_g, tail) blocks,
// rows_g = offsets[g+1] - offsets[g], numbered group after group -- ceil(rows_g / BM), but
// with tail > 0 a last partial block of at most `tail` rows is left out (those rows are
// another kernel's).  One wavefront scans the offsets; the results are equal in every lane.
template <int BM>
__host__ __device__ __forceinline__ int row_blocks(int rows, int tail) { return rows / BM + (rows % BM > tail ? 1 : 0); }

// Block index m_lin -> its group (-1 past the last block), the group's first block and
// its block count.
template <int BM>
__device__ __forceinline__ void find_row_block(const int32_t *offsets, int G, int m_lin, int &g_out, int &first,
                                               int &count, int tail = 0) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  g_out = -1;
  first = 0;
  count = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    const int g = g0 + lane;
    int mt = 0;
    if (g < G) mt = row_blocks<BM>(offsets[g + 1] - offsets[g], tail);
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
      first = base + __shfl(incl - mt, l, 64);
      count = __shfl(mt, l, 64);
      return;
    }
    base += __shfl(incl, 63, 64);
  }
}

// Total row blocks over all groups, sum_g ceil(rows_g / BM).
template <int BM>
__device__ __forceinline__ int total_row_blocks(const int32_t *offsets, int G, int tail = 0) {
  const int lane = threadIdx.x & 63;
  int sum = 0;
  for (int g = lane; g < G; g += 64) sum += row_blocks<BM>(offsets[g + 1] - offsets[g], tail);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  return sum;
}

// silu(z) = z sigmoid(z), the sigmoid with the hardware reciprocal (about 1 ulp) instead of
// an IEEE division: the SwiGLU epilogue evaluates it for every output of a large tile while
// the matrix cores wait (Mixtral-shaped gate_up 1475 -> 1443 us), and its result is rounded
// to bf16.  z -> -inf gives -0, as the division does.
__device__ __forceinline__ float silu_f32(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// sigmoid(z) with the hardware reciprocal (about 1 ulp): for gradients rounded to bf16.
__device__ __forceinline__ float sigmoid_fast(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// d silu / dz = s (1 + z (1 - s)) with s = sigmoid(z).
__device__ __forceinline__ float silu_grad_f32(float z) {
  const float s = 1.0f / (1.0f + __expf(-z));
  return s * (1.0f + z * (1.0f - s));
}

}  // namespace moe
