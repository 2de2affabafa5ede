// Device-side building blocks shared by the dpfused kernels (gfx950 only).
//
//  * bf16 / fp32 operand types and the two MFMA shapes used here:
//      v_mfma_f32_32x32x16_bf16 (dense bf16 tiles, fp32 accumulate)
//      v_mfma_f32_32x32x2_f32   (fp32 inputs stay fp32 end to end)
//    Lane layouts (64-lane wave, lane l):
//      operand "row" r = l % 32, k-slice = l / 32 (8 bf16 values, or 1 fp32)
//      accumulator register j holds D[8*(j/4) + 4*(l/32) + (j%4)][l % 32]
//  * Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC'11) and Box-Muller,
//    which draw the Gaussian noise added to the clipped sum.
//  * Wave- and workgroup-level fp64 sums with a fixed order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dpf {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Element types
// ---------------------------------------------------------------------------
struct BF16 {
  typedef uint16_t storage;             // raw bits in memory and LDS
  static constexpr int kVec = 8;        // elements per 16-byte chunk
  static constexpr int kMfmaK = 16;     // K of one MFMA
  static __device__ __forceinline__ float to_float(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
  }
};

struct F32 {
  typedef float storage;
  static constexpr int kVec = 4;
  static constexpr int kMfmaK = 2;
  static __device__ __forceinline__ float to_float(float f) { return f; }
};

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// MFMA wrappers
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma_32x32x16(const u16x8& a, const u16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_32x32x2(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row (M index within a 32x32 block) held by accumulator register j of lane l.
__device__ __forceinline__ int acc_row(int j, int lane) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

// LDS transpose read: from a [k][m] tile (m contiguous) give this lane the 4
// consecutive-k values of one m.  Within each group of 16 lanes, lane j's
// address names row (j/4) and the 4-element chunk (j%4) of a 4x16 block; the
// result in lane j is column j of that block, rows 0..3.
__device__ __forceinline__ u16x4 lds_read_tr16(const uint16_t* p) {
  bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
  return __builtin_bit_cast(u16x4, v);
}

// ---------------------------------------------------------------------------
// Philox4x32-10 and Box-Muller
// ---------------------------------------------------------------------------
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

// Words of block `block` under key (lo32(seed), hi32(seed)); counter =
// (lo32(block), hi32(block), 0, 0).
__device__ __forceinline__ u32x4 philox_block(uint64_t seed, uint64_t block) {
  uint32_t c0 = (uint32_t)block, c1 = (uint32_t)(block >> 32), c2 = 0u, c3 = 0u;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += kPhiloxW0; k1 += kPhiloxW1; }
    // One 32 x 32 -> 64-bit multiply per product (v_mad_u64_u32).
    const uint64_t p0 = (uint64_t)kPhiloxM0 * c0, p1 = (uint64_t)kPhiloxM1 * c2;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
  }
  u32x4 w; w.x = c0; w.y = c1; w.z = c2; w.w = c3;
  return w;
}

// u = ((w >> 9) + 0.5) * 2^-23, exact in fp32 and strictly inside (0, 1).
__device__ __forceinline__ float word_to_uniform(uint32_t w) {
  return ((float)(w >> 9) + 0.5f) * 1.1920928955078125e-07f;
}

// Four standard normals from one Philox block: (z0, z1) from (u0, u1) and
// (z2, z3) from (u2, u3); radius sqrt(-2 ln ua), angle 2 pi ub.
__device__ __forceinline__ f32x4 normals_of_block(u32x4 w) {
  const float r01 = sqrtf(-2.0f * logf(word_to_uniform(w.x)));
  const float r23 = sqrtf(-2.0f * logf(word_to_uniform(w.z)));
  float s1, c1, s3, c3;
  sincospif(2.0f * word_to_uniform(w.y), &s1, &c1);   // 2*u is exact
  sincospif(2.0f * word_to_uniform(w.w), &s3, &c3);
  f32x4 z;
  z.x = r01 * c1; z.y = r01 * s1; z.z = r23 * c3; z.w = r23 * s3;
  return z;
}

__device__ __forceinline__ float normal_at(uint64_t seed, uint64_t offset, uint64_t e) {
  const f32x4 z = normals_of_block(philox_block(seed, offset + (e >> 2)));
  switch (e & 3) { case 0: return z.x; case 1: return z.y; case 2: return z.z; default: return z.w; }
}

// ---------------------------------------------------------------------------
// Fixed-order reductions (fp64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Sum of one double per thread over the workgroup; result valid in thread 0.
// `scratch` needs (blockDim.x / 64) doubles of LDS.
__device__ __forceinline__ double block_sum_f64(double v, double* scratch) {
  v = wave_sum_f64(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) scratch[wave] = v;
  __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0) {
    const int nw = blockDim.x >> 6;
    for (int w = 0; w < nw; ++w) s += scratch[w];
  }
  return s;
}

// ---------------------------------------------------------------------------
// Operand description passed to kernels (element strides; last dim contiguous)
// ---------------------------------------------------------------------------
struct Act {
  const void* data;
  int64_t stride_b, stride_t;
};

__device__ __forceinline__ bool row_active(const uint8_t* mask, int T, int b, int t) {
  return t < T && (mask == nullptr || mask[(int64_t)b * T + t] != 0);
}

}  // namespace dpf
