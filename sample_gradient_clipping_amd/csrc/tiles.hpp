// Tile loaders and MFMA fragment readers shared by the GEMM-shaped kernels.
//
// Two operand layouts occur on this path:
//   K-outer : global [k][m] with m contiguous.  The weight-gradient
//             contraction G_i^T X_i sums over tokens, and both X and G are
//             stored token-major, so both operands are K-outer there.
//             LDS keeps the global layout ([k][m]); gfx950's transposing LDS
//             read hands each lane its 8 consecutive-k values.
//   K-inner : global [m][k] with k contiguous (the Gram products X X^T and
//             G G^T, and X in the projection X P).  LDS keeps [m][k]; a lane
//             reads its 8 k-values with one 16-byte LDS read.
// Rows that are masked, past T, or past the end of a dimension load as zero
// (selection: the memory of a masked row is never read).
#pragma once

#include "common.hpp"

namespace dpf {

// Raw 16-byte chunk of E elements.
template <class E>
struct Chunk {
  u32x4 v;
};

template <class E, bool VEC>
__device__ __forceinline__ u32x4 load_chunk(const typename E::storage* p, int avail) {
  // avail: number of valid elements starting at p (<= 0 means none).
  if (avail <= 0) return u32x4{0u, 0u, 0u, 0u};
  if constexpr (VEC) {
    return *(const u32x4*)(p);
  } else {
    typename E::storage tmp[E::kVec];
#pragma unroll
    for (int e = 0; e < E::kVec; ++e) tmp[e] = (e < avail) ? p[e] : (typename E::storage)0;
    return __builtin_bit_cast(u32x4, tmp);
  }
}

// K-outer tile: KT token rows x TILE columns of one sample, into registers.
//   base   : start of sample b's rows (element pointer)
//   t0     : first token of the tile; col0: first column
template <class E, int TILE, int KT, int NT, bool VEC>
struct KOuterLoader {
  static constexpr int CPR = TILE / E::kVec;          // chunks per row
  static constexpr int N = KT * CPR / NT;             // chunks per thread
  static_assert((KT * CPR) % NT == 0, "tile does not split evenly over the workgroup");
  u32x4 r[N];

  __device__ __forceinline__ void load(const typename E::storage* base, int64_t stride_t, int T,
                                       const uint8_t* mask_b, int t0, int col0, int D) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = threadIdx.x + NT * i;
      const int row = q / CPR, cc = q % CPR;
      const int t = t0 + row, col = col0 + cc * E::kVec;
      const bool active = t < T && (mask_b == nullptr || mask_b[t] != 0);
      r[i] = load_chunk<E, VEC>(base + (int64_t)t * stride_t + col, active ? (D - col) : 0);
    }
  }

  template <int LD>
  __device__ __forceinline__ void store(typename E::storage* lds) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = threadIdx.x + NT * i;
      const int row = q / CPR, cc = q % CPR;
      *(u32x4*)(lds + row * LD + cc * E::kVec) = r[i];
    }
  }
};

// K-inner tile: ROWS token rows x KT features of one sample.
template <class E, int ROWS, int KT, int NT, bool VEC>
struct KInnerLoader {
  static constexpr int CPR = KT / E::kVec;
  static constexpr int N = ROWS * CPR / NT;
  static_assert((ROWS * CPR) % NT == 0, "tile does not split evenly over the workgroup");
  u32x4 r[N];

  __device__ __forceinline__ void load(const typename E::storage* base, int64_t stride_t, int T,
                                       const uint8_t* mask_b, int r0, int k0, int K) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = threadIdx.x + NT * i;
      const int row = q / CPR, cc = q % CPR;
      const int t = r0 + row, k = k0 + cc * E::kVec;
      const bool active = t < T && (mask_b == nullptr || mask_b[t] != 0);
      r[i] = load_chunk<E, VEC>(base + (int64_t)t * stride_t + k, active ? (K - k) : 0);
    }
  }

  // Same, but the ROWS rows are flat token indices over all samples (b = q / T).
  __device__ __forceinline__ void load_flat(const typename E::storage* data, int64_t stride_b,
                                            int64_t stride_t, int B, int T, const uint8_t* mask,
                                            int64_t q0, int k0, int K) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = threadIdx.x + NT * i;
      const int row = q / CPR, cc = q % CPR;
      const int64_t flat = q0 + row;
      const int b = (int)(flat / T), t = (int)(flat % T);
      const bool active = b < B && (mask == nullptr || mask[flat] != 0);
      const int k = k0 + cc * E::kVec;
      r[i] = load_chunk<E, VEC>(data + (int64_t)b * stride_b + (int64_t)t * stride_t + k,
                                active ? (K - k) : 0);
    }
  }

  template <int LD>
  __device__ __forceinline__ void store(typename E::storage* lds) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int q = threadIdx.x + NT * i;
      const int row = q / CPR, cc = q % CPR;
      *(u32x4*)(lds + row * LD + cc * E::kVec) = r[i];
    }
  }
};

// ---------------------------------------------------------------------------
// Fragment readers.  Frag<E> is one MFMA operand for one 32-row block.
// ---------------------------------------------------------------------------
template <class E> struct Frag;
template <> struct Frag<BF16> { typedef u16x8 type; };
template <> struct Frag<F32> { typedef float type; };

// From a K-outer LDS tile [k][m] (row length LD): rows m0..m0+31, k-step ks.
template <class E, int LD>
__device__ __forceinline__ typename Frag<E>::type frag_kouter(const typename E::storage* lds,
                                                              int m0, int ks) {
  const int lane = threadIdx.x & 63;
  if constexpr (sizeof(typename E::storage) == 2) {
    const int krow = ks * 16 + 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int col = m0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const u16x4 lo = lds_read_tr16(lds + krow * LD + col);
    const u16x4 hi = lds_read_tr16(lds + (krow + 4) * LD + col);
    u16x8 f;
    f.s0 = lo.s0; f.s1 = lo.s1; f.s2 = lo.s2; f.s3 = lo.s3;
    f.s4 = hi.s0; f.s5 = hi.s1; f.s6 = hi.s2; f.s7 = hi.s3;
    return f;
  } else {
    return lds[(ks * 2 + (lane >> 5)) * LD + m0 + (lane & 31)];
  }
}

// From a K-inner LDS tile [m][k] (row length LD): rows m0..m0+31, k-step ks.
template <class E, int LD>
__device__ __forceinline__ typename Frag<E>::type frag_kinner(const typename E::storage* lds,
                                                              int m0, int ks) {
  const int lane = threadIdx.x & 63;
  if constexpr (sizeof(typename E::storage) == 2) {
    return *(const u16x8*)(lds + (m0 + (lane & 31)) * LD + ks * 16 + 8 * (lane >> 5));
  } else {
    return lds[(m0 + (lane & 31)) * LD + ks * 2 + (lane >> 5)];
  }
}

template <class E>
__device__ __forceinline__ f32x16 mfma(const typename Frag<E>::type& a,
                                       const typename Frag<E>::type& b, const f32x16& c) {
  if constexpr (sizeof(typename E::storage) == 2) return mfma_32x32x16(a, b, c);
  else return mfma_32x32x2(a, b, c);
}

// One 16-byte chunk of a projection P regenerated instead of read:
// P[d][c .. c + 16/sizeof(storage)) = scale * xi_e for e = d*r + c ..,
// xi from Philox4x32-10 (seed, offset) and Box-Muller, rounded to the storage
// type exactly as the Gaussian fill writes it; zero for d >= din or c >= r.
// r is a multiple of 8, so a chunk covers whole Philox blocks (two for bf16,
// one for fp32).
template <class E>
__device__ __forceinline__ u32x4 gen_p_chunk(uint64_t seed, uint64_t offset, float scale, int din,
                                             int r, int d, int c) {
  if (d >= din || c >= r) return u32x4{0u, 0u, 0u, 0u};
  const uint64_t blk = offset + (((uint64_t)d * (uint64_t)r + (uint64_t)c) >> 2);
  if constexpr (sizeof(typename E::storage) == 2) {
    const f32x4 z0 = normals_of_block(philox_block(seed, blk));
    const f32x4 z1 = normals_of_block(philox_block(seed, blk + 1));
    const float v[8] = {scale * z0.x, scale * z0.y, scale * z0.z, scale * z0.w,
                        scale * z1.x, scale * z1.y, scale * z1.z, scale * z1.w};
    uint16_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = f32_to_bf16_rne(v[e]);
    return __builtin_bit_cast(u32x4, h);
  } else {
    const f32x4 z = normals_of_block(philox_block(seed, blk));
    const float v[4] = {scale * z.x, scale * z.y, scale * z.z, scale * z.w};
    return __builtin_bit_cast(u32x4, v);
  }
}

}  // namespace dpf
