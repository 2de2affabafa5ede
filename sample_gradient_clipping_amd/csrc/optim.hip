// Projected Adam step: the optimizer states live in the projected space
// (Memory-Efficient Differentially Private Training with Gradient Random
// Projection, English explainer, Methodology, "Projected Optimizer States"),
// and the update reaches the full weight through the projection:
//
//   m <- beta1 m + (1 - beta1) h          h, m, v, U : [dout, r] float32
//   v <- beta2 v + (1 - beta2) h^2
//   U  = (m / bc1) / (sqrt(v / bc2) + eps),   bc_k = 1 - beta_k^step
//   W <- W - lr * U P^T                   W : [dout, din] float32, P : [din, r]
//
//  adam_moments_kernel : the elementwise part, 4 elements per thread
//  adam_update_kernel  : W -= lr * U P^T, fp32 MFMA (v_mfma_f32_32x32x2f32)
//                        on 128 x 128 tiles of W, or 64 x 64 when the larger
//                        tiles would leave compute units idle; P is read
//                        (bf16 or fp32) or drawn again from its seed exactly
//                        as gaussian_fill writes it, then widened to fp32.
//                        With more than one row of W tiles a seeded P is drawn
//                        once into workspace by the gaussian fill instead.
#include "kernels.hpp"
#include "tiles.hpp"

namespace dpf {
namespace optim {

constexpr int kNT = 256;                 // 4 waves, 2 x 2
constexpr int kKT = 32;                  // r per LDS step
constexpr int kLD = kKT + 4;             // LDS row (floats), padded against bank conflicts
// W tile: TILE (din) x TILE (dout); P and U slices double-buffered in LDS
template <int TILE>
constexpr int lds_bytes() { return 2 * 2 * TILE * kLD * (int)sizeof(float); }

__global__ void __launch_bounds__(256) adam_moments_kernel(AdamArgs a) {
  const int64_t n = a.dout * a.r;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;   // n is a multiple of 4 (r is)
  const f32x4 g = *(const f32x4*)(a.grad + i);
  f32x4 m = *(const f32x4*)(a.m + i), v = *(const f32x4*)(a.v + i), u;
  const float b1 = a.beta1, b2 = a.beta2;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m[e] = b1 * m[e] + (1.0f - b1) * g[e];
    v[e] = b2 * v[e] + (1.0f - b2) * (g[e] * g[e]);
    u[e] = (m[e] / a.bc1) / (sqrtf(v[e] / a.bc2) + a.eps);
  }
  *(f32x4*)(a.m + i) = m;
  *(f32x4*)(a.v + i) = v;
  *(f32x4*)(a.u + i) = u;
}

// Four consecutive P entries P[d][j .. j+3] (j a multiple of 4) as float32.
__device__ __forceinline__ f32x4 p_chunk(const AdamArgs& a, int64_t d, int j) {
  if (d >= a.din || j >= a.r) return f32x4{0.f, 0.f, 0.f, 0.f};
  const int64_t e = d * a.r + j;
  f32x4 w;
  if (a.gen) {
    const f32x4 z = normals_of_block(philox_block(a.p_seed, a.p_offset + (uint64_t)(e >> 2)));
    const float v[4] = {a.p_scale * z.x, a.p_scale * z.y, a.p_scale * z.z, a.p_scale * z.w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = a.p_dtype == kBF16 ? BF16::to_float(f32_to_bf16_rne(v[k])) : v[k];
  } else if (a.p_dtype == kBF16) {
    const u16x4 h = *(const u16x4*)((const uint16_t*)a.P + e);
    w.x = BF16::to_float(h.s0); w.y = BF16::to_float(h.s1);
    w.z = BF16::to_float(h.s2); w.w = BF16::to_float(h.s3);
  } else {
    w = *(const f32x4*)((const float*)a.P + e);
  }
  return w;
}

__device__ __forceinline__ f32x4 u_chunk(const AdamArgs& a, int64_t o, int j) {
  if (o >= a.dout || j >= a.r) return f32x4{0.f, 0.f, 0.f, 0.f};
  return *(const f32x4*)(a.u + o * a.r + j);
}

// One W tile.  MFMA "A" = P rows (din), "B" = U rows (dout), both with r
// contiguous ("K-inner"), so D[d][o] gives each lane 4 consecutive din
// columns of one W row: a 16-byte read-modify-write.  Each wave owns NB x NB
// blocks of 32 x 32.
template <int TILE>
__global__ void __launch_bounds__(kNT) adam_update_kernel(AdamArgs a) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  constexpr int NB = TILE / 64;
  constexpr int kTileFloats = TILE * kLD;
  const int ntd = (int)((a.din + TILE - 1) / TILE);
  const int64_t d0 = (int64_t)(blockIdx.x % ntd) * TILE, o0 = (int64_t)(blockIdx.x / ntd) * TILE;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int kChunks = TILE * (kKT / 4) / kNT;   // chunks of each operand per thread
  f32x16 acc[NB][NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  f32x4 pr[kChunks], ur[kChunks];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int q = threadIdx.x + kNT * c;
      const int row = q / (kKT / 4), col = (q % (kKT / 4)) * 4;
      pr[c] = p_chunk(a, d0 + row, k0 + col);
      ur[c] = u_chunk(a, o0 + row, k0 + col);
    }
  };
  auto stash = [&](float* buf) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int q = threadIdx.x + kNT * c;
      const int row = q / (kKT / 4), col = (q % (kKT / 4)) * 4;
      *(f32x4*)(buf + row * kLD + col) = pr[c];
      *(f32x4*)(buf + kTileFloats + row * kLD + col) = ur[c];
    }
  };
  const int nk = (int)((a.r + kKT - 1) / kKT);
  fetch(0);
  stash(lds);
  __syncthreads();
  for (int kk = 0; kk < nk; ++kk) {
    const bool more = kk + 1 < nk;
    if (more) fetch((kk + 1) * kKT);
    const float* Ps = lds + (kk & 1) * 2 * kTileFloats;
    const float* Us = Ps + kTileFloats;
#pragma unroll
    for (int ks = 0; ks < kKT / 2; ++ks) {
      float fa[NB], fb[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) fa[i] = frag_kinner<F32, kLD>(Ps, (wm * NB + i) * 32, ks);
#pragma unroll
      for (int j = 0; j < NB; ++j) fb[j] = frag_kinner<F32, kLD>(Us, (wn * NB + j) * 32, ks);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma<F32>(fa[i], fb[j], acc[i][j]);
    }
    if (!more) break;
    stash(lds + ((kk + 1) & 1) * 2 * kTileFloats);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int64_t o = o0 + (wn * NB + j) * 32 + acc_col(lane);
      if (o >= a.dout) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t d = d0 + (wm * NB + i) * 32 + acc_row(4 * g, lane);
        if (d >= a.din) continue;   // din % 4 == 0: d .. d+3 all in range
        f32x4* w = (f32x4*)(a.W + o * a.din + d);
        f32x4 x = *w;
        x.x -= a.lr * acc[i][j][4 * g + 0];
        x.y -= a.lr * acc[i][j][4 * g + 1];
        x.z -= a.lr * acc[i][j][4 * g + 2];
        x.w -= a.lr * acc[i][j][4 * g + 3];
        *w = x;
      }
    }
}

}  // namespace optim

namespace {
template <int TILE>
hipError_t launch_update(const AdamArgs& a, hipStream_t s) {
  static hipError_t once = hipFuncSetAttribute((const void*)optim::adam_update_kernel<TILE>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               optim::lds_bytes<TILE>());
  if (once != hipSuccess) return once;
  const int64_t tiles = ((a.din + TILE - 1) / TILE) * ((a.dout + TILE - 1) / TILE);
  timing_begin("adam_update", s);
  hipLaunchKernelGGL(optim::adam_update_kernel<TILE>, dim3((unsigned)tiles), dim3(optim::kNT),
                     optim::lds_bytes<TILE>(), s, a);
  const hipError_t e = hipGetLastError();
  timing_end("adam_update", s);
  return e;
}

// 128 x 128 W tiles unless that leaves fewer workgroups than compute units.
bool small_tiles(const AdamArgs& a) {
  return ((a.din + 127) / 128) * ((a.dout + 127) / 128) < device_cus();
}
}  // namespace

bool adam_draws_p_once(const AdamArgs& a) {
  const int tile = small_tiles(a) ? 64 : 128;
  return a.gen != 0 && !p_in_kernels() && a.dout > tile;
}

hipError_t launch_projected_adam(const AdamArgs& a, hipStream_t s) {
  AdamArgs q = a;
  if (adam_draws_p_once(a)) {
    if (a.pbuf == nullptr) return hipErrorInvalidValue;
    hipError_t e = launch_gaussian_fill(a.p_seed, a.p_offset, a.din * a.r, a.p_scale, a.p_dtype,
                                        a.pbuf, s);
    if (e != hipSuccess) return e;
    q.P = a.pbuf;
    q.gen = 0;
  }
  const int64_t n = a.dout * a.r;
  timing_begin("adam_moments", s);
  hipLaunchKernelGGL(optim::adam_moments_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256),
                     0, s, q);
  hipError_t e = hipGetLastError();
  timing_end("adam_moments", s);
  if (e != hipSuccess) return e;
  return small_tiles(q) ? launch_update<64>(q, s) : launch_update<128>(q, s);
}

}  // namespace dpf
