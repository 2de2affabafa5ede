// The whole per-layer DP step in one workgroup, for layers small enough that
// one workgroup holds every sample's gradient: the single fused pass (FlashDP
// abstract: each per-sample gradient computed once, clipped and summed in
// one task) without any cross-workgroup synchronisation.
//
//   stage every sample's rows of X and G in LDS as float32 (masked rows
//   selected to zero, rows padded with zeros to 4 / 2 columns);
//   each thread owns a 2 (dout) x 4 (din) block of outputs for all B samples:
//     g_b[block] = sum over t of G_b[t][o] X_b[t][a]          (fp32, t order)
//   n_b = ||g_b||: fp32 per thread, fp64 per wave, waves in a fixed order;
//   c_b = 1 if n_b <= C else C / n_b;
//   out = beta * out + (sum_b c_b g_b + noise_std * xi) / denom   (b order)
#include "kernels.hpp"

namespace dpf {
namespace {

constexpr int kTinyThreads = 1024;
constexpr int kTinyWaves = kTinyThreads / 64;
constexpr int kTO = 2, kTA = 4;   // outputs per thread: kTO rows (dout) x kTA columns (din)

// Same rule as the ordered finalize: n = sqrt(max(sq, 0)), c = 1 when n <= C.
__device__ __forceinline__ void tiny_clip(double sq, float C, float* c, float* n) {
  const double nn = sqrt(sq < 0.0 ? 0.0 : sq);
  *n = (float)nn;
  *c = (nn <= (double)C) ? 1.0f : (float)((double)C / nn);
}

__host__ __device__ inline int pad_to(int v, int m) { return (v + m - 1) / m * m; }

template <class E>
__global__ void __launch_bounds__(kTinyThreads) tiny_layer_kernel(LayerArgs p, float C,
                                                                  float* norms_out) {
  using S = typename E::storage;
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ double red[kTinyMaxB][kTinyWaves];
  __shared__ float cs[kTinyMaxB];
  const int B = p.B, T = p.T;
  const int dinp = pad_to(p.din, kTA), doutp = pad_to(p.dout, kTO);
  float* xs = lds;                                  // [B][T][dinp]
  float* gs = lds + (size_t)B * T * dinp;           // [B][T][doutp]
  for (int i = threadIdx.x; i < B * T * dinp; i += kTinyThreads) {
    const int a = i % dinp, bt = i / dinp, t = bt % T, b = bt / T;
    const bool on = a < p.din && (p.mask == nullptr || p.mask[(int64_t)b * T + t] != 0);
    xs[i] = on ? E::to_float(((const S*)p.X.data)[(int64_t)b * p.X.stride_b +
                                                  (int64_t)t * p.X.stride_t + a])
               : 0.f;
  }
  for (int i = threadIdx.x; i < B * T * doutp; i += kTinyThreads) {
    const int o = i % doutp, bt = i / doutp, t = bt % T, b = bt / T;
    const bool on = o < p.dout && (p.mask == nullptr || p.mask[(int64_t)b * T + t] != 0);
    gs[i] = on ? E::to_float(((const S*)p.G.data)[(int64_t)b * p.G.stride_b +
                                                  (int64_t)t * p.G.stride_t + o])
               : 0.f;
  }
  __syncthreads();
  const int nab = dinp / kTA, nblk = (doutp / kTO) * nab;
  const bool mine = (int)threadIdx.x < nblk;
  const int o0 = mine ? (threadIdx.x / nab) * kTO : 0, a0 = mine ? (threadIdx.x % nab) * kTA : 0;
  float acc[kTinyMaxB][kTO][kTA];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int b = 0; b < kTinyMaxB; ++b) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kTO; ++i)
#pragma unroll
      for (int j = 0; j < kTA; ++j) acc[b][i][j] = 0.f;
    if (b < B && mine) {
      const float* xb = xs + (size_t)b * T * dinp + a0;
      const float* gb = gs + (size_t)b * T * doutp + o0;
      for (int t = 0; t < T; ++t) {
        const f32x4 x = *(const f32x4*)(xb + (size_t)t * dinp);
        const float g0 = gb[(size_t)t * doutp], g1 = gb[(size_t)t * doutp + 1];
        acc[b][0][0] += g0 * x.x; acc[b][0][1] += g0 * x.y;
        acc[b][0][2] += g0 * x.z; acc[b][0][3] += g0 * x.w;
        acc[b][1][0] += g1 * x.x; acc[b][1][1] += g1 * x.y;
        acc[b][1][2] += g1 * x.z; acc[b][1][3] += g1 * x.w;
      }
#pragma unroll
      for (int i = 0; i < kTO; ++i)
#pragma unroll
        for (int j = 0; j < kTA; ++j) ss += acc[b][i][j] * acc[b][i][j];   // padding is zero
    }
    if (b < B) {
      const double w = wave_sum_f64((double)ss);
      if (lane == 0) red[b][wave] = w;
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < B) {
    const int b = threadIdx.x;
    double sq = 0.0;
    for (int w = 0; w < kTinyWaves; ++w) sq += red[b][w];
    float c, n;
    tiny_clip(sq, C, &c, &n);
    if (norms_out != nullptr) norms_out[b] = n;
    cs[b] = c;
  }
  __syncthreads();
  if (!mine) return;
#pragma unroll
  for (int i = 0; i < kTO; ++i) {
    const int o = o0 + i;
    if (o >= p.dout) continue;
#pragma unroll
    for (int j = 0; j < kTA; ++j) {
      const int a = a0 + j;
      if (a >= p.din) continue;
      float v = 0.f;
#pragma unroll
      for (int b = 0; b < kTinyMaxB; ++b)
        if (b < B) v += cs[b] * acc[b][i][j];
      const uint64_t e = (uint64_t)o * p.din + a;
      if (p.noise_std != 0.0f) v += p.noise_std * normal_at(p.seed, p.offset, e);
      v = v / p.denom;
      if (p.beta) v += p.out[e];
      p.out[e] = v;
    }
  }
}

}  // namespace

bool tiny_eligible(const LayerArgs& p) {
  const int64_t dinp = pad_to(p.din, kTA), doutp = pad_to(p.dout, kTO);
  return p.B <= kTinyMaxB && (doutp / kTO) * (dinp / kTA) <= kTinyThreads &&
         (int64_t)p.B * p.T * (dinp + doutp) * (int64_t)sizeof(float) <= kTinyLdsBytes &&
         2.0 * p.B * p.T * (double)p.din * p.dout <= kTinyMaxFlops;
}

hipError_t launch_tiny_layer(const LayerArgs& p, float C, float* norms_out, hipStream_t s) {
  if (!tiny_eligible(p)) return hipErrorInvalidValue;
  const size_t lds = (size_t)p.B * p.T * (pad_to(p.din, kTA) + pad_to(p.dout, kTO)) * sizeof(float);
  timing_begin("tiny_layer", s);
  if (p.dtype == kBF16)
    hipLaunchKernelGGL(tiny_layer_kernel<BF16>, dim3(1), dim3(kTinyThreads), lds, s, p, C,
                       norms_out);
  else
    hipLaunchKernelGGL(tiny_layer_kernel<F32>, dim3(1), dim3(kTinyThreads), lds, s, p, C,
                       norms_out);
  const hipError_t e = hipGetLastError();
  timing_end("tiny_layer", s);
  return e;
}

}  // namespace dpf
