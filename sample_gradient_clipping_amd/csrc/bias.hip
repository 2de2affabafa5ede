// Bias gradients of a linear layer y = x W^T + b, clipped together with the
// weight gradient (the layer's parameters are W and b: sample i's gradient
// is the pair (g_i, gb_i), whose norm is sqrt(||g_i||^2 + ||gb_i||^2)).
//
//   bias_grad_kernel       gb[b][o] = sum over the active tokens t of G[b][t][o]
//                          (float32, token order; masked rows selected to zero)
//   bias_sq_kernel         sq[b] += ||gb[b]||^2 (float64, fixed order)
//   bias_accumulate_kernel out[o] = (sum_b c[b] gb[b][o] + noise_std xi_o) / B
//                          (samples in order; xi from the given Philox offset)
#include "kernels.hpp"

namespace dpf {
namespace {

constexpr int kCols = 256;

template <class E>
__global__ void __launch_bounds__(kCols) bias_grad_kernel(Act G, int T, int dout,
                                                          const uint8_t* mask, float* gb) {
  using S = typename E::storage;
  const int b = blockIdx.y;
  const int o = blockIdx.x * kCols + threadIdx.x;
  if (o >= dout) return;
  const S* g = (const S*)G.data + (int64_t)b * G.stride_b + o;
  const uint8_t* m = mask != nullptr ? mask + (int64_t)b * T : nullptr;
  float sum = 0.f;
#pragma unroll 8
  for (int t = 0; t < T; ++t) {
    const float v = E::to_float(g[(int64_t)t * G.stride_t]);
    if (m == nullptr || m[t] != 0) sum += v;   // select: a masked row is never added
  }
  gb[(int64_t)b * dout + o] = sum;
}

__global__ void __launch_bounds__(kCols) bias_sq_kernel(const float* gb, int dout, double* sq) {
  __shared__ double red[kCols / 64];
  const int b = blockIdx.x;
  double s = 0.0;
  for (int o = threadIdx.x; o < dout; o += kCols) {
    const double v = gb[(int64_t)b * dout + o];
    s += v * v;
  }
  const double tot = block_sum_f64(s, red);
  if (threadIdx.x == 0) sq[b] += tot;
}

__global__ void __launch_bounds__(kCols) bias_accumulate_kernel(const float* gb, const float* c,
                                                                int B, int dout, float noise_std,
                                                                uint64_t seed, uint64_t offset,
                                                                float* out) {
  const int64_t j = (int64_t)blockIdx.x * kCols + threadIdx.x;   // Philox block: columns 4j..4j+3
  const int64_t e0 = 4 * j;
  if (e0 >= dout) return;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < B; ++b) {
    const float cb = c[b];
    for (int k = 0; k < 4; ++k)
      if (e0 + k < dout) v[k] += cb * gb[(int64_t)b * dout + e0 + k];
  }
  const float rB = 1.0f / (float)B;   // as the weight epilogue
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  if (noise_std != 0.0f) z = normals_of_block(philox_block(seed, offset + (uint64_t)j));
  const float zz[4] = {z.x, z.y, z.z, z.w};
  for (int k = 0; k < 4; ++k)
    if (e0 + k < dout) out[e0 + k] = (v[k] + noise_std * zz[k]) * rB;
}

}  // namespace

hipError_t launch_bias_grads(const Act& G, int dtype, int B, int T, int dout, const uint8_t* mask,
                             float* gb, double* sq, hipStream_t s) {
  timing_begin("bias_grad", s);
  const dim3 grid((unsigned)((dout + kCols - 1) / kCols), (unsigned)B);
  if (dtype == kBF16)
    hipLaunchKernelGGL(bias_grad_kernel<BF16>, grid, dim3(kCols), 0, s, G, T, dout, mask, gb);
  else
    hipLaunchKernelGGL(bias_grad_kernel<F32>, grid, dim3(kCols), 0, s, G, T, dout, mask, gb);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    hipLaunchKernelGGL(bias_sq_kernel, dim3((unsigned)B), dim3(kCols), 0, s, (const float*)gb,
                       dout, sq);
    e = hipGetLastError();
  }
  timing_end("bias_grad", s);
  return e;
}

hipError_t launch_bias_accumulate(const float* gb, const float* c, int B, int dout,
                                  float noise_std, uint64_t seed, uint64_t offset, float* out,
                                  hipStream_t s) {
  timing_begin("bias_accumulate", s);
  const int64_t blocks = ((int64_t)dout + 3) / 4;
  hipLaunchKernelGGL(bias_accumulate_kernel, dim3((unsigned)((blocks + kCols - 1) / kCols)),
                     dim3(kCols), 0, s, gb, c, B, dout, noise_std, seed, offset, out);
  timing_end("bias_accumulate", s);
  return hipGetLastError();
}

}  // namespace dpf
