// Bias gradients of a linear layer y = x W^T + b, clipped together with the
// weight gradient (the layer's parameters are W and b: sample i's gradient
// is the pair (g_i, gb_i), whose norm is sqrt(||g_i||^2 + ||gb_i||^2)).
//
//   bias_grad_kernel       part[z][b][o] = sum over the active tokens t of chunk z
//                          of G[b][t][o] (float32, token order; masked rows
//                          selected to zero); the token chunks spread the
//                          latency-bound column sums over enough workgroups
//   bias_sq_kernel         gb[b][o] = sum over z of part[z][b][o] (chunk order),
//                          sq[b] += ||gb[b]||^2 (float64, fixed order)
//   bias_accumulate_kernel out[o] = (sum_b c[b] gb[b][o] + noise_std xi_o) / B
//                          (samples in order; xi from the given Philox offset)
#include <algorithm>

#include "kernels.hpp"

namespace dpf {
namespace {

constexpr int kCols = 256;

// V consecutive columns per thread: 8 bf16 columns as one 16-byte load when
// the rows allow it, else one column.
template <class E, int V>
__global__ void __launch_bounds__(kCols) bias_grad_kernel(Act G, int B, int T, int dout,
                                                          const uint8_t* mask, int chunk,
                                                          float* part) {
  using S = typename E::storage;
  const int b = blockIdx.y, z = blockIdx.z;
  const int o = (blockIdx.x * kCols + threadIdx.x) * V;
  if (o >= dout) return;
  const int t0 = z * chunk, t1 = min(T, t0 + chunk);
  const S* g = (const S*)G.data + (int64_t)b * G.stride_b + o;
  const uint8_t* m = mask != nullptr ? mask + (int64_t)b * T : nullptr;
  float sum[V];
#pragma unroll
  for (int k = 0; k < V; ++k) sum[k] = 0.f;
#pragma unroll 4
  for (int t = t0; t < t1; ++t) {
    if (m != nullptr && m[t] == 0) continue;   // a masked row is never read
    const S* row = g + (int64_t)t * G.stride_t;
    if constexpr (V == 8) {
      const u16x8 h = *(const u16x8*)row;
      sum[0] += E::to_float(h.s0); sum[1] += E::to_float(h.s1);
      sum[2] += E::to_float(h.s2); sum[3] += E::to_float(h.s3);
      sum[4] += E::to_float(h.s4); sum[5] += E::to_float(h.s5);
      sum[6] += E::to_float(h.s6); sum[7] += E::to_float(h.s7);
    } else {
      sum[0] += E::to_float(row[0]);
    }
  }
  float* dst = part + ((int64_t)z * B + b) * dout + o;
#pragma unroll
  for (int k = 0; k < V; ++k) dst[k] = sum[k];
}

constexpr int kSqThreads = 1024;
__global__ void __launch_bounds__(kSqThreads) bias_sq_kernel(const float* part, int nz, int B,
                                                             int dout, float* gb, double* sq) {
  __shared__ double red[kSqThreads / 64];
  const int b = blockIdx.x;
  double s = 0.0;
  for (int o = threadIdx.x; o < dout; o += kSqThreads) {
    float v = 0.f;
    for (int z = 0; z < nz; ++z) v += part[((int64_t)z * B + b) * dout + o];
    gb[(int64_t)b * dout + o] = v;
    s += (double)v * (double)v;
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
  const int nk = (int)min((int64_t)4, dout - e0);
  // samples in order, eight at a time with their loads in flight together
  for (int b0 = 0; b0 < B; b0 += 8) {
    float w[8][4], cb[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int b = min(b0 + q, B - 1);
      cb[q] = c[b];
#pragma unroll
      for (int k = 0; k < 4; ++k) w[q][k] = k < nk ? gb[(int64_t)b * dout + e0 + k] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (b0 + q < B) {
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] += cb[q] * w[q][k];
      }
  }
  const float rB = 1.0f / (float)B;   // as the weight epilogue
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  if (noise_std != 0.0f) z = normals_of_block(philox_block(seed, offset + (uint64_t)j));
  const float zz[4] = {z.x, z.y, z.z, z.w};
  for (int k = 0; k < 4; ++k)
    if (e0 + k < dout) out[e0 + k] = (v[k] + noise_std * zz[k]) * rB;
}

}  // namespace

// Columns per thread: 8 (one 16-byte load) for bf16 rows that are 16-byte
// aligned, else 1.
int bias_vec(const Act& G, int dtype, int dout) {
  return dtype == kBF16 && dout % 8 == 0 && G.stride_t % 8 == 0 && G.stride_b % 8 == 0 &&
                 ((uintptr_t)G.data & 15) == 0
             ? 8
             : 1;
}

// Token chunks per column sum: enough (column block, sample, chunk) workgroups
// to cover the chip a few times, chunks of at least 32 tokens.
int bias_chunks(int B, int T, int dout, int vec) {
  const int64_t blocks = (int64_t)((dout + kCols * vec - 1) / (kCols * vec)) * B;
  const int64_t want = (2048 + blocks - 1) / blocks;
  const int64_t most = ((int64_t)T + 31) / 32;
  return (int)std::max<int64_t>(1, std::min<int64_t>(want, most));
}

// Fewer column blocks mean more chunks: size for whichever width is used.
size_t bias_workspace_bytes(int B, int T, int dout) {
  const int nz = std::max(bias_chunks(B, T, dout, 1), bias_chunks(B, T, dout, 8));
  return (size_t)nz * B * dout * sizeof(float);
}

hipError_t launch_bias_grads(const Act& G, int dtype, int B, int T, int dout, const uint8_t* mask,
                             float* part, float* gb, double* sq, hipStream_t s) {
  const int vec = bias_vec(G, dtype, dout);
  const int nz = bias_chunks(B, T, dout, vec);
  const int chunk = (T + nz - 1) / nz;
  timing_begin("bias_grad", s);
  const dim3 grid((unsigned)((dout + kCols * vec - 1) / (kCols * vec)), (unsigned)B, (unsigned)nz);
  if (vec == 8)
    hipLaunchKernelGGL((bias_grad_kernel<BF16, 8>), grid, dim3(kCols), 0, s, G, B, T, dout, mask,
                       chunk, part);
  else if (dtype == kBF16)
    hipLaunchKernelGGL((bias_grad_kernel<BF16, 1>), grid, dim3(kCols), 0, s, G, B, T, dout, mask,
                       chunk, part);
  else
    hipLaunchKernelGGL((bias_grad_kernel<F32, 1>), grid, dim3(kCols), 0, s, G, B, T, dout, mask,
                       chunk, part);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) {
    hipLaunchKernelGGL(bias_sq_kernel, dim3((unsigned)B), dim3(kSqThreads), 0, s,
                       (const float*)part, nz, B, dout, gb, sq);
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
