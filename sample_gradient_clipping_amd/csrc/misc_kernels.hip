// Small kernels: Philox/Gaussian fills, mask tile flags, ordered finalize.
#include <atomic>

#include "kernels.hpp"

namespace dpf {

// out[4j..4j+3] = Philox4x32-10 words of block offset + j.
__global__ void philox_fill_kernel(uint64_t seed, uint64_t offset, int64_t nblocks, u32x4* out) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < nblocks) out[j] = philox_block(seed, offset + (uint64_t)j);
}

// out[e] = scale * xi_e, four elements (one Philox block) per thread.
__global__ void gaussian_fill_kernel(uint64_t seed, uint64_t offset, int64_t n, float scale,
                                     int dtype, void* out) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t e0 = 4 * j;
  if (e0 >= n) return;
  const f32x4 z = normals_of_block(philox_block(seed, offset + (uint64_t)j));
  const float v[4] = {scale * z.x, scale * z.y, scale * z.z, scale * z.w};
  if (dtype == kF32) {
    float* o = (float*)out + e0;
    if (e0 + 4 <= n) {
      f32x4 w; w.x = v[0]; w.y = v[1]; w.z = v[2]; w.w = v[3];
      *(f32x4*)o = w;
    } else {
      for (int e = 0; e < 4 && e0 + e < n; ++e) o[e] = v[e];
    }
  } else {
    uint16_t* o = (uint16_t*)out + e0;
    if (e0 + 4 <= n) {
      u16x4 w;
      w.s0 = f32_to_bf16_rne(v[0]); w.s1 = f32_to_bf16_rne(v[1]);
      w.s2 = f32_to_bf16_rne(v[2]); w.s3 = f32_to_bf16_rne(v[3]);
      *(u16x4*)o = w;
    } else {
      for (int e = 0; e < 4 && e0 + e < n; ++e) o[e] = f32_to_bf16_rne(v[e]);
    }
  }
}

// bits[b, w] bit r = token 32 w + r of sample b is active (< T and mask != 0).
// One wave per two words: lanes 0..31 -> word 2j, lanes 32..63 -> word 2j+1.
__global__ void row_bits_kernel(const uint8_t* mask, int B, int T, uint32_t* bits, int nwords) {
  const int64_t pair = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t wi = 2 * pair + (lane >> 5);
  const int64_t total = (int64_t)B * nwords;
  bool a = false;
  if (wi < total) {
    const int b = (int)(wi / nwords), w = (int)(wi % nwords);
    const int t = w * kBitsTokens + (lane & 31);
    a = t < T && mask[(int64_t)b * T + t] != 0;
  }
  const uint64_t ball = __ballot(a);
  if (wi < total && (lane & 31) == 0) bits[wi] = (uint32_t)(ball >> (lane & 32));
}

// Active-step list (layout in kernels.hpp) from the row bits: one workgroup
// walks the words in order, 1024 at a time; an entry's index is the number
// of active words before it (ballot counts within a wave, then wave totals).
// Each word also checks that its sample stays a prefix through it: an empty
// word is followed by an empty one, and a word that is not full is a run of
// low bits followed by an empty one (the last word of a sample counts as
// followed by an empty one).
constexpr int kListThreads = 1024;
__global__ void __launch_bounds__(kListThreads) step_list_kernel(const uint32_t* bits, int B,
                                                                 int nwords, uint32_t* steps) {
  __shared__ uint32_t wave_count[kListThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t total = (int64_t)B * nwords;
  uint32_t* entries = steps + 2 + B;
  uint32_t base = 0;                  // active words before this chunk (same in every thread)
  int prefix = 1;                     // every word so far keeps its sample a prefix
  for (int64_t c0 = 0; c0 < total; c0 += kListThreads) {
    const int64_t i = c0 + tid;
    const bool act = i < total && bits[i] != 0u;
    bool ok = true;
    if (i < total) {
      const uint32_t x = bits[i];
      const uint32_t next = (i % nwords) + 1 < nwords ? bits[i + 1] : 0u;
      ok = x == 0u ? next == 0u : ((x & (x + 1u)) == 0u && (x == 0xffffffffu || next == 0u));
    }
    prefix = __syncthreads_and(prefix && ok);
    const uint64_t ball = __ballot(act);
    const uint32_t below = (uint32_t)__popcll(ball & ((1ull << lane) - 1ull));
    if (lane == 0) wave_count[wave] = (uint32_t)__popcll(ball);
    __syncthreads();
    uint32_t before = 0, chunk = 0;
    for (int w = 0; w < kListThreads / 64; ++w) {
      if (w < wave) before += wave_count[w];
      chunk += wave_count[w];
    }
    const uint32_t idx = base + before + below;
    if (i < total) {
      const int b = (int)(i / nwords), w = (int)(i % nwords);
      if (w == 0) steps[1 + b] = idx;
      if (act) entries[idx] = ((uint32_t)b << 16) | (uint32_t)w;
    }
    base += chunk;
    __syncthreads();                  // wave_count is rewritten by the next chunk
  }
  if (tid == 0) {
    steps[0] = base | (prefix ? kStepsPrefix : 0u);
    steps[1 + B] = base;
    entries[base] = 0u;               // spare entry
  }
}

__device__ __forceinline__ void clip_of_sq(double sq, float C, float* c, float* n) {
  // Rounding can leave a tiny negative sum when g_i ~ 0; NaN must pass through.
  const double nn = sqrt(sq < 0.0 ? 0.0 : sq);
  *n = (float)nn;
  *c = (nn <= (double)C) ? 1.0f : (float)((double)C / nn);
}

// One workgroup per sample.  Thread t sums partials t, t + 1024, ... in index
// order (four loads in flight at a time); the 1024 sums are then combined by
// the fixed tree of block_sum_f64, so the result does not depend on timing.
constexpr int kFinThreads = 1024;
__global__ void __launch_bounds__(kFinThreads) finalize_kernel(const double* partials, int np,
                                                               double* sq_io, int accumulate,
                                                               float C, float* c_out,
                                                               float* norms_out) {
  __shared__ double red[kFinThreads / 64];
  const int b = blockIdx.x;
  const double* row = partials + (int64_t)b * np;
  double part = 0.0;
  int i = threadIdx.x;
  for (; i + 3 * kFinThreads < np; i += 4 * kFinThreads) {
    const double v0 = row[i], v1 = row[i + kFinThreads];
    const double v2 = row[i + 2 * kFinThreads], v3 = row[i + 3 * kFinThreads];
    part += v0;
    part += v1;
    part += v2;
    part += v3;
  }
  for (; i < np; i += kFinThreads) part += row[i];
  double sq = block_sum_f64(part, red);
  if (threadIdx.x != 0) return;
  if (sq_io != nullptr) {
    if (accumulate) sq += sq_io[b];
    sq_io[b] = sq;
  }
  if (c_out != nullptr) {
    float c, n;
    clip_of_sq(sq, C, &c, &n);
    c_out[b] = c;
    if (norms_out != nullptr) norms_out[b] = n;
  }
}

__global__ void clip_from_sq_kernel(const double* sq, int64_t n, float C, float* c_out,
                                    float* norms_out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float c, nn;
  clip_of_sq(sq[i], C, &c, &nn);
  c_out[i] = c;
  if (norms_out != nullptr) norms_out[i] = nn;
}

// ---------------------------------------------------------------------------
static inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

hipError_t launch_philox_fill(uint64_t seed, uint64_t offset, int64_t nblocks, uint32_t* out,
                              hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  timing_begin("philox_fill", s);
  hipLaunchKernelGGL(philox_fill_kernel, dim3(blocks_for(nblocks, 256)), dim3(256), 0, s, seed,
                     offset, nblocks, (u32x4*)out);
  timing_end("philox_fill", s);
  return hipGetLastError();
}

hipError_t launch_gaussian_fill(uint64_t seed, uint64_t offset, int64_t n, float scale, int dtype,
                                void* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  timing_begin("gaussian_fill", s);
  hipLaunchKernelGGL(gaussian_fill_kernel, dim3(blocks_for((n + 3) / 4, 256)), dim3(256), 0, s,
                     seed, offset, n, scale, dtype, out);
  timing_end("gaussian_fill", s);
  return hipGetLastError();
}

hipError_t launch_row_bits(const uint8_t* mask, int B, int T, uint32_t* bits, int nwords,
                           hipStream_t s) {
  const int64_t waves = ((int64_t)B * nwords + 1) / 2;
  timing_begin("row_bits", s);
  hipLaunchKernelGGL(row_bits_kernel, dim3(blocks_for(waves, 4)), dim3(256), 0, s, mask, B, T,
                     bits, nwords);
  timing_end("row_bits", s);
  return hipGetLastError();
}

hipError_t launch_step_list(const uint32_t* bits, int B, int nwords, uint32_t* steps,
                            hipStream_t s) {
  timing_begin("step_list", s);
  hipLaunchKernelGGL(step_list_kernel, dim3(1), dim3(kListThreads), 0, s, bits, B, nwords, steps);
  timing_end("step_list", s);
  return hipGetLastError();
}

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  int n = cache[dev].load();
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 1;
    cache[dev].store(n);
  }
  return n;
}

hipError_t launch_finalize(const double* partials, int B, int np, double* sq_io, int accumulate,
                           float C, float* c_out, float* norms_out, hipStream_t s) {
  timing_begin("finalize", s);
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)B), dim3(kFinThreads), 0, s, partials, np,
                     sq_io, accumulate, C, c_out, norms_out);
  timing_end("finalize", s);
  return hipGetLastError();
}

hipError_t launch_clip_from_sq(const double* sq, int64_t n, float C, float* c_out,
                               float* norms_out, hipStream_t s) {
  timing_begin("clip_factors", s);
  hipLaunchKernelGGL(clip_from_sq_kernel, dim3(blocks_for(n, 64)), dim3(64), 0, s, sq, n, C,
                     c_out, norms_out);
  timing_end("clip_factors", s);
  return hipGetLastError();
}

}  // namespace dpf
