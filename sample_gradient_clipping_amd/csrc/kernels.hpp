// Internal (C++) interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dpf {

enum DType { kF32 = 0, kBF16 = 1 };
enum class NormPath { kAuto = 0, kGram = 1, kDirect = 2 };

// Tokens covered by one word of the per-sample row-activity bits.
constexpr int kBitsTokens = 32;

struct LayerArgs {
  Act X, G;                 // [B, T, din] and [B, T, dout]
  int dtype;                // DType
  int B, T, din, dout;
  const uint8_t* mask;      // [B, T] or null
  const uint32_t* rowbits;  // [B, nwords]: bit r of word w = token 32 w + r is active; null = no mask
  int nwords;               // ceil(T / 32)
  const float* c;           // [B] clip factors (accumulate only)
  float noise_std;          // sigma * C (0 = no noise)
  uint64_t seed, offset;
  float* out;               // [dout, din]
  double* partials;         // [B, norm_partials_per_sample] (norm kernels)
};

struct ProjArgs {
  Act X;                    // [B, T, din]
  const void* P;            // [din, r]
  void* Y;                  // [B, T, r] contiguous, X's dtype
  int dtype;
  int B, T, din, r;
  const uint8_t* mask;
};

// Launchers (gemm_kernels.hip).  `vec` selects 16-byte vector loads; the
// caller has checked alignment of every pointer, dimension and stride.
hipError_t launch_accumulate(const LayerArgs& p, bool vec, hipStream_t s);
hipError_t launch_norm(const LayerArgs& p, NormPath path, bool vec, hipStream_t s);
hipError_t launch_project(const ProjArgs& p, bool vec, hipStream_t s);
// Partials per sample written by the norm kernel launch_norm picks for (p, path, vec).
int norm_partials_per_sample(const LayerArgs& p, NormPath path, bool vec);

// Large-tile bf16 kernels (accum_big.hip).
int big_tiles(int din, int dout);
hipError_t launch_accumulate_big(const LayerArgs& p, hipStream_t s);
hipError_t launch_direct_norm_big(const LayerArgs& p, hipStream_t s);

// Large-tile bf16 Gram-norm kernel (gram_big.hip).
int gram_big_items_per_sample(int T);
hipError_t launch_gram_norm_big(const LayerArgs& p, hipStream_t s);

// Small kernels (misc_kernels.hip).
hipError_t launch_row_bits(const uint8_t* mask, int B, int T, uint32_t* bits, int nwords,
                           hipStream_t s);
// Per sample: sq = ordered sum of np partials; optionally added into sq_io;
// then c = clip factor and norms = sqrt(sq) when c_out is given.
hipError_t launch_finalize(const double* partials, int B, int np, double* sq_io, int accumulate,
                           float C, float* c_out, float* norms_out, hipStream_t s);
hipError_t launch_clip_from_sq(const double* sq, int64_t n, float C, float* c_out,
                               float* norms_out, hipStream_t s);
hipError_t launch_philox_fill(uint64_t seed, uint64_t offset, int64_t nblocks, uint32_t* out,
                              hipStream_t s);
hipError_t launch_gaussian_fill(uint64_t seed, uint64_t offset, int64_t n, float scale, int dtype,
                                void* out, hipStream_t s);

// Timing hooks (api.cpp): bracket one kernel launch on `s` when enabled.
void timing_begin(const char* name, hipStream_t s);
void timing_end(const char* name, hipStream_t s);

}  // namespace dpf
