// Internal (C++) interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dpf {

enum DType { kF32 = 0, kBF16 = 1 };
// kStaged (large-tile path only): the direct kernel also stores every
// per-sample gradient tile (fp32) in the workspace, and the accumulate phase
// is launch_staged_combine over those tiles instead of a second contraction.
// kOnePass (large-tile layout, single-layer calls only): one cooperative
// kernel computes each per-sample gradient tile once, reduces the per-sample
// norms across workgroups and adds c_i g_i to a running sum in registers
// (launch_onepass); no separate norm or accumulate phase.
enum class NormPath { kAuto = 0, kGram = 1, kDirect = 2, kStaged = 3, kOnePass = 4 };

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
  float denom;              // the sum is divided by this (B unless the caller gives another)
  int beta;                 // 1: out += result; 0: out = result
  float* out;               // [dout, din]
  double* partials;         // [B, norm_partials_per_sample] (norm kernels)
  const uint32_t* steps;    // active-step list (large-tile kernels, masked calls) or null
  float* skws;              // partials of split tiles / items (large-tile kernels), or null
  int max_split;            // 1: never split a tile or Gram item (no split partials in
                            // skws); 0: as the cost model picks
  int small_tiles;          // few-tile outputs (the projected variant's r-space sums):
                            // 1 accumulate over 128 x 128 tiles whose samples are cut
                            // into pieces (partials in skws); 2 also the direct norm
                            // over 128 x 128 tiles; 0 the large tiles
};

// Active-step list of a masked call, built from the row bits:
//   steps[0]          n, the number of (sample, 32-token step) pairs with an active
//                     token, in bits 0-30; bit 31 set when every sample's active
//                     tokens are a prefix of its rows (its steps 0 .. k - 1, all rows
//                     active except in step k - 1)
//   steps[1 + b]      index of sample b's first entry (b = 0..B; steps[1 + B] = n)
//   steps[2 + B + k]  entry k = sample << 16 | step, sample-major (k < n), then one
//                     spare zero entry, so that reading entry n stays in bounds.
constexpr uint32_t kStepCountMask = 0x7fffffffu;
constexpr uint32_t kStepsPrefix = 0x80000000u;
inline size_t step_list_words(int B, int nwords) { return (size_t)B * nwords + B + 3; }

struct ProjArgs {
  Act X;                    // [B, T, din]
  const void* P;            // [din, r]
  void* Y;                  // [B, T, r] contiguous, X's dtype
  int dtype;
  int B, T, din, r;
  const uint8_t* mask;
  float* part;              // [splits, B*T, r] fp32 partial products when splits > 1
  int splits;               // din chunks, one workgroup each per output tile
  // gen != 0: P is not read but regenerated, P[d][j] = p_scale * xi_{d*r+j}
  // from Philox (p_seed, p_offset), rounded to X's dtype (as gaussian_fill).
  int gen;
  uint64_t p_seed, p_offset;
  float p_scale;
};

// Bias gradients (bias.hip): gb[b][o] = sum of the active rows of G_b, and
// sq[b] += ||gb[b]||^2; then out[o] = (sum_b c[b] gb[b][o] + noise_std xi_o) / B.
// part: bias_workspace_bytes(B, T, dout) of scratch for the token-chunk sums.
size_t bias_workspace_bytes(int B, int T, int dout);
hipError_t launch_bias_grads(const Act& G, int dtype, int B, int T, int dout, const uint8_t* mask,
                             float* part, float* gb, double* sq, hipStream_t s);
hipError_t launch_bias_accumulate(const float* gb, const float* c, int B, int dout,
                                  float noise_std, uint64_t seed, uint64_t offset, float* out,
                                  hipStream_t s);

// The whole step in one workgroup for tiny layers (tiny.hip): eligible when
// B <= kTinyMaxB, one thread per 2 x 4 block of outputs fits the workgroup,
// every sample's X and G rows fit kTinyLdsBytes as float32, and the call is
// at most kTinyMaxFlops.  Writes out and norms_out.
constexpr int kTinyMaxB = 8;
constexpr int kTinyLdsBytes = 64 * 1024;
constexpr double kTinyMaxFlops = 4.0e6;
bool tiny_eligible(const LayerArgs& p);
hipError_t launch_tiny_layer(const LayerArgs& p, float C, float* norms_out, hipStream_t s);

// One projected Adam step (optim.hip).
struct AdamArgs {
  const float* grad;        // [dout, r] privatised projected gradient
  float* m;                 // [dout, r] first moment, updated in place
  float* v;                 // [dout, r] second moment, updated in place
  float* u;                 // [dout, r] workspace: the bias-corrected direction
  float* W;                 // [dout, din] float32 weight, updated in place
  int64_t dout, din, r;
  float lr, beta1, beta2, eps, bc1, bc2;   // bc_k = 1 - beta_k^step
  const void* P;            // [din, r] of p_dtype, unless gen
  int p_dtype;
  int gen;                  // P[d][j] = p_scale * xi_{d*r+j}(p_seed, p_offset), rounded to p_dtype
  uint64_t p_seed, p_offset;
  float p_scale;
  void* pbuf;               // [din, r] of p_dtype, workspace when adam_draws_p_once(a)
};
// True when a seeded P is drawn once into a.pbuf (gaussian fill) and read
// from there, rather than drawn again by every row of W tiles.
bool adam_draws_p_once(const AdamArgs& a);
// Process-wide: when on, a seeded P is always drawn inside the projection
// and update kernels where it is used, and never exists in memory.
void set_p_in_kernels(bool on);
bool p_in_kernels();
hipError_t launch_projected_adam(const AdamArgs& a, hipStream_t s);

// Launchers (gemm_kernels.hip).  `vec` selects 16-byte vector loads; the
// caller has checked alignment of every pointer, dimension and stride.
// True when (p, vec) runs on the large-tile bf16 kernels; a masked call on
// them needs the active-step list (p.steps).
bool big_path(const LayerArgs& p, bool vec);
// Device workspace bytes launch_accumulate / launch_norm need for (p, vec),
// passed in as p.skws (0: none).  The two phases run one after the other on
// one stream and may share the buffer.
size_t accumulate_workspace_bytes(const LayerArgs& p, bool vec);
size_t norm_workspace_bytes(const LayerArgs& p, NormPath path, bool vec);
hipError_t launch_accumulate(const LayerArgs& p, bool vec, hipStream_t s);
// Accumulate phase of the staged path: out from the tiles launch_norm stored.
hipError_t launch_staged_combine(const LayerArgs& p, hipStream_t s);
hipError_t launch_norm(const LayerArgs& p, NormPath path, bool vec, hipStream_t s);
hipError_t launch_project(const ProjArgs& p, bool vec, hipStream_t s);
// Number of din chunks launch_project splits Y = X P into, and the fp32
// partial buffer (p.part) that takes when above 1.
int project_splits(const ProjArgs& p, bool vec);
size_t project_workspace_bytes(const ProjArgs& p, bool vec);
// The bf16 projection kernel (proj_big.hip): the shape conditions alone, and
// with the pointers of a call (P 16-byte, Y 8-byte aligned).
bool project_big_shape_ok(const ProjArgs& p, bool vec);
bool project_big_eligible(const ProjArgs& p, bool vec);
hipError_t launch_project_big(const ProjArgs& p, hipStream_t s);
// Partials per sample written by the norm kernel launch_norm picks for (p, path, vec).
int norm_partials_per_sample(const LayerArgs& p, NormPath path, bool vec);

// Large-tile bf16 kernels (accum_big.hip).
int big_tiles(int din, int dout);
size_t accumulate_big_workspace_bytes(const LayerArgs& p);
hipError_t launch_accumulate_big(const LayerArgs& p, hipStream_t s);
hipError_t launch_direct_norm_big(const LayerArgs& p, hipStream_t s);
size_t staged_big_workspace_bytes(const LayerArgs& p);
int staged_big_partials_per_sample(const LayerArgs& p);
int direct_big_partials_per_sample(const LayerArgs& p);
hipError_t launch_staged_norm_big(const LayerArgs& p, hipStream_t s);
hipError_t launch_staged_combine_big(const LayerArgs& p, hipStream_t s);

// Single-pass fused kernel (onepass.hip): one workgroup per 128 x 128 output
// tile, all resident at once.  p.partials: onepass_workspace_bytes(p) of
// per-(sample, tile) slots.  Writes p.out (with noise, / denom, beta) and
// norms_out.  hipErrorCooperativeLaunchTooLarge when the tiles cannot all
// be resident.
int onepass_tiles(int din, int dout);
int onepass_resident_limit();
size_t onepass_workspace_bytes(const LayerArgs& p);
hipError_t launch_onepass(const LayerArgs& p, float C, float* norms_out, hipStream_t s);
// Testing hooks of the single-pass kernel's bounded waits: tries of a
// blocking poll (default 2^20), and never_ready != 0 to treat every fetch of
// partials as incomplete (every bounded wait then gives up: NaN outputs).
void set_onepass_testing(int spin_limit, int never_ready);

// Large-tile bf16 Gram-norm kernel (gram_big.hip).
int gram_big_items_per_sample(int T);
size_t gram_big_workspace_bytes(const LayerArgs& p);
hipError_t launch_gram_norm_big(const LayerArgs& p, hipStream_t s);

// Small kernels (misc_kernels.hip).
hipError_t launch_row_bits(const uint8_t* mask, int B, int T, uint32_t* bits, int nwords,
                           hipStream_t s);
hipError_t launch_step_list(const uint32_t* bits, int B, int nwords, uint32_t* steps, hipStream_t s);
// Compute units of the current device (cached per device).
int device_cus();
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
