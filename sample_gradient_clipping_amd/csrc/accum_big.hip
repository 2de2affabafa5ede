// Large-tile bf16 kernels for the token-contraction G~^T X~ (K-outer x K-outer):
//
//   accumulate_big_kernel : grad = (sum_i c_i G~_i^T X~_i + noise_std xi) / B
//   direct_norm_big_kernel: per (output tile, sample) sum of squares of g_i's tile
//   staged_norm_big_kernel: the same, and g_i's tile itself stored (fp32) in a
//                           workspace; staged_combine_kernel then forms
//                           (sum_i c_i g_i + noise_std xi) / B from those tiles,
//                           so each per-sample gradient is computed only once
//
// Workgroup: 512 threads = 8 waves (2 x 4, two per SIMD); workgroup tile 256
// (din) x 256 (dout); each wave owns 128 x 64 = 4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16 accumulators (128 fp32 per lane).  K advances 32
// tokens per step.
//
// Data movement per step (32 tokens): global memory -> LDS by 16-byte-per-lane
// buffer loads that write LDS directly (no staging registers), into a ring
// of five 32 KiB slots, refilled four steps ahead.  LDS rows are 512 bytes with no
// padding; the 16-byte chunk c of row k is stored at chunk c ^ (4 (k mod 4)),
// which keeps the transposing 8-byte reads (ds_read_b64_tr_b16) free of bank
// conflicts on gfx950's 64 banks.  Masked rows and columns past the end are
// read through out-of-range buffer offsets, which return zeros.
//
// Output tiles are ordered so that the workgroups resident on one XCD at a
// time cover a compact block of tiles (shared X and G strips stay in that
// XCD's L2).
#include <algorithm>

#include "kernels.hpp"
#include "tiles.hpp"

namespace dpf {
namespace big {

constexpr int kNT = 512;                // 8 waves: two per SIMD
constexpr int kWaveRows = 2, kWaveCols = 4;   // wave grid over the 256 x 256 tile
constexpr int kBA = 4, kBO = 2;         // 32x32 accumulator blocks per wave: 128 (din) x 64 (dout)
constexpr int kTile = 256;              // both output dims
constexpr int kKT = 32;                 // tokens per step (one LDS slot)
constexpr int kRowBytes = kTile * 2;    // one LDS row (bf16)
constexpr int kOpBytes = kKT * kRowBytes;      // one operand, one slot: 16 KiB
constexpr int kStageBytes = 2 * kOpBytes;      // X and G: 32 KiB
constexpr int kStages = 5;                     // 160 KiB: all of gfx950's LDS
constexpr int kLdsBytes = kStages * kStageBytes;
constexpr int kWaves = kNT / 64;
constexpr int kRowsPerWave = kKT / kWaves;        // 4 rows of each operand per wave per step
constexpr int kDmaPerOp = kRowsPerWave / 2;       // 2 DMAs (2 rows each) per operand
constexpr int kDmaPerStep = 2 * kDmaPerOp;        // per wave
constexpr int kGroupRows = 4;           // grouped raster: tiles of 4 rows share an L2 window

typedef __attribute__((address_space(4))) const uint32_t c_u32;
typedef __attribute__((address_space(4))) const float c_f32;

__device__ __forceinline__ int swz(int k, int c16) { return c16 ^ ((k & 3) << 2); }

// Out-of-range buffer offsets read as zero without touching memory.
constexpr int kOOB = 0x7ffffff0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sample_rsrc(const Act& a, int b, int T, int D) {
  const char* base = (const char*)a.data + (int64_t)b * a.stride_b * 2;
  const int64_t bytes = ((int64_t)(T - 1) * a.stride_t + D) * 2;
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0,
                                           (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff),
                                           0x00020000);
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane.
// Issued from inline asm so that the compiler does not put a vmcnt(0) wait
// in front of every LDS read; completion is awaited explicitly (wait_dma).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, int voffset, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(lds)
               : "memory");
}

// Wait until at most `steps` of this wave's most recent DMA steps are in flight.
__device__ __forceinline__ void wait_dma(int steps) {
  static_assert(kDmaPerStep == 4, "wait_dma encodes 4 DMAs per step");
  if (steps <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (steps == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if (steps == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (steps == 3) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const unsigned char*)p;
}

// Token masks come in three forms (MASK): 0 none; 1 a mask, stepped through
// by the call's active-step list (one list entry and one row-bit word read
// per step); 2 a mask in which every sample's active tokens are a prefix of
// its rows (padding at the end), stepped through by the samples' step
// ranges, so that only a change of sample reads memory.
//
// Active-row bits of the 32 tokens of step s of sample b.  With a mask they
// are in memory; otherwise only the tail past T is inactive, and no memory
// is read -- which keeps scalar loads out of the main loop, so the compiler
// can wait for LDS reads precisely.
template <int MASK>
__device__ __forceinline__ uint32_t step_bits(const LayerArgs& p, int b, int s) {
  if constexpr (MASK) return ((c_u32*)p.rowbits)[(int64_t)b * p.nwords + s];
  const int n = p.T - s * kKT;
  return n >= 32 ? 0xffffffffu : ((1u << n) - 1u);
}

// MASK 2: the sample whose step range holds position k0 of the call's steps
// (k0 < n): the last b with first step <= k0, by bisection over the samples'
// first-step indices (samples without a step share their successor's).
__device__ __forceinline__ int prefix_sample_of(const LayerArgs& p, int k0) {
  int lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int)((c_u32*)p.steps)[1 + mid] <= k0) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Per-lane, per-step-invariant part of the DMA addressing: lane l of DMA j
// (of this wave) fills physical 16-byte chunk l % 32 of tile row r =
// 4 wave + 2 j + l / 32, i.e. logical chunk (l % 32) ^ swizzle(r).  A column
// past the end of the row gets an offset of kOOB or more, which stays out of
// range once the step's row offset (< 2 GiB) is added.
struct DmaLane {
  uint32_t xoff[kDmaPerOp], goff[kDmaPerOp];
  __device__ __forceinline__ void init(const LayerArgs& p, int a0, int o0) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < kDmaPerOp; ++j) {
      const int r = kRowsPerWave * wave + 2 * j + (lane >> 5);
      const int c16 = (lane & 31) ^ ((r & 3) << 2);
      const int ca = a0 + c16 * 8, co = o0 + c16 * 8;
      xoff[j] = ca < p.din ? (uint32_t)(((int64_t)r * p.X.stride_t + ca) * 2) : (uint32_t)kOOB;
      goff[j] = co < p.dout ? (uint32_t)(((int64_t)r * p.G.stride_t + co) * 2) : (uint32_t)kOOB;
    }
  }
};

// Issue side of the pipeline: the next step to queue, with the buffer
// descriptors of its sample (rebuilt only when the sample changes) and the
// byte offsets of its first token row in X and G.  Without a mask, steps
// run through every sample in order and the offsets advance by constant
// increments; with one, the active-step list gives each step.
template <int MASK>
struct Issue {
  __amdgpu_buffer_rsrc_t rx, rg;
  int b, s, k, nsteps;
  uint32_t xs, gs, dx, dg;     // byte offsets of the step; per-step increments
  uint32_t wdst;               // this wave's rows within a slot (LDS bytes)
  uint32_t bits;               // with a mask: this wave's rows' activity bits of the step
  const uint32_t* list;
  int ns, nxt;                 // MASK 2: steps of sample b, index of sample b + 1's first step
  uint32_t last;               // MASK 2: row bits of sample b's last step
  __device__ __forceinline__ void rsrc(const LayerArgs& p) {
    rx = sample_rsrc(p.X, b, p.T, p.din);
    rg = sample_rsrc(p.G, b, p.T, p.dout);
  }
  __device__ __forceinline__ void load(const LayerArgs& p) {
    const uint32_t v = ((c_u32*)list)[k];
    const int nb = (int)(v >> 16);
    s = (int)(v & 0xffffu);
    xs = (uint32_t)s * dx;     // < 2^31: span checked on the host
    gs = (uint32_t)s * dg;
    if (nb != b) {
      b = nb;
      rsrc(p);
    }
    bits = step_bits<MASK>(p, b, s) >> (wdst / kRowBytes);
  }
  // MASK 2: sample b's steps are 0 .. ns - 1, every row active but in the
  // last step, whose bits are `last`.
  __device__ __forceinline__ void prefix_bits() {
    bits = (s == ns - 1 ? last : 0xffffffffu) >> (wdst / kRowBytes);
  }
  __device__ __forceinline__ void prefix_enter(const LayerArgs& p) {
    last = ((c_u32*)p.rowbits)[(int64_t)b * p.nwords + ns - 1];
    rsrc(p);
  }
  __device__ __forceinline__ void start(const LayerArgs& p, int k0) {
    nsteps = (p.T + kKT - 1) / kKT;
    dx = (uint32_t)kKT * (uint32_t)p.X.stride_t * 2u;
    dg = (uint32_t)kKT * (uint32_t)p.G.stride_t * 2u;
    wdst = (uint32_t)(kRowsPerWave * __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * kRowBytes);
    k = k0;
    if constexpr (MASK == 2) {
      b = prefix_sample_of(p, k0);
      const int first = (int)((c_u32*)p.steps)[1 + b];
      nxt = (int)((c_u32*)p.steps)[2 + b];
      ns = nxt - first;
      s = k0 - first;
      xs = (uint32_t)s * dx;
      gs = (uint32_t)s * dg;
      prefix_enter(p);
      prefix_bits();
    } else if constexpr (MASK) {
      list = p.steps + 2 + p.B;
      b = -1;
      load(p);
    } else {
      b = k0 / nsteps;
      s = k0 - b * nsteps;
      xs = (uint32_t)s * dx;
      gs = (uint32_t)s * dg;
      rsrc(p);
    }
  }
  // Only called while another step remains, so b stays a valid sample.
  __device__ __forceinline__ void advance(const LayerArgs& p) {
    ++k;
    if constexpr (MASK == 2) {
      if (++s == ns) {
        int first;
        do {                           // the next sample with a step
          ++b;
          first = nxt;
          nxt = (int)((c_u32*)p.steps)[2 + b];
        } while (nxt == first);
        ns = nxt - first;
        s = 0;
        xs = gs = 0u;
        prefix_enter(p);
      } else {
        xs += dx;
        gs += dg;
      }
      prefix_bits();
    } else if constexpr (MASK) {
      load(p);
    } else if (++s == nsteps) {
      s = 0;
      xs = gs = 0u;
      ++b;
      rsrc(p);
    } else {
      xs += dx;
      gs += dg;
    }
  }
  // DMA `d` (0..3) of this step into the slot at LDS address `stage`: pair
  // d / 2 (rows 4 wave + 2 (d / 2) + {0, 1}) of X (d even) or G (d odd).
  // With a mask, inactive rows read through out-of-range offsets.  Without
  // one, the rows past T of a tail step are already past the end of the
  // sample's buffer descriptor (row stride >= row length), so they read
  // zeros as they are.
  __device__ __forceinline__ void dma(const LayerArgs& p, const DmaLane& dl, uint32_t stage,
                                      int d) const {
    const int j = d >> 1;
    const int lane = threadIdx.x & 63;
    const uint32_t dst = stage + wdst + 2 * j * kRowBytes + (d & 1) * kOpBytes;
    uint32_t off = (d & 1) ? dl.goff[j] + gs : dl.xoff[j] + xs;
    if constexpr (MASK) {
      if (!((bits >> (2 * j + (lane >> 5))) & 1u)) off = (uint32_t)kOOB;
    }
    dma16((d & 1) ? rg : rx, (int)off, dst);
  }
  __device__ __forceinline__ void step(const LayerArgs& p, const DmaLane& dl, uint32_t stage) const {
#pragma unroll
    for (int d = 0; d < 2 * kDmaPerOp; ++d) dma(p, dl, stage, d);
  }
};

// MFMA operands of one 16-token k-substep for this wave: 4 X blocks (din
// rows) and 2 G blocks (dout rows), each read with two transposing 8-byte
// LDS reads (12 reads: within the 15 the LDS counter can track).
struct Frags {
  u16x8 a[kBA], b[kBO];
};

__device__ __forceinline__ u16x8 frag(const unsigned char* op, int m0, int ks) {
  const int lane = threadIdx.x & 63;
  const int krow = ks * 16 + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = m0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int c16 = col >> 3, half = (col >> 2) & 1;
  const unsigned char* p0 = op + krow * kRowBytes + swz(krow, c16) * 16 + half * 8;
  const unsigned char* p1 = op + (krow + 4) * kRowBytes + swz(krow + 4, c16) * 16 + half * 8;
  const u16x4 lo = lds_read_tr16((const uint16_t*)p0);
  const u16x4 hi = lds_read_tr16((const uint16_t*)p1);
  u16x8 f;
  f.s0 = lo.s0; f.s1 = lo.s1; f.s2 = lo.s2; f.s3 = lo.s3;
  f.s4 = hi.s0; f.s5 = hi.s1; f.s6 = hi.s2; f.s7 = hi.s3;
  return f;
}

__device__ __forceinline__ int wave_row() { return (threadIdx.x >> 6) / kWaveCols; }
__device__ __forceinline__ int wave_col() { return (threadIdx.x >> 6) % kWaveCols; }

__device__ __forceinline__ void read_frags(Frags& f, const unsigned char* stage, int ks) {
  const int wm = wave_row(), wn = wave_col();
#pragma unroll
  for (int i = 0; i < kBA; ++i) f.a[i] = frag(stage, wm * (kBA * 32) + i * 32, ks);
#pragma unroll
  for (int j = 0; j < kBO; ++j) f.b[j] = frag(stage + kOpBytes, wn * (kBO * 32) + j * 32, ks);
}

// Fragment q of a k-substep: q = 0, 1 are the G blocks b[0], b[1]; q = 2..5
// the X blocks a[0..3].  This is the order in which the MFMAs first need them.
__device__ __forceinline__ void read_frag(Frags& f, const unsigned char* stage, int ks, int q) {
  if (q < kBO) f.b[q] = frag(stage + kOpBytes, wave_col() * (kBO * 32) + q * 32, ks);
  else f.a[q - kBO] = frag(stage, wave_row() * (kBA * 32) + (q - kBO) * 32, ks);
}

// Nothing is scheduled across this point: it fixes the interleaving of
// MFMAs with LDS reads and DMA issue that the main loop spells out.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

struct Acc {
  f32x16 v[kBA][kBO];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kBA; ++i)
#pragma unroll
      for (int j = 0; j < kBO; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) v[i][j][r] = 0.f;
  }
  // Rescale block by block; the empty asm statements pin each block's
  // product back into accumulation registers, which keeps the scaled copy
  // from occupying ordinary VGPRs across the loop.
  __device__ __forceinline__ void scale(float s) {
#pragma unroll
    for (int i = 0; i < kBA; ++i)
#pragma unroll
      for (int j = 0; j < kBO; ++j) {
        f32x16 t = v[i][j];
        asm volatile("" : "+v"(t));
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] *= s;
        asm volatile("" : "+a"(t));
        v[i][j] = t;
      }
  }
  // Keep every MFMA issued so far on this side of the statement (an
  // ordering point; no instruction is emitted).
  __device__ __forceinline__ void pin() {
    asm volatile("" : "+a"(v[0][0]), "+a"(v[0][1]), "+a"(v[1][0]), "+a"(v[1][1]),
                      "+a"(v[2][0]), "+a"(v[2][1]), "+a"(v[3][0]), "+a"(v[3][1]));
  }
  // MFMA k of a k-substep: block (k / kBO, k % kBO).
  __device__ __forceinline__ void mma1(const Frags& f, int k) {
    v[k / kBO][k % kBO] = mfma_32x32x16(f.a[k / kBO], f.b[k % kBO], v[k / kBO][k % kBO]);
  }
  __device__ __forceinline__ void mma(const Frags& f) {
#pragma unroll
    for (int i = 0; i < kBA; ++i)
#pragma unroll
      for (int j = 0; j < kBO; ++j) v[i][j] = mfma_32x32x16(f.a[i], f.b[j], v[i][j]);
  }
};

// Cursor over the active (sample, 32-token step) pairs of a call, in order:
// without a mask every step of every sample, with one the call's active-step
// list.  k is the position in that sequence.
template <int MASK>
struct Cursor {
  int k, b, s, nsteps;
  const uint32_t* list;
  const uint32_t* steps;       // MASK 2: the call's step header
  int ns, nxt, B;              // MASK 2: steps of sample b, next sample's first step, samples
  __device__ __forceinline__ void load() {
    if constexpr (MASK == 1) {
      const uint32_t v = ((c_u32*)list)[k];
      b = (int)(v >> 16);
      s = (int)(v & 0xffffu);
    }
  }
  __device__ __forceinline__ void start(const LayerArgs& p, int k0) {
    nsteps = (p.T + kKT - 1) / kKT;
    k = k0;
    if constexpr (MASK == 2) {
      steps = p.steps;
      B = p.B;
      b = prefix_sample_of(p, k0);
      const int first = (int)((c_u32*)steps)[1 + b];
      nxt = (int)((c_u32*)steps)[2 + b];
      ns = nxt - first;
      s = k0 - first;
    } else if constexpr (MASK) {
      list = p.steps + 2 + p.B;
      load();
    } else {
      b = k0 / nsteps;
      s = k0 - b * nsteps;
    }
  }
  // Also called after a run's last step (the result is then unused): the
  // prefix form stops at the last sample instead of reading past the header.
  __device__ __forceinline__ void advance() {
    ++k;
    if constexpr (MASK == 2) {
      if (++s == ns) {
        int first;
        do {
          ++b;
          first = nxt;
          nxt = (int)((c_u32*)steps)[2 + b];
        } while (nxt == first && b + 1 < B);
        ns = nxt - first;
        s = 0;
      }
    } else if constexpr (MASK) {
      load();
    } else if (++s == nsteps) {
      s = 0;
      ++b;
    }
  }
};

// All of this wave's LDS reads have returned.  Issued as the compiler's own
// wait instruction, so that its bookkeeping of outstanding LDS reads (whose
// counter tracks at most 15) starts again from zero: the reads issued next
// are then waited for on their own, not together with older ones.
__device__ __forceinline__ void lds_reads_done() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt(63) expcnt(7) lgkmcnt(0)
}

// Workgroup barrier without a memory fence: each wave has seen its LDS reads
// return (lds_reads_done) and its DMA writes land (wait_dma) before it.  The
// empty asm statements keep the compiler from moving LDS accesses across.
__device__ __forceinline__ void step_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Main loop over n active steps, from position k0 of the call's sequence.
//
// Five 32 KiB LDS slots.  Barrier i (between the two k-substeps of step i)
// certifies that step i+1 has landed for every wave and that every wave's
// reads of step i-1 are complete; slot (i-1) is then refilled with step i+4.
//
// Both waves of a SIMD pass each barrier together, so neither can cover the
// other's non-MFMA work: each wave interleaves its own.  Each k-substep is
// eight MFMAs on fragments already in registers, with the LDS reads of the
// other k-substep's fragments (and, after the barrier, the DMA of step i+4)
// issued between them:
//
//   k-substep 0 of step i : MFMAs on f0, reads of f1 (step i, tokens 16..31)
//   wait for f1, wait for step i+1's DMA, barrier
//   k-substep 1 of step i : MFMAs on f1, DMA of step i+4, reads of f0 (step i+1)
//
// SCALE: rescale the accumulator at sample boundaries so that it ends as
// sum_i (c_i / c_last) g_i; c_last is returned.
// Pipeline state of one run over an output tile: the lanes' DMA offsets,
// the issue side, and the consumer side (the sample of the step being
// consumed and, without a mask, the steps left before the next sample).
template <int MASK>
struct Pipe {
  DmaLane dl;
  Issue<MASK> is;
  Cursor<MASK> cc;
  int left, n;
};

// Queue the first min(kStages, n) steps of a run into the slot ring.
template <int MASK>
__device__ __forceinline__ void prologue(const LayerArgs& p, int k0, int n, int a0, int o0,
                                         Pipe<MASK>& ps, uint32_t base) {
  ps.n = n;
  if (n <= 0) return;
  ps.dl.init(p, a0, o0);
  ps.is.start(p, k0);
  ps.cc.start(p, k0);
  ps.left = ps.cc.nsteps - ps.cc.s;
#pragma unroll
  for (int k = 0; k < kStages; ++k) {
    if (k < n) {
      ps.is.step(p, ps.dl, base + k * kStageBytes);
      if (k + 1 < n) ps.is.advance(p);
    }
  }
}

// Wait until step 0 of a run has landed for this wave, `steps` of its DMA
// steps having been queued after step 0.  after_stores: at least 32 vector
// memory stores were issued after the whole prologue (the previous unit's
// tile, in the staged kernel).  Loads complete in order among themselves, so
// allowing for those stores (and no more than their minimum count) still
// guarantees step 0; allowing for fewer would only wait longer.
__device__ __forceinline__ void wait_first(int steps, bool after_stores) {
  if (!after_stores) {
    wait_dma(steps);
  } else if (steps <= 0) {
    asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
  } else if (steps == 1) {
    asm volatile("s_waitcnt vmcnt(36)" ::: "memory");
  } else if (steps == 2) {
    asm volatile("s_waitcnt vmcnt(40)" ::: "memory");
  } else if (steps == 3) {
    asm volatile("s_waitcnt vmcnt(44)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(48)" ::: "memory");
  }
}

// The run whose first steps `prologue` queued: the main loop below.
template <bool SCALE, int MASK>
__device__ __forceinline__ float run_queued(const LayerArgs& p, Pipe<MASK>& ps, Acc& acc,
                                            unsigned char* lds, bool after_stores) {
  static_assert(kKT == kBitsTokens, "one row-bit word per step");
  static_assert(kBA * kBO == 8 && kBA + kBO == 6, "interleave encodes 8 MFMAs and 6 fragments");
  static_assert(2 * kDmaPerOp == 4, "one DMA after every other one of eight MFMAs");
  static_assert(kDmaPerStep * (kStages - 1) + 32 <= 63, "vmcnt field");
  acc.zero();
  const int n = ps.n;
  if (n <= 0) return 1.0f;
  const uint32_t base = lds_addr(lds);
  const DmaLane& dl = ps.dl;
  Issue<MASK>& is = ps.is;               // next step to queue
  Cursor<MASK>& cc = ps.cc;
  int left = ps.left;
  float c_last = SCALE ? ((c_f32*)p.c)[cc.b] : 1.0f;
  int cb = cc.b;
  wait_first(min(kStages - 1, n - 1), after_stores);   // step 0 has landed for this wave
  step_barrier();
  Frags f0, f1;
#pragma unroll
  for (int q = 0; q < 6; ++q) read_frag(f0, lds, 0, q);
  int slot = 0;                        // i % kStages
  for (int i = 0; i < n; ++i) {
    if (SCALE && cc.b != cb) {
      // acc holds sum_{j<=cb} (c_j / c_cb) g_j; re-express it in units of the
      // new sample's factor before its tiles are added.
      const float cn = ((c_f32*)p.c)[cc.b];
      acc.scale(c_last / cn);
      c_last = cn;
      cb = cc.b;
    }
    const unsigned char* st = lds + slot * kStageBytes;
    sched_fence();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      acc.mma1(f0, k);
      sched_fence();
      if (k < 6) read_frag(f1, st, 1, k);
      if (k == 7) {
        // Consumer cursor to step i+1.
        if constexpr (MASK) {
          cc.advance();
        } else if (--left == 0) {
          left = cc.nsteps;
          ++cc.b;
        }
      }
      sched_fence();
    }
    lds_reads_done();                  // f1 is in registers; slot i-1 is no longer read
    const int next = (slot + 1 == kStages) ? 0 : slot + 1;
    const unsigned char* sn = lds + next * kStageBytes;
    // Issued so far: steps 0 .. min(4, n-1) before the loop, then step j+4
    // at barrier j >= 1, i.e. up to max(4, i+3).  Wait for step i+1: in the
    // steady state that leaves two steps in flight.
    const bool steady = i >= 1 && i + kStages - 1 < n;
    if (steady) {
      wait_dma(2);
      step_barrier();
    } else if (i + 1 < n) {
      wait_dma(min(n - 1, i <= 1 ? kStages - 1 : i + kStages - 2) - (i + 1));
      step_barrier();
    }
    // slot (i-1) % kStages is free: queue step i+4 into it, one DMA after
    // every other MFMA.  The reads of f0 follow; on the last step
    // they read the next slot's stale contents, which are never used.
    const uint32_t prev = base + ((slot == 0) ? kStages - 1 : slot - 1) * kStageBytes;
    sched_fence();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      acc.mma1(f1, k);
      sched_fence();
      if ((k & 1) == 0 && steady) is.dma(p, dl, prev, k >> 1);
      if (k == 7 && steady && i + kStages < n) is.advance(p);
      if (k >= 1 && k <= 6) read_frag(f0, sn, 0, k - 1);
      sched_fence();
    }
    slot = next;
  }
  return c_last;
}

// One run over n steps from position k0 of the call's sequence.
template <bool SCALE, int MASK>
__device__ __forceinline__ float run(const LayerArgs& p, int k0, int n, int a0, int o0, Acc& acc,
                                     unsigned char* lds) {
  Pipe<MASK> ps;
  prologue<MASK>(p, k0, n, a0, o0, ps, lds_addr(lds));
  return run_queued<SCALE, MASK>(p, ps, acc, lds, false);
}

// Grouped raster order of the output tiles: tile index L -> (tm, tn), kGroupRows
// tile-rows at a time, so that consecutive tiles share X and G strips.
__device__ __forceinline__ void raster(int L, int ntm, int ntn, int* tm, int* tn) {
  const int gsz = kGroupRows * ntn;
  const int g = L / gsz, r = L % gsz;
  const int rows = min(kGroupRows, ntm - g * kGroupRows);
  *tm = g * kGroupRows + r % rows;
  *tn = r / rows;
}

// Workgroups are dealt to the 8 XCDs round robin; logical index of this
// workgroup such that XCD x holds the contiguous range [x*G/8, (x+1)*G/8).
__device__ __forceinline__ int logical_wg(int id, int G) {
  return (G % 8 == 0) ? (id & 7) * (G / 8) + (id >> 3) : id;
}

constexpr int kTileElems = kTile * kTile;

// Store one output tile from the accumulator.  part == nullptr: the final
// result (acc * c_last + noise) / denom into p.out (added to it when beta).  Otherwise the raw partial
// acc * c_last into part[256 x 256] (row o - o0, column a - a0), which the
// fixup kernel sums.  The waves park their accumulator blocks in LDS one
// 32-row block-row (i) at a time as [o][a] (64 a values: 32 from each wave
// row); every thread then takes 4 consecutive a of one o -- one Philox block
// of noise and one 16-byte store.
__device__ __forceinline__ void store_tile(const LayerArgs& p, const Acc& acc, float c_last, int a0,
                                           int o0, float* part, unsigned char* smem) {
  static_assert(256 * (64 + 4) * 4 <= kLdsBytes, "epilogue staging fits in the stage ring");
  const int lane = threadIdx.x & 63;
  const int wm = wave_row(), wn = wave_col();
  // 1/denom: exact for a power of two, else within one ulp of dividing.
  const float rB = 1.0f / p.denom;
  const bool noise = p.noise_std != 0.0f;
  float* park = (float*)smem;
  constexpr int kParkLd = 64 + 4;     // floats per o row (padding against bank conflicts)
  __syncthreads();                    // all waves are done reading the last slot
#pragma unroll
  for (int i = 0; i < kBA; ++i) {
#pragma unroll
    for (int j = 0; j < kBO; ++j) {
      const int ol = wn * (kBO * 32) + j * 32 + acc_col(lane);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int al = wm * 32 + acc_row(4 * q, lane);
        f32x4 v;
        v.x = acc.v[i][j][4 * q + 0]; v.y = acc.v[i][j][4 * q + 1];
        v.z = acc.v[i][j][4 * q + 2]; v.w = acc.v[i][j][4 * q + 3];
        *(f32x4*)(park + ol * kParkLd + al) = v;
      }
    }
    __syncthreads();
#pragma unroll 1
    for (int e = threadIdx.x; e < 256 * 16; e += kNT) {
      const int ol = e >> 4, a4 = (e & 15) * 4;            // a4 in [0, 64)
      const int al = (a4 >> 5) * (kBA * 32) + i * 32 + (a4 & 31);
      f32x4 v = *(const f32x4*)(park + ol * kParkLd + a4);
      v.x *= c_last; v.y *= c_last; v.z *= c_last; v.w *= c_last;
      if (part != nullptr) {
        *(f32x4*)(part + ol * kTile + al) = v;
        continue;
      }
      const int o = o0 + ol, a = a0 + al;
      if (o < p.dout && a < p.din) {   // din % 8 == 0 on this path: a..a+3 all in range
        const uint64_t e0 = (uint64_t)o * (uint64_t)p.din + (uint64_t)a;
        if (noise) {
          const f32x4 z = normals_of_block(philox_block(p.seed, p.offset + (e0 >> 2)));
          v.x += p.noise_std * z.x; v.y += p.noise_std * z.y;
          v.z += p.noise_std * z.z; v.w += p.noise_std * z.w;
        }
        v.x *= rB; v.y *= rB; v.z *= rB; v.w *= rB;
        if (p.beta) {
          const f32x4 old = *(const f32x4*)(p.out + e0);
          v.x += old.x; v.y += old.y; v.z += old.z; v.w += old.w;
        }
        *(f32x4*)(p.out + e0) = v;
      }
    }
    __syncthreads();
  }
}

// Work plan of one accumulate launch (host-computed).  G persistent
// workgroups, one per compute unit.  Tiles in grouped raster order; the first
// D*G tiles go in D full rounds (tile d*G + L to workgroup L).  Each of the R
// remaining tiles is split into P token chunks (P == 1: not split); piece
// pi = c*R + r (chunk c of remaining tile r) goes to workgroup pi mod G, so
// the workgroups running at the same time stream the same token rows and
// share them in L2.  Pieces store partials; the fixup kernel sums them.
struct SkPlan {
  int G, D, R, P;
  int ntm, ntn;
};

constexpr int kMaxSplit = 16;   // P never exceeds this

// P for the R tiles of the last, partial round over n steps, at most maxP.
// Cost model in microseconds, fitted to sweeps of P on MI355X at the
// Llama-13B shapes (dense and ragged): one 32-token step of a 256 x 256 tile
// ~0.8 us, a piece's pipeline fill and epilogue ~4 us (workgroups left alone
// in a partly filled round run faster, which hides most of it), the fixup
// ~5 us plus 0.06 us per partial (256 KiB written, then read).  Pieces are
// at least 4 steps long: layers with a handful of tiles (the RoBERTa
// r-space calls: 4 tiles, 128 steps) then spread over 64 workgroups instead
// of 32; at the Llama and GPT-2 shapes the model's choice is the same as
// with a 16-step minimum.  Runs on the host over every step, and on the
// device for masked calls, over the active steps only the device knows.
__host__ __device__ inline int split_tiles(int R, int G, int n, int maxP) {
  if (R == 0) return 1;
  const double step_us = 0.8, piece_us = 4.0;
  double best = n * step_us + piece_us;   // P = 1: one more round
  int bestP = 1;
  for (int P = 2; P <= maxP; ++P) {
    if ((double)n / P < 4.0) break;       // pieces of >= 4 steps
    const int S = (R * P + G - 1) / G;
    const double t = S * ((double)n / P * step_us + piece_us) + 5.0 + 0.06 * R * P;
    if (t < best) {
      best = t;
      bestP = P;
    }
  }
  return bestP;
}

// Active steps per tile: all of them without a mask, else the list's count.
__device__ __forceinline__ int active_steps(const LayerArgs& p) {
  return p.steps != nullptr ? (int)(((c_u32*)p.steps)[0] & kStepCountMask)
                            : p.B * ((p.T + kKT - 1) / kKT);
}

template <int MASK>
__device__ __forceinline__ void accumulate_body(const LayerArgs& p, SkPlan sk,
                                                unsigned char* smem) {
  const int n = active_steps(p);
  if (MASK) sk.P = split_tiles(sk.R, sk.G, n, sk.P);   // the host's P is for every step
  const int L = logical_wg(blockIdx.x, sk.G);
  Acc acc;
  auto full_tile = [&](int t) {
    int tm, tn;
    raster(t, sk.ntm, sk.ntn, &tm, &tn);
    const float c_last = run<true, MASK>(p, 0, n, tm * kTile, tn * kTile, acc, smem);
    store_tile(p, acc, c_last, tm * kTile, tn * kTile, nullptr, smem);
  };
  for (int d = 0; d < sk.D; ++d) full_tile(d * sk.G + L);
  if (sk.P == 1) {
    if (L < sk.R) full_tile(sk.D * sk.G + L);
    return;
  }
  for (int pi = L; pi < sk.R * sk.P; pi += sk.G) {
    const int c = pi / sk.R, t = sk.D * sk.G + pi % sk.R;
    const int k0 = (int)((int64_t)c * n / sk.P), k1 = (int)((int64_t)(c + 1) * n / sk.P);
    int tm, tn;
    raster(t, sk.ntm, sk.ntn, &tm, &tn);
    const float c_last = run<true, MASK>(p, k0, k1 - k0, tm * kTile, tn * kTile, acc, smem);
    store_tile(p, acc, c_last, tm * kTile, tn * kTile, p.skws + (int64_t)pi * kTileElems, smem);
  }
}

__global__ void __launch_bounds__(kNT, 1) accumulate_big_kernel(LayerArgs p, SkPlan sk) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  if (p.steps == nullptr) accumulate_body<0>(p, sk, smem);
  else if (((c_u32*)p.steps)[0] & kStepsPrefix) accumulate_body<2>(p, sk, smem);
  else accumulate_body<1>(p, sk, smem);
}

// Split tiles: sum their P partials in chunk order, add the noise, divide by
// B.  One thread per 4 consecutive outputs, one workgroup per 4 rows of a
// split tile, so a 256 x 256 tile spreads over 64 workgroups.  Each thread
// keeps the loads of up to kFixBatch partials in flight at once (indices past
// P are clamped to the last partial and their values dropped).
constexpr int kFixThreads = 256;
constexpr int kFixRows = kFixThreads / (kTile / 4);     // 4 tile rows per workgroup
constexpr int kFixBlocksPerTile = kTile / kFixRows;     // 64
constexpr int kFixBatch = 8;
__global__ void __launch_bounds__(kFixThreads) accumulate_fixup_kernel(LayerArgs p, SkPlan sk) {
  if (p.steps != nullptr) sk.P = split_tiles(sk.R, sk.G, active_steps(p), sk.P);
  if (sk.P == 1) return;            // masked: the active steps did not call for a split
  const int r = blockIdx.x / kFixBlocksPerTile, rows = blockIdx.x % kFixBlocksPerTile;
  int tm, tn;
  raster(sk.D * sk.G + r, sk.ntm, sk.ntn, &tm, &tn);
  const int ol = rows * kFixRows + (int)(threadIdx.x >> 6), al = (int)(threadIdx.x & 63) * 4;
  const int o = tn * kTile + ol, a = tm * kTile + al;
  if (o >= p.dout || a >= p.din) return;
  const float* part = p.skws + (int64_t)r * kTileElems + ol * kTile + al;
  const int64_t stride = (int64_t)sk.R * kTileElems;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int c0 = 0; c0 < sk.P; c0 += kFixBatch) {
    f32x4 w[kFixBatch];
#pragma unroll
    for (int j = 0; j < kFixBatch; ++j)
      w[j] = *(const f32x4*)(part + (int64_t)min(c0 + j, sk.P - 1) * stride);
#pragma unroll
    for (int j = 0; j < kFixBatch; ++j) {
      if (c0 + j < sk.P) {
        v.x += w[j].x; v.y += w[j].y; v.z += w[j].z; v.w += w[j].w;
      }
    }
  }
  const float rB = 1.0f / p.denom;   // as in store_tile
  const uint64_t e0 = (uint64_t)o * (uint64_t)p.din + (uint64_t)a;
  if (p.noise_std != 0.0f) {
    const f32x4 z = normals_of_block(philox_block(p.seed, p.offset + (e0 >> 2)));
    v.x += p.noise_std * z.x; v.y += p.noise_std * z.y;
    v.z += p.noise_std * z.z; v.w += p.noise_std * z.w;
  }
  v.x *= rB; v.y *= rB; v.z *= rB; v.w *= rB;
  if (p.beta) {
    const f32x4 old = *(const f32x4*)(p.out + e0);
    v.x += old.x; v.y += old.y; v.z += old.z; v.w += old.w;
  }
  *(f32x4*)(p.out + e0) = v;
}

__global__ void __launch_bounds__(kNT, 1) direct_norm_big_kernel(LayerArgs p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int ntm = (p.din + kTile - 1) / kTile, ntn = (p.dout + kTile - 1) / kTile;
  const int ntiles = ntm * ntn;
  // blockIdx.x enumerates (sample, tile) with the tile fastest
  const int b = blockIdx.x / ntiles;
  const int local = blockIdx.x % ntiles;
  const int tm = local % ntm, tn = local / ntm;
  Acc acc;
  if (p.steps != nullptr) {
    const int k0 = (int)((c_u32*)p.steps)[1 + b], k1 = (int)((c_u32*)p.steps)[2 + b];
    run<false, true>(p, k0, k1 - k0, tm * kTile, tn * kTile, acc, smem);
  } else {
    const int nsteps = (p.T + kKT - 1) / kKT;
    run<false, false>(p, b * nsteps, nsteps, tm * kTile, tn * kTile, acc, smem);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kBA; ++i)
#pragma unroll
    for (int j = 0; j < kBO; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc.v[i][j][r] * acc.v[i][j][r];
  __syncthreads();   // the slot ring is free: reuse its first bytes for the reduction
  const double tot = block_sum_f64((double)s, (double*)smem);
  if (threadIdx.x == 0) p.partials[(int64_t)b * ntiles + local] = tot;
}

// Staged per-sample gradients.  Unit u = b * ntiles + L is sample b's output
// tile L (grouped raster order); its 256 x 256 fp32 tile is stored at
// skws + u * 65536 as the accumulator's register image: 16-byte chunk
// (w * 32 + k) * 64 + lane holds v[i][j][4g .. 4g+3] of lane `lane` of wave
// w, with k = (i * kBO + j) * 4 + g.  Each store instruction writes 1 KiB
// contiguously and needs no LDS; the combine kernel decodes the image.
constexpr int kImgChunks = kBA * kBO * 4;   // 16-byte chunks per lane
constexpr int64_t kImgStride = kTileElems;   // floats from one unit's image to the next

// Persistent: G workgroups (one per compute unit) take units u = L, L + G,
// ... (L the XCD-aware logical index), so the workgroups resident on one XCD
// work on neighbouring tiles of one sample at a time and share its X and G
// strips in that XCD's L2.  Once every wave is done with a unit's LDS slots,
// the next unit's first steps are queued before this unit's tile is stored,
// so the stores overlap the next unit's pipeline fill.  Each wave writes its
// own fp64 partial (np = 8 per tile), so no LDS is needed between units.
// Without STORE the same loop is the persistent form of the direct norm:
// each tile is squared, summed and dropped, and the next unit's pipeline
// fill overlaps this unit's reduction instead of a new workgroup's start.
constexpr int kStagedParts = kWaves;

template <int MASK, bool NT, bool STORE>
__device__ __forceinline__ void staged_units(const LayerArgs& p, int G, unsigned char* smem) {
  const int ntm = (p.din + kTile - 1) / kTile, ntn = (p.dout + kTile - 1) / kTile;
  const int ntiles = ntm * ntn;
  const int N = ntiles * p.B;
  const int nsteps = (p.T + kKT - 1) / kKT;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t base = lds_addr(smem);
  // queue the first steps of unit u
  auto queue = [&](int u, Pipe<MASK>& ps) {
    const int b = u / ntiles, L = u - b * ntiles;
    int tm, tn;
    raster(L, ntm, ntn, &tm, &tn);
    int k0, n;
    if constexpr (MASK) {
      k0 = (int)((c_u32*)p.steps)[1 + b];
      n = (int)((c_u32*)p.steps)[2 + b] - k0;
    } else {
      k0 = b * nsteps;
      n = nsteps;
    }
    prologue<MASK>(p, k0, n, tm * kTile, tn * kTile, ps, base);
  };
  Acc acc;
  Pipe<MASK> ps;
  int u = logical_wg(blockIdx.x, G);
  if (u < N) queue(u, ps);
  bool after_stores = false;
  for (; u < N; u += G) {
    const int b = u / ntiles, L = u - b * ntiles;
    run_queued<false, MASK>(p, ps, acc, smem, after_stores);
    // Every wave's LDS reads of this unit have returned before any wave
    // refills the ring; then the next unit's first steps go out.
    lds_reads_done();
    step_barrier();
    after_stores = false;
    if (u + G < N) {
      queue(u + G, ps);
      after_stores = STORE && ps.n > 0;
    }
    float* img = STORE ? p.skws + (int64_t)u * kImgStride + ((int64_t)wave * kImgChunks * 64 + lane) * 4
                       : nullptr;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kBA; ++i)
#pragma unroll
      for (int j = 0; j < kBO; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v;
          v.x = acc.v[i][j][4 * g + 0]; v.y = acc.v[i][j][4 * g + 1];
          v.z = acc.v[i][j][4 * g + 2]; v.w = acc.v[i][j][4 * g + 3];
          s += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
          if constexpr (!STORE) continue;
          // Plain (cached) stores leave the most recently written tiles in
          // the 256 MB MALL for the combine kernel: 13% faster combines at
          // 5120 x 5120.  Non-temporal stores (NT) suit the calls whose tiles
          // mostly leave the MALL anyway, or whose short units store so often
          // that cached stores crowd out the operands of the next units.
          f32x4* dst = (f32x4*)(img + ((i * kBO + j) * 4 + g) * 256);
          if constexpr (NT) __builtin_nontemporal_store(v, dst);
          else *dst = v;
        }
    const double tot = wave_sum_f64((double)s);
    if (lane == 0) p.partials[((int64_t)b * ntiles + L) * kStagedParts + wave] = tot;
  }
}

template <bool NT>
__global__ void __launch_bounds__(kNT, 1) staged_norm_big_kernel(LayerArgs p, int G) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  if (p.steps != nullptr) staged_units<true, NT, true>(p, G, smem);
  else staged_units<false, NT, true>(p, G, smem);
}

__global__ void __launch_bounds__(kNT, 1) direct_norm_units_kernel(LayerArgs p, int G) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  if (p.steps != nullptr) staged_units<true, false, false>(p, G, smem);
  else staged_units<false, false, false>(p, G, smem);
}

// out = (sum_b c_b g_b + noise_std xi) / B from the staged tiles: one thread
// per 16-byte chunk of a tile image, i.e. 4 consecutive din columns of one
// output row; samples summed in order, kCombBatch loads in flight (indices
// past B clamped to the last sample and their values dropped).
constexpr int kCombThreads = 256;
constexpr int kCombBlocksPerTile = kTileElems / 4 / kCombThreads;   // 64
constexpr int kCombBatch = 8;

__global__ void __launch_bounds__(kCombThreads) staged_combine_kernel(LayerArgs p) {
  const int ntm = (p.din + kTile - 1) / kTile, ntn = (p.dout + kTile - 1) / kTile;
  const int ntiles = ntm * ntn;
  const int L = blockIdx.x / kCombBlocksPerTile;
  const int chunk = (blockIdx.x % kCombBlocksPerTile) * kCombThreads + (int)threadIdx.x;
  const int lane = chunk & 63, k = (chunk >> 6) % kImgChunks, wave = (chunk >> 6) / kImgChunks;
  const int g = k & 3, j = (k >> 2) % kBO, i = (k >> 2) / kBO;
  int tm, tn;
  raster(L, ntm, ntn, &tm, &tn);
  const int a = tm * kTile + (wave / kWaveCols) * (kBA * 32) + i * 32 + acc_row(4 * g, lane);
  const int o = tn * kTile + (wave % kWaveCols) * (kBO * 32) + j * 32 + acc_col(lane);
  if (o >= p.dout || a >= p.din) return;   // din % 8 == 0 on this path: a..a+3 all in range
  const float* src = p.skws + (int64_t)L * kImgStride + (int64_t)chunk * 4;
  const int64_t stride = (int64_t)ntiles * kImgStride;   // one sample's tiles
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int b0 = 0; b0 < p.B; b0 += kCombBatch) {
    f32x4 w[kCombBatch];
    float cb[kCombBatch];
#pragma unroll
    for (int q = 0; q < kCombBatch; ++q) {
      const int b = min(b0 + q, p.B - 1);
      w[q] = __builtin_nontemporal_load((const f32x4*)(src + (int64_t)b * stride));
      cb[q] = p.c[b];
    }
#pragma unroll
    for (int q = 0; q < kCombBatch; ++q) {
      if (b0 + q < p.B) {
        v.x += cb[q] * w[q].x; v.y += cb[q] * w[q].y;
        v.z += cb[q] * w[q].z; v.w += cb[q] * w[q].w;
      }
    }
  }
  const float rB = 1.0f / p.denom;   // as in store_tile
  const uint64_t e0 = (uint64_t)o * (uint64_t)p.din + (uint64_t)a;
  if (p.noise_std != 0.0f) {
    const f32x4 z = normals_of_block(philox_block(p.seed, p.offset + (e0 >> 2)));
    v.x += p.noise_std * z.x; v.y += p.noise_std * z.y;
    v.z += p.noise_std * z.z; v.w += p.noise_std * z.w;
  }
  v.x *= rB; v.y *= rB; v.z *= rB; v.w *= rB;
  if (p.beta) {
    const f32x4 old = *(const f32x4*)(p.out + e0);
    v.x += old.x; v.y += old.y; v.z += old.z; v.w += old.w;
  }
  *(f32x4*)(p.out + e0) = v;
}

}  // namespace big

namespace {
template <auto Kernel>
hipError_t allow_lds_big(int bytes) {
  static hipError_t once = hipFuncSetAttribute((const void*)Kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  return once;
}
}  // namespace

int big_tiles(int din, int dout) {
  return ((din + big::kTile - 1) / big::kTile) * ((dout + big::kTile - 1) / big::kTile);
}

namespace {
big::SkPlan plan_accumulate(const LayerArgs& p) {
  big::SkPlan sk{};
  sk.ntm = (p.din + big::kTile - 1) / big::kTile;
  sk.ntn = (p.dout + big::kTile - 1) / big::kTile;
  const int ntiles = sk.ntm * sk.ntn;
  const int cus = device_cus();
  int G = std::min(cus, ntiles * 16);
  if (G >= 8) G -= G % 8;
  sk.G = G;
  sk.D = ntiles / G;
  sk.R = ntiles - sk.D * G;
  const int n = p.B * ((p.T + big::kKT - 1) / big::kKT);   // every step (an upper bound if masked)
  sk.P = big::split_tiles(sk.R, G, n, p.max_split == 1 ? 1 : big::kMaxSplit);
  if (sk.P == 1 && sk.D == 0) sk.G = sk.R;   // one tile per workgroup, no idle ones
  return sk;
}
}  // namespace

size_t accumulate_big_workspace_bytes(const LayerArgs& p) {
  const big::SkPlan sk = plan_accumulate(p);
  return sk.P == 1 ? 0 : (size_t)sk.R * sk.P * big::kTileElems * sizeof(float);
}

hipError_t launch_accumulate_big(const LayerArgs& p, hipStream_t s) {
  hipError_t e = allow_lds_big<big::accumulate_big_kernel>(big::kLdsBytes);
  if (e != hipSuccess) return e;
  const big::SkPlan sk = plan_accumulate(p);
  if (sk.P != 1 && p.skws == nullptr) return hipErrorInvalidValue;
  timing_begin("accumulate", s);
  hipLaunchKernelGGL(big::accumulate_big_kernel, dim3(sk.G), dim3(big::kNT), big::kLdsBytes, s, p, sk);
  e = hipGetLastError();
  timing_end("accumulate", s);
  if (e != hipSuccess || sk.P == 1) return e;
  timing_begin("accumulate_fixup", s);
  hipLaunchKernelGGL(big::accumulate_fixup_kernel, dim3(big::kFixBlocksPerTile * sk.R),
                     dim3(big::kFixThreads), 0, s, p, sk);
  e = hipGetLastError();
  timing_end("accumulate_fixup", s);
  return e;
}

size_t staged_big_workspace_bytes(const LayerArgs& p) {
  return (size_t)p.B * big_tiles(p.din, p.dout) * big::kImgStride * sizeof(float);
}

int staged_big_partials_per_sample(const LayerArgs& p) {
  return big_tiles(p.din, p.dout) * big::kStagedParts;
}

// Non-temporal tile stores where measured faster on MI355X: units of at most
// 16 token steps (GPT-2 MLP, T = 512: 7% faster calls), or more than 1.5 GB
// of tiles (Llama-13B gate/up/down, 2.3 GB: 1%).  Cached stores otherwise
// (q/k/v/o, 0.84 GB: the combine reads recent tiles from the MALL, 2% faster).
static bool staged_nontemporal(const LayerArgs& p) {
  const int nsteps = (p.T + big::kKT - 1) / big::kKT;
  return nsteps <= 16 || (double)staged_big_workspace_bytes(p) > 1.5e9;
}

template <bool NT>
static hipError_t launch_staged_norm_t(const LayerArgs& p, int G, hipStream_t s) {
  hipError_t e = allow_lds_big<big::staged_norm_big_kernel<NT>>(big::kLdsBytes);
  if (e != hipSuccess) return e;
  timing_begin("staged_norm", s);
  hipLaunchKernelGGL(big::staged_norm_big_kernel<NT>, dim3((unsigned)G), dim3(big::kNT),
                     big::kLdsBytes, s, p, G);
  e = hipGetLastError();
  timing_end("staged_norm", s);
  return e;
}

hipError_t launch_staged_norm_big(const LayerArgs& p, hipStream_t s) {
  const int64_t units = (int64_t)big_tiles(p.din, p.dout) * p.B;
  if (p.skws == nullptr || units > 0x7fffffff) return hipErrorInvalidValue;
  int G = (int)std::min<int64_t>(device_cus(), units);
  if (G >= 8) G -= G % 8;
  return staged_nontemporal(p) ? launch_staged_norm_t<true>(p, G, s)
                               : launch_staged_norm_t<false>(p, G, s);
}

hipError_t launch_staged_combine_big(const LayerArgs& p, hipStream_t s) {
  const int64_t blocks = (int64_t)big_tiles(p.din, p.dout) * big::kCombBlocksPerTile;
  if (p.skws == nullptr || blocks > 0x7fffffff) return hipErrorInvalidValue;
  timing_begin("staged_combine", s);
  hipLaunchKernelGGL(big::staged_combine_kernel, dim3((unsigned)blocks), dim3(big::kCombThreads),
                     0, s, p);
  const hipError_t e = hipGetLastError();
  timing_end("staged_combine", s);
  return e;
}

// The direct norm runs persistent (one workgroup per compute unit walking
// the (sample, tile) units, eight partials per tile) when the units fill
// more than one round of the chip; one workgroup per unit otherwise.
static int direct_units_grid(const LayerArgs& p) {
  const int64_t units = (int64_t)big_tiles(p.din, p.dout) * p.B;
  const int cus = device_cus();
  if (units <= cus || units > 0x7fffffff) return 0;
  return cus >= 8 ? cus - cus % 8 : cus;
}

int direct_big_partials_per_sample(const LayerArgs& p) {
  return big_tiles(p.din, p.dout) * (direct_units_grid(p) > 0 ? big::kStagedParts : 1);
}

hipError_t launch_direct_norm_big(const LayerArgs& p, hipStream_t s) {
  const int G = direct_units_grid(p);
  if (G > 0) {
    hipError_t e = allow_lds_big<big::direct_norm_units_kernel>(big::kLdsBytes);
    if (e != hipSuccess) return e;
    timing_begin("direct_norm", s);
    hipLaunchKernelGGL(big::direct_norm_units_kernel, dim3((unsigned)G), dim3(big::kNT),
                       big::kLdsBytes, s, p, G);
    e = hipGetLastError();
    timing_end("direct_norm", s);
    return e;
  }
  hipError_t e = allow_lds_big<big::direct_norm_big_kernel>(big::kLdsBytes);
  if (e != hipSuccess) return e;
  const int nt = big_tiles(p.din, p.dout);
  timing_begin("direct_norm", s);
  hipLaunchKernelGGL(big::direct_norm_big_kernel, dim3(nt * p.B), dim3(big::kNT), big::kLdsBytes,
                     s, p);
  e = hipGetLastError();
  timing_end("direct_norm", s);
  return e;
}

}  // namespace dpf
