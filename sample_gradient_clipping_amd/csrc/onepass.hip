// Single-pass fused kernel for layers whose per-sample gradients fit on chip
// (FlashDP abstract: the per-layer DP step as one fused task that computes
// each per-sample gradient only once; aibr.jp FlashDP explainer, section 3:
// a block-wise reduction across thread blocks, designed around the GPU's
// synchronisation constraints).
//
// One cooperative launch: one workgroup per 128 (din) x 128 (dout) output
// tile, every workgroup resident at once.  Each workgroup walks the samples in
// order; for sample b it
//   1. computes its tile of g_b = G~_b^T X~_b by MFMA over sample b's active
//      tokens (never stored anywhere: the tile stays in registers);
//   2. publishes the tile's sum of squares as its partial for sample b, one
//      64-bit slot per (sample, tile) in device memory, written once;
//   3. folds an earlier sample f whose partials are all published: the
//      partials of f summed in tile order (the same fp64 sum in every
//      workgroup) give n_f and c_f = min(1, C / n_f), and the tile of g_f,
//      still in registers, is added to the running sum as c_f g_f.
// Up to two computed samples wait in registers for their factors, and the
// loads that fetch a sample's partials are issued one sample before they are
// needed, so the cross-workgroup reduction overlaps the next contraction
// instead of stalling it.  No workgroup ever waits at a grid-wide barrier; a
// workgroup that finds a factor missing when both waiting places are full
// polls for it, with a bounded number of tries (a timeout poisons the
// outputs with NaN rather than hanging).  After the last sample:
// (sum_b c_b g_b + noise_std xi) / denom, written from the registers with
// the library's Philox noise layout.
//
// Workgroup: 512 threads, 8 waves (2 per SIMD) as 2 (din) x 4 (dout); each
// wave owns 64 x 32 of the tile, 2 x 1 blocks of v_mfma_f32_32x32x16_bf16
// accumulators, in four sets (running sum, two waiting samples, current).
// Operands are token-major ("K-outer") as in the large-tile accumulate
// kernel: 32-token steps of the tile's 128 X columns and 128 G columns
// (16 KiB) go from global memory into a ring of nine LDS slots by 16-byte
// buffer loads that write LDS directly; rows are 256 bytes, the 16-byte chunk
// c of row k at chunk c ^ 4 (k mod 4), read back with gfx950's transposing
// LDS read.  Waves 4..7 issue all the loads; waves 0..3 issue none, so wave 0
// can wait for its own loads of partials without waiting for any operand.
#include <algorithm>
#include <atomic>

#include "kernels.hpp"

namespace dpf {
namespace onepass {

constexpr int kNT = 512;
constexpr int kWaves = kNT / 64;
constexpr int kWaveRows = 2, kWaveCols = 4;   // waves along din (a) and along dout (o)
constexpr int kBA = 2;                        // 32-wide din blocks per wave (64 a x 32 o)
constexpr int kTile = 128;                    // the tile: 128 (a) x 128 (o)
constexpr int kKT = 32;                       // tokens per step
constexpr int kRowBytes = kTile * 2;          // one token row of one operand, bf16
constexpr int kOpBytes = kKT * kRowBytes;     // 8 KiB
constexpr int kStageBytes = 2 * kOpBytes;     // 16 KiB: the X rows, then the G rows
constexpr int kStages = 9;
constexpr int kRingBytes = kStages * kStageBytes;   // 144 KiB
constexpr int kRedBytes = 256;                      // wave sums, factor, flags
constexpr int kLdsBytes = kRingBytes + kRedBytes;
constexpr int kFirstDmaWave = 4;                    // waves 4..7 load the operands
constexpr int kDmaPerWave = 4;                      // per step: 2 X and 2 G row groups
constexpr int kOOB = 0x7ffffff0;
constexpr int kMaxPoll = 4;                         // partials per lane of wave 0 (<= 256 tiles)
// Content of a partial's slot until its workgroup publishes it: a NaN whose
// low bits no sum of squares can produce (fp32-derived NaNs have them zero).
constexpr uint64_t kEmpty = 0x7ff4deadbeef1234ull;

static_assert(kWaveRows * kBA * 32 == kTile && kWaveCols * 32 == kTile, "wave grid covers the tile");
static_assert(kWaves - kFirstDmaWave == 4 && kDmaPerWave * 4 == 16, "16 row groups per step");

typedef __attribute__((address_space(4))) const uint32_t c_u32;

__device__ __forceinline__ int swz(int k, int c16) { return c16 ^ ((k & 3) << 2); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const unsigned char*)p;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sample_rsrc(const Act& a, int b, int T, int D) {
  const char* base = (const char*)a.data + (int64_t)b * a.stride_b * 2;
  const int64_t bytes = ((int64_t)(T - 1) * a.stride_t + D) * 2;
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0,
                                           (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff),
                                           0x00020000);
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane;
// completion is awaited explicitly (wait_dma).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, int voffset, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(lds)
               : "memory");
}

// Wait until at most `steps` of this wave's most recent DMA steps are in flight.
__device__ __forceinline__ void wait_dma(int steps) {
  static_assert(kDmaPerWave == 4, "wait_dma encodes 4 DMAs per step");
  static_assert(kStages <= 9, "wait_dma encodes at most 8 steps in flight");
  switch (steps) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(28)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
  }
}

__device__ __forceinline__ void lds_reads_done() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt(63) expcnt(7) lgkmcnt(0)
}

__device__ __forceinline__ void step_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Active-row bits of the 32 tokens of step s of sample b: with a mask the
// row bits, else only the tail past T is inactive.
template <bool MASK>
__device__ __forceinline__ uint32_t step_bits(const LayerArgs& p, int b, int s) {
  if constexpr (MASK) return ((c_u32*)p.rowbits)[(int64_t)b * p.nwords + s];
  const int n = p.T - s * kKT;
  return n >= 32 ? 0xffffffffu : ((1u << n) - 1u);
}

// Issue side of the operand pipeline (waves 4..7).  DMA d of wave w loads
// rows 8 (w - 4) + 4 (d & 1) .. +3 of the step's X (d < 2) or G (d >= 2)
// rows; lane l writes physical chunk l % 16 of row l / 16 of that group,
// i.e. logical chunk (l % 16) ^ 4 (row mod 4): features 8 c .. 8 c + 7 of the
// tile's columns.  A chunk past the end of the row gets an offset of kOOB or
// more, which stays out of range once the step's row offset (< 2 GiB) is
// added; so do rows past T (the row stride is at least the row length).
template <bool MASK>
struct Issue {
  __amdgpu_buffer_rsrc_t rx, rg;
  uint32_t off[kDmaPerWave];   // lane offset within a step (bytes), or kOOB
  int row[kDmaPerWave];        // row of the step each DMA's lane fills
  int b, s, k, nsteps;
  uint32_t xs, gs, dx, dg;     // byte offsets of the step's first row; per-step increments
  uint32_t bits;
  const uint32_t* list;

  __device__ __forceinline__ void rsrc(const LayerArgs& p) {
    rx = sample_rsrc(p.X, b, p.T, p.din);
    rg = sample_rsrc(p.G, b, p.T, p.dout);
  }
  __device__ __forceinline__ void load(const LayerArgs& p) {
    const uint32_t v = ((c_u32*)list)[k];
    const int nb = (int)(v >> 16);
    s = (int)(v & 0xffffu);
    xs = (uint32_t)s * dx;
    gs = (uint32_t)s * dg;
    if (nb != b) {
      b = nb;
      rsrc(p);
    }
    bits = step_bits<MASK>(p, b, s);
  }
  __device__ __forceinline__ void init(const LayerArgs& p, int a0, int o0, int k0) {
    const int w = wave_id() - kFirstDmaWave, lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 0; d < kDmaPerWave; ++d) {
      const int r = 8 * w + 4 * (d & 1) + (lane >> 4);
      const int c = (lane & 15) ^ ((r & 3) << 2);
      row[d] = r;
      if (d < 2) {
        const int a = a0 + 8 * c;
        off[d] = a < p.din ? (uint32_t)(((int64_t)r * p.X.stride_t + a) * 2) : (uint32_t)kOOB;
      } else {
        const int o = o0 + 8 * c;
        off[d] = o < p.dout ? (uint32_t)(((int64_t)r * p.G.stride_t + o) * 2) : (uint32_t)kOOB;
      }
    }
    nsteps = (p.T + kKT - 1) / kKT;
    dx = (uint32_t)kKT * (uint32_t)p.X.stride_t * 2u;
    dg = (uint32_t)kKT * (uint32_t)p.G.stride_t * 2u;
    k = k0;
    if constexpr (MASK) {
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
    if constexpr (MASK) {
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
  // The four DMAs of the current step into the slot at LDS address `stage`.
  __device__ __forceinline__ void step(uint32_t stage) const {
    const int w = wave_id() - kFirstDmaWave;
#pragma unroll
    for (int d = 0; d < kDmaPerWave; ++d) {
      uint32_t o = off[d] + (d < 2 ? xs : gs);
      if constexpr (MASK) {
        if (!((bits >> row[d]) & 1u)) o = (uint32_t)kOOB;
      }
      const uint32_t dst = stage + (d >> 1) * kOpBytes + (8 * w + 4 * (d & 1)) * kRowBytes;
      dma16(d < 2 ? rx : rg, (int)o, dst);
    }
  }
};

// MFMA operand of one 16-token substep ks for the 32 columns m0.. of an
// operand's rows in a slot: two transposing 8-byte reads give each lane its
// 8 consecutive tokens of one column.
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

// The six operands of one step for this wave: per substep two X blocks and
// one G block.
struct Frags {
  u16x8 a[2][kBA], g[2];
};

// Operand q (0..5) of a step: q = 3 ks + {0: G block, 1, 2: X blocks}.
__device__ __forceinline__ void read_frag(Frags& f, const unsigned char* slot, int q) {
  const int wave = threadIdx.x >> 6;
  const int ks = q / 3, r = q % 3;
  if (r == 0) f.g[ks] = frag(slot + kOpBytes, (wave % kWaveCols) * 32, ks);
  else f.a[ks][r - 1] = frag(slot, (wave / kWaveCols) * (kBA * 32) + (r - 1) * 32, ks);
}

typedef f32x16 Tile[kBA];

__device__ __forceinline__ void zero(Tile& t) {
#pragma unroll
  for (int i = 0; i < kBA; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) t[i][r] = 0.f;
}

// MFMA j (0..3) of a step: substep j / 2, X block j % 2.
__device__ __forceinline__ void mma(Tile& acc, const Frags& f, int j) {
  const int ks = j >> 1, i = j & 1;
  acc[i] = mfma_32x32x16(f.a[ks][i], f.g[ks], acc[i]);
}

__device__ __forceinline__ void axpy(Tile& run, float c, const Tile& t) {
#pragma unroll
  for (int i = 0; i < kBA; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) run[i][r] += c * t[i][r];
}

__device__ __forceinline__ void copy(Tile& dst, const Tile& src) {
#pragma unroll
  for (int i = 0; i < kBA; ++i) dst[i] = src[i];
}

// Wave 0's fetch of one sample's partials: lane l holds the slots of tiles
// l, l + 64, ... (fewer than kMaxPoll * 64 tiles).
struct Poll {
  uint64_t v[kMaxPoll];
  __device__ __forceinline__ void issue(const uint64_t* slots, int ntiles) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int m = 0; m < kMaxPoll; ++m) {
      const int t = lane + 64 * m;
      v[m] = t < ntiles ? __hip_atomic_load(slots + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                        : 0ull;
    }
  }
  // True when every tile has published (the same answer in every lane).
  __device__ __forceinline__ bool complete() const {
    bool ok = true;
#pragma unroll
    for (int m = 0; m < kMaxPoll; ++m) ok = ok && v[m] != kEmpty;
    return __all(ok);
  }
  // The sample's squared norm: each lane sums its slots in tile order, then
  // a fixed butterfly across the wave -- the same bits in every workgroup.
  __device__ __forceinline__ double total() const {
    double s = 0.0;
#pragma unroll
    for (int m = 0; m < kMaxPoll; ++m) s += __longlong_as_double((long long)v[m]);
    return wave_sum_f64(s);
  }
};

// LDS words of the per-sample exchange between wave 0 and the others.
struct Shared {
  double red[kWaves];   // wave sums of squares of the current sample
  float fac;            // factor of the sample being folded
  int ready;            // 1: fac holds the factor of the oldest waiting sample
};

// Factor and norm of a squared norm (the rule of the ordered finalize).
__device__ __forceinline__ void clip_of(double sq, float C, float* c, float* n) {
  const double nn = sqrt(sq < 0.0 ? 0.0 : sq);
  *n = (float)nn;
  *c = (nn <= (double)C) ? 1.0f : (float)((double)C / nn);
}

struct Params {
  float C;
  float* norms_out;      // [B] or null
  uint64_t* slots;       // [B][ntiles] partial slots, kEmpty on entry
  int ntiles, ntm;       // tiles, tiles along din
  int spin_limit;        // tries of a blocking poll before it gives up
  int never_ready;       // testing: treat every fetch as incomplete (forces the timeout path)
};

template <bool MASK>
__device__ void body(const LayerArgs& p, const Params& q, unsigned char* smem) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const bool dma_wave = wave >= kFirstDmaWave;
  const int G = q.ntiles;
  const int L = (G % 8 == 0) ? (int)(blockIdx.x & 7) * (G / 8) + (int)(blockIdx.x >> 3)
                             : (int)blockIdx.x;
  const int tm = L % q.ntm, tn = L / q.ntm;
  const int a0 = tm * kTile, o0 = tn * kTile;
  Shared* sh = (Shared*)(smem + kRingBytes);
  const uint32_t base = lds_addr(smem);

  // The active steps: with a mask the call's list (sample-major), else every
  // step of every sample.
  const int nsteps = (p.T + kKT - 1) / kKT;
  const int N = MASK ? (int)(((c_u32*)p.steps)[0] & kStepCountMask) : p.B * nsteps;
  auto first_step = [&](int b) {
    return MASK ? (int)((c_u32*)p.steps)[1 + b] : b * nsteps;
  };

  Tile run, w0, w1, cur;
  zero(run);
  zero(cur);
  zero(w0);
  zero(w1);
  int fold_next = 0;     // samples < fold_next have been added to run
  bool failed = false;   // a blocking poll gave up: every later factor is NaN
  Poll poll;
  bool poll_on = false;  // wave 0: poll holds loads of fold_next's slots

  // Wave 0: wait (bounded) until fold_next's partials are all published, then
  // post its factor for the other waves; the caller then passes a barrier.
  auto fetch_blocking = [&](int f) {
    const uint64_t* sl = q.slots + (int64_t)f * G;
    bool ok = false;
    if (!failed) {
      for (int it = 0; it <= q.spin_limit; ++it) {
        if (!poll_on) poll.issue(sl, G);
        poll_on = false;
        if (!q.never_ready && poll.complete()) {
          ok = true;
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
    }
    failed = failed || !ok;
    float c, n;
    if (ok) {
      clip_of(poll.total(), q.C, &c, &n);
    } else {
      c = __builtin_nanf("");
      n = __builtin_nanf("");
    }
    if (lane == 0) {
      sh->fac = c;
      sh->ready = 1;
      if (L == 0 && q.norms_out != nullptr) q.norms_out[f] = n;
    }
  };

  // Fold the oldest waiting sample with the factor wave 0 posted.
  auto fold = [&]() {
    const float c = sh->fac;
    if ((fold_next & 1) == 0) axpy(run, c, w0);
    else axpy(run, c, w1);
    ++fold_next;
  };

  // ---- prologue: the first kStages steps into the ring
  Issue<MASK> is;
  if (dma_wave && N > 0) {
    is.init(p, a0, o0, 0);
#pragma unroll 1
    for (int k = 0; k < kStages && k < N; ++k) {
      is.step(base + k * kStageBytes);
      if (k + 1 < N) is.advance(p);
    }
    wait_dma(min(kStages, N) - 1);
  }
  step_barrier();
  Frags fa, fb;
  if (N > 0) {
#pragma unroll
    for (int r = 0; r < 6; ++r) read_frag(fa, smem, r);
  }
  int i = 0;          // global step index
  int slot = 0;       // i % kStages

#pragma unroll 1
  for (int b = 0; b < p.B; ++b) {
    const int nb = first_step(b + 1) - first_step(b);
    // ---- sample b's contraction
#pragma unroll 1
    for (int j = 0; j < nb; ++j, ++i) {
      lds_reads_done();                 // fa (step i) is in registers
      const int nxt = slot + 1 == kStages ? 0 : slot + 1;
      if (i + 1 < N) {
        if (dma_wave) {
          // steps 0 .. min(i + kStages - 1, N - 1) are queued; step i+1 must land
          wait_dma(min(i + kStages - 1, N - 1) - (i + 1));
        }
        step_barrier();
        if (dma_wave && i + kStages < N) {
          is.step(base + slot * kStageBytes);   // slot i % kStages takes step i + kStages
          if (i + kStages + 1 < N) is.advance(p);
        }
      }
      const unsigned char* sn = smem + nxt * kStageBytes;
      sched_fence();
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        mma(cur, fa, m);
        sched_fence();
        if (i + 1 < N) {
          if (m < 3) {
            read_frag(fb, sn, 2 * m);
            read_frag(fb, sn, 2 * m + 1);
          }
        }
        sched_fence();
      }
      fa = fb;
      slot = nxt;
    }

    // ---- sample b done: publish the tile's partial
    float ss = 0.f;
#pragma unroll
    for (int ii = 0; ii < kBA; ++ii)
#pragma unroll
      for (int r = 0; r < 16; ++r) ss += cur[ii][r] * cur[ii][r];
    const double ws = wave_sum_f64((double)ss);
    if (lane == 0) sh->red[wave] = ws;
    if (wave == 0) {
      // the factor of fold_next, if the fetch issued at the last boundary
      // found every partial
      int rdy = 0;
      if (poll_on) {
        if (!q.never_ready && poll.complete()) {
          float c, n;
          clip_of(poll.total(), q.C, &c, &n);
          if (lane == 0) {
            sh->fac = c;
            if (L == 0 && q.norms_out != nullptr) q.norms_out[fold_next] = n;
          }
          rdy = 1;
        }
        poll_on = false;   // incomplete: fetched again below
      }
      if (lane == 0) sh->ready = rdy;
    }
    // Barriers here are plain (no memory fence): the waves exchange data
    // through LDS only, and a fence would make the loading waves wait for
    // every operand load in flight.
    lds_reads_done();
    step_barrier();
    if (wave == 0 && lane == 0) {
      double tot = 0.0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) tot += sh->red[w];
      __hip_atomic_store(q.slots + (int64_t)b * G + L, (uint64_t)__double_as_longlong(tot),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (sh->ready) fold();
    // both waiting places full: the oldest must be folded before b can wait
    if (b - fold_next == 2) {
      lds_reads_done();                 // every wave has read sh->ready / sh->fac
      step_barrier();
      if (wave == 0) fetch_blocking(fold_next);
      lds_reads_done();
      step_barrier();
      fold();
    }
    if ((b & 1) == 0) copy(w0, cur);
    else copy(w1, cur);
    zero(cur);
    // wave 0: fetch the oldest waiting sample's partials, checked at the next
    // boundary (issued fresh if an earlier fetch came back incomplete)
    if (wave == 0 && !poll_on && fold_next <= b) {
      poll.issue(q.slots + (int64_t)fold_next * G, G);
      poll_on = true;
    }
    // sh is rewritten at the next boundary.  A plain barrier (no memory
    // fence): a fence would wait for the fetch just issued.
    lds_reads_done();
    step_barrier();
  }

  // ---- the samples still waiting
#pragma unroll 1
  while (fold_next < p.B) {
    if (wave == 0) fetch_blocking(fold_next);
    lds_reads_done();
    step_barrier();
    fold();
    lds_reads_done();
    step_barrier();
  }

  // ---- epilogue: (run + noise_std xi) / denom, from the registers
  const int wm = wave / kWaveCols, wn = wave % kWaveCols;
  const float rD = 1.0f / p.denom;
  const int o = o0 + wn * 32 + acc_col(lane);
#pragma unroll
  for (int ii = 0; ii < kBA; ++ii) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int a = a0 + wm * (kBA * 32) + ii * 32 + acc_row(4 * g, lane);
      if (o >= p.dout || a >= p.din) continue;   // din % 8 == 0: a .. a+3 all in range
      f32x4 v;
      v.x = run[ii][4 * g + 0]; v.y = run[ii][4 * g + 1];
      v.z = run[ii][4 * g + 2]; v.w = run[ii][4 * g + 3];
      const uint64_t e0 = (uint64_t)o * (uint64_t)p.din + (uint64_t)a;
      if (p.noise_std != 0.0f) {
        const f32x4 z = normals_of_block(philox_block(p.seed, p.offset + (e0 >> 2)));
        v.x += p.noise_std * z.x; v.y += p.noise_std * z.y;
        v.z += p.noise_std * z.z; v.w += p.noise_std * z.w;
      }
      v.x *= rD; v.y *= rD; v.z *= rD; v.w *= rD;
      if (p.beta) {
        const f32x4 old = *(const f32x4*)(p.out + e0);
        v.x += old.x; v.y += old.y; v.z += old.z; v.w += old.w;
      }
      *(f32x4*)(p.out + e0) = v;
    }
  }
}

__global__ void __launch_bounds__(kNT, 1) onepass_kernel(LayerArgs p, Params q) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  if (p.steps != nullptr) body<true>(p, q, smem);
  else body<false>(p, q, smem);
}

__global__ void fill_empty_kernel(uint64_t* slots, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) slots[i] = kEmpty;
}

}  // namespace onepass

namespace {
std::atomic<int> g_spin_limit{1 << 20};
std::atomic<int> g_never_ready{0};
}  // namespace

void set_onepass_testing(int spin_limit, int never_ready) {
  g_spin_limit.store(spin_limit);
  g_never_ready.store(never_ready);
}
int onepass_spin_limit() { return g_spin_limit.load(); }
int onepass_never_ready() { return g_never_ready.load(); }

int onepass_tiles(int din, int dout) {
  return ((din + onepass::kTile - 1) / onepass::kTile) *
         ((dout + onepass::kTile - 1) / onepass::kTile);
}

// Workgroups of the kernel that can be resident at once on the current
// device (0 if it cannot be told).
int onepass_resident_limit() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load();
  if (n == 0) {
    if (hipFuncSetAttribute((const void*)onepass::onepass_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            onepass::kLdsBytes) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, onepass::onepass_kernel,
                                                     onepass::kNT, onepass::kLdsBytes) !=
            hipSuccess ||
        per_cu < 1) {
      (void)hipGetLastError();
      return 0;
    }
    n = per_cu * device_cus();
    cache[dev].store(n);
  }
  return n;
}

size_t onepass_workspace_bytes(const LayerArgs& p) {
  return (size_t)p.B * onepass_tiles(p.din, p.dout) * sizeof(uint64_t);
}

hipError_t launch_onepass(const LayerArgs& p, float C, float* norms_out, hipStream_t s) {
  const int ntiles = onepass_tiles(p.din, p.dout);
  if (p.partials == nullptr || ntiles > 64 * onepass::kMaxPoll) return hipErrorInvalidValue;
  const int limit = onepass_resident_limit();
  if (limit < ntiles) return hipErrorCooperativeLaunchTooLarge;
  onepass::Params q{};
  q.C = C;
  q.norms_out = norms_out;
  q.slots = reinterpret_cast<uint64_t*>(p.partials);
  q.ntiles = ntiles;
  q.ntm = (p.din + onepass::kTile - 1) / onepass::kTile;
  q.spin_limit = onepass_spin_limit();
  q.never_ready = onepass_never_ready();
  const int64_t n = (int64_t)p.B * ntiles;
  timing_begin("onepass_fill", s);
  hipLaunchKernelGGL(onepass::fill_empty_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     q.slots, n);
  hipError_t e = hipGetLastError();
  timing_end("onepass_fill", s);
  if (e != hipSuccess) return e;
  LayerArgs pa = p;
  void* args[] = {&pa, &q};
  timing_begin("onepass", s);
  e = hipLaunchCooperativeKernel((const void*)onepass::onepass_kernel, dim3((unsigned)ntiles),
                                 dim3(onepass::kNT), args, onepass::kLdsBytes, s);
  if (e == hipSuccess) e = hipGetLastError();
  timing_end("onepass", s);
  return e;
}

}  // namespace dpf
