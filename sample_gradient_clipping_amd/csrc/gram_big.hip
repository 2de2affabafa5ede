// Large-tile bf16 kernel for the Gram form of the per-sample squared norm:
//
//   ||G~_i^T X~_i||^2 = sum_{s,t} (X~_i X~_i^T)[s,t] (G~_i G~_i^T)[s,t]
//
// One workgroup per (sample, 256-token row block S, 128-token column block
// Tb) with Tb >= 2S, i.e. every tile that touches the upper triangle s <= t.
// Each element is weighted 2 above the diagonal, 1 on it and 0 below, so the
// symmetric sum is counted once.  The X Gram tile (K = din) and the G Gram
// tile (K = dout) accumulate one after the other in registers; their
// elementwise product is reduced wave -> LDS -> one fp64 partial per
// workgroup, summed in a fixed order later (finalize_kernel).
//
// Workgroup: 512 threads = 8 waves (4 along s, 2 along t; two per SIMD);
// each wave owns 64 x 64 of both Gram tiles: 2 x 2 blocks of
// v_mfma_f32_32x32x16_bf16 accumulators per Gram (128 fp32 per lane).
// Operands are feature-contiguous ("K-inner"): each lane's MFMA fragment is
// one 16-byte LDS read.  Data moves global -> LDS by 16-byte-per-lane buffer
// loads that write LDS directly into a ring of three 48 KiB slots (64
// features of 256 + 128 token rows); rows are 128 bytes with the 16-byte
// chunk c of row r stored at c ^ ((r >> 1) & 7), which keeps both the DMA
// writes and the fragment reads free of bank conflicts.  Masked tokens and
// rows past T read through out-of-range buffer offsets (zeros).
#include <algorithm>

#include "kernels.hpp"
#include "tiles.hpp"

namespace dpf {
namespace gram {

constexpr int kNT = 512;
constexpr int kWaveRows = 4, kWaveCols = 2;
constexpr int kRowsS = 256, kRowsT = 128;
constexpr int kKF = 64;                         // features per step
constexpr int kRowBytes = kKF * 2;              // 128
constexpr int kSBytes = kRowsS * kRowBytes;     // 32 KiB
constexpr int kSlotBytes = kSBytes + kRowsT * kRowBytes;   // 48 KiB
constexpr int kStages = 3;
constexpr int kLdsBytes = kStages * kSlotBytes;            // 144 KiB
constexpr int kDmaPerStep = kSlotBytes / 1024 / (kNT / 64);  // 6 per wave
constexpr int kOOB = 0x7ffffff0;

typedef __attribute__((address_space(4))) const uint32_t c_u32;

__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row >> 1) & 7); }

// 16 bytes per lane from rsrc at voffset + soffset straight into LDS at
// m0 + 16 * lane.  soffset is wave-uniform (the step's feature offset).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, int voffset, uint32_t lds,
                                      uint32_t soffset) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(lds), "s"(soffset)
               : "memory");
}

// Wait until at most `steps` of this wave's most recent DMA steps are in flight.
__device__ __forceinline__ void wait_dma(int steps) {
  static_assert(kDmaPerStep == 6, "wait_dma encodes 6 DMAs per step");
  if (steps <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (steps == 1) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
}

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

// Work items per sample for T tokens.
__device__ __host__ __forceinline__ int items_per_sample(int T) {
  const int nS = (T + kRowsS - 1) / kRowsS, nTb = (T + kRowsT - 1) / kRowsT;
  int n = 0;
  for (int S = 0; S < nS; ++S) n += (nTb - 2 * S > 0) ? nTb - 2 * S : 0;
  return n;
}

// Per-lane DMA addressing for this workgroup's rows.  DMA j of wave w is
// instruction q = 6 w + j of the slot: q < 32 fills s-rows 8q .. 8q+7, the
// rest t-rows; lane l fills physical chunk l % 8 of row l / 8 of that group,
// i.e. logical feature chunk (l % 8) ^ swizzle(row).
struct DmaLane {
  uint32_t xoff[kDmaPerStep], goff[kDmaPerStep];   // row offset + chunk, or kOOB
  int cfeat[kDmaPerStep];                          // first feature of the chunk
  __device__ __forceinline__ void init(const LayerArgs& p, int b, int S, int Tb) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < kDmaPerStep; ++j) {
      const int q = kDmaPerStep * wave + j;
      const bool sreg = q < kRowsS / 8;
      const int row = (sreg ? 8 * q : 8 * (q - kRowsS / 8)) + (lane >> 3);
      const int tok = sreg ? kRowsS * S + row : kRowsT * Tb + row;
      bool active = tok < p.T;
      if (active && p.rowbits != nullptr)
        active = (p.rowbits[(int64_t)b * p.nwords + (tok >> 5)] >> (tok & 31)) & 1u;
      const int c = swz(row, lane & 7);
      cfeat[j] = c * 8;
      xoff[j] = active ? (uint32_t)(((int64_t)tok * p.X.stride_t + c * 8) * 2) : (uint32_t)kOOB;
      goff[j] = active ? (uint32_t)(((int64_t)tok * p.G.stride_t + c * 8) * 2) : (uint32_t)kOOB;
    }
  }
};

// What the DMAs of one feature step need, computed once per step: the
// descriptor and feature offset (the instruction's scalar offset) of the X
// or G rows, and whether the step runs past D (then each lane tests its
// chunk and sends the chunks past D out of range).
// Steps are queued in order, X steps first: the lane's row offsets in dl.xoff
// are replaced by its G offsets once, when the first G step is queued.
struct StepDma {
  __amdgpu_buffer_rsrc_t r;
  uint32_t soff;
  int k0, D;
  bool tail;
  __device__ __forceinline__ void at(const LayerArgs& p, DmaLane& dl, __amdgpu_buffer_rsrc_t rx,
                                     __amdgpu_buffer_rsrc_t rg, int step, int nkx, bool& on_g) {
    const bool xs = step < nkx;
    if (!xs && !on_g) {
#pragma unroll
      for (int j = 0; j < kDmaPerStep; ++j) dl.xoff[j] = dl.goff[j];
      on_g = true;
    }
    k0 = (xs ? step : step - nkx) * kKF;
    D = xs ? p.din : p.dout;
    r = xs ? rx : rg;
    soff = (uint32_t)k0 * 2u;
    tail = k0 + kKF > D;
  }
  // DMA j of the step into the slot whose address for this wave's DMAs is
  // `dst`; TAIL: the step runs past D.
  template <bool TAIL>
  __device__ __forceinline__ void dma_(const DmaLane& dl, uint32_t dst, int j) const {
    int off = (int)dl.xoff[j];
    if (TAIL && k0 + dl.cfeat[j] >= D) off = kOOB;
    dma16(r, off, dst + (uint32_t)j * 1024u, soff);
  }
  // DMAs j0 .. j0+cnt-1.  Tail steps (only when D is not a multiple of the
  // step's 64 features) take a separate branch, so that the common path
  // carries no per-lane test.
  __device__ __forceinline__ void dmas(const DmaLane& dl, uint32_t dst, int j0, int cnt) const {
    if (__builtin_expect(tail, 0)) {
      for (int j = j0; j < j0 + cnt; ++j) dma_<true>(dl, dst, j);
    } else {
      for (int j = j0; j < j0 + cnt; ++j) dma_<false>(dl, dst, j);
    }
  }
};

__device__ __forceinline__ void issue_step(const LayerArgs& p, DmaLane& dl,
                                           __amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rg,
                                           int step, int nkx, uint32_t dst, bool& on_g) {
  StepDma sd;
  sd.at(p, dl, rx, rg, step, nkx, on_g);
  sd.dmas(dl, dst, 0, kDmaPerStep);
}

// All of this wave's LDS reads have returned.  Issued as the compiler's own
// wait instruction, so that its bookkeeping of outstanding LDS reads restarts
// from zero.
__device__ __forceinline__ void lds_reads_done() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt(63) expcnt(7) lgkmcnt(0)
}

// Workgroup barrier without a memory fence: each wave has seen its LDS reads
// return (lds_reads_done) and its DMA writes land (wait_dma) before it.
__device__ __forceinline__ void step_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Nothing is scheduled across this point: it fixes the interleaving of
// MFMAs with LDS reads and DMA issue that the main loop spells out.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// MFMA operand for rows m0..m0+31 of a region, 16-feature substep ks.
__device__ __forceinline__ u16x8 frag(const unsigned char* region, int m0, int ks) {
  const int lane = threadIdx.x & 63;
  const int row = m0 + (lane & 31);
  const int c = 2 * ks + (lane >> 5);
  return *(const u16x8*)(region + row * kRowBytes + swz(row, c) * 16);
}

struct Acc2 {
  f32x16 v[2][2];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) v[i][j][r] = 0.f;
  }
  // Keep the accumulators in accumulation registers (AGPRs): with two Gram
  // tiles live, ordinary VGPRs would overflow.
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) asm volatile("" : "+a"(v[i][j]));
  }
  // MFMA k of a 16-feature substep: block (k / 2, k % 2).
  __device__ __forceinline__ void mma1(const u16x8 (&f)[4], int k) {
    v[k >> 1][k & 1] = mfma_32x32x16(f[k >> 1], f[2 + (k & 1)], v[k >> 1][k & 1]);
  }
};

// Fragment q of 16-feature substep ks of this wave: q = 0, 1 the s blocks
// (rows wm*64 + 32q), q = 2, 3 the t blocks (rows wn*64 + 32(q-2)).
__device__ __forceinline__ void read_frag(u16x8 (&f)[4], const unsigned char* slot, int ks, int q) {
  const int wave = threadIdx.x >> 6;
  const int wm = wave / kWaveCols, wn = wave % kWaveCols;
  f[q] = q < 2 ? frag(slot, wm * 64 + q * 32, ks) : frag(slot + kSBytes, wn * 64 + (q - 2) * 32, ks);
}

// Sample, row block S and column block Tb of item L (L = b * per_sample +
// index of (S, Tb) within the sample, S-major).
__device__ __forceinline__ void item_coords(int L, int per_sample, int T, int* b, int* S, int* Tb) {
  *b = L / per_sample;
  int r = L % per_sample;
  const int nTb = (T + kRowsT - 1) / kRowsT;
  int s = 0;
  while (r >= nTb - 2 * s) { r -= nTb - 2 * s; ++s; }
  *S = s;
  *Tb = 2 * s + r;
}

// Workgroups are dealt to the 8 XCDs round robin; logical index of this
// workgroup such that XCD x holds the contiguous range [x*G/8, (x+1)*G/8):
// consecutive items (same sample, shared rows) meet in one L2.
__device__ __forceinline__ int logical_wg(int id, int G) {
  return (G % 8 == 0) ? (id & 7) * (G / 8) + (id >> 3) : id;
}

// Feature steps [k0, k1) of item (b, S, Tb) into ax (steps < nkx: X Gram)
// and ag (the rest: G Gram).
//
// Three 48 KiB slots of 64 features = four 16-feature substeps.  Fragments
// are double-buffered: the MFMAs of one substep run on registers while the
// next substep's fragments are read, one read between consecutive MFMAs.
// Barrier i comes before the last substep of step i: it certifies that step
// i+1 has landed for every wave and that every wave has read all of step i,
// whose slot is then refilled with step i+3 (its DMAs interleaved with the
// last substep's MFMAs), leaving two steps in flight.
__device__ __forceinline__ void run_item(const LayerArgs& p, int b, int S, int Tb, int k0, int k1,
                                         Acc2& ax, Acc2& ag, unsigned char* smem) {
  static_assert(kKF / 16 == 4 && kDmaPerStep == 6, "the interleave encodes 4 substeps, 6 DMAs");
  const int nkx = (p.din + kKF - 1) / kKF;
  const int n = k1 - k0;
  const __amdgpu_buffer_rsrc_t rx = sample_rsrc(p.X, b, p.T, p.din);
  const __amdgpu_buffer_rsrc_t rg = sample_rsrc(p.G, b, p.T, p.dout);
  DmaLane dl;
  dl.init(p, b, S, Tb);
  const uint32_t base = lds_addr(smem);
  // This wave's DMAs fill kDmaPerStep consecutive KiB of a slot.
  const uint32_t wdst =
      base + (uint32_t)(kDmaPerStep * __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * 1024u;
  bool on_g = false;
#pragma unroll
  for (int k = 0; k < kStages; ++k)
    if (k < n) issue_step(p, dl, rx, rg, k0 + k, nkx, wdst + k * kSlotBytes, on_g);
  ax.zero();
  ag.zero();
  wait_dma(min(kStages - 1, n - 1));   // step 0 has landed for this wave
  step_barrier();
  u16x8 f0[4], f1[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) read_frag(f0, smem, 0, (q == 1) ? 2 : (q == 2) ? 3 : (q == 3) ? 1 : 0);
  int slot = 0;
  // Fragments in the order the MFMAs first need them: s block 0, t blocks
  // 0 and 1, s block 1; two reads before a substep's first MFMA (the
  // previous substep released their registers) and two after it.
  constexpr int kNeed[4] = {0, 2, 3, 1};
  auto substep = [&](Acc2& acc, const u16x8 (&f)[4], u16x8 (&g)[4], const unsigned char* st,
                     int ks) {
    read_frag(g, st, ks, kNeed[0]);
    read_frag(g, st, ks, kNeed[1]);
    sched_fence();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc.mma1(f, k);
      sched_fence();
      if (k == 0) {
        read_frag(g, st, ks, kNeed[2]);
        read_frag(g, st, ks, kNeed[3]);
      }
      sched_fence();
    }
  };
  auto body = [&](int i, Acc2& acc) {
    const unsigned char* st = smem + slot * kSlotBytes;
    sched_fence();
    substep(acc, f0, f1, st, 1);             // substep 0 on f0, read substep 1
    substep(acc, f1, f0, st, 2);             // substep 1 on f1, read substep 2
    substep(acc, f0, f1, st, 3);             // substep 2 on f0, read substep 3
    lds_reads_done();                        // all of step i is in registers
    const int next = (slot + 1 == kStages) ? 0 : slot + 1;
    if (i + 1 < n) {
      // Issued so far: steps 0..2 before the loop, then step j+3 at barrier
      // j < i, i.e. up to i+2.  Wait for step i+1.
      wait_dma(min(n - 1, i + kStages - 1) - (i + 1));
      step_barrier();
    }
    const bool refill = i + kStages < n;
    const uint32_t dst = wdst + slot * kSlotBytes;
    StepDma sd;
    if (refill) sd.at(p, dl, rx, rg, k0 + i + kStages, nkx, on_g);
    const unsigned char* sn = smem + next * kSlotBytes;
    // substep 3 on f1, reads of step i+1 (stale on the last step, never
    // used), DMA of step i+3
    read_frag(f0, sn, 0, kNeed[0]);
    read_frag(f0, sn, 0, kNeed[1]);
    sched_fence();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc.mma1(f1, k);
      sched_fence();
      if (k == 0) {
        read_frag(f0, sn, 0, kNeed[2]);
        read_frag(f0, sn, 0, kNeed[3]);
      }
      if (k >= 1 && refill) sd.dmas(dl, dst, 2 * (k - 1), 2);
      sched_fence();
    }
    slot = next;
  };
  const int nx = max(0, min(k1, nkx) - k0);   // X steps of this range
  int i = 0;
  for (; i < nx; ++i) body(i, ax);   // X Gram, K = din
  for (; i < n; ++i) body(i, ag);    // G Gram, K = dout
  __syncthreads();                   // every wave is done with the slot ring
}

// Weighted sum of ax .* ag over this thread's elements of item (S, Tb):
// weight 2 above the diagonal (s < t), 1 on it, 0 below.  Rows past T and
// masked rows are zero in both Grams.
__device__ __forceinline__ float weighted_product(const Acc2& ax, const Acc2& ag, int S, int Tb) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave / kWaveCols, wn = wave % kWaveCols;
  const bool above = kRowsT * Tb >= kRowsS * (S + 1);   // whole tile has s < t
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float prod = ax.v[i][j][r] * ag.v[i][j][r];
        if (above) {
          sum += 2.0f * prod;
        } else {
          const int s = kRowsS * S + wm * 64 + i * 32 + acc_row(r, lane);
          const int t = kRowsT * Tb + wn * 64 + j * 32 + acc_col(lane);
          sum += (s < t) ? 2.0f * prod : ((s == t) ? prod : 0.0f);
        }
      }
  return sum;
}

// Work plan (host-computed): G persistent workgroups; the first D*G items in
// D full rounds (item d*G + L to workgroup L); each of the R remaining items
// split into P chunks of its feature steps (P == 1: not split), piece
// pi = c*R + r going to workgroup pi mod G.  A piece stores its partial
// Grams; the fixup kernel finishes split items.
struct GramPlan {
  int G, D, R, P;
};

constexpr int kMaxSplit = 16;

// D, R and P for `items` items of n feature steps on G workgroups, with at
// most `cap` pieces.  Cost model from measurements on MI355X: a 64-feature
// step of a 256 x 128 item ~0.8 us; a piece's fill and partial store ~10 us;
// the fixup ~10 us plus 0.13 us per piece.  Runs on the host, and on the
// device for masked calls, where only the device knows how many items hold
// an active token.
__host__ __device__ inline GramPlan split_items(int items, int G, int n, int cap) {
  GramPlan gp{G, items / G, items % G, 1};
  if (gp.R == 0) return gp;
  const double step_us = 0.8, piece_us = 10.0;
  double best = n * step_us + piece_us;
  for (int P = 2; P <= kMaxSplit; ++P) {
    if ((double)n / P < 8.0 || gp.R * P > cap) break;
    const int S = (gp.R * P + G - 1) / G;
    const double t = S * ((double)n / P * step_us + piece_us) + 10.0 + 0.13 * gp.R * P;
    if (t < best) {
      best = t;
      gp.P = P;
    }
  }
  return gp;
}

// A piece's partial Grams: 128 floats per thread (64 of X, then 64 of G),
// stored as f32x4 q of thread tid at [q][tid] so that stores and loads of
// consecutive threads are contiguous.
constexpr int kPieceFloats = 128 * kNT;

__device__ __forceinline__ void store_piece(float* dst, const Acc2& ax, const Acc2& ag) {
  f32x4* d = (f32x4*)dst;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int x = (i * 2 + j) * 4 + q;
        f32x4 v;
        v.x = ax.v[i][j][4 * q]; v.y = ax.v[i][j][4 * q + 1];
        v.z = ax.v[i][j][4 * q + 2]; v.w = ax.v[i][j][4 * q + 3];
        d[x * kNT + threadIdx.x] = v;
        v.x = ag.v[i][j][4 * q]; v.y = ag.v[i][j][4 * q + 1];
        v.z = ag.v[i][j][4 * q + 2]; v.w = ag.v[i][j][4 * q + 3];
        d[(16 + x) * kNT + threadIdx.x] = v;
      }
}

__device__ __forceinline__ void add_piece(const float* src, Acc2& ax, Acc2& ag) {
  const f32x4* d = (const f32x4*)src;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int x = (i * 2 + j) * 4 + q;
        const f32x4 u = d[x * kNT + threadIdx.x], w = d[(16 + x) * kNT + threadIdx.x];
        ax.v[i][j][4 * q] += u.x; ax.v[i][j][4 * q + 1] += u.y;
        ax.v[i][j][4 * q + 2] += u.z; ax.v[i][j][4 * q + 3] += u.w;
        ag.v[i][j][4 * q] += w.x; ag.v[i][j][4 * q + 1] += w.y;
        ag.v[i][j][4 * q + 2] += w.z; ag.v[i][j][4 * q + 3] += w.w;
      }
}

// Masked calls: live[0] = n, the number of items with an active token in
// both of their row blocks, live[1 .. n] their indices in increasing order.
// The other items are exactly zero; the list kernel stores their partials.
// The plan over the n live items is made here, with at most `cap` pieces.
__global__ void __launch_bounds__(kNT, 1) gram_norm_big_kernel(LayerArgs p, GramPlan gp,
                                                               const uint32_t* live, int cap,
                                                               float* ws) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int per_sample = items_per_sample(p.T);
  const int n = (p.din + kKF - 1) / kKF + (p.dout + kKF - 1) / kKF;
  const int L = logical_wg(blockIdx.x, gp.G);
  if (live != nullptr) gp = split_items((int)((c_u32*)live)[0], gp.G, n, cap);
  auto item_at = [&](int i) { return live != nullptr ? (int)((c_u32*)live)[1 + i] : i; };
  Acc2 ax, ag;
  auto full_item = [&](int item) {
    int b, S, Tb;
    item_coords(item, per_sample, p.T, &b, &S, &Tb);
    run_item(p, b, S, Tb, 0, n, ax, ag, smem);
    const double tot = block_sum_f64((double)weighted_product(ax, ag, S, Tb), (double*)smem);
    if (threadIdx.x == 0) p.partials[item] = tot;
    __syncthreads();                 // the reduction scratch is the next item's ring
  };
  for (int d = 0; d < gp.D; ++d) full_item(item_at(d * gp.G + L));
  if (gp.P == 1) {
    if (L < gp.R) full_item(item_at(gp.D * gp.G + L));
    return;
  }
  for (int pi = L; pi < gp.R * gp.P; pi += gp.G) {
    const int c = pi / gp.R, item = item_at(gp.D * gp.G + pi % gp.R);
    int b, S, Tb;
    item_coords(item, per_sample, p.T, &b, &S, &Tb);
    run_item(p, b, S, Tb, (int)((int64_t)c * n / gp.P), (int)((int64_t)(c + 1) * n / gp.P), ax, ag,
             smem);
    store_piece(ws + (int64_t)pi * kPieceFloats, ax, ag);
  }
}

// Split items: sum the P partial Grams in chunk order, then the weighted
// product and its reduction, as for a whole item.  One workgroup per item,
// with the main kernel's thread layout.  Masked calls launch one workgroup
// per possible split item and make the plan as the main kernel does.
__global__ void __launch_bounds__(kNT, 1) gram_fixup_kernel(LayerArgs p, GramPlan gp,
                                                            const uint32_t* live, int cap,
                                                            const float* ws) {
  __shared__ double red[kNT / 64];
  const int n = (p.din + kKF - 1) / kKF + (p.dout + kKF - 1) / kKF;
  if (live != nullptr) gp = split_items((int)((c_u32*)live)[0], gp.G, n, cap);
  const int r = blockIdx.x;
  if (gp.P == 1 || r >= gp.R) return;
  const int i = gp.D * gp.G + r;
  const int item = live != nullptr ? (int)((c_u32*)live)[1 + i] : i;
  int b, S, Tb;
  item_coords(item, items_per_sample(p.T), p.T, &b, &S, &Tb);
  Acc2 ax, ag;
  ax.zero();
  ag.zero();
  for (int c = 0; c < gp.P; ++c) add_piece(ws + (int64_t)(c * gp.R + r) * kPieceFloats, ax, ag);
  const double tot = block_sum_f64((double)weighted_product(ax, ag, S, Tb), red);
  if (threadIdx.x == 0) p.partials[item] = tot;
}

// Live-item list of a masked call (layout at gram_norm_big_kernel) from the
// row bits; items with no active token in one of their row blocks get a zero
// partial here.  One workgroup walks the items in order, 1024 at a time; an
// entry's index is the number of live items before it.
constexpr int kListThreads = 1024;
__global__ void __launch_bounds__(kListThreads) live_items_kernel(LayerArgs p, uint32_t* live) {
  __shared__ uint32_t wave_count[kListThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per_sample = items_per_sample(p.T);
  const int64_t total = (int64_t)p.B * per_sample;
  uint32_t base = 0;
  for (int64_t c0 = 0; c0 < total; c0 += kListThreads) {
    const int64_t i = c0 + tid;
    bool act = false;
    if (i < total) {
      int b, S, Tb;
      item_coords((int)i, per_sample, p.T, &b, &S, &Tb);
      const uint32_t* w = p.rowbits + (int64_t)b * p.nwords;
      uint32_t ws = 0, wt = 0;
      for (int k = S * (kRowsS / 32); k < min((S + 1) * (kRowsS / 32), p.nwords); ++k) ws |= w[k];
      for (int k = Tb * (kRowsT / 32); k < min((Tb + 1) * (kRowsT / 32), p.nwords); ++k) wt |= w[k];
      act = ws != 0u && wt != 0u;
      if (!act) p.partials[i] = 0.0;
    }
    const uint64_t ball = __ballot(act);
    const uint32_t below = (uint32_t)__popcll(ball & ((1ull << lane) - 1ull));
    if (lane == 0) wave_count[wave] = (uint32_t)__popcll(ball);
    __syncthreads();
    uint32_t before = 0, chunk = 0;
    for (int w = 0; w < kListThreads / 64; ++w) {
      if (w < wave) before += wave_count[w];
      chunk += wave_count[w];
    }
    if (act) live[1 + base + before + below] = (uint32_t)i;
    base += chunk;
    __syncthreads();                  // wave_count is rewritten by the next chunk
  }
  if (tid == 0) live[0] = base;
}

}  // namespace gram

int gram_big_items_per_sample(int T) { return gram::items_per_sample(T); }

namespace {
gram::GramPlan plan_gram(const LayerArgs& p) {
  const int items = p.B * gram::items_per_sample(p.T);
  const int cus = device_cus();
  int G = std::min(cus, items * 16);
  if (G >= 8) G -= G % 8;
  const int n = (p.din + gram::kKF - 1) / gram::kKF + (p.dout + gram::kKF - 1) / gram::kKF;
  gram::GramPlan gp = gram::split_items(items, G, n, 1 << 30);
  if (gp.P == 1 && gp.D == 0) gp.G = gp.R;
  return gp;
}

// Workspace of a masked call: the live-item list, then room for G pieces
// (the device-side plan never splits into more).
size_t live_list_bytes(const LayerArgs& p) {
  const size_t b = ((size_t)p.B * gram::items_per_sample(p.T) + 1) * sizeof(uint32_t);
  return (b + 255) & ~(size_t)255;
}
}  // namespace

size_t gram_big_workspace_bytes(const LayerArgs& p) {
  const gram::GramPlan gp = plan_gram(p);
  if (p.mask != nullptr)
    return live_list_bytes(p) + (size_t)gp.G * gram::kPieceFloats * sizeof(float);
  return gp.P == 1 ? 0 : (size_t)gp.R * gp.P * gram::kPieceFloats * sizeof(float);
}

hipError_t launch_gram_norm_big(const LayerArgs& p, hipStream_t s) {
  static hipError_t once = hipFuncSetAttribute((const void*)gram::gram_norm_big_kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               gram::kLdsBytes);
  if (once != hipSuccess) return once;
  const gram::GramPlan gp = plan_gram(p);
  const bool masked = p.rowbits != nullptr;
  if ((masked || gp.P != 1) && p.skws == nullptr) return hipErrorInvalidValue;
  uint32_t* live = nullptr;
  float* pieces = p.skws;
  hipError_t e;
  if (masked) {
    live = reinterpret_cast<uint32_t*>(p.skws);
    pieces = p.skws + live_list_bytes(p) / sizeof(float);
    timing_begin("live_items", s);
    hipLaunchKernelGGL(gram::live_items_kernel, dim3(1), dim3(gram::kListThreads), 0, s, p, live);
    e = hipGetLastError();
    timing_end("live_items", s);
    if (e != hipSuccess) return e;
  }
  timing_begin("gram_norm", s);
  hipLaunchKernelGGL(gram::gram_norm_big_kernel, dim3(gp.G), dim3(gram::kNT), gram::kLdsBytes, s, p,
                     gp, (const uint32_t*)live, gp.G, pieces);
  e = hipGetLastError();
  timing_end("gram_norm", s);
  if (e != hipSuccess || (!masked && gp.P == 1)) return e;
  timing_begin("gram_fixup", s);
  hipLaunchKernelGGL(gram::gram_fixup_kernel, dim3(masked ? gp.G : gp.R), dim3(gram::kNT), 0, s, p,
                     gp, (const uint32_t*)live, gp.G, (const float*)pieces);
  e = hipGetLastError();
  timing_end("gram_fixup", s);
  return e;
}

}  // namespace dpf
