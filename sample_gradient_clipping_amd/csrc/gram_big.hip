// Large-tile bf16 kernel for the Gram form of the per-sample squared norm:
//
//   ||G~_i^T X~_i||^2 = sum_{s,t} (X~_i X~_i^T)[s,t] (G~_i G~_i^T)[s,t]
//
// Work item: (sample, 256-token row block S, 256-token column block Tb) with
// S <= Tb, i.e. every block that touches the upper triangle s <= t.  Each
// element is weighted 2 above the diagonal, 1 on it and 0 below, so the
// symmetric sum is counted once (for a diagonal item that is the plain sum
// of its block, which is symmetric).
//
// Workgroup: 512 threads = 8 waves (2 along s, 4 along t; two per SIMD);
// each wave owns 128 x 64 of the item's Gram tile: 4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16 accumulators (128 fp32 per lane), the shape of
// the accumulate kernel's wave tile.  Only one Gram fits in registers, so an
// item runs in two phases: the X Gram (K = din) is computed and parked in a
// per-workgroup scratch buffer (256 KiB, thread-major, read back only by the
// thread that wrote it), then the G Gram (K = dout); the epilogue multiplies
// the two elementwise, weights and reduces wave -> LDS -> one fp64 partial per
// item, summed in a fixed order later (finalize_kernel).
//
// Operands are feature-contiguous ("K-inner"): each lane's MFMA fragment is
// one 16-byte LDS read.  A phase computes 32-feature steps (two 16-feature
// substeps of eight MFMAs), but loads 64-feature chunks: one side's 256 rows
// of a chunk (a "half", 32 KiB) is one whole 128-byte line per row, so every
// 16-byte-per-lane buffer load that writes LDS directly covers 8 full lines
// (32-feature loads covered 16 half lines per instruction and kept the
// address unit busy for twice as long per byte).  Five 32 KiB LDS slots
// hold halves: s halves of chunk c in slot 2 (c mod 3), t halves in slot
// 1 + 2 (c mod 2).  Rows are 128 bytes with the 16-byte chunk c of row r
// stored at c ^ ((r >> 1) & 7), which keeps the fragment reads free of bank
// conflicts.  Each wave reads all of a chunk's t fragments (its 64 t rows,
// 64 features: 32 registers) as the chunk starts, so the t slot is free one
// substep into the chunk; the s fragments are read one substep ahead of
// their MFMAs.  That lets the t half of chunk c + 2 be queued a quarter of
// the way into chunk c and the s half of chunk c + 3 three quarters of the
// way (three and four steps ahead of their first use).  Masked tokens and
// rows past T read through out-of-range buffer offsets (zeros).
#include <algorithm>
#include <type_traits>

#include "kernels.hpp"
#include "tiles.hpp"

namespace dpf {
namespace gram {

constexpr int kNT = 512;
constexpr int kWaveRows = 2, kWaveCols = 4;    // wave grid: 2 along s, 4 along t
constexpr int kBA = 4, kBO = 2;                // 32x32 blocks per wave: 128 (s) x 64 (t)
constexpr int kRows = 256;                     // token rows on each side of an item
constexpr int kKF = 32;                        // features per step
constexpr int kChunkF = 2 * kKF;               // features per load chunk: two steps
constexpr int kRowBytes = kChunkF * 2;         // 128: one cache line
constexpr int kHalfBytes = kRows * kRowBytes;  // 32 KiB: one side's rows of one chunk
constexpr int kSlots = 5;
constexpr int kLdsBytes = kSlots * kHalfBytes; // 160 KiB: all of gfx950's LDS
constexpr int kWaves = kNT / 64;
constexpr int kDmaPerHalf = kHalfBytes / 1024 / kWaves;   // 4 per wave, 8 rows each
constexpr int kOOB = 0x7ffffff0;
constexpr int kAccFloats = kBA * kBO * 16;            // 128 per lane
constexpr int kGramFloats = kAccFloats * kNT;         // one Gram tile, thread-major
constexpr int kMaxSplit = 16;

typedef __attribute__((address_space(4))) const uint32_t c_u32;

__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row >> 1) & 7); }

// The thread index, hidden from the optimiser: addressing derived from it
// is then computed where it is used, once per item, instead of being hoisted
// out of the item loop and kept live (in registers it does not have) across
// the whole kernel.
__device__ __forceinline__ int opaque_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// 16 bytes per lane from rsrc at voffset + soffset straight into LDS at
// m0 + 16 * lane.  soffset is wave-uniform (the step's feature offset).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, int voffset, uint32_t lds,
                                      uint32_t soffset) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(lds), "s"(soffset)
               : "memory");
}

// Wait until at most `halves` of this wave's most recently queued halves
// are in flight (0 to kSlots - 2 of them).
__device__ __forceinline__ void wait_halves(int halves) {
  static_assert(kDmaPerHalf == 4, "wait_halves encodes 4 DMAs per half");
  if (halves <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (halves == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if (halves == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
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

// Work items per sample for T tokens: the upper triangle (with the diagonal)
// of nB x nB blocks of 256 tokens.
__device__ __host__ __forceinline__ int items_per_sample(int T) {
  const int nB = (T + kRows - 1) / kRows;
  return nB * (nB + 1) / 2;
}

// Sample, row block S and column block Tb >= S of item L (L = b * per_sample
// + index of (S, Tb) within the sample, S-major).
__device__ __forceinline__ void item_coords(int L, int per_sample, int T, int* b, int* S, int* Tb) {
  *b = L / per_sample;
  int r = L % per_sample;
  const int nB = (T + kRows - 1) / kRows;
  int s = 0;
  while (r >= nB - s) { r -= nB - s; ++s; }
  *S = s;
  *Tb = s + r;
}

// Lane l of DMA j of wave w fills physical chunk l % 8 of row
// 8 (4 w + j) + l / 8 of a half, i.e. logical 16-byte chunk
// swz(row, l % 8) of that row's 128 bytes.
__device__ __forceinline__ int dma_row(int wave, int lane, int j) {
  return 8 * (kDmaPerHalf * wave + j) + (lane >> 3);
}
__device__ __forceinline__ int dma_chunk(int lane, int j) {
  // (row >> 1) & 7 of dma_row does not depend on the wave
  return (lane & 7) ^ ((4 * j + (lane >> 4)) & 7);
}

// Per-lane DMA addressing of an item's two row blocks (one side, X or G):
// byte offset of the lane's token row and 16-byte chunk, or kOOB for masked
// tokens and rows past T.
struct DmaLane {
  uint32_t s[kDmaPerHalf], t[kDmaPerHalf];
  __device__ __forceinline__ void init(const LayerArgs& p, const Act& a, int b, int S, int Tb,
                                       int tid) {
    const int wave = tid >> 6, lane = tid & 63;
    auto offset = [&](int tok, int c) {
      bool active = tok < p.T;
      if (active && p.rowbits != nullptr)
        active = (p.rowbits[(int64_t)b * p.nwords + (tok >> 5)] >> (tok & 31)) & 1u;
      return active ? (uint32_t)(((int64_t)tok * a.stride_t + 8 * c) * 2) : (uint32_t)kOOB;
    };
#pragma unroll
    for (int j = 0; j < kDmaPerHalf; ++j) {
      const int row = dma_row(wave, lane, j), c = dma_chunk(lane, j);
      s[j] = offset(kRows * S + row, c);
      t[j] = offset(kRows * Tb + row, c);
    }
  }
};

// The DMAs of one half: chunk m of a side with D features.  The chunk's
// byte offset rides in the instruction's scalar offset; only a chunk that
// runs past D tests each lane's 8 features (D is a multiple of 8 on this
// path, so they are wholly inside or wholly past the end).
struct HalfDma {
  uint32_t soff;
  int f0, D;
  bool tail;
  __device__ __forceinline__ void at(int m, int Dd) {
    f0 = m * kChunkF;
    D = Dd;
    soff = (uint32_t)f0 * 2u;
    tail = f0 + kChunkF > D;
  }
  __device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t dst,
                                      int j) const {
    if (__builtin_expect(tail, 0) && f0 + 8 * dma_chunk(opaque_tid() & 63, j) >= D) off = kOOB;
    dma16(r, (int)off, __builtin_amdgcn_readfirstlane(dst + (uint32_t)j * 1024u),
          __builtin_amdgcn_readfirstlane(soff));
  }
};

// All of this wave's LDS reads have returned.  Issued as the compiler's own
// wait instruction, so that its bookkeeping of outstanding LDS reads restarts
// from zero.
__device__ __forceinline__ void lds_reads_done() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt(63) expcnt(7) lgkmcnt(0)
}

// Workgroup barrier without a memory fence: each wave has seen its LDS reads
// return (lds_reads_done) and its DMA writes land (wait_halves) before it.
__device__ __forceinline__ void step_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Nothing is scheduled across this point: it fixes the interleaving of
// MFMAs with LDS reads and DMA issue that the main loop spells out.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// MFMA operands: lane l reads row l % 32 of a 32-row block, 16-byte chunk
// 2 q + l / 32 of the row (features 16 q .. 16 q + 15 of the chunk).  For
// a block starting at a multiple of 32 rows the swizzle depends on l alone
// and 2 q enters it by XOR below the row's 128 bytes, so a fragment's LDS
// address is half + (lane part ^ 32 q) + 128 * (block's first row): the
// last term is the instruction's immediate offset, and one register per
// side holds the lane part (with the wave's first row of that side).
__device__ __forceinline__ uint32_t frag_lane(int row0) {
  const int lane = threadIdx.x & 63, lrow = lane & 31;
  return (uint32_t)((row0 + lrow) * kRowBytes + (swz(lrow, lane >> 5) << 4));
}
// Address of substep q's fragments in the half at LDS address half, computed
// where it is used (not kept live across the loop).
__device__ __forceinline__ uint32_t sub_addr(uint32_t half, uint32_t lane_part, int q) {
  asm volatile("" : "+v"(lane_part));
  return half + (lane_part ^ (uint32_t)(32 * q));
}
typedef __attribute__((address_space(3))) const u16x8 lds_u16x8;
__device__ __forceinline__ u16x8 frag(uint32_t addr, int block) {
  return *(lds_u16x8*)(size_t)(addr + (uint32_t)(block * 32 * kRowBytes));
}


__device__ __forceinline__ int wave_row() { return (threadIdx.x >> 6) / kWaveCols; }
__device__ __forceinline__ int wave_col() { return (threadIdx.x >> 6) % kWaveCols; }


// A wave's fragments: s fragments of two substeps (the MFMAs' and the next
// one's), t fragments of all four substeps of a chunk.
struct Frags {
  u16x8 a[2][kBA];
  u16x8 b[4][kBO];
};

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
  // Keep the accumulators in accumulation registers (AGPRs), which the MFMAs
  // read and write directly; in ordinary VGPRs they would not fit beside the
  // fragments and addresses.
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int i = 0; i < kBA; ++i)
#pragma unroll
      for (int j = 0; j < kBO; ++j) asm volatile("" : "+a"(v[i][j]));
  }
  // MFMA k of substep q: block (k / kBO, k % kBO).
  __device__ __forceinline__ void mma1(const Frags& f, int q, int k) {
    v[k / kBO][k % kBO] =
        mfma_32x32x16(f.a[q & 1][k / kBO], f.b[q][k % kBO], v[k / kBO][k % kBO]);
  }
};

// Slots of chunk c's halves (c counted from the run's first chunk).
__device__ __forceinline__ int slot_s(int c) { return 2 * (c % 3); }
__device__ __forceinline__ int slot_t(int c) { return 1 + 2 * (c & 1); }

// Steps k0 .. k0+n-1 (32 features each) of one side (a: X or G, D features)
// of item (b, S, Tb) into acc, as 16-feature substeps u = 2 k0 .. 2 (k0+n) - 1
// (chunk u / 4, substep q = u % 4 of it).  Halves h = 0, 1, 2, ... of the run
// (h / 2 the chunk counted from the one holding step k0, h % 2 the side)
// are queued in that order: five up front, then the t half of chunk c + 2
// in substep 1 of chunk c and the s half of chunk c + 3 in its substep 3.
//
//   substep q of chunk c : eight MFMAs; between them the reads of the next
//     substep's s fragments, in substep 3 also the t fragments 0-2 of chunk
//     c + 1, in substep 0 the t fragment 3 of chunk c; in substeps 1 and 3
//     the DMAs of the half named above
//   after substep 0 : barrier (every wave holds chunk c's t fragments: its t
//     slot is free)
//   after substep 2 (chunk c + 1 follows) : wait for chunk c + 1, barrier
//     (it has landed, and every wave's reads of chunk c's s half are done)
__device__ __forceinline__ void run(const LayerArgs& p, const Act& a, int D, int b, int S, int Tb,
                                    int k0, int n, Acc& acc, unsigned char* lds) {
  static_assert(kBA == 4 && kBO == 2, "the interleave encodes 8 MFMAs per substep");
  static_assert(kWaveRows * kWaveCols == kWaves, "wave grid");
  static_assert(kSlots == 5, "the slot rota assumes five halves");
  acc.zero();
  if (n <= 0) return;
  const __amdgpu_buffer_rsrc_t r = sample_rsrc(a, b, p.T, D);
  const int tid = opaque_tid();
  DmaLane dl;
  dl.init(p, a, b, S, Tb, tid);
  const uint32_t base = lds_addr(lds);
  // This wave's DMAs fill kDmaPerHalf consecutive KiB of a slot.
  const uint32_t wdst = (uint32_t)(kDmaPerHalf * __builtin_amdgcn_readfirstlane(tid >> 6)) * 1024u;
  const int m0 = k0 >> 1;
  const int nc = ((k0 + n - 1) >> 1) - m0 + 1;      // chunks of the run
  const int nh = 2 * nc;                            // halves of the run
  const int u0 = 2 * k0 - 4 * m0, u1 = 2 * (k0 + n) - 4 * m0;   // substeps, from chunk 0
  auto half_slot = [&](int h) { return (h & 1) ? slot_t(h >> 1) : slot_s(h >> 1); };
#pragma unroll
  for (int h = 0; h < kSlots; ++h) {
    if (h < nh) {
      HalfDma hd;
      hd.at(m0 + (h >> 1), D);
      const uint32_t dst = base + (uint32_t)half_slot(h) * kHalfBytes + wdst;
#pragma unroll
      for (int j = 0; j < kDmaPerHalf; ++j) hd.dma(r, (h & 1) ? dl.t[j] : dl.s[j], dst, j);
    }
  }
  int issued = min(nh, kSlots);
  wait_halves(issued - 2);             // chunk 0 has landed for this wave
  step_barrier();
  Frags f;
  // lane parts of the s blocks (rows wave_row * 128 + 32 i) and the t blocks
  // (rows wave_col * 64 + 32 j)
  const uint32_t ls = frag_lane(wave_row() * (kBA * 32));
  const uint32_t lt = frag_lane(wave_col() * (kBO * 32));
  auto half_at = [&](int slot) { return base + (uint32_t)slot * kHalfBytes; };
  {
    const int q0 = u0 & 3;             // 0 or 2: s fragments in f.a[0]
    const uint32_t as = sub_addr(half_at(slot_s(0)), ls, q0);
#pragma unroll
    for (int i = 0; i < kBA; ++i) f.a[0][i] = frag(as, i);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t at = sub_addr(half_at(slot_t(0)), lt, q);
#pragma unroll
      for (int j = 0; j < kBO; ++j) f.b[q][j] = frag(at, j);
    }
  }
  lds_reads_done();
  step_barrier();                      // chunk 0's t slot is free
  // The next half in line goes out now if it is the t half of chunk 2.
  HalfDma hd;
  uint32_t dst = 0;
  bool tside = false;
  auto prepare = [&](int h) {          // true: DMAs of half h to issue
    if (h != issued || h >= nh) return false;
    hd.at(m0 + (h >> 1), D);
    dst = base + (uint32_t)half_slot(h) * kHalfBytes + wdst;
    tside = h & 1;
    ++issued;
    return true;
  };
  if (prepare(5)) {
#pragma unroll
    for (int j = 0; j < kDmaPerHalf; ++j) hd.dma(r, tside ? dl.t[j] : dl.s[j], dst, j);
  }
  // Substep q of chunk c: its eight MFMAs, with the reads of the next
  // substep's fragments and the DMAs of the half queued now between them,
  // then the barrier after it.  Returns false after the run's last substep.
  // STEADY: a full chunk with three more after it (both of its halves to
  // queue, both barriers taken), where nothing needs testing.
  auto substep = [&](auto qc, auto steady, int c, uint32_t hs, uint32_t ht, uint32_t ns,
                     uint32_t nt) -> bool {
    constexpr int q = decltype(qc)::value;
    constexpr bool STEADY = decltype(steady)::value;
    const int u = 4 * c + q;
    if (!STEADY && (u < u0 || u >= u1)) return true;
    const bool more = STEADY || u + 1 < u1;
    bool dma = false;
    if constexpr (q == 1 || q == 3) {
      if constexpr (STEADY) {
        // the t half of chunk c + 2 into chunk c's t slot, or the s half of
        // chunk c + 3 into its s slot
        hd.at(m0 + c + (q == 1 ? 2 : 3), D);
        dst = (q == 1 ? ht : hs) + wdst;
        tside = q == 1;
        ++issued;
        dma = true;
      } else {
        dma = prepare(q == 1 ? 2 * c + 5 : 2 * c + 6);
      }
    }
    // addresses of this substep's reads
    const uint32_t an = q < 3 ? sub_addr(hs, ls, q + 1) : sub_addr(ns, ls, 0);
    uint32_t at = 0;
    if constexpr (q == 0) at = sub_addr(ht, lt, 3);
    acc.pin();
    sched_fence();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      acc.mma1(f, q, k);
      sched_fence();
      if (dma && (k & 1) == 0) hd.dma(r, tside ? dl.t[k >> 1] : dl.s[k >> 1], dst, k >> 1);
      if (more) {
        if (k < kBA) {
          f.a[(q + 1) & 1][k] = frag(an, k);
        } else if constexpr (q == 3) {
          // t fragments of substeps 0..2 of chunk c + 1 (3 is in use)
          const int x = k - kBA;
          if (x < 3) {
            const uint32_t ax = sub_addr(nt, lt, x);
            f.b[x][0] = frag(ax, 0);
            f.b[x][1] = frag(ax, 1);
          }
        } else if constexpr (q == 0) {
          if (k == kBA && (STEADY || c >= 1)) {
            f.b[3][0] = frag(at, 0);
            f.b[3][1] = frag(at, 1);
          }
        }
      }
      sched_fence();
    }
    if (!more) return false;
    if constexpr (q == 0) {
      if (STEADY || c >= 1) {
        lds_reads_done();
        step_barrier();                // chunk c's t slot is free
      }
    } else if constexpr (q == 2) {
      if (STEADY || u + 2 < u1) {
        lds_reads_done();
        // halves up to 2c + 3 are needed; those queued after may fly
        wait_halves(STEADY ? 2 : issued - (2 * c + 4));
        step_barrier();
      }
    }
    return true;
  };
  auto chunk = [&](auto steady, int c) -> bool {
    const uint32_t hs = half_at(slot_s(c)), ht = half_at(slot_t(c));
    const uint32_t ns = half_at(slot_s(c + 1)), nt = half_at(slot_t(c + 1));
    return substep(std::integral_constant<int, 0>{}, steady, c, hs, ht, ns, nt) &&
           substep(std::integral_constant<int, 1>{}, steady, c, hs, ht, ns, nt) &&
           substep(std::integral_constant<int, 2>{}, steady, c, hs, ht, ns, nt) &&
           substep(std::integral_constant<int, 3>{}, steady, c, hs, ht, ns, nt);
  };
  // chunk 0, then the steady chunks 1 .. nc - 4, then the last ones
  bool go = chunk(std::false_type{}, 0);
  int c = 1;
  for (; go && c <= nc - 4; ++c) chunk(std::true_type{}, c);
  for (; go && c < nc; ++c) go = chunk(std::false_type{}, c);
  __syncthreads();                     // every wave is done with the slot ring
}

// A Gram tile's accumulators, thread-major: f32x4 x of thread tid at
// [x][tid], so that the stores and loads of consecutive threads are
// contiguous.  Quad x = (i * kBO + j) * 4 + q holds block (i, j) registers
// 4q .. 4q+3.
__device__ __forceinline__ void store_gram(float* dst, const Acc& acc) {
  const int tid = opaque_tid();
  f32x4* d = (f32x4*)dst + tid;
#pragma unroll
  for (int i = 0; i < kBA; ++i)
#pragma unroll
    for (int j = 0; j < kBO; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 v;
        v.x = acc.v[i][j][4 * q]; v.y = acc.v[i][j][4 * q + 1];
        v.z = acc.v[i][j][4 * q + 2]; v.w = acc.v[i][j][4 * q + 3];
        d[((i * kBO + j) * 4 + q) * kNT] = v;
        if (q == 3) sched_fence();   // one block's registers at a time
      }
}

// Weight of an item's elements in the symmetric sum.  Off the diagonal
// (S < Tb) every element has s < t: weight 2.  A diagonal item (S == Tb)
// pairs the same 256 tokens on both sides, so both of its Gram blocks are
// symmetric and the sum above its diagonal equals the sum below: weighting
// 2 above, 1 on and 0 below gives the plain sum of the whole block.
__device__ __forceinline__ float item_weight(int S, int Tb) { return S < Tb ? 2.0f : 1.0f; }

// Sum over this thread's elements of xg * gg, with xg a thread-major Gram
// tile (layout at store_gram) and gg the accumulators.
__device__ __forceinline__ float product_sum(const float* xg, const Acc& gg) {
  const int tid = opaque_tid();
  const f32x4* dx = (const f32x4*)xg + tid;
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kBA; ++i)
#pragma unroll
    for (int j = 0; j < kBO; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 u = dx[((i * kBO + j) * 4 + q) * kNT];
        sum += u.x * gg.v[i][j][4 * q] + u.y * gg.v[i][j][4 * q + 1] +
               u.z * gg.v[i][j][4 * q + 2] + u.w * gg.v[i][j][4 * q + 3];
      }
      if (j == kBO - 1) sched_fence();   // 8 loaded quads at a time
    }
  return sum;
}

// Work plan: G persistent workgroups; the first D*G items in D full rounds
// (item d*G + L to workgroup L); each of the R remaining items split into P
// chunks of its feature steps (X steps first, then G steps; P == 1: not
// split), piece pi = c*R + r going to workgroup pi mod G.  A piece stores
// the partial Gram of each side it touches; the fixup kernel finishes split
// items.
struct GramPlan {
  int G, D, R, P;
};

// D, R and P for `items` items of n feature steps on G workgroups, with at
// most `cap` pieces.  Cost model in microseconds from measurements on MI355X:
// a 32-feature step of a 256 x 256 item ~0.8 us; a piece's pipeline fill and
// partial store ~8 us; the fixup ~10 us plus 0.1 us per piece.  Runs on the
// host, and on the device for masked calls, where only the device knows how
// many items hold an active token.
__host__ __device__ inline GramPlan split_items(int items, int G, int n, int cap) {
  GramPlan gp{G, items / G, items % G, 1};
  if (gp.R == 0) return gp;
  const double step_us = 0.8, piece_us = 8.0;
  double best = n * step_us + piece_us;
  for (int P = 2; P <= kMaxSplit; ++P) {
    if ((double)n / P < 8.0 || gp.R * P > cap) break;
    const int S = (gp.R * P + G - 1) / G;
    const double t = S * ((double)n / P * step_us + piece_us) + 10.0 + 0.1 * gp.R * P;
    if (t < best) {
      best = t;
      gp.P = P;
    }
  }
  return gp;
}

// Workgroups are dealt to the 8 XCDs round robin; logical index of this
// workgroup such that XCD x holds the contiguous range [x*G/8, (x+1)*G/8):
// consecutive items (same sample, shared rows) meet in one L2.
__device__ __forceinline__ int logical_wg(int id, int G) {
  return (G % 8 == 0) ? (id & 7) * (G / 8) + (id >> 3) : id;
}

// Feature steps [c0, c1) of the concatenated sequence (X steps, then G
// steps) split into the X part [x0, x1) and the G part [g0, g1).
struct Parts {
  int x0, x1, g0, g1;
  __device__ __forceinline__ Parts(int c0, int c1, int nkx) {
    x0 = min(c0, nkx);
    x1 = min(c1, nkx);
    g0 = max(c0, nkx) - nkx;
    g1 = max(c1, nkx) - nkx;
  }
};

// Masked calls: live[0] = n, the number of items with an active token in
// both of their row blocks, live[1 .. n] their indices in increasing order.
// The other items are exactly zero; the list kernel stores their partials.
// The plan over the n live items is made here, with at most `cap` pieces.
// Workspace: xs = one X Gram per workgroup; pieces = two Gram tiles (X part,
// G part) per piece.
__global__ void __launch_bounds__(kNT, 1) gram_norm_big_kernel(LayerArgs p, GramPlan gp,
                                                               const uint32_t* live, int cap,
                                                               float* xs, float* pieces) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int per_sample = items_per_sample(p.T);
  const int nkx = (p.din + kKF - 1) / kKF, nkg = (p.dout + kKF - 1) / kKF;
  const int n = nkx + nkg;
  const int L = logical_wg(blockIdx.x, gp.G);
  if (live != nullptr) gp = split_items((int)((c_u32*)live)[0], gp.G, n, cap);
  auto item_at = [&](int i) { return live != nullptr ? (int)((c_u32*)live)[1 + i] : i; };
  // This workgroup's units: whole items d*G + L, then pieces L, L+G, ...
  const int nfull = gp.D + ((gp.P == 1 && L < gp.R) ? 1 : 0);
  const int npiece = gp.P == 1 ? 0 : (gp.R * gp.P - L + gp.G - 1) / gp.G;
  float* mine = xs + (int64_t)L * kGramFloats;   // this workgroup's X Gram
  Acc acc;
  // Whole items: the X Gram to scratch, then the G Gram, multiplied with the
  // X Gram read back by the threads that stored it.
#pragma unroll 1
  for (int u = 0; u < nfull; ++u) {
    const int item = item_at(u * gp.G + L);
    int b, S, Tb;
    item_coords(item, per_sample, p.T, &b, &S, &Tb);
    run(p, p.X, p.din, b, S, Tb, 0, nkx, acc, smem);
    store_gram(mine, acc);
    run(p, p.G, p.dout, b, S, Tb, 0, nkg, acc, smem);
    const double tot =
        block_sum_f64((double)(item_weight(S, Tb) * product_sum(mine, acc)), (double*)smem);
    if (threadIdx.x == 0) p.partials[item] = tot;
    __syncthreads();                 // the reduction scratch is the next unit's ring
  }
  // Pieces: the partial Gram of each side the piece touches.
#pragma unroll 1
  for (int u = 0; u < npiece; ++u) {
    const int pi = L + u * gp.G;
    const int c = pi / gp.R;
    const int item = item_at(gp.D * gp.G + pi % gp.R);
    int b, S, Tb;
    item_coords(item, per_sample, p.T, &b, &S, &Tb);
    const Parts pt((int)((int64_t)c * n / gp.P), (int)((int64_t)(c + 1) * n / gp.P), nkx);
    float* dst = pieces + (int64_t)pi * 2 * kGramFloats;
#pragma unroll 1
    for (int side = 0; side < 2; ++side) {
      const int k0 = side ? pt.g0 : pt.x0, k1 = side ? pt.g1 : pt.x1;
      if (k1 <= k0) continue;
      run(p, side ? p.G : p.X, side ? p.dout : p.din, b, S, Tb, k0, k1 - k0, acc, smem);
      store_gram(dst + side * kGramFloats, acc);
    }
  }
}

// Split items: sum the partial X and G Grams of the P pieces in chunk order,
// then the weighted product and its reduction, as for a whole item.  Each
// item spreads over kFixParts workgroups (with the main kernel's thread
// layout), workgroup h taking quads [h, h+1) * kAccFloats / 4 / kFixParts of
// every thread; their fp64 sums go to part[r][h], which gram_fixup_sum_kernel
// adds in order.  Masked calls launch workgroups for every possible split
// item and make the plan as the main kernel does.
constexpr int kFixParts = 8;
constexpr int kFixQuads = kAccFloats / 4 / kFixParts;   // 4
constexpr int kFixBatch = 4;                            // pieces whose loads are in flight together
__global__ void __launch_bounds__(kNT, 1) gram_fixup_kernel(LayerArgs p, GramPlan gp,
                                                            const uint32_t* live, int cap,
                                                            const float* pieces, double* part) {
  __shared__ double red[kNT / 64];
  const int nkx = (p.din + kKF - 1) / kKF, nkg = (p.dout + kKF - 1) / kKF;
  const int n = nkx + nkg;
  if (live != nullptr) gp = split_items((int)((c_u32*)live)[0], gp.G, n, cap);
  const int r = blockIdx.x / kFixParts, h = blockIdx.x % kFixParts;
  if (gp.P == 1 || r >= gp.R) return;
  const int i = gp.D * gp.G + r;
  const int item = live != nullptr ? (int)((c_u32*)live)[1 + i] : i;
  int b, S, Tb;
  item_coords(item, items_per_sample(p.T), p.T, &b, &S, &Tb);
  f32x4 sx[kFixQuads], sg[kFixQuads];
#pragma unroll
  for (int x = 0; x < kFixQuads; ++x) {
    sx[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    sg[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // The loads of kFixBatch pieces are issued before any of their sums, so
  // that they are in flight together; each piece's load covers only the
  // sides it touched, and the sums run in piece order.
  for (int c0 = 0; c0 < gp.P; c0 += kFixBatch) {
    f32x4 wx[kFixBatch][kFixQuads], wg[kFixBatch][kFixQuads];
    bool tx[kFixBatch], tg[kFixBatch];
#pragma unroll
    for (int j = 0; j < kFixBatch; ++j) {
      const int c = c0 + j;
      const Parts pt((int)((int64_t)c * n / gp.P), (int)((int64_t)(c + 1) * n / gp.P), nkx);
      tx[j] = c < gp.P && pt.x1 > pt.x0;
      tg[j] = c < gp.P && pt.g1 > pt.g0;
      const f32x4* src = (const f32x4*)(pieces + (int64_t)(min(c, gp.P - 1) * gp.R + r) * 2 *
                                                     kGramFloats) +
                         (h * kFixQuads) * kNT + threadIdx.x;
#pragma unroll
      for (int x = 0; x < kFixQuads; ++x) {
        wx[j][x] = tx[j] ? src[x * kNT] : f32x4{0.f, 0.f, 0.f, 0.f};
        wg[j][x] = tg[j] ? src[kGramFloats / 4 + x * kNT] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int j = 0; j < kFixBatch; ++j) {
#pragma unroll
      for (int x = 0; x < kFixQuads; ++x) {
        if (tx[j]) sx[x] += wx[j][x];
        if (tg[j]) sg[x] += wg[j][x];
      }
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int x = 0; x < kFixQuads; ++x)
    sum += sx[x].x * sg[x].x + sx[x].y * sg[x].y + sx[x].z * sg[x].z + sx[x].w * sg[x].w;
  const double tot = block_sum_f64((double)(item_weight(S, Tb) * sum), red);
  if (threadIdx.x == 0) part[r * kFixParts + h] = tot;
}

// partials[item] = sum over h of part[r][h], in order; one thread per split
// item.
__global__ void gram_fixup_sum_kernel(LayerArgs p, GramPlan gp, const uint32_t* live, int cap,
                                      const double* part) {
  const int nkx = (p.din + kKF - 1) / kKF, nkg = (p.dout + kKF - 1) / kKF;
  if (live != nullptr) gp = split_items((int)((c_u32*)live)[0], gp.G, nkx + nkg, cap);
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (gp.P == 1 || r >= gp.R) return;
  const int i = gp.D * gp.G + r;
  const int item = live != nullptr ? (int)((c_u32*)live)[1 + i] : i;
  double s = 0.0;
  for (int h = 0; h < kFixParts; ++h) s += part[r * kFixParts + h];
  p.partials[item] = s;
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
  constexpr int kWords = kRows / 32;   // row-bit words per block
  uint32_t base = 0;
  for (int64_t c0 = 0; c0 < total; c0 += kListThreads) {
    const int64_t i = c0 + tid;
    bool act = false;
    if (i < total) {
      int b, S, Tb;
      item_coords((int)i, per_sample, p.T, &b, &S, &Tb);
      const uint32_t* w = p.rowbits + (int64_t)b * p.nwords;
      uint32_t ws = 0, wt = 0;
      for (int k = S * kWords; k < min((S + 1) * kWords, p.nwords); ++k) ws |= w[k];
      for (int k = Tb * kWords; k < min((Tb + 1) * kWords, p.nwords); ++k) wt |= w[k];
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
  gram::GramPlan gp = gram::split_items(items, G, n, p.max_split == 1 ? 0 : 1 << 30);
  if (gp.P == 1 && gp.D == 0) gp.G = gp.R;
  return gp;
}

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace layout: [live-item list (masked calls)] [one X Gram per
// workgroup] [two Gram tiles per piece] [fixup sums].  A masked call reserves room for G
// pieces: the device-side plan never splits into more.
struct GramWs {
  size_t xs = 0, pieces = 0, part = 0, total = 0;
};
GramWs gram_ws(const LayerArgs& p, const gram::GramPlan& gp) {
  GramWs w;
  const size_t tile = (size_t)gram::kGramFloats * sizeof(float);
  if (p.mask != nullptr) w.xs = round256(((size_t)p.B * gram::items_per_sample(p.T) + 1) * 4);
  w.pieces = w.xs + (size_t)gp.G * tile;
  const size_t npieces = p.max_split == 1 ? 0
                        : p.mask != nullptr ? (size_t)gp.G : (gp.P == 1 ? 0 : (size_t)gp.R * gp.P);
  w.part = w.pieces + npieces * 2 * tile;
  // fixup sums: one row per possible split item (R < G)
  w.total = w.part + round256((size_t)gp.G * gram::kFixParts * sizeof(double));
  return w;
}
}  // namespace

size_t gram_big_workspace_bytes(const LayerArgs& p) { return gram_ws(p, plan_gram(p)).total; }

hipError_t launch_gram_norm_big(const LayerArgs& p, hipStream_t s) {
  static hipError_t once = hipFuncSetAttribute((const void*)gram::gram_norm_big_kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               gram::kLdsBytes);
  if (once != hipSuccess) return once;
  const gram::GramPlan gp = plan_gram(p);
  const bool masked = p.rowbits != nullptr;
  if (p.skws == nullptr) return hipErrorInvalidValue;
  const GramWs w = gram_ws(p, gp);
  char* base = reinterpret_cast<char*>(p.skws);
  uint32_t* live = masked ? reinterpret_cast<uint32_t*>(base) : nullptr;
  float* xs = reinterpret_cast<float*>(base + w.xs);
  float* pieces = reinterpret_cast<float*>(base + w.pieces);
  double* part = reinterpret_cast<double*>(base + w.part);
  // pieces the device-side plan of a masked call may use (0: no split)
  const int cap = p.max_split == 1 ? 0 : gp.G;
  hipError_t e;
  if (masked) {
    timing_begin("live_items", s);
    hipLaunchKernelGGL(gram::live_items_kernel, dim3(1), dim3(gram::kListThreads), 0, s, p, live);
    e = hipGetLastError();
    timing_end("live_items", s);
    if (e != hipSuccess) return e;
  }
  timing_begin("gram_norm", s);
  hipLaunchKernelGGL(gram::gram_norm_big_kernel, dim3(gp.G), dim3(gram::kNT), gram::kLdsBytes, s, p,
                     gp, (const uint32_t*)live, cap, xs, pieces);
  e = hipGetLastError();
  timing_end("gram_norm", s);
  if (e != hipSuccess || (!masked && gp.P == 1)) return e;
  const int nfix = masked ? gp.G : gp.R;   // items that may be split
  timing_begin("gram_fixup", s);
  hipLaunchKernelGGL(gram::gram_fixup_kernel, dim3(nfix * gram::kFixParts), dim3(gram::kNT), 0, s,
                     p, gp, (const uint32_t*)live, cap, (const float*)pieces, part);
  e = hipGetLastError();
  if (e == hipSuccess)
    hipLaunchKernelGGL(gram::gram_fixup_sum_kernel, dim3((nfix + 63) / 64), dim3(64), 0, s, p, gp,
                       (const uint32_t*)live, cap, (const double*)part);
  if (e == hipSuccess) e = hipGetLastError();
  timing_end("gram_fixup", s);
  return e;
}

}  // namespace dpf
