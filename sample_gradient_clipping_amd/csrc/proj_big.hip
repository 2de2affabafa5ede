// Projection Y = X~ P of the projected variant (Memory-Efficient
// Differentially Private Training with Gradient Random Projection, English
// explainer, Methodology: project first, then clip and add noise), bf16, for
// 16-byte-aligned shapes.
//
//   X~ [B*T, din]  (masked rows read as zero)      P [din, r]      Y [B*T, r]
//
// The RoBERTa-sized calls this serves are small GEMMs (a few GFLOP), so the
// tile is chosen for parallelism, not reuse: 64 r columns x 64 tokens per
// workgroup, the whole din range in one workgroup (no split along din, hence
// no partial products and no second kernel).  4096 tokens x r = 256 give 256
// workgroups, one per compute unit.
//
// Workgroup: 512 threads = 8 waves, two per SIMD.  Waves w and w + 4 own the
// same 32 x 32 block of v_mfma_f32_32x32x16_bf16 accumulators (A = P^T: rows
// along r; B = X~^T: columns along tokens; the 2 x 2 blocks of the tile), the
// first on features 0..63 of every 128-feature step, the second on 64..127,
// each in two accumulator sets (alternate 16-feature substeps) so that its
// MFMAs form two independent chains.  At these sizes a step's cost is its
// serial chain (barrier, LDS read latency, dependent MFMAs), not its data or
// arithmetic, so each step carries as many features as the LDS ring allows.
// At the end each wave adds its two sets, the second group's sums go through
// LDS to the first, which adds them (fixed order) and stores Y; each lane
// ends with 4 consecutive r of one token.  Both operands go from global
// memory to LDS with 16-byte-per-lane buffer loads that write LDS directly,
// into a ring of four 32 KiB slots filled three steps ahead, one barrier per
// step.
//   X rows (tokens, features contiguous: "K-inner", 256 B per step) are read
//   back as whole 16-byte fragments; chunk c of row t sits at c ^ (t % 16).
//   P rows (features, r contiguous: "K-outer", 128 B per step) are read with
//   the transposing ds_read_b64_tr_b16; chunk c of row k sits at
//   c ^ (4 ((k >> 1) & 1)).
// Both placements keep the reads free of bank conflicts.  Rows past the end,
// masked tokens and features past din read through out-of-range buffer
// offsets, which return zeros.
#include "kernels.hpp"
#include "tiles.hpp"

namespace dpf {
namespace proj {

constexpr int kNT = 512;
constexpr int kTile = 64;                      // r columns and tokens per tile
constexpr int kKF = 128;                       // features per step
constexpr int kXRowBytes = kKF * 2;            // an X row of one step: 256 B
constexpr int kPRowBytes = kTile * 2;          // a P row (64 r columns): 128 B
constexpr int kXBytes = kTile * kXRowBytes;    // 16 KiB: 64 token rows
constexpr int kPBytes = kKF * kPRowBytes;      // 16 KiB: 128 feature rows
constexpr int kStageBytes = kXBytes + kPBytes; // X rows, then P rows
constexpr int kStages = 4;
constexpr int kLdsBytes = kStages * kStageBytes;   // 128 KiB
constexpr int kDmaPerOp = 2;                   // per wave per step: 2 KiB of X, 2 KiB of P
constexpr int kDmaPerStep = 2 * kDmaPerOp;
constexpr int kOOB = 0x7ffffff0;
// Largest byte span of X or P this kernel addresses (32-bit buffer offsets,
// with room above for the out-of-range offset).
constexpr int64_t kMaxSpan = ((int64_t)1 << 31) - ((int64_t)1 << 20);

__device__ __forceinline__ int swz_x(int row, int c) { return c ^ (row & 15); }
__device__ __forceinline__ int swz_p(int k, int c) { return c ^ (((k >> 1) & 1) << 2); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const unsigned char*)p;
}

// 16 bytes per lane from rsrc at voffset + soffset straight into LDS at
// m0 + 16 * lane; soffset is wave-uniform (the step's offset).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, int voffset, uint32_t lds,
                                      uint32_t soffset) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(lds), "s"(soffset)
               : "memory");
}

// Wait until at most `steps` (0 .. kStages - 2) of this wave's most recent
// DMA steps are in flight: four DMAs per step, or two when P is drawn in the
// kernel (GEN).
template <bool GEN>
__device__ __forceinline__ void wait_dma(int steps) {
  static_assert(kDmaPerStep == 4 && kStages == 4, "wait_dma encodes up to 2 steps ahead");
  if (steps <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (steps == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(GEN ? 2 : 4) : "memory");
  else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(GEN ? 4 : 8) : "memory");
}

// Workgroup barrier without a memory fence: each wave has seen its own DMA
// writes land (wait_dma) before it; the empty asm statements keep the
// compiler from moving LDS accesses across.
__device__ __forceinline__ void step_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Byte span of X that rows of B samples x T tokens x din features cover.
__host__ __device__ inline int64_t x_span(const ProjArgs& p) {
  return ((int64_t)(p.B - 1) * p.X.stride_b + (int64_t)(p.T - 1) * p.X.stride_t + p.din) * 2;
}

// Per-lane DMA addressing, fixed for the whole K loop.  Wave w fills X rows
// 8 w .. 8 w + 7 (DMA j: rows 8 w + 4 j .. +3, lane l physical chunk l % 16
// of row 8 w + 4 j + l / 16) and P rows 16 w .. 16 w + 15 (DMA j: rows
// 16 w + 8 j .. +7, lane l physical chunk l % 8 of row 16 w + 8 j + l / 8):
// 1 KiB of consecutive LDS per DMA.
struct Lanes {
  uint32_t xoff[kDmaPerOp];   // X: token row + logical chunk, bytes (kOOB: inactive)
  int xf[kDmaPerOp];          // first feature of the lane's X chunk within a step
  uint32_t poff[kDmaPerOp];   // P: row within the step + column chunk, bytes (kOOB: past r)
  int pk[kDmaPerOp];          // the P row (feature) within a step
  int pcol[kDmaPerOp];        // the first r column of the lane's P chunk
  __device__ __forceinline__ void init(const ProjArgs& p, int64_t q0, int j0) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t ntok = (int64_t)p.B * p.T;
#pragma unroll
    for (int j = 0; j < kDmaPerOp; ++j) {
      const int row = 8 * wave + 4 * j + (lane >> 4);
      const int cx = swz_x(row, lane & 15);
      const int64_t tok = q0 + row;
      bool on = tok < ntok;
      if (on && p.mask != nullptr) on = p.mask[tok] != 0;
      const int64_t b = tok / p.T, t = tok - b * p.T;
      xf[j] = 8 * cx;
      xoff[j] = on ? (uint32_t)((b * p.X.stride_b + t * p.X.stride_t + 8 * cx) * 2)
                   : (uint32_t)kOOB;
      const int k = 16 * wave + 8 * j + (lane >> 3);
      const int cp = swz_p(k, lane & 7);
      const int col = j0 + 8 * cp;
      pk[j] = k;
      pcol[j] = col;
      poff[j] = col < p.r ? (uint32_t)(((int64_t)k * p.r + col) * 2) : (uint32_t)kOOB;
    }
  }
};

// Step k's rows of this wave into the slot at LDS offset `slot`: X by DMA;
// P by DMA, or (GEN) drawn from its seed here and written to the place the
// DMA would have filled (the LDS reads that follow wait for these writes,
// which complete in order with them, before the next barrier).
template <bool GEN>
__device__ __forceinline__ void issue(const ProjArgs& p, __amdgpu_buffer_rsrc_t rx,
                                      __amdgpu_buffer_rsrc_t rp, const Lanes& ln, int k,
                                      unsigned char* lds, uint32_t base, uint32_t slot,
                                      uint32_t wdst) {
  const int k0 = k * kKF;
  const bool tail = k0 + kKF > p.din;
  const uint32_t sx = (uint32_t)k0 * 2u;
#pragma unroll
  for (int j = 0; j < kDmaPerOp; ++j) {
    int xo = (int)ln.xoff[j];
    if (tail && k0 + ln.xf[j] >= p.din) xo = kOOB;
    dma16(rx, xo, base + slot + wdst + (uint32_t)j * 1024u, sx);
  }
#pragma unroll
  for (int j = 0; j < kDmaPerOp; ++j) {
    if constexpr (GEN) {
      const int lane = threadIdx.x & 63;
      const int col = ln.poff[j] == (uint32_t)kOOB ? p.r : ln.pcol[j];
      *(u32x4*)(lds + slot + kXBytes + wdst + j * 1024 + 16 * lane) =
          gen_p_chunk<BF16>(p.p_seed, p.p_offset, p.p_scale, p.din, p.r, k0 + ln.pk[j], col);
    } else {
      const uint32_t sp = (uint32_t)k0 * (uint32_t)p.r * 2u;
      int po = (int)ln.poff[j];
      if (tail && k0 + ln.pk[j] >= p.din) po = kOOB;
      dma16(rp, po, base + slot + kXBytes + wdst + (uint32_t)j * 1024u, sp);
    }
  }
}

// A operand: P^T rows m0 .. m0+31 (r), 16-feature substep ks, by two
// transposing reads.
__device__ __forceinline__ u16x8 frag_p(const unsigned char* op, int m0, int ks) {
  const int lane = threadIdx.x & 63;
  const int krow = ks * 16 + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = m0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int c16 = col >> 3, half = (col >> 2) & 1;
  const unsigned char* p0 = op + krow * kPRowBytes + swz_p(krow, c16) * 16 + half * 8;
  const unsigned char* p1 = op + (krow + 4) * kPRowBytes + swz_p(krow + 4, c16) * 16 + half * 8;
  const u16x4 lo = lds_read_tr16((const uint16_t*)p0);
  const u16x4 hi = lds_read_tr16((const uint16_t*)p1);
  u16x8 f;
  f.s0 = lo.s0; f.s1 = lo.s1; f.s2 = lo.s2; f.s3 = lo.s3;
  f.s4 = hi.s0; f.s5 = hi.s1; f.s6 = hi.s2; f.s7 = hi.s3;
  return f;
}

// B operand: X~ rows m0 .. m0+31 (tokens), 16-feature substep ks, one
// 16-byte read per lane.
__device__ __forceinline__ u16x8 frag_x(const unsigned char* op, int m0, int ks) {
  const int lane = threadIdx.x & 63;
  const int row = m0 + (lane & 31);
  const int c = 2 * ks + (lane >> 5);
  return *(const u16x8*)(op + row * kXRowBytes + swz_x(row, c) * 16);
}

// Tiles in token-major order (the r tiles of one token block adjacent), and
// workgroups dealt to the 8 XCDs round robin, so workgroup id takes logical
// tile (id % 8) * (G / 8) + id / 8: each XCD runs a contiguous range of
// tiles, and the r tiles that read one X block meet in one L2 instead of
// fetching it into several.
template <bool GEN>
__global__ void __launch_bounds__(kNT) project_big_kernel(ProjArgs p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int ntr = (p.r + kTile - 1) / kTile;
  const int G = (int)gridDim.x, id = (int)blockIdx.x;
  const int L = (G % 8 == 0) ? (id & 7) * (G >> 3) + (id >> 3) : id;
  const int64_t q0 = (int64_t)(L / ntr) * kTile;
  const int j0 = (L % ntr) * kTile;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int half = wave >> 2;               // features 64 half .. 64 half + 63 of each step
  const int wm = (wave >> 1) & 1, wn = wave & 1;

  const __amdgpu_buffer_rsrc_t rx = rsrc(p.X.data, x_span(p));
  const __amdgpu_buffer_rsrc_t rp = rsrc(GEN ? p.X.data : p.P, GEN ? 0 : (int64_t)p.din * p.r * 2);
  Lanes ln;
  ln.init(p, q0, j0);
  const uint32_t base = lds_addr(lds);
  const uint32_t wdst = (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 2048u;
  const int n = (p.din + kKF - 1) / kKF;

  f32x16 acc[2];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[0][e] = acc[1][e] = 0.f;

  // Steps 0 .. kStages-2 before the loop; step i + kStages - 1 at iteration
  // i, into the slot that step i - 1 used (free once every wave has passed
  // iteration i's barrier).  At iteration i's wait, min(n, kStages - 1 + i)
  // steps have been issued, min(n - 1 - i, kStages - 2) of them after step i.
#pragma unroll
  for (int k = 0; k < kStages - 1; ++k)
    if (k < n) issue<GEN>(p, rx, rp, ln, k, lds, base, (uint32_t)k * kStageBytes, wdst);
  int slot = 0;
  for (int i = 0; i < n; ++i) {
    wait_dma<GEN>(min(n - 1 - i, kStages - 2));
    if constexpr (GEN) __builtin_amdgcn_s_waitcnt(0xC07F);   // this wave's P writes (lgkmcnt(0))
    step_barrier();
    if (i + kStages - 1 < n) {
      const int fs = slot == 0 ? kStages - 1 : slot - 1;
      issue<GEN>(p, rx, rp, ln, i + kStages - 1, lds, base, (uint32_t)fs * kStageBytes, wdst);
    }
    const unsigned char* st = lds + slot * kStageBytes;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int ks = 4 * half + h;
      const u16x8 a = frag_p(st + kXBytes, wm * 32, ks);
      const u16x8 b = frag_x(st, wn * 32, ks);
      acc[h & 1] = mfma_32x32x16(a, b, acc[h & 1]);
    }
    slot = slot + 1 == kStages ? 0 : slot + 1;
  }

  // Each wave's two sets added, then the second group's sums to the first
  // through LDS (every DMA has landed and every operand read has returned
  // before the barrier), lane-major so that the stores and loads of
  // consecutive lanes are contiguous.
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[0][e] += acc[1][e];
  __syncthreads();
  f32x4* red = (f32x4*)lds + (wave & 3) * 4 * 64 + lane;
  if (half == 1) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      red[g * 64] = f32x4{acc[0][4 * g], acc[0][4 * g + 1], acc[0][4 * g + 2], acc[0][4 * g + 3]};
  }
  __syncthreads();
  if (half == 1) return;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 u = red[g * 64];
    acc[0][4 * g] += u.x; acc[0][4 * g + 1] += u.y; acc[0][4 * g + 2] += u.z; acc[0][4 * g + 3] += u.w;
  }

  // Y[token][j .. j+3] in bf16, 8 bytes per lane and register group.
  const int64_t ntok = (int64_t)p.B * p.T;
  const int64_t q = q0 + wn * 32 + acc_col(lane);
  if (q >= ntok) return;
  uint16_t* yrow = (uint16_t*)p.Y + q * p.r;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int j = j0 + wm * 32 + acc_row(4 * g, lane);
    if (j >= p.r) continue;
    u16x4 w;
    w.s0 = f32_to_bf16_rne(acc[0][4 * g + 0]);
    w.s1 = f32_to_bf16_rne(acc[0][4 * g + 1]);
    w.s2 = f32_to_bf16_rne(acc[0][4 * g + 2]);
    w.s3 = f32_to_bf16_rne(acc[0][4 * g + 3]);
    *(u16x4*)(yrow + j) = w;
  }
}

}  // namespace proj

bool project_big_shape_ok(const ProjArgs& p, bool vec) {
  return p.dtype == kBF16 && vec && p.r % 8 == 0 && p.din % 8 == 0 &&
         p.B >= 1 && p.T >= 1 && p.din >= 1 && proj::x_span(p) <= proj::kMaxSpan &&
         (int64_t)p.din * p.r * 2 <= proj::kMaxSpan;
}

bool project_big_eligible(const ProjArgs& p, bool vec) {
  return project_big_shape_ok(p, vec) && (p.gen != 0 || ((uintptr_t)p.P & 15) == 0) &&
         ((uintptr_t)p.Y & 7) == 0;
}

hipError_t launch_project_big(const ProjArgs& p, hipStream_t s) {
  static const hipError_t lds_ok = hipFuncSetAttribute(
      (const void*)proj::project_big_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
      proj::kLdsBytes);
  static const hipError_t lds_gen_ok = hipFuncSetAttribute(
      (const void*)proj::project_big_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
      proj::kLdsBytes);
  if (lds_ok != hipSuccess) return lds_ok;
  if (lds_gen_ok != hipSuccess) return lds_gen_ok;
  const int64_t ntok = (int64_t)p.B * p.T;
  const int64_t grid = ((ntok + proj::kTile - 1) / proj::kTile) * ((p.r + proj::kTile - 1) / proj::kTile);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  timing_begin("project", s);
  if (p.gen)
    hipLaunchKernelGGL(proj::project_big_kernel<true>, dim3((unsigned)grid), dim3(proj::kNT),
                       proj::kLdsBytes, s, p);
  else
    hipLaunchKernelGGL(proj::project_big_kernel<false>, dim3((unsigned)grid), dim3(proj::kNT),
                       proj::kLdsBytes, s, p);
  const hipError_t e = hipGetLastError();
  timing_end("project", s);
  return e;
}

}  // namespace dpf
