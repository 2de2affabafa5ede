// Large-tile bf16 kernels for the token-contraction G~^T X~ (K-outer x K-outer):
//
//   accumulate_big_kernel : grad = (sum_i c_i G~_i^T X~_i + noise_std xi) / B
//   direct_norm_big_kernel: per (output tile, sample) sum of squares of g_i's tile
//
// Workgroup: 256 threads = 4 waves (2 x 2); workgroup tile 256 (din) x 256
// (dout); each wave owns 128 x 128 = 4 x 4 blocks of v_mfma_f32_32x32x16_bf16
// accumulators (256 fp32 per lane).  K advances 32 tokens per step.
//
// Data movement per step: global memory -> LDS by 16-byte-per-lane buffer
// loads that write LDS directly (no staging registers), into a ring of four
// 32 KiB stages filled three steps ahead.  LDS rows are 512 bytes with no
// padding; the 16-byte chunk c of row k is stored at chunk c ^ (4 (k mod 4)),
// which keeps the transposing 8-byte reads (ds_read_b64_tr_b16) free of bank
// conflicts on gfx950's 64 banks.  Masked rows and columns past the end are
// read through out-of-range buffer offsets, which return zeros.
//
// Output tiles are ordered so that the workgroups resident on one XCD at a
// time cover a compact block of tiles (shared X and G strips stay in that
// XCD's L2).
#include "kernels.hpp"
#include "tiles.hpp"

namespace dpf {
namespace big {

constexpr int kNT = 256;
constexpr int kTile = 256;              // both output dims
constexpr int kKT = 32;                 // tokens per step
constexpr int kRowBytes = kTile * 2;    // one LDS row (bf16)
constexpr int kOpBytes = kKT * kRowBytes;      // one operand, one stage: 16 KiB
constexpr int kStageBytes = 2 * kOpBytes;      // X and G
constexpr int kStages = 4;
constexpr int kLdsBytes = kStages * kStageBytes;   // 128 KiB
constexpr int kDmaPerStep = 8;          // per wave: 4 for X, 4 for G (2 rows each)
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

// Wait until at most n of this wave's DMA steps are still in flight.
__device__ __forceinline__ void wait_dma(int steps_outstanding) {
  switch (steps_outstanding) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
  }
}
static_assert(kDmaPerStep == 8 && kStages - 2 <= 2, "wait_dma encodes 8 DMAs per step, <= 2 steps");

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const unsigned char*)p;
}

// Active-row bits of the 32 tokens starting at t0 of sample b.
__device__ __forceinline__ uint32_t step_bits(const LayerArgs& p, int b, int s) {
  if (p.rowbits != nullptr) return ((c_u32*)p.rowbits)[(int64_t)b * p.nwords + s];
  const int n = p.T - s * kKT;
  return n >= 32 ? 0xffffffffu : ((1u << n) - 1u);
}

// Queue step (b, s): X[tokens, a0:a0+256] and G[tokens, o0:o0+256] into one
// LDS stage.  Each wave moves 8 rows of each operand, 2 rows per DMA; lane l
// of a DMA fills physical chunk l % 32 of its row, i.e. logical chunk
// (l % 32) ^ swizzle(row).  Inactive rows and columns past the end read as 0.
__device__ __forceinline__ void issue_step(const LayerArgs& p, int b, int s, int a0, int o0,
                                           uint32_t stage) {
  const __amdgpu_buffer_rsrc_t rx = sample_rsrc(p.X, b, p.T, p.din);
  const __amdgpu_buffer_rsrc_t rg = sample_rsrc(p.G, b, p.T, p.dout);
  const uint32_t bits = step_bits(p, b, s);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = s * kKT;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r0 = 8 * wave + 2 * j;
    const int r = r0 + (lane >> 5);
    const int c16 = (lane & 31) ^ ((r & 3) << 2);
    const bool active = (bits >> r) & 1u;
    const int64_t t = t0 + r;
    const int ca = a0 + c16 * 8, co = o0 + c16 * 8;
    const int ox = (active && ca < p.din) ? (int)((t * p.X.stride_t + ca) * 2) : kOOB;
    const int og = (active && co < p.dout) ? (int)((t * p.G.stride_t + co) * 2) : kOOB;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(stage + r0 * kRowBytes);
    dma16(rx, ox, dst);
    dma16(rg, og, dst + kOpBytes);
  }
}

// MFMA operand for rows m0..m0+31 (within the 256-wide tile), k-substep ks.
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

struct Acc {
  f32x16 v[4][4];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) v[i][j][r] = 0.f;
  }
  // Rescale block by block; the empty asm statements pin each block's
  // product back into accumulation registers, which keeps the scaled copy
  // from occupying 256 ordinary VGPRs across the loop.
  __device__ __forceinline__ void scale(float s) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x16 t = v[i][j];
        asm volatile("" : "+v"(t));
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] *= s;
        asm volatile("" : "+a"(t));
        v[i][j] = t;
      }
  }
  __device__ __forceinline__ void compute(const unsigned char* stage) {
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int ks = 0; ks < kKT / 16; ++ks) {
      u16x8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = frag(stage, wm * 128 + i * 32, ks);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = frag(stage + kOpBytes, wn * 128 + j * 32, ks);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) v[i][j] = mfma_32x32x16(fa[i], fb[j], v[i][j]);
    }
  }
};

// (sample, step) cursor over the active steps of samples [b, b_end).
struct Cursor {
  int b, s, b_end, nsteps;
  __device__ __forceinline__ bool active(const LayerArgs& p) const {
    return p.rowbits == nullptr || ((c_u32*)p.rowbits)[(int64_t)b * p.nwords + s] != 0u;
  }
  __device__ __forceinline__ void settle(const LayerArgs& p) {
    while (b < b_end && !active(p)) {
      if (++s == nsteps) { s = 0; ++b; }
    }
  }
  __device__ __forceinline__ void advance(const LayerArgs& p) {
    if (++s == nsteps) { s = 0; ++b; }
    settle(p);
  }
};

__device__ __forceinline__ int count_active(const LayerArgs& p, int b0, int b1, int nsteps) {
  if (p.rowbits == nullptr) return (b1 - b0) * nsteps;
  int n = 0;
  for (int b = b0; b < b1; ++b)
    for (int s = 0; s < nsteps; ++s) n += ((c_u32*)p.rowbits)[(int64_t)b * p.nwords + s] != 0u;
  return n;
}

// Main loop over the active steps of samples [b0, b1): kStages-deep LDS ring
// filled by DMA kStages-1 steps ahead, one barrier per step.  SCALE: rescale
// the accumulator at sample boundaries so that it ends as
// sum_i (c_i / c_last) g_i; c_last is returned.
template <bool SCALE>
__device__ __forceinline__ float run(const LayerArgs& p, int b0, int b1, int a0, int o0, Acc& acc,
                                     unsigned char* lds) {
  static_assert(kKT == kBitsTokens, "one row-bit word per step");
  const int nsteps = (p.T + kKT - 1) / kKT;
  const int n = count_active(p, b0, b1, nsteps);
  acc.zero();
  if (n == 0) return 1.0f;
  const uint32_t base = lds_addr(lds);
  Cursor ic{b0, 0, b1, nsteps};
  ic.settle(p);
#pragma unroll
  for (int k = 0; k < kStages - 1; ++k) {
    if (k < n) {
      issue_step(p, ic.b, ic.s, a0, o0, base + k * kStageBytes);
      ic.advance(p);
    }
  }
  Cursor cc{b0, 0, b1, nsteps};
  cc.settle(p);
  int cb = cc.b;
  float c_last = SCALE ? ((c_f32*)p.c)[cb] : 1.0f;
  for (int i = 0; i < n; ++i) {
    wait_dma(min(kStages - 2, n - 1 - i));
    __syncthreads();
    if (i + kStages - 1 < n) {
      issue_step(p, ic.b, ic.s, a0, o0, base + ((i + kStages - 1) % kStages) * kStageBytes);
      ic.advance(p);
    }
    if constexpr (SCALE) {
      if (cc.b != cb) {
        // acc holds sum_{j<i} (c_j / c_prev) g_j; re-express it in units of
        // this sample's factor before its tiles are added.
        const float cn = ((c_f32*)p.c)[cc.b];
        acc.scale(c_last / cn);
        c_last = cn;
        cb = cc.b;
      }
    }
    acc.compute(lds + (i % kStages) * kStageBytes);
    cc.advance(p);
  }
  return c_last;
}

// Tile index for this workgroup: workgroups are dealt to the 8 XCDs round
// robin, so give XCD x the contiguous range [x*per, (x+1)*per) of a grouped
// raster order (kGroupRows tile-rows at a time).
__device__ __forceinline__ bool tile_of(int id, int ntm, int ntn, int* tm, int* tn) {
  const int ntiles = ntm * ntn;
  const int per = (ntiles + 7) / 8;
  const int L = (id & 7) * per + (id >> 3);
  if (L >= ntiles) return false;
  const int gsz = kGroupRows * ntn;
  const int g = L / gsz, r = L % gsz;
  const int rows = min(kGroupRows, ntm - g * kGroupRows);
  *tm = g * kGroupRows + r % rows;
  *tn = r / rows;
  return true;
}

__global__ void __launch_bounds__(kNT, 1) accumulate_big_kernel(LayerArgs p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int ntm = (p.din + kTile - 1) / kTile, ntn = (p.dout + kTile - 1) / kTile;
  int tm, tn;
  if (!tile_of(blockIdx.x, ntm, ntn, &tm, &tn)) return;
  const int a0 = tm * kTile, o0 = tn * kTile;
  Acc acc;
  const float c_last = run<true>(p, 0, p.B, a0, o0, acc, smem);
  static_assert(256 * (64 + 4) * 4 <= kLdsBytes, "epilogue staging fits in the stage ring");

  // Epilogue, one 32-row block-row (i) at a time: the waves park their
  // accumulator blocks in LDS as [o][a] (o = dout index, 64 a values: 32 from
  // each wave row), then every thread takes 4 consecutive a of one o -- one
  // Philox block of noise and one 16-byte store.
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const float fB = (float)p.B;
  const bool noise = p.noise_std != 0.0f;
  float* park = (float*)smem;
  constexpr int kParkLd = 64 + 4;     // floats per o row (padding against bank conflicts)
  __syncthreads();                    // all waves are done reading the last stage
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ol = wn * 128 + j * 32 + acc_col(lane);
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
      const int o = o0 + ol;
      const int a = a0 + (a4 >> 5) * 128 + i * 32 + (a4 & 31);
      if (o < p.dout && a < p.din) {   // din % 8 == 0 on this path: a..a+3 all in range
        f32x4 v = *(const f32x4*)(park + ol * kParkLd + a4);
        v.x *= c_last; v.y *= c_last; v.z *= c_last; v.w *= c_last;
        const uint64_t e0 = (uint64_t)o * (uint64_t)p.din + (uint64_t)a;
        if (noise) {
          const f32x4 z = normals_of_block(philox_block(p.seed, p.offset + (e0 >> 2)));
          v.x += p.noise_std * z.x; v.y += p.noise_std * z.y;
          v.z += p.noise_std * z.z; v.w += p.noise_std * z.w;
        }
        v.x = v.x / fB; v.y = v.y / fB; v.z = v.z / fB; v.w = v.w / fB;
        *(f32x4*)(p.out + e0) = v;
      }
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(kNT, 1) direct_norm_big_kernel(LayerArgs p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ double red[kNT / 64];
  const int ntm = (p.din + kTile - 1) / kTile, ntn = (p.dout + kTile - 1) / kTile;
  const int ntiles = ntm * ntn;
  // blockIdx.x enumerates (sample, tile) with the tile fastest
  const int b = blockIdx.x / ntiles;
  const int local = blockIdx.x % ntiles;
  const int tm = local % ntm, tn = local / ntm;
  Acc acc;
  run<false>(p, b, b + 1, tm * kTile, tn * kTile, acc, smem);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += acc.v[i][j][r] * acc.v[i][j][r];
  const double tot = block_sum_f64((double)s, red);
  if (threadIdx.x == 0) p.partials[(int64_t)b * ntiles + local] = tot;
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

hipError_t launch_accumulate_big(const LayerArgs& p, hipStream_t s) {
  hipError_t e = allow_lds_big<big::accumulate_big_kernel>(big::kLdsBytes);
  if (e != hipSuccess) return e;
  const int nt = big_tiles(p.din, p.dout);
  const int grid = 8 * ((nt + 7) / 8);
  timing_begin("accumulate", s);
  hipLaunchKernelGGL(big::accumulate_big_kernel, dim3(grid), dim3(big::kNT), big::kLdsBytes, s, p);
  e = hipGetLastError();
  timing_end("accumulate", s);
  return e;
}

hipError_t launch_direct_norm_big(const LayerArgs& p, hipStream_t s) {
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
