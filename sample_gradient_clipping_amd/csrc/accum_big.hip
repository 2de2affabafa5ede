// Large-tile bf16 kernels for the token-contraction G~^T X~ (K-outer x K-outer):
//
//   accumulate_big_kernel : grad = (sum_i c_i G~_i^T X~_i + noise_std xi) / B
//   direct_norm_big_kernel: per (output tile, sample) sum of squares of g_i's tile
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

// Active-row bits of the 32 tokens of step s of sample b.  MASK: the call
// has a token mask (row bits in memory); otherwise only the tail past T is
// inactive, and no memory is read -- which keeps scalar loads out of the
// main loop, so the compiler can wait for LDS reads precisely.
template <bool MASK>
__device__ __forceinline__ uint32_t step_bits(const LayerArgs& p, int b, int s) {
  if constexpr (MASK) return ((c_u32*)p.rowbits)[(int64_t)b * p.nwords + s];
  const int n = p.T - s * kKT;
  return n >= 32 ? 0xffffffffu : ((1u << n) - 1u);
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

// Queue step (b, s) into the LDS slot at `stage`: X[tokens, a0:a0+256] and
// G[tokens, o0:o0+256].  Inactive rows read through out-of-range offsets.
template <bool MASK>
__device__ __forceinline__ void issue_step(const LayerArgs& p, const DmaLane& dl, int b, int s,
                                           uint32_t stage) {
  const __amdgpu_buffer_rsrc_t rx = sample_rsrc(p.X, b, p.T, p.din);
  const __amdgpu_buffer_rsrc_t rg = sample_rsrc(p.G, b, p.T, p.dout);
  const uint32_t bits = step_bits<MASK>(p, b, s);
  const int t0 = s * kKT;
  const uint32_t xs = (uint32_t)((int64_t)t0 * p.X.stride_t * 2);
  const uint32_t gs = (uint32_t)((int64_t)t0 * p.G.stride_t * 2);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t wbase = stage + kRowsPerWave * wave * kRowBytes;
  const uint32_t mine = bits >> (kRowsPerWave * wave);   // bit 2j + l/32 = row of DMA j
#pragma unroll
  for (int j = 0; j < kDmaPerOp; ++j) {
    const bool act = (mine >> (2 * j + (lane >> 5))) & 1u;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(wbase + 2 * j * kRowBytes);
    dma16(rx, act ? (int)(dl.xoff[j] + xs) : kOOB, dst);
    dma16(rg, act ? (int)(dl.goff[j] + gs) : kOOB, dst + kOpBytes);
  }
}

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
  __device__ __forceinline__ void mma(const Frags& f) {
#pragma unroll
    for (int i = 0; i < kBA; ++i)
#pragma unroll
      for (int j = 0; j < kBO; ++j) v[i][j] = mfma_32x32x16(f.a[i], f.b[j], v[i][j]);
  }
};

// (sample, step) cursor over the active steps of samples [b, b_end).
template <bool MASK>
struct Cursor {
  int b, s, b_end, nsteps;
  __device__ __forceinline__ bool active(const LayerArgs& p) const {
    if constexpr (!MASK) return true;
    else return ((c_u32*)p.rowbits)[(int64_t)b * p.nwords + s] != 0u;
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

template <bool MASK>
__device__ __forceinline__ int count_active(const LayerArgs& p, int b0, int b1, int nsteps) {
  if constexpr (!MASK) return (b1 - b0) * nsteps;
  int n = 0;
  Cursor<MASK> c{b0, 0, b1, nsteps};
  for (c.settle(p); c.b < b1; c.advance(p)) ++n;
  return n;
}

// Main loop over the active steps of samples [b0, b1).
//
// Five 32 KiB LDS slots.  A slot is refilled as soon as every wave's reads
// of it are complete (the barrier of the next step), so the DMA of step i+4
// is queued at the start of step i and has three steps to land: up to 128 KiB
// per CU in flight, which is what it takes to keep the MFMAs fed through L2
// misses.  Two waves share each SIMD, so one
// wave's LDS-read and barrier waits are covered by the other's MFMAs.
//
// SCALE: rescale the accumulator at sample boundaries so that it ends as
// sum_i (c_i / c_last) g_i; c_last is returned.
template <bool SCALE, bool MASK>
__device__ __forceinline__ float run(const LayerArgs& p, int b0, int b1, int a0, int o0, Acc& acc,
                                     unsigned char* lds) {
  static_assert(kKT == kBitsTokens, "one row-bit word per step");
  const int nsteps = (p.T + kKT - 1) / kKT;
  const int n = count_active<MASK>(p, b0, b1, nsteps);
  acc.zero();
  if (n == 0) return 1.0f;
  const uint32_t base = lds_addr(lds);
  DmaLane dl;
  dl.init(p, a0, o0);

  Cursor<MASK> ic{b0, 0, b1, nsteps};   // next step to issue
  ic.settle(p);
  Cursor<MASK> cc = ic;                  // step being consumed
#pragma unroll
  for (int k = 0; k < kStages; ++k) {
    if (k < n) {
      issue_step<MASK>(p, dl, ic.b, ic.s, base + k * kStageBytes);
      ic.advance(p);
    }
  }
  float c_last = SCALE ? ((c_f32*)p.c)[cc.b] : 1.0f;
  int cb = cc.b;
  int slot = 0;                        // i % kStages
  for (int i = 0; i < n; ++i) {
    // Issued so far: steps 0 .. min(4, n-1) before the loop, then step j+4
    // in iteration j >= 1, i.e. up to min(i+3, n-1) once i >= 1.  Wait until
    // step i has landed for this wave; the barrier extends that to every
    // wave and also certifies that all reads of step i-1 are complete.
    wait_dma(i == 0 ? min(kStages - 1, n - 1) : min(kStages - 2, n - 1 - i));
    __syncthreads();
    if (i >= 1 && i + kStages - 1 < n) {
      // refill slot (i-1) % kStages, drained before the barrier, with step i+4
      const int prev = (slot == 0) ? kStages - 1 : slot - 1;
      issue_step<MASK>(p, dl, ic.b, ic.s, base + prev * kStageBytes);
      ic.advance(p);
    }
    if (SCALE && cc.b != cb) {
      // acc holds sum_{j<=cb} (c_j / c_cb) g_j; re-express it in units of the
      // new sample's factor before its tiles are added.
      const float cn = ((c_f32*)p.c)[cc.b];
      acc.scale(c_last / cn);
      c_last = cn;
      cb = cc.b;
    }
    const unsigned char* st = lds + slot * kStageBytes;
    Frags f;
    read_frags(f, st, 0);
    acc.mma(f);
    read_frags(f, st, 1);
    acc.mma(f);
    cc.advance(p);
    slot = (slot + 1 == kStages) ? 0 : slot + 1;
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
  const float c_last = p.rowbits != nullptr ? run<true, true>(p, 0, p.B, a0, o0, acc, smem)
                                            : run<true, false>(p, 0, p.B, a0, o0, acc, smem);
  static_assert(256 * (64 + 4) * 4 <= kLdsBytes, "epilogue staging fits in the stage ring");

  // Epilogue, one 32-row block-row (i) at a time: the waves park their
  // accumulator blocks in LDS as [o][a] (o = dout index, 64 a values: 32 from
  // each wave row), then every thread takes 4 consecutive a of one o -- one
  // Philox block of noise and one 16-byte store.
  const int lane = threadIdx.x & 63;
  const int wm = wave_row(), wn = wave_col();
  const float fB = (float)p.B;
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
      const int o = o0 + ol;
      const int a = a0 + (a4 >> 5) * (kBA * 32) + i * 32 + (a4 & 31);
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
  const int ntm = (p.din + kTile - 1) / kTile, ntn = (p.dout + kTile - 1) / kTile;
  const int ntiles = ntm * ntn;
  // blockIdx.x enumerates (sample, tile) with the tile fastest
  const int b = blockIdx.x / ntiles;
  const int local = blockIdx.x % ntiles;
  const int tm = local % ntm, tn = local / ntm;
  Acc acc;
  if (p.rowbits != nullptr) run<false, true>(p, b, b + 1, tm * kTile, tn * kTile, acc, smem);
  else run<false, false>(p, b, b + 1, tm * kTile, tn * kTile, acc, smem);
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
