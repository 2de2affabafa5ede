// GEMM-shaped kernels of the per-layer DP step for fp32 inputs and for the
// shapes the large-tile bf16 kernels (accum_big.hip, gram_big.hip) do not
// take, plus the projection of the projected variant for every shape.
//
//  accumulate_kernel : grad = (sum_i c_i G~_i^T X~_i + noise_std * xi) / B
//                      One GEMM whose K runs over every active token of every
//                      sample; the clip factor is applied to the accumulator
//                      at each sample boundary, so no per-sample gradient is
//                      stored (FlashDP abstract: gradients computed once,
//                      fused, per layer).
//  direct_norm_kernel: per (output tile, sample) sum of squares of the tile of
//                      g_i = G~_i^T X~_i, computed and dropped in registers.
//  gram_norm_kernel  : per (sample, upper-triangular token-tile pair) partial
//                      of <X~X~^T, G~G~^T> (the Gram form of ||g_i||^2).
//  project_kernel    : Y = X~ P for the projected variant (DP-GRAPE explainer,
//                      Methodology: project before clipping and noise),
//                      optionally split along din into fp32 partials that
//                      project_reduce_kernel sums in chunk order; P is read,
//                      or (GEN) drawn from its seed where it is loaded.
//  accumulate_pieces_kernel: the accumulation for outputs of few tiles (the
//                      projected variant's r-space sum), each tile's samples
//                      cut into pieces; accumulate_pieces_fixup_kernel adds
//                      the pieces' parts in order, with the noise.
//
// All of them: 256 threads = 4 waves in a 2 x 2 grid, each wave owning 2 x 2
// blocks of 32 x 32 accumulators (a 128 x 128 workgroup tile), LDS double
// buffered along K.  Partial results leave as fp64 per workgroup and are
// summed in index order by finalize_kernel, so every reduction is fixed-order.
#include <algorithm>

#include <atomic>

#include "kernels.hpp"
#include "tiles.hpp"

namespace dpf {

constexpr int kNT = 256;          // threads per workgroup
constexpr int kWM = 2, kWN = 2;   // waves along the two tile dims
constexpr int kBM = 2, kBN = 2;   // 32x32 blocks per wave along each dim
constexpr int kTileM = kWM * kBM * 32;
constexpr int kTileN = kWN * kBN * 32;

template <class E> struct Cfg;
template <> struct Cfg<BF16> { static constexpr int KT = 64; static constexpr int PAD = 16; };
template <> struct Cfg<F32>  { static constexpr int KT = 32; static constexpr int PAD = 4; };

// ===========================================================================
// K-outer x K-outer main loop over a list of (sample, token-tile) steps.
// MFMA operand "A" = X (rows along din), "B" = G (rows along dout), so the
// accumulator block D[a][o] gives each lane 4 consecutive din columns of one
// output row: one Philox block per lane-group and 16-byte stores.
// ===========================================================================
template <class E, bool VEC>
struct KOuterGemm {
  using S = typename E::storage;
  static constexpr int KT = Cfg<E>::KT;
  static constexpr int LDA = kTileM + Cfg<E>::PAD;
  static constexpr int LDB = kTileN + Cfg<E>::PAD;
  static constexpr int A_ELEMS = KT * LDA, B_ELEMS = KT * LDB;
  static constexpr int LDS_BYTES = 2 * (A_ELEMS + B_ELEMS) * (int)sizeof(S);

  f32x16 acc[kBM][kBN];
  KOuterLoader<E, kTileM, KT, kNT, VEC> la;
  KOuterLoader<E, kTileN, KT, kNT, VEC> lb;

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kBM; ++i)
#pragma unroll
      for (int j = 0; j < kBN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  __device__ __forceinline__ void scale(float s) {
#pragma unroll
    for (int i = 0; i < kBM; ++i)
#pragma unroll
      for (int j = 0; j < kBN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] *= s;
  }

  __device__ __forceinline__ void fetch(const LayerArgs& p, int b, int kt, int a0, int o0) {
    const S* xb = (const S*)p.X.data + (int64_t)b * p.X.stride_b;
    const S* gb = (const S*)p.G.data + (int64_t)b * p.G.stride_b;
    const uint8_t* mb = p.mask ? p.mask + (int64_t)b * p.T : nullptr;
    la.load(xb, p.X.stride_t, p.T, mb, kt * KT, a0, p.din);
    lb.load(gb, p.G.stride_t, p.T, mb, kt * KT, o0, p.dout);
  }

  __device__ __forceinline__ void stash(S* lds) const {
    la.template store<LDA>(lds);
    lb.template store<LDB>(lds + A_ELEMS);
  }

  __device__ __forceinline__ void compute(const S* lds) {
    const int wave = threadIdx.x >> 6;
    const int wm = wave / kWN, wn = wave % kWN;
    const S* As = lds;
    const S* Bs = lds + A_ELEMS;
#pragma unroll
    for (int ks = 0; ks < KT / E::kMfmaK; ++ks) {
      typename Frag<E>::type fa[kBM], fb[kBN];
#pragma unroll
      for (int i = 0; i < kBM; ++i) fa[i] = frag_kouter<E, LDA>(As, (wm * kBM + i) * 32, ks);
#pragma unroll
      for (int j = 0; j < kBN; ++j) fb[j] = frag_kouter<E, LDB>(Bs, (wn * kBN + j) * 32, ks);
#pragma unroll
      for (int i = 0; i < kBM; ++i)
#pragma unroll
        for (int j = 0; j < kBN; ++j) acc[i][j] = mfma<E>(fa[i], fb[j], acc[i][j]);
    }
  }
};

// Step cursor over (sample, token tile) pairs in [b_begin, b_end), skipping
// token tiles with no active row when per-tile flags are given.
// Any active token among tokens [t0, t0 + n) of sample b (n a multiple of 32).
__device__ __forceinline__ bool any_active(const uint32_t* bits, int nwords, int b, int t0, int n) {
  if (bits == nullptr) return true;
  const int w0 = t0 / kBitsTokens;
  uint32_t acc = 0u;
  for (int w = w0; w < w0 + n / kBitsTokens && w < nwords; ++w) acc |= bits[(int64_t)b * nwords + w];
  return acc != 0u;
}

struct StepCursor {
  int b, kt, b_end, nkt;
  const uint32_t* bits;   // [B][nwords] row-activity bits or null
  int nwords, kt_tokens;
  __device__ __forceinline__ bool valid() const { return b < b_end; }
  __device__ __forceinline__ bool active() const {
    return any_active(bits, nwords, b, kt * kt_tokens, kt_tokens);
  }
  __device__ __forceinline__ void skip_inactive() {
    while (b < b_end && !active()) {
      if (++kt == nkt) { kt = 0; ++b; }
    }
  }
  __device__ __forceinline__ void advance() {
    if (++kt == nkt) { kt = 0; ++b; }
    skip_inactive();
  }
};

template <class E, bool VEC, bool NORM>
__device__ __forceinline__ void kouter_run(const LayerArgs& p, int b_begin, int b_end, int a0,
                                           int o0, KOuterGemm<E, VEC>& g,
                                           typename E::storage* lds, float* c_last) {
  using S = typename E::storage;
  using KG = KOuterGemm<E, VEC>;
  const int nkt = (p.T + KG::KT - 1) / KG::KT;
  static_assert(KG::KT % kBitsTokens == 0, "row-bit granularity");
  StepCursor cur{b_begin, 0, b_end, nkt, p.rowbits, p.nwords, KG::KT};
  cur.skip_inactive();
  g.zero();
  *c_last = 1.0f;
  if (!cur.valid()) return;
  int cur_b = cur.b;
  if constexpr (!NORM) *c_last = p.c[cur_b];
  g.fetch(p, cur.b, cur.kt, a0, o0);
  g.stash(lds);
  __syncthreads();
  int buf = 0;
  while (true) {
    StepCursor nxt = cur;
    nxt.advance();
    if (nxt.valid()) g.fetch(p, nxt.b, nxt.kt, a0, o0);
    g.compute(lds + buf * (KG::A_ELEMS + KG::B_ELEMS));
    if (!nxt.valid()) break;
    if constexpr (!NORM) {
      if (nxt.b != cur_b) {
        // acc holds sum_{j<=cur} (c_j / c_cur) g_j; re-express it in units
        // of the next sample's factor before that sample's tiles are added.
        const float c_next = p.c[nxt.b];
        g.scale(*c_last / c_next);
        *c_last = c_next;
        cur_b = nxt.b;
      }
    }
    g.stash(lds + (buf ^ 1) * (KG::A_ELEMS + KG::B_ELEMS));
    __syncthreads();
    buf ^= 1;
    cur = nxt;
  }
}

// ---------------------------------------------------------------------------
template <class E, bool VEC>
__global__ void __launch_bounds__(kNT) accumulate_kernel(LayerArgs p) {
  using KG = KOuterGemm<E, VEC>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  auto* lds = (typename E::storage*)smem;
  const int ntm = (p.din + kTileM - 1) / kTileM;
  const int a0 = (blockIdx.x % ntm) * kTileM;
  const int o0 = (blockIdx.x / ntm) * kTileN;
  KG g;
  float c_last;
  kouter_run<E, VEC, false>(p, 0, p.B, a0, o0, g, lds, &c_last);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
  const float inv_scale = c_last;
  const float denom = p.denom;
  const bool vec_store = (p.din & 3) == 0;
#pragma unroll
  for (int i = 0; i < kBM; ++i) {
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      const int o = o0 + (wn * kBN + j) * 32 + acc_col(lane);
      if (o >= p.dout) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int a = a0 + (wm * kBM + i) * 32 + acc_row(4 * q, lane);   // 4 consecutive a
        if (a >= p.din) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = g.acc[i][j][4 * q + e] * inv_scale;
        const uint64_t e0 = (uint64_t)o * (uint64_t)p.din + (uint64_t)a;
        if (p.noise_std != 0.0f) {
          if (vec_store) {
            const f32x4 z = normals_of_block(philox_block(p.seed, p.offset + (e0 >> 2)));
            v[0] += p.noise_std * z.x; v[1] += p.noise_std * z.y;
            v[2] += p.noise_std * z.z; v[3] += p.noise_std * z.w;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (a + e < p.din) v[e] += p.noise_std * normal_at(p.seed, p.offset, e0 + e);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = v[e] / denom;
        float* dst = p.out + e0;
        if (vec_store) {
          f32x4 w; w.x = v[0]; w.y = v[1]; w.z = v[2]; w.w = v[3];
          if (p.beta) {
            const f32x4 old = *(const f32x4*)dst;
            w.x += old.x; w.y += old.y; w.z += old.z; w.w += old.w;
          }
          *(f32x4*)dst = w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (a + e < p.din) dst[e] = p.beta ? dst[e] + v[e] : v[e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Few-tile accumulation: outputs of a few 128 x 128 tiles over many tokens
// (the projected variant's r-space sum G~^T Y, [dout, r]: 16 to 64 tiles at
// r = 256).  One workgroup per tile and none else would leave most compute
// units idle, and the large tiles are fewer still; so the samples of each
// tile are cut into P consecutive pieces [b0, b1), one workgroup each.  Piece
// q stores its part of the sum, acc * c_last = sum over its samples of
// c_i g_i (the clip factors already applied), as a 128 x 128 fp32 tile
// [o - o0][a - a0] at part + (q * ntiles + tile) * 16384; a piece without an
// active token stores zeros.  accumulate_pieces_fixup_kernel then adds the P
// parts of every output in piece order, the noise and 1/denom.
constexpr int kPieceFloats = kTileM * kTileN;

template <class E, bool VEC>
__global__ void __launch_bounds__(kNT) accumulate_pieces_kernel(LayerArgs p, int P, float* part) {
  using KG = KOuterGemm<E, VEC>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  auto* lds = (typename E::storage*)smem;
  const int ntm = (p.din + kTileM - 1) / kTileM;
  const int ntiles = ntm * ((p.dout + kTileN - 1) / kTileN);
  const int tile = (int)(blockIdx.x % (unsigned)ntiles), q = (int)(blockIdx.x / (unsigned)ntiles);
  const int a0 = (tile % ntm) * kTileM;
  const int o0 = (tile / ntm) * kTileN;
  const int b0 = (int)((int64_t)q * p.B / P), b1 = (int)((int64_t)(q + 1) * p.B / P);
  KG g;
  float c_last;
  kouter_run<E, VEC, false>(p, b0, b1, a0, o0, g, lds, &c_last);
  float* dst = part + ((int64_t)q * ntiles + tile) * kPieceFloats;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
#pragma unroll
  for (int i = 0; i < kBM; ++i) {
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      const int ol = (wn * kBN + j) * 32 + acc_col(lane);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int al = (wm * kBM + i) * 32 + acc_row(4 * qq, lane);   // 4 consecutive a
        f32x4 v;
        v.x = g.acc[i][j][4 * qq + 0] * c_last;
        v.y = g.acc[i][j][4 * qq + 1] * c_last;
        v.z = g.acc[i][j][4 * qq + 2] * c_last;
        v.w = g.acc[i][j][4 * qq + 3] * c_last;
        *(f32x4*)(dst + ol * kTileM + al) = v;
      }
    }
  }
}

// One thread per 4 consecutive outputs (o, a .. a+3) of the [dout, din]
// result (din a multiple of 4): the P parts summed in piece order, then the
// noise (one Philox block), 1/denom and the prior value when beta.  Each
// thread keeps the loads of up to kPieceBatch parts in flight (indices past
// P clamped to the last part, their values dropped).
constexpr int kPieceFixThreads = 256;
constexpr int kPieceBatch = 8;
__global__ void __launch_bounds__(kPieceFixThreads) accumulate_pieces_fixup_kernel(LayerArgs p,
                                                                                   int P,
                                                                                   const float* part) {
  const int nq = p.din >> 2;
  const int64_t idx = (int64_t)blockIdx.x * kPieceFixThreads + threadIdx.x;
  if (idx >= (int64_t)p.dout * nq) return;
  const int o = (int)(idx / nq), a = (int)(idx % nq) * 4;
  const int ntm = (p.din + kTileM - 1) / kTileM;
  const int ntiles = ntm * ((p.dout + kTileN - 1) / kTileN);
  const int tile = (o / kTileN) * ntm + a / kTileM;
  const float* src = part + (int64_t)tile * kPieceFloats + (o % kTileN) * kTileM + (a % kTileM);
  const int64_t stride = (int64_t)ntiles * kPieceFloats;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int c0 = 0; c0 < P; c0 += kPieceBatch) {
    f32x4 w[kPieceBatch];
#pragma unroll
    for (int j = 0; j < kPieceBatch; ++j)
      w[j] = *(const f32x4*)(src + (int64_t)min(c0 + j, P - 1) * stride);
#pragma unroll
    for (int j = 0; j < kPieceBatch; ++j) {
      if (c0 + j < P) {
        v.x += w[j].x; v.y += w[j].y; v.z += w[j].z; v.w += w[j].w;
      }
    }
  }
  const float rB = 1.0f / p.denom;   // exact for a power of two, else within one ulp
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

// ---------------------------------------------------------------------------
template <class E, bool VEC>
__global__ void __launch_bounds__(kNT) direct_norm_kernel(LayerArgs p) {
  using KG = KOuterGemm<E, VEC>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  auto* lds = (typename E::storage*)smem;
  __shared__ double red[kNT / 64];
  const int ntm = (p.din + kTileM - 1) / kTileM;
  const int ntiles = ntm * ((p.dout + kTileN - 1) / kTileN);
  const int tile = blockIdx.x;
  const int b = blockIdx.y;
  const int a0 = (tile % ntm) * kTileM;
  const int o0 = (tile / ntm) * kTileN;
  KG g;
  float unused;
  kouter_run<E, VEC, true>(p, b, b + 1, a0, o0, g, lds, &unused);
  // Out-of-range rows/columns loaded as zero, so their accumulators are 0.
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kBM; ++i)
#pragma unroll
    for (int j = 0; j < kBN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += g.acc[i][j][r] * g.acc[i][j][r];
  const double tot = block_sum_f64((double)s, red);
  if (threadIdx.x == 0) p.partials[(int64_t)b * ntiles + tile] = tot;
}

// ===========================================================================
// Gram form of the per-sample norm:
//   ||G~^T X~||^2 = sum_{s,t} (X~X~^T)[s,t] (G~G~^T)[s,t]
// One workgroup per (sample, token-tile pair (S <= T)): the two 128 x 128
// Gram tiles are accumulated one after the other (K = din, then K = dout)
// and multiplied elementwise in registers; off-diagonal pairs count twice.
// ===========================================================================
template <class E, bool VEC>
struct GramTile {
  using S = typename E::storage;
  static constexpr int KT = Cfg<E>::KT;
  static constexpr int LD = KT + (sizeof(S) == 2 ? 8 : 4);
  static constexpr int ELEMS = kTileM * LD;         // one operand tile
  static constexpr int LDS_BYTES = 2 * 2 * ELEMS * (int)sizeof(S);
  KInnerLoader<E, kTileM, KT, kNT, VEC> ls, lt;

  __device__ __forceinline__ void run(const Act& A, int K, const LayerArgs& p, int b, int s0,
                                      int t0, S* lds, f32x16 (&acc)[kBM][kBN]) {
#pragma unroll
    for (int i = 0; i < kBM; ++i)
#pragma unroll
      for (int j = 0; j < kBN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    const S* base = (const S*)A.data + (int64_t)b * A.stride_b;
    const uint8_t* mb = p.mask ? p.mask + (int64_t)b * p.T : nullptr;
    const int nk = (K + KT - 1) / KT;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / kWN, wn = wave % kWN;
    ls.load(base, A.stride_t, p.T, mb, s0, 0, K);
    lt.load(base, A.stride_t, p.T, mb, t0, 0, K);
    ls.template store<LD>(lds);
    lt.template store<LD>(lds + ELEMS);
    __syncthreads();
    int buf = 0;
    for (int kk = 0; kk < nk; ++kk) {
      const bool more = kk + 1 < nk;
      if (more) {
        ls.load(base, A.stride_t, p.T, mb, s0, (kk + 1) * KT, K);
        lt.load(base, A.stride_t, p.T, mb, t0, (kk + 1) * KT, K);
      }
      const S* Ss = lds + buf * 2 * ELEMS;
      const S* Ts = Ss + ELEMS;
#pragma unroll
      for (int ks = 0; ks < KT / E::kMfmaK; ++ks) {
        typename Frag<E>::type fa[kBM], fb[kBN];
#pragma unroll
        for (int i = 0; i < kBM; ++i) fa[i] = frag_kinner<E, LD>(Ss, (wm * kBM + i) * 32, ks);
#pragma unroll
        for (int j = 0; j < kBN; ++j) fb[j] = frag_kinner<E, LD>(Ts, (wn * kBN + j) * 32, ks);
#pragma unroll
        for (int i = 0; i < kBM; ++i)
#pragma unroll
          for (int j = 0; j < kBN; ++j) acc[i][j] = mfma<E>(fa[i], fb[j], acc[i][j]);
      }
      if (!more) break;
      S* nbuf = lds + (buf ^ 1) * 2 * ELEMS;
      ls.template store<LD>(nbuf);
      lt.template store<LD>(nbuf + ELEMS);
      __syncthreads();
      buf ^= 1;
    }
    __syncthreads();   // LDS is reused by the next phase
  }
};

// Pair index p -> (S, T) token-tile indices with S <= T, row-major over S.
__device__ __forceinline__ void pair_of_index(int pidx, int nt, int* s, int* t) {
  int row = 0, start = 0;
  while (pidx >= start + (nt - row)) { start += nt - row; ++row; }
  *s = row;
  *t = row + (pidx - start);
}

template <class E, bool VEC>
__global__ void __launch_bounds__(kNT) gram_norm_kernel(LayerArgs p) {
  using GT = GramTile<E, VEC>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  auto* lds = (typename E::storage*)smem;
  __shared__ double red[kNT / 64];
  const int nt = (p.T + kTileM - 1) / kTileM;
  const int npairs = nt * (nt + 1) / 2;
  const int pidx = blockIdx.x;
  const int b = blockIdx.y;
  int st, tt;
  pair_of_index(pidx, nt, &st, &tt);
  // Skip pairs whose token tiles hold no active row.
  const bool live = any_active(p.rowbits, p.nwords, b, st * kTileM, kTileM) &&
                    any_active(p.rowbits, p.nwords, b, tt * kTileM, kTileM);
  double tot = 0.0;
  if (live) {
    GT gt;
    f32x16 ax[kBM][kBN], ag[kBM][kBN];
    gt.run(p.X, p.din, p, b, st * kTileM, tt * kTileM, lds, ax);
    gt.run(p.G, p.dout, p, b, st * kTileM, tt * kTileM, lds, ag);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kBM; ++i)
#pragma unroll
      for (int j = 0; j < kBN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += ax[i][j][r] * ag[i][j][r];
    tot = block_sum_f64((double)s, red);
    if (st != tt) tot *= 2.0;
  }
  if (threadIdx.x == 0) p.partials[(int64_t)b * npairs + pidx] = tot;
}

// ===========================================================================
// Projection Y = X~ P.  MFMA "A" = P^T (rows along r, K-outer in memory),
// "B" = X (rows along tokens, K-inner).  Each lane ends with 4 consecutive r
// of one token.  Y is [B, T, r] contiguous in X's dtype.  With p.splits > 1
// the din range is cut into that many chunks, one workgroup per (output
// tile, chunk), each storing its fp32 partial product; project_reduce_kernel
// sums the chunks in order and rounds.
// ===========================================================================
template <class E, bool VEC, bool GEN>
__global__ void __launch_bounds__(kNT) project_kernel(ProjArgs p) {
  using S = typename E::storage;
  constexpr int KT = Cfg<E>::KT;
  constexpr int LDP = kTileM + Cfg<E>::PAD;        // P tile [KT][TileM] (r)
  constexpr int LDX = KT + (sizeof(S) == 2 ? 8 : 4);  // X tile [TileN][KT]
  constexpr int P_ELEMS = KT * LDP, X_ELEMS = kTileN * LDX;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  S* lds = (S*)smem;
  const int64_t ntok = (int64_t)p.B * p.T;
  const int ntr = (p.r + kTileM - 1) / kTileM;
  const int64_t ntiles = (int64_t)ntr * ((ntok + kTileN - 1) / kTileN);
  const int64_t tile = blockIdx.x % ntiles;
  const int split = (int)(blockIdx.x / ntiles);
  const int j0 = (int)(tile % ntr) * kTileM;
  const int64_t q0 = (tile / ntr) * kTileN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave / kWN, wn = wave % kWN;

  KOuterLoader<E, kTileM, KT, kNT, VEC> lp;
  KInnerLoader<E, kTileN, KT, kNT, VEC> lx;
  f32x16 acc[kBM][kBN];
#pragma unroll
  for (int i = 0; i < kBM; ++i)
#pragma unroll
    for (int j = 0; j < kBN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const S* P = (const S*)p.P;
  const S* Xd = (const S*)p.X.data;
  const int nk_all = (p.din + KT - 1) / KT;
  const int kb = (int)((int64_t)split * nk_all / p.splits);
  const int nk = (int)((int64_t)(split + 1) * nk_all / p.splits);
  // P rows are "tokens" of the K-outer loader: row k of P, T = din, no mask.
  using LP = decltype(lp);
  auto load_p = [&](int k0) {
    if constexpr (GEN) {
#pragma unroll
      for (int i = 0; i < LP::N; ++i) {
        const int q = threadIdx.x + kNT * i;
        lp.r[i] = gen_p_chunk<E>(p.p_seed, p.p_offset, p.p_scale, p.din, p.r, k0 + q / LP::CPR,
                                 j0 + (q % LP::CPR) * E::kVec);
      }
    } else {
      lp.load(P, p.r, p.din, nullptr, k0, j0, p.r);
    }
  };
  load_p(kb * KT);
  lx.load_flat(Xd, p.X.stride_b, p.X.stride_t, p.B, p.T, p.mask, q0, kb * KT, p.din);
  lp.template store<LDP>(lds);
  lx.template store<LDX>(lds + P_ELEMS);
  __syncthreads();
  int buf = 0;
  for (int kk = kb; kk < nk; ++kk) {
    const bool more = kk + 1 < nk;
    if (more) {
      load_p((kk + 1) * KT);
      lx.load_flat(Xd, p.X.stride_b, p.X.stride_t, p.B, p.T, p.mask, q0, (kk + 1) * KT, p.din);
    }
    const S* Ps = lds + buf * (P_ELEMS + X_ELEMS);
    const S* Xs = Ps + P_ELEMS;
#pragma unroll
    for (int ks = 0; ks < KT / E::kMfmaK; ++ks) {
      typename Frag<E>::type fa[kBM], fb[kBN];
#pragma unroll
      for (int i = 0; i < kBM; ++i) fa[i] = frag_kouter<E, LDP>(Ps, (wm * kBM + i) * 32, ks);
#pragma unroll
      for (int j = 0; j < kBN; ++j) fb[j] = frag_kinner<E, LDX>(Xs, (wn * kBN + j) * 32, ks);
#pragma unroll
      for (int i = 0; i < kBM; ++i)
#pragma unroll
        for (int j = 0; j < kBN; ++j) acc[i][j] = mfma<E>(fa[i], fb[j], acc[i][j]);
    }
    if (!more) break;
    S* nb = lds + (buf ^ 1) * (P_ELEMS + X_ELEMS);
    lp.template store<LDP>(nb);
    lx.template store<LDX>(nb + P_ELEMS);
    __syncthreads();
    buf ^= 1;
  }

#pragma unroll
  for (int i = 0; i < kBM; ++i) {
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      const int64_t q = q0 + (wn * kBN + j) * 32 + acc_col(lane);
      if (q >= ntok) continue;
      S* yrow = (S*)p.Y + q * p.r;
      float* prow = p.part + ((int64_t)split * ntok + q) * p.r;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int jj = j0 + (wm * kBM + i) * 32 + acc_row(4 * g, lane);
        if (jj >= p.r) continue;
        if (p.splits > 1) {
          if ((p.r & 3) == 0) {
            f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                       acc[i][j][4 * g + 3]};
            *(f32x4*)(prow + jj) = v;
          } else {
            for (int e = 0; e < 4; ++e) if (jj + e < p.r) prow[jj + e] = acc[i][j][4 * g + e];
          }
        } else if constexpr (sizeof(S) == 2) {
          u16x4 w;
          w.s0 = f32_to_bf16_rne(acc[i][j][4 * g + 0]);
          w.s1 = f32_to_bf16_rne(acc[i][j][4 * g + 1]);
          w.s2 = f32_to_bf16_rne(acc[i][j][4 * g + 2]);
          w.s3 = f32_to_bf16_rne(acc[i][j][4 * g + 3]);
          if ((p.r & 3) == 0) {
            *(u16x4*)(yrow + jj) = w;
          } else {
            const uint16_t ww[4] = {w.s0, w.s1, w.s2, w.s3};
            for (int e = 0; e < 4; ++e) if (jj + e < p.r) yrow[jj + e] = ww[e];
          }
        } else {
          for (int e = 0; e < 4; ++e) if (jj + e < p.r) yrow[jj + e] = acc[i][j][4 * g + e];
        }
      }
    }
  }
}

// Y = sum of the p.splits partial products, chunk by chunk in order, rounded
// to Y's dtype.  Four consecutive elements per thread.
template <class E>
__global__ void __launch_bounds__(256) project_reduce_kernel(ProjArgs p) {
  using S = typename E::storage;
  const int64_t n = (int64_t)p.B * p.T * p.r;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if ((n & 3) == 0) {
    for (int c = 0; c < p.splits; ++c) {
      const f32x4 w = *(const f32x4*)(p.part + c * n + i);
      v[0] += w.x; v[1] += w.y; v[2] += w.z; v[3] += w.w;
    }
  } else {
    for (int c = 0; c < p.splits; ++c)
      for (int e = 0; e < 4; ++e)
        if (i + e < n) v[e] += p.part[c * n + i + e];
  }
  S* y = (S*)p.Y + i;
  for (int e = 0; e < 4; ++e) {
    if (i + e >= n) break;
    if constexpr (sizeof(S) == 2) y[e] = f32_to_bf16_rne(v[e]);
    else y[e] = v[e];
  }
}

// ===========================================================================
// Host-side launchers
// ===========================================================================
namespace {
// Kernels here use more than the default 64 KiB of dynamic LDS; raise the
// per-kernel limit once per instantiation.
template <auto Kernel>
hipError_t allow_lds(int bytes) {
  static hipError_t once = hipFuncSetAttribute((const void*)Kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  return once;
}

template <class E, bool VEC>
hipError_t launch_accumulate_t(const LayerArgs& p, hipStream_t s) {
  using KG = KOuterGemm<E, VEC>;
  const int grid = ((p.din + kTileM - 1) / kTileM) * ((p.dout + kTileN - 1) / kTileN);
  hipError_t e = allow_lds<accumulate_kernel<E, VEC>>(KG::LDS_BYTES);
  if (e != hipSuccess) return e;
  timing_begin("accumulate", s);
  hipLaunchKernelGGL((accumulate_kernel<E, VEC>), dim3(grid), dim3(kNT), KG::LDS_BYTES, s, p);
  e = hipGetLastError();
  timing_end("accumulate", s);
  return e;
}
// Pieces per tile of the few-tile accumulation: enough for every compute
// unit to take one, at most one per sample and at most kMaxPieces.
constexpr int kMaxPieces = 32;
int small_tile_count(const LayerArgs& p) {
  return ((p.din + kTileM - 1) / kTileM) * ((p.dout + kTileN - 1) / kTileN);
}
int pieces_per_tile(const LayerArgs& p) {
  const int P = std::max(1, device_cus() / small_tile_count(p));
  return std::min(P, std::min(p.B, kMaxPieces));
}

template <class E, bool VEC>
hipError_t launch_pieces_t(const LayerArgs& p, hipStream_t s) {
  using KG = KOuterGemm<E, VEC>;
  const int P = pieces_per_tile(p);
  if (P == 1) return launch_accumulate_t<E, VEC>(p, s);
  if (p.skws == nullptr || (p.din & 3) != 0) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)small_tile_count(p) * P;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipError_t e = allow_lds<accumulate_pieces_kernel<E, VEC>>(KG::LDS_BYTES);
  if (e != hipSuccess) return e;
  timing_begin("accumulate", s);
  hipLaunchKernelGGL((accumulate_pieces_kernel<E, VEC>), dim3((unsigned)grid), dim3(kNT),
                     KG::LDS_BYTES, s, p, P, p.skws);
  e = hipGetLastError();
  timing_end("accumulate", s);
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)p.dout * (p.din >> 2);
  timing_begin("accumulate_fixup", s);
  hipLaunchKernelGGL(accumulate_pieces_fixup_kernel,
                     dim3((unsigned)((n + kPieceFixThreads - 1) / kPieceFixThreads)),
                     dim3(kPieceFixThreads), 0, s, p, P, (const float*)p.skws);
  e = hipGetLastError();
  timing_end("accumulate_fixup", s);
  return e;
}
template <class E, bool VEC>
hipError_t launch_direct_t(const LayerArgs& p, hipStream_t s) {
  using KG = KOuterGemm<E, VEC>;
  const int grid = ((p.din + kTileM - 1) / kTileM) * ((p.dout + kTileN - 1) / kTileN);
  hipError_t e = allow_lds<direct_norm_kernel<E, VEC>>(KG::LDS_BYTES);
  if (e != hipSuccess) return e;
  timing_begin("direct_norm", s);
  hipLaunchKernelGGL((direct_norm_kernel<E, VEC>), dim3(grid, p.B), dim3(kNT), KG::LDS_BYTES, s, p);
  e = hipGetLastError();
  timing_end("direct_norm", s);
  return e;
}
template <class E, bool VEC>
hipError_t launch_gram_t(const LayerArgs& p, hipStream_t s) {
  using GT = GramTile<E, VEC>;
  const int nt = (p.T + kTileM - 1) / kTileM;
  hipError_t e = allow_lds<gram_norm_kernel<E, VEC>>(GT::LDS_BYTES);
  if (e != hipSuccess) return e;
  timing_begin("gram_norm", s);
  hipLaunchKernelGGL((gram_norm_kernel<E, VEC>), dim3(nt * (nt + 1) / 2, p.B), dim3(kNT),
                     GT::LDS_BYTES, s, p);
  e = hipGetLastError();
  timing_end("gram_norm", s);
  return e;
}
template <class E, bool VEC, bool GEN>
hipError_t launch_project_t(const ProjArgs& p, hipStream_t s) {
  using S = typename E::storage;
  constexpr int KT = Cfg<E>::KT;
  constexpr int bytes = 2 * (KT * (kTileM + Cfg<E>::PAD) + kTileN * (KT + (sizeof(S) == 2 ? 8 : 4))) *
                        (int)sizeof(S);
  const int64_t ntok = (int64_t)p.B * p.T;
  const int64_t tiles = ((p.r + kTileM - 1) / kTileM) * ((ntok + kTileN - 1) / kTileN);
  if (p.splits < 1 || (p.splits > 1 && p.part == nullptr)) return hipErrorInvalidValue;
  hipError_t e = allow_lds<project_kernel<E, VEC, GEN>>(bytes);
  if (e != hipSuccess) return e;
  timing_begin("project", s);
  hipLaunchKernelGGL((project_kernel<E, VEC, GEN>), dim3((unsigned)(tiles * p.splits)), dim3(kNT),
                     bytes, s, p);
  e = hipGetLastError();
  timing_end("project", s);
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t n = ntok * p.r;
  timing_begin("project_reduce", s);
  hipLaunchKernelGGL((project_reduce_kernel<E>), dim3((unsigned)((n + 1023) / 1024)), dim3(256), 0,
                     s, p);
  e = hipGetLastError();
  timing_end("project_reduce", s);
  return e;
}
}  // namespace

// The large-tile kernels take bf16 inputs with 16-byte vector loads and
// address one sample's rows with 32-bit byte offsets, including the rows of
// the last (partial) tile past T, which must land past the end of the
// sample's buffer range rather than wrap around into it: the padded span must
// stay below 2 GiB.  Active-step entries pack the sample and the step into
// 16 bits each.
static bool use_big(const LayerArgs& p, bool vec) {
  const int64_t lim = (int64_t)1 << 30;   // elements: 2 GiB of bf16
  const int64_t Tp = ((int64_t)p.T + 255) / 256 * 256;
  return p.dtype == kBF16 && vec && Tp * p.X.stride_t + p.din < lim &&
         Tp * p.G.stride_t + p.dout < lim && p.B < 65536 && p.nwords < 65536;
}

bool big_path(const LayerArgs& p, bool vec) { return use_big(p, vec); }

// The few-tile kernels (128 x 128 tiles, samples cut into pieces) for a call
// that asks for them (small_tiles), with 16-byte rows (din a multiple of 4,
// 8 for bf16) and at most half as many of those tiles as compute units.
// Where the large tiles could run the call instead (bf16), only if the
// pieces keep at least half of the compute units busy and each piece stays
// short (at most 32 of the generic loop's steps): the large-tile loop is the
// faster one per step, and splits a long token range of few samples itself.
static bool use_pieces(const LayerArgs& p, bool vec) {
  if (p.small_tiles == 0 || !vec || (p.din & 3) != 0) return false;
  const int64_t cus = device_cus(), nt = small_tile_count(p);
  if (2 * nt > cus) return false;
  if (!use_big(p, vec)) return true;
  const int P = pieces_per_tile(p);
  const int kt = p.dtype == kBF16 ? Cfg<BF16>::KT : Cfg<F32>::KT;
  const int64_t steps = (int64_t)((p.B + P - 1) / P) * ((p.T + kt - 1) / kt);
  return 2 * nt * P >= cus && steps <= 32;
}
// ... and, with small_tiles == 2, the direct norm over the same tiles.
static bool small_norm(const LayerArgs& p, bool vec) {
  return p.small_tiles == 2 && use_pieces(p, vec);
}

size_t accumulate_workspace_bytes(const LayerArgs& p, bool vec) {
  if (use_pieces(p, vec)) {
    const int P = pieces_per_tile(p);
    return P == 1 ? 0 : (size_t)P * small_tile_count(p) * kPieceFloats * sizeof(float);
  }
  return use_big(p, vec) ? accumulate_big_workspace_bytes(p) : 0;
}

size_t norm_workspace_bytes(const LayerArgs& p, NormPath path, bool vec) {
  if (!use_big(p, vec) || path == NormPath::kOnePass) return 0;
  if (path == NormPath::kGram) return gram_big_workspace_bytes(p);
  return path == NormPath::kStaged ? staged_big_workspace_bytes(p) : 0;
}

int norm_partials_per_sample(const LayerArgs& p, NormPath path, bool vec) {
  if (path == NormPath::kOnePass) return onepass_tiles(p.din, p.dout);
  if (path == NormPath::kGram && use_big(p, vec)) return gram_big_items_per_sample(p.T);
  if (path == NormPath::kGram) {
    const int nt = (p.T + kTileM - 1) / kTileM;
    return nt * (nt + 1) / 2;
  }
  if (path == NormPath::kStaged && use_big(p, vec)) return staged_big_partials_per_sample(p);
  if (use_big(p, vec) && !small_norm(p, vec)) return direct_big_partials_per_sample(p);
  return ((p.din + kTileM - 1) / kTileM) * ((p.dout + kTileN - 1) / kTileN);
}

hipError_t launch_accumulate(const LayerArgs& p, bool vec, hipStream_t s) {
  if (use_pieces(p, vec))
    return p.dtype == kBF16 ? launch_pieces_t<BF16, true>(p, s) : launch_pieces_t<F32, true>(p, s);
  if (use_big(p, vec)) return launch_accumulate_big(p, s);
  if (p.dtype == kBF16) return vec ? launch_accumulate_t<BF16, true>(p, s) : launch_accumulate_t<BF16, false>(p, s);
  return vec ? launch_accumulate_t<F32, true>(p, s) : launch_accumulate_t<F32, false>(p, s);
}
hipError_t launch_staged_combine(const LayerArgs& p, hipStream_t s) {
  return launch_staged_combine_big(p, s);
}
hipError_t launch_norm(const LayerArgs& p, NormPath path, bool vec, hipStream_t s) {
  if (path == NormPath::kStaged) {
    if (!use_big(p, vec)) return hipErrorInvalidValue;
    return launch_staged_norm_big(p, s);
  }
  if (path == NormPath::kGram) {
    if (use_big(p, vec)) return launch_gram_norm_big(p, s);
    if (p.dtype == kBF16) return vec ? launch_gram_t<BF16, true>(p, s) : launch_gram_t<BF16, false>(p, s);
    return vec ? launch_gram_t<F32, true>(p, s) : launch_gram_t<F32, false>(p, s);
  }
  if (use_big(p, vec) && !small_norm(p, vec)) return launch_direct_norm_big(p, s);
  if (p.dtype == kBF16) return vec ? launch_direct_t<BF16, true>(p, s) : launch_direct_t<BF16, false>(p, s);
  return vec ? launch_direct_t<F32, true>(p, s) : launch_direct_t<F32, false>(p, s);
}
// A projection drawn from its seed regenerates its slice of P in every token
// tile.  With more than one token tile it is cheaper to draw P once into the
// call's workspace (din*r elements, after the split partials) with the
// gaussian fill, whose values are the ones the kernel would draw, and read
// it like a stored P.  P still lives only for the call.
static std::atomic<int> g_p_in_kernels{0};
void set_p_in_kernels(bool on) { g_p_in_kernels.store(on ? 1 : 0); }
bool p_in_kernels() { return g_p_in_kernels.load() != 0; }

static bool project_draws_p_once(const ProjArgs& p) {
  const int64_t ntok = (int64_t)p.B * p.T;
  return p.gen != 0 && !p_in_kernels() && (ntok + kTileN - 1) / kTileN > 1;
}

// din chunks of the projection.  One wherever the bf16 projection kernel
// (proj_big.hip, never split) takes the shape; it also draws P in its own
// tiles when asked, so a P drawn in the kernel, drawn once into workspace or
// stored meets the same arithmetic and gives the same bits.  Otherwise (the
// generic tiles) enough (output tile, chunk) workgroups for one per compute
// unit, each chunk at least 4 K-steps long, at most 8 chunks.
int project_splits(const ProjArgs& p, bool vec) {
  ProjArgs q = p;
  q.gen = 0;
  if (project_big_shape_ok(q, vec)) return 1;
  const int KT = p.dtype == kBF16 ? Cfg<BF16>::KT : Cfg<F32>::KT;
  const int64_t ntok = (int64_t)p.B * p.T;
  const int64_t tiles = ((p.r + kTileM - 1) / kTileM) * ((ntok + kTileN - 1) / kTileN);
  const int nk = (p.din + KT - 1) / KT;
  const int64_t want = (device_cus() + tiles - 1) / tiles;
  return (int)std::max<int64_t>(1, std::min<int64_t>({want, 8, nk / 4}));
}

static size_t project_split_bytes(const ProjArgs& p, int sp) {
  const size_t b = sp == 1 ? 0 : (size_t)sp * p.B * p.T * p.r * sizeof(float);
  return (b + 255) & ~(size_t)255;
}

size_t project_workspace_bytes(const ProjArgs& p, bool vec) {
  const int sp = project_splits(p, vec);
  if (!project_draws_p_once(p)) return project_split_bytes(p, sp);
  return project_split_bytes(p, sp) + (size_t)p.din * p.r * (p.dtype == kBF16 ? 2 : 4);
}

hipError_t launch_project(const ProjArgs& p, bool vec, hipStream_t s) {
  if (project_draws_p_once(p)) {
    if (p.part == nullptr) return hipErrorInvalidValue;
    ProjArgs q = p;
    q.P = reinterpret_cast<char*>(p.part) + project_split_bytes(p, p.splits);
    q.gen = 0;
    hipError_t e = launch_gaussian_fill(p.p_seed, p.p_offset, (int64_t)p.din * p.r, p.p_scale,
                                        p.dtype, const_cast<void*>(q.P), s);
    if (e != hipSuccess) return e;
    return launch_project(q, vec, s);
  }
  if (p.splits == 1 && project_big_eligible(p, vec)) return launch_project_big(p, s);
  if (p.gen) {
    if (p.dtype == kBF16)
      return vec ? launch_project_t<BF16, true, true>(p, s) : launch_project_t<BF16, false, true>(p, s);
    return vec ? launch_project_t<F32, true, true>(p, s) : launch_project_t<F32, false, true>(p, s);
  }
  if (p.dtype == kBF16)
    return vec ? launch_project_t<BF16, true, false>(p, s) : launch_project_t<BF16, false, false>(p, s);
  return vec ? launch_project_t<F32, true, false>(p, s) : launch_project_t<F32, false, false>(p, s);
}

}  // namespace dpf
