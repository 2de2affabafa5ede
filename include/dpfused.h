/*
 * dpfused: per-layer DP-SGD clip-and-accumulate for one linear layer, on
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * What the library computes (FlashDP: Private Training Large Language Models
 * with Efficient DP-SGD, Abstract: per-sample gradient clipping done per
 * layer, gradients computed once, in one fused task; Memory-Efficient
 * Differentially Private Training with Gradient Random Projection, English
 * explainer, Problem Statement and Methodology: clip each sample's gradient
 * before the noise is added, and in the projected variant project first):
 *
 *   X~_i, G~_i   rows of sample i whose mask byte is 0 are taken as zero
 *   g_i          = G~_i^T X~_i                        [dout, din]
 *   n_i          = ||g_i||_F
 *   c_i          = 1 if n_i <= C, else C / n_i
 *   grad_out     = (sum_i c_i g_i + sigma * C * xi) / B
 *   norms_out[i] = n_i   (before clipping)
 *
 * xi_e, for the row-major element index e of grad_out, is the standard normal
 * number e mod 4 of Philox4x32-10 block (offset + floor(e/4)): key =
 * (lo32(seed), hi32(seed)), counter = (lo32(block), hi32(block), 0, 0); the
 * four words w give uniforms u = ((w >> 9) + 0.5) * 2^-23, and Box-Muller
 * maps (u0,u1) -> (z0,z1) and (u2,u3) -> (z2,z3).  A call consumes
 * dpfused_noise_blocks(dout*din) blocks: advance `offset` by that much
 * between calls to draw fresh noise.
 *
 * Each call picks one of two ways to the norms, both giving the same n_i and
 * grad_out up to rounding, and neither storing a per-sample gradient: the
 * Gram identity ||G~^T X~||^2 = <X~ X~^T, G~ G~^T> (T short relative to the
 * layer), or the per-sample gradient tiles computed and dropped (a second
 * contraction then forms the clipped sum).  A third way, on request only
 * (the "norm_path" option set to 3), computes each tile once and stages it
 * in device memory (fp32, B * dout * din values rounded up to 256 x 256
 * tiles, at most 16 GiB per call) for the clipped sum to read back; that is
 * the explicit per-sample storage the FlashDP abstract sets its method
 * against, kept for comparison.  Staged tiles are given back at the end of
 * the call unless the "staged_keep_bytes" option keeps them.
 * Tiny dense calls (B <= 8, about 8192 outputs, every sample's rows within
 * 64 KiB as float32, at most 4 MFLOP) run the whole step in one workgroup
 * instead: one launch, the per-sample gradients never leave the chip.
 *
 * Conventions for every entry point
 *   - Every data pointer is DEVICE memory owned by the caller; the library
 *     never keeps, frees or reallocates it.  Outputs are overwritten.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *     queued on it asynchronously; temporary workspace is taken and given
 *     back in stream order: a block kept from an earlier call is used only
 *     after that call's last use of it (the stream waits for it on the GPU).
 *     Calls on different streams may run concurrently, except that staged
 *     calls take a kept staged-tile buffer in turn when the
 *     "staged_keep_bytes" option keeps one (each call's stream waits, on the
 *     GPU, for the previous holder's last use).
 *   - Arguments are checked before anything is queued: on any error nothing
 *     is launched and nothing is written; the status says why and
 *     dpfused_last_error() gives a message (per thread).
 *   - Faults inside a kernel surface at the caller's next synchronisation.
 *   - NaN or Inf in an ACTIVE row propagates to the outputs; masked rows are
 *     never read into the arithmetic, whatever they hold.
 *   - Results are bit-identical from run to run on the same device and build
 *     (every reduction has a fixed order; no floating-point atomics).
 *   - Noise: two outputs must never draw the same Philox block under one
 *     seed.  Shared normals cancel when the two outputs are subtracted, and
 *     the privacy the noise buys is lost.  Advance `offset` by
 *     dpfused_noise_blocks(n) after each call; the group call and the seeded
 *     projected call reject overlapping ranges that they can see.
 */
#ifndef DPFUSED_H
#define DPFUSED_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DPFUSED_ABI_VERSION 1

typedef enum {
  DPF_OK = 0,
  DPF_ERR_INVALID_ARGUMENT = 1, /* a shape, value or pointer is not acceptable */
  DPF_ERR_UNSUPPORTED = 2,      /* acceptable in principle, not handled (alignment, dtype mix) */
  DPF_ERR_OUT_OF_MEMORY = 3,    /* workspace allocation failed */
  DPF_ERR_HIP = 4               /* the HIP runtime reported an error while queueing */
} dpf_status;

typedef enum { DPF_F32 = 0, DPF_BF16 = 1 } dpf_dtype;

/* One [B, T, D] activation-like tensor in device memory.  The last dimension
 * is contiguous; stride_b and stride_t are in ELEMENTS.  `data` must be
 * 16-byte aligned, and for the vectorised loads also D * elemsize and both
 * strides * elemsize should be multiples of 16 bytes (other layouts are
 * accepted and run on a slower element-wise load path). */
typedef struct {
  const void* data;
  int32_t dtype;     /* dpf_dtype */
  int32_t reserved;  /* must be 0 */
  int64_t B, T, D;
  int64_t stride_b, stride_t;
} dpf_act;

/* The fused per-layer DP step for one linear layer (FlashDP abstract: one
 * fused per-layer task; the clip rule, noise law and orientation follow the
 * contract above).
 *
 *   X         activations        [B, T, din]   (bf16 or f32)
 *   G         output gradients   [B, T, dout]  (same dtype as X, same B and T)
 *   mask      [B, T] uint8, contiguous, 1 = active token; NULL = all active
 *   C         clip norm, finite and > 0
 *   sigma     noise multiplier, finite and >= 0 (0 = no noise, no Philox work)
 *   seed, offset   Philox key and first block (see above)
 *   grad_out  [dout, din] float32, row-major, overwritten
 *   norms_out [B] float32, pre-clip n_i; may be NULL
 *   stream    hipStream_t
 *
 * Errors: DPF_ERR_INVALID_ARGUMENT for NULL X/G data or grad_out, B/T/D < 1,
 * X.B != G.B or X.T != G.T, C not finite or <= 0, sigma not finite or < 0,
 * strides smaller than the row they step over; DPF_ERR_UNSUPPORTED for mixed
 * dtypes, an unknown dtype, a non-zero reserved field or a data pointer not
 * 16-byte aligned; DPF_ERR_OUT_OF_MEMORY if workspace cannot be allocated;
 * DPF_ERR_HIP if a launch fails. */
dpf_status dpfused_linear_clip_accumulate(const dpf_act* X, const dpf_act* G,
                                          const uint8_t* mask, float C, float sigma,
                                          uint64_t seed, uint64_t offset,
                                          float* grad_out, float* norms_out,
                                          void* stream);

/* The same step with an explicit denominator, added into grad_out on request:
 *
 *   grad_out = beta * grad_out + (sum_i c_i g_i + sigma * C * xi) / denom,
 *   beta = accumulate (0 or 1)
 *
 * For gradient accumulation over micro-batches of one logical batch, and for
 * a batch split across devices: each part is called with the logical batch
 * size as denom and sigma = 0 except for one part, which adds the noise.  The
 * per-sample clipping is unchanged (each sample is clipped on its own,
 * FlashDP abstract: per-layer clipping of each sample's gradient), so the
 * parts add up to the call on the whole batch.  With denom = B and
 * accumulate = 0 the result is dpfused_linear_clip_accumulate's, bit for bit.
 *
 *   denom       finite and > 0
 *   accumulate  0: grad_out is overwritten; 1: the result is added to it
 *               (grad_out must then hold finite values)
 *   other arguments, layouts and errors as dpfused_linear_clip_accumulate;
 *   a bad denom or accumulate gives DPF_ERR_INVALID_ARGUMENT. */
dpf_status dpfused_linear_clip_accumulate_ex(const dpf_act* X, const dpf_act* G,
                                             const uint8_t* mask, float C, float sigma,
                                             uint64_t seed, uint64_t offset, float denom,
                                             int32_t accumulate, float* grad_out,
                                             float* norms_out, void* stream);

/* dpfused_linear_clip_accumulate for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The call allocates nothing -- no hipMalloc, hipFree or
 * pool allocation.  Its workspace is a static device array of 80 MiB that
 * the library holds on each GPU it runs on until the process ends.
 *
 * Same arguments, result and errors as dpfused_linear_clip_accumulate.  The
 * norm path is that call's automatic choice (or the "norm_path" option's
 * Gram or direct; never the staged form).  When that plan's workspace is
 * larger than the scratch, the call runs without split tiles (same path),
 * then, for the Gram path, the direct form: results then equal the
 * allocating call's up to fp32 summation order, not bit for bit.
 *
 * Extra error: DPF_ERR_UNSUPPORTED when even that workspace (norm partials
 * B * tiles * 8 bytes, mask bits and lists) exceeds 80 MiB; nothing is then
 * launched or written.
 *
 * Every call on one GPU uses that GPU's one scratch array, and a call
 * leaves its contents behind (every kernel writes what it later reads, so
 * nothing needs clearing).  Calls that overlap in time on one GPU -- on two
 * streams, or from two threads without ordering -- race on it and give
 * wrong results; order them (one stream, or events). */
dpf_status dpfused_linear_clip_accumulate_noalloc(const dpf_act* X, const dpf_act* G,
                                                  const uint8_t* mask, float C, float sigma,
                                                  uint64_t seed, uint64_t offset,
                                                  float* grad_out, float* norms_out,
                                                  void* stream);

/* Projected variant (Memory-Efficient Differentially Private Training with
 * Gradient Random Projection, English explainer, Methodology: "Random
 * Projection over SVD" and "Order of Operations").  Each sample's gradient is
 * projected by a Gaussian matrix P before it is clipped and summed:
 *
 *   Y_i = X~_i P                 [T, r]  (rounded to X's dtype in workspace)
 *   h_i = G~_i^T Y_i             [dout, r]
 *   then clip, sum, noise and 1/B exactly as above, with r in place of din.
 *
 *   P         [din, r] row-major, same dtype as X, 16-byte aligned
 *   r         projection rank >= 1
 *   grad_out  [dout, r] float32, row-major, overwritten
 *   norms_out [B] float32, pre-clip ||h_i||; may be NULL
 *
 * Errors as above, plus DPF_ERR_INVALID_ARGUMENT for NULL P or r < 1. */
dpf_status dpfused_linear_clip_accumulate_projected(const dpf_act* X, const dpf_act* G,
                                                    const uint8_t* mask, const void* P,
                                                    int64_t r, float C, float sigma,
                                                    uint64_t seed, uint64_t offset,
                                                    float* grad_out, float* norms_out,
                                                    void* stream);

/* Several independent projected calls queued together, for example the six
 * linears of one RoBERTa layer: call l is
 *
 *   dpfused_linear_clip_accumulate_projected(&X[l], &G[l], masks[l], P[l], r,
 *       C, sigma, seed, offsets[l], grad_out[l], norms_out[l], stream)
 *
 * each clipped on its own (per-layer clipping, as in the single call).  The
 * calls run on streams of the library, forked from `stream` after its earlier
 * work and joined back into it, so that the small launches of different
 * linears overlap on the GPU; every output is bitwise that of the single
 * call.  Call l runs on branch l mod (k + 1): branch 0 is `stream` itself,
 * branch j the library's stream j - 1, with k = the "side_streams" option
 * (default 1, at most 4; 0 queues every call on `stream`).  When `stream` is
 * being captured into a graph, with n = 1, or with the staged norm path
 * forced, the calls run one after another on `stream`.  The library's streams
 * (four per device, default priority) live until the process ends.
 *
 *   n          number of calls, 1 .. 64
 *   X, G       HOST arrays of n descriptors (each call its own B, T, din, dout)
 *   masks      HOST array of n mask pointers ([B_l, T_l] or NULL), or NULL
 *   P          HOST array of n DEVICE pointers, P[l] [din_l, r] in X[l]'s dtype
 *   r          projection width, shared
 *   offsets    HOST array of n Philox offsets; with sigma > 0 the block ranges
 *              [offsets[l], offsets[l] + dpfused_noise_blocks(dout_l * r)) must
 *              be pairwise disjoint, else DPF_ERR_INVALID_ARGUMENT
 *   grad_out   HOST array of n DEVICE pointers, grad_out[l] [dout_l, r]
 *   norms_out  HOST array of n DEVICE pointers ([B_l] float32 or NULL), or NULL
 *
 * Errors as for the single call, checked for every call before anything is
 * queued; the workspace of all calls is taken at once, so an allocation
 * failure leaves every output untouched.  Calls that overlap in time on one
 * GPU from several host threads are queued one at a time. */
dpf_status dpfused_linear_clip_accumulate_projected_many(
    int32_t n, const dpf_act* X, const dpf_act* G, const uint8_t* const* masks,
    const void* const* P, int64_t r, float C, float sigma, uint64_t seed, const uint64_t* offsets,
    float* const* grad_out, float* const* norms_out, void* stream);

/* Projected variant with the projection regenerated from a seed instead of
 * stored (same explainer, Methodology, "Random Projection over SVD": the
 * random matrices need not be kept, since they can be drawn again from their
 * seed).  Identical to dpfused_linear_clip_accumulate_projected with
 *
 *   P[d][j] = p_scale * xi_{d*r + j}   (d < din, j < r)
 *
 * rounded to X's dtype, xi from Philox4x32-10 (p_seed, p_offset) as above --
 * i.e. with the P that dpfused_gaussian_fill(p_seed, p_offset, din*r,
 * p_scale, X's dtype) writes -- but P is not kept: with one tile of tokens
 * (B*T <= 128), or with the "p_in_kernels" option on, the projection kernel
 * draws each element where it needs it and P never exists in memory; with
 * more, P is drawn once into the call's workspace (din*r elements, released
 * with it) and read from there, which is cheaper than drawing it again in
 * every token tile.  Both give the same bits.
 *
 *   r         projection rank, a positive multiple of 8
 *   p_scale   the entries' standard deviation; NaN or <= 0 selects the
 *             method's N(0, 1/r) entries, p_scale = 1/sqrt(r) (same
 *             explainer and section: Gaussian entries whose variance is
 *             the inverse of the rank)
 *
 * Errors as for the projected variant; r not a multiple of 8 gives
 * DPF_ERR_UNSUPPORTED; an infinite p_scale gives DPF_ERR_INVALID_ARGUMENT;
 * with sigma > 0 and seed == p_seed, noise blocks [offset, offset +
 * dpfused_noise_blocks(dout*r)) that overlap P's blocks [p_offset, p_offset +
 * dpfused_noise_blocks(din*r)) give DPF_ERR_INVALID_ARGUMENT (the noise would
 * be a scaled copy of P's entries, known to anyone who can draw P again). */
dpf_status dpfused_linear_clip_accumulate_projected_seeded(
    const dpf_act* X, const dpf_act* G, const uint8_t* mask, int64_t r, uint64_t p_seed,
    uint64_t p_offset, float p_scale, float C, float sigma, uint64_t seed, uint64_t offset,
    float* grad_out, float* norms_out, void* stream);

/* The projection step of the projected variant alone (same explainer,
 * Methodology, "Order of Operations": the activations are projected before
 * the per-sample gradient is formed, clipped and noised):
 *
 *   Y[b][t][j] = sum_d X~[b][t][d] P[d][j]     (X~: X with masked rows zero)
 *
 * accumulated in float32 and rounded to X's dtype (round to nearest even for
 * bf16) -- exactly the Y that the projected calls form in their workspace.
 *
 *   X     as for the dense call (bf16 or float32)
 *   mask  [B, T] uint8 or NULL; masked rows of Y are zero
 *   P     [din, r] row-major, X's dtype, 16-byte aligned
 *   r     >= 1
 *   Y     [B, T, r] row-major, contiguous, X's dtype, 16-byte aligned;
 *         owned by the caller, overwritten
 *
 * Errors: DPF_ERR_INVALID_ARGUMENT for NULL P or Y or r < 1; as for the
 * dense call for X; DPF_ERR_UNSUPPORTED for unaligned P or Y or r too large;
 * DPF_ERR_OUT_OF_MEMORY when the split-K workspace of the fallback tiles
 * (used for float32 and for shapes the bf16 kernel does not take) cannot be
 * allocated. */
dpf_status dpfused_project(const dpf_act* X, const uint8_t* mask, const void* P, int64_t r,
                           void* Y, void* stream);

/* Per-sample squared norms ||G~_i^T X~_i||^2 only, in float64, written to
 * sqnorms_out[B] (device).  With accumulate != 0 the values are ADDED to what
 * sqnorms_out holds (summing over several linears gives the squared norm of
 * a sample's gradient across those layers).  Same argument rules as
 * dpfused_linear_clip_accumulate. */
dpf_status dpfused_per_sample_sqnorms(const dpf_act* X, const dpf_act* G, const uint8_t* mask,
                                      double* sqnorms_out, int32_t accumulate, void* stream);

/* Clip factors from squared norms: c[i] = 1 if sqrt(sqnorms[i]) <= C else
 * C / sqrt(sqnorms[i]) (float32), and norms_out[i] = sqrt(sqnorms[i]) when
 * norms_out is not NULL.  All pointers are device memory; n >= 1. */
dpf_status dpfused_clip_factors(const double* sqnorms, int64_t n, float C, float* c_out,
                                float* norms_out, void* stream);

/* grad_out = (sum_i c[i] G~_i^T X~_i + noise_std * xi) / B for given factors
 * c[B] (device float32, each finite and > 0), with xi as above (noise_std = 0
 * disables the noise).  Same argument rules as dpfused_linear_clip_accumulate;
 * noise_std must be finite and >= 0. */
dpf_status dpfused_scaled_accumulate(const dpf_act* X, const dpf_act* G, const uint8_t* mask,
                                     const float* c, float noise_std, uint64_t seed,
                                     uint64_t offset, float* grad_out, void* stream);

/* The dense step for a linear layer with a bias, y = x W^T + b: the layer's
 * parameters are W and b, so sample i's gradient is the pair (g_i, gb_i) and
 * both parts are clipped by the norm of the pair (the per-layer clipping of
 * the FlashDP abstract, applied to the whole layer):
 *
 *   gb_i             = sum over the active tokens t of G~_i[t]       [dout]
 *   n_i              = sqrt(||g_i||_F^2 + ||gb_i||^2)
 *   grad_out         = (sum_i c_i g_i  + sigma * C * xi) / B          [dout, din]
 *   bias_grad_out    = (sum_i c_i gb_i + sigma * C * xi') / B         [dout]
 *
 * xi as for dpfused_linear_clip_accumulate (offset); xi' continues the same
 * Philox stream after it: element o of the bias uses block
 * offset + dpfused_noise_blocks(dout*din) + floor(o/4), lane o mod 4.  A call
 * consumes dpfused_noise_blocks(dout*din) + dpfused_noise_blocks(dout) blocks.
 * Equivalently: the dense call on the input [X, 1] (a constant-one column
 * whose weight is the bias), up to the noise layout.
 *
 *   bias_grad_out  [dout] float32 (device), 4-byte aligned, overwritten
 *
 * Other arguments and errors as for dpfused_linear_clip_accumulate. */
dpf_status dpfused_linear_clip_accumulate_bias(const dpf_act* X, const dpf_act* G,
                                               const uint8_t* mask, float C, float sigma,
                                               uint64_t seed, uint64_t offset, float* grad_out,
                                               float* bias_grad_out, float* norms_out,
                                               void* stream);

/* Group (joint) clipping over n linears that see the same samples, e.g. the
 * seven linears of one decoder layer.  The FlashDP pages clip per layer
 * (FlashDP, Abstract: per-layer DP-SGD, gradients computed once); this is the
 * same step with the clipping norm taken over a group of layers instead of
 * one, the form standard (flat) DP-SGD uses for the whole model:
 *
 *   n_i^2           = sum_l ||G~_il^T X~_il||_F^2
 *   c_i             = 1 if n_i <= C, else C / n_i
 *   grad_out[l]     = (sum_i c_i G~_il^T X~_il + sigma * C * xi^(l)) / B
 *   norms_out[i]    = n_i (the group norm, before clipping)
 *
 * xi^(l) is the noise of the dense call with (seed, offsets[l]).  With n = 1
 * it is dpfused_linear_clip_accumulate.  With sigma > 0 the block ranges
 * [offsets[l], offsets[l] + dpfused_noise_blocks(dout_l * din_l)) must be
 * pairwise disjoint, else DPF_ERR_INVALID_ARGUMENT (consecutive ranges,
 * offsets[l+1] = offsets[l] + dpfused_noise_blocks(dout_l * din_l), are the
 * usual choice).
 *
 *   n          number of linears, >= 1
 *   X, G       HOST arrays of n descriptors; every linear has the same B and T
 *   mask       [B, T] or NULL, shared by the linears
 *   offsets    HOST array of n Philox offsets
 *   grad_out   HOST array of n DEVICE pointers, grad_out[l] [dout_l, din_l]
 *   norms_out  [B] float32 or NULL
 *
 * Errors as for dpfused_linear_clip_accumulate, checked for every linear
 * before anything is queued; B or T differing between linears gives
 * DPF_ERR_INVALID_ARGUMENT. */
dpf_status dpfused_group_clip_accumulate(int32_t n, const dpf_act* X, const dpf_act* G,
                                         const uint8_t* mask, float C, float sigma, uint64_t seed,
                                         const uint64_t* offsets, float* const* grad_out,
                                         float* norms_out, void* stream);

/* One step of the projected Adam optimizer (Memory-Efficient Differentially
 * Private Training with Gradient Random Projection, English explainer,
 * Methodology, "Projected Optimizer States": the Adam moments are kept in the
 * projected space, and the update goes back to the weight through the
 * projection).  With h = grad, the privatised projected gradient of a linear
 * (the grad_out of a projected call):
 *
 *   m <- beta1 m + (1 - beta1) h,   v <- beta2 v + (1 - beta2) h*h
 *   U  = (m / (1 - beta1^step)) / (sqrt(v / (1 - beta2^step)) + eps)
 *   W <- W - lr * U P^T
 *
 * (plain Adam, no weight decay; elementwise in float32, U P^T with float32
 * MFMA).
 *
 *   grad       [dout, r] float32 (device), read
 *   m, v       [dout, r] float32 (device), updated in place
 *   W          [dout, din] float32 row-major (device), updated in place
 *   r, din     multiples of 4
 *   step       >= 1, the number of this update (1 for the first)
 *   beta1, beta2 in [0, 1); eps finite and > 0; lr finite
 *   P          [din, r] row-major, p_dtype (DPF_F32 or DPF_BF16), 16-byte
 *              aligned -- or NULL: then P[d][j] = p_scale * xi_{d*r+j} from
 *              Philox (p_seed, p_offset) rounded to p_dtype, the P of
 *              dpfused_linear_clip_accumulate_projected_seeded (NaN or <= 0
 *              p_scale: 1/sqrt(r), as there), drawn again
 *              inside the kernel, or once into workspace (din*r elements of
 *              p_dtype, for this call only) when W has more than one row of
 *              the kernel's tiles and the "p_in_kernels" option is off
 *
 * All pointers 16-byte aligned.  Errors as above; nothing is written on
 * error.  m, v and W must not overlap each other or grad. */
dpf_status dpfused_projected_adam_step(const float* grad, float* m, float* v, float* W,
                                       int64_t dout, int64_t din, int64_t r, int64_t step,
                                       float lr, float beta1, float beta2, float eps,
                                       const void* P, int32_t p_dtype, uint64_t p_seed,
                                       uint64_t p_offset, float p_scale, void* stream);

/* Raw Philox4x32-10 words of the noise generator (the noise added after
 * clipping in the FlashDP abstract and in the DP-GRAPE explainer,
 * Methodology, is drawn from this counter-based generator; Salmon, Moraes,
 * Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11):
 * out[4*j + k] = word k of block (offset + j), j < nblocks, with the
 * key/counter layout above.  For checking the generator and for callers
 * that draw their own noise.  out: device, 16-byte aligned, 4*nblocks
 * uint32.  nblocks >= 0 (0 = nothing queued).  Errors: NULL or misaligned
 * out, negative nblocks. */
dpf_status dpfused_philox4x32_10(uint64_t seed, uint64_t offset, int64_t nblocks,
                                 uint32_t* out, void* stream);

/* Gaussian numbers of the noise law above: out[e] = scale * xi_e for e < n
 * (four normals per block, starting at block `offset`), stored as float32
 * or as bfloat16 rounded to nearest-even from the float32 product.  Draws
 * the Gaussian projection P of the DP-GRAPE explainer (Methodology, "Random
 * Projection over SVD": random Gaussian matrices, drawn again from their
 * seed; entries N(0, 1/r): scale = 1/sqrt(r)), and the noise
 * sigma * C * xi of the FlashDP abstract's noise step on its own.  out:
 * device, 16-byte aligned.  n >= 0.  Errors: unknown dtype, infinite scale,
 * NULL or misaligned out, negative n. */
dpf_status dpfused_gaussian_fill(uint64_t seed, uint64_t offset, int64_t n, float scale,
                                 int32_t dtype, void* out, void* stream);

/* Philox blocks consumed by n noise elements (four normals per block, by
 * the noise layout above): ceil(n / 4); 0 for n <= 0.  Advance `offset` by
 * this much between calls so that no two outputs share noise. */
uint64_t dpfused_noise_blocks(int64_t n_elements);

/* Library options (process-wide).  Names:
 *   "norm_path"  0 = choose per call between Gram and direct (default);
 *                1 = always Gram; 2 = always direct (gradient tiles
 *                computed and dropped, then a second contraction); 3 =
 *                staged where the call allows it (bf16 single-layer and
 *                group calls whose staged tiles fit in 16 GiB), else direct;
 *                4 = single pass where the call allows it (the dense
 *                single-layer calls, bf16 on the large-tile layout, at most
 *                256 output tiles of 128 x 128 that can all be resident at
 *                once, not under graph capture: one cooperative kernel that
 *                computes each per-sample gradient tile once and reduces the
 *                norms across workgroups while the next sample is
 *                contracted), else the automatic choice
 *   "onepass_spin_limit"  single pass: tries of a blocked wait for another
 *                workgroup's partial norms before the call gives up and
 *                writes NaN to its outputs (default 2^20; 0..2^30)
 *   "onepass_never_ready"  testing only: 1 = every fetch of partials in the
 *                single pass counts as incomplete, so every blocked wait
 *                gives up after "onepass_spin_limit" tries (the kernel still
 *                exits; the outputs are NaN); 0 (default) = normal
 *   "timing"     1 = record a HIP event pair around every kernel the library
 *                launches, on the launch stream (see dpfused_timing_*); 0 = off
 *   "workspace_keep_bytes"  bytes of workspace the library keeps reserved
 *                for later calls (default 512 MiB, about twice the largest
 *                Llama-13B-layer call's workspace), each of: workspace
 *                blocks freed by calls and kept for reuse (a later call's
 *                stream waits on the GPU for the block's last use, so blocks
 *                move between streams safely), and freed memory in the
 *                per-device pool behind them.  Setting it trims both;
 *                trimming kept blocks waits for their last users.
 *   "staged_keep_bytes"  staged path only: a per-device buffer of staged
 *                tiles up to this size is kept for the next call (calls on
 *                any stream then take it in turn, the stream waiting on the
 *                GPU for its previous holder); 0 (default) = the tiles are
 *                taken and given back within each call, stream-ordered
 *   "workspace_limit_bytes"  a workspace request larger than this (one
 *                call's pool allocation, or its staged tile buffer) fails
 *                with DPF_ERR_OUT_OF_MEMORY before any output is written, as a
 *                failed hipMallocAsync would; 0 (default) = no limit
 *   "p_in_kernels"  1 = a P given by its seed is always drawn inside the
 *                kernels that use it, never stored (slower at many token
 *                tiles); 0 (default) = drawn once per call into workspace
 *                where that is cheaper.  Results are identical.
 *   "side_streams"  0 .. 4: library streams that
 *                dpfused_linear_clip_accumulate_projected_many spreads its
 *                calls over beside the caller's stream (default 1; 0 = all
 *                on the caller's stream).  Results are identical.
 *   "rspace_tiles"  projected calls: the r-space sum G~^T Y ([dout, r],
 *                a few tiles over B*T tokens) accumulated on 128 x 128 tiles
 *                whose samples are cut into pieces spread over the compute
 *                units, the pieces' fp32 parts added in a fixed order by a
 *                second kernel (1, the default); that and the direct norm
 *                on the same tiles (2); the 256 x 256 tiles (0).  Results
 *                agree within rounding (a different summation order), and
 *                each setting is deterministic.
 *   "trace"      1 = push a roctx range named after the entry point around
 *                every call, for rocprofv3 --marker-trace; 0 = off (default)
 *   "debug"      1 = synchronise the launch stream after every kernel and
 *                print the kernel's name and the HIP error to stderr if it
 *                failed; slow, for finding a failing launch; 0 = off (default)
 * Defaults are read from the environment when the library is loaded:
 * DPFUSED_NORM_PATH ("auto", "gram", "direct", "staged", "onepass" or 0-4),
 * DPFUSED_TRACE and DPFUSED_DEBUG (0/1), DPFUSED_WS_LIMIT (bytes).
 * Read-only (dpfused_get_option): "workspace_reserved_bytes" and
 * "workspace_reserved_high", what the current device's pool holds now and at
 * most (-1 without a pool); "workspace_call_bytes", the device memory the
 * last call on this thread took beyond its inputs and outputs (workspace
 * plus staged tiles), and "workspace_call_high", the most any call took
 * since the library was loaded or since dpfused_set_option(
 * "workspace_call_high", 0).
 * Returns DPF_ERR_INVALID_ARGUMENT for an unknown name or value. */
dpf_status dpfused_set_option(const char* name, int64_t value);
int64_t dpfused_get_option(const char* name);

/* Kernel timing, when the "timing" option is on.  dpfused_timing_collect()
 * waits for every recorded event pair, adds its duration to a per-kernel
 * total and returns the number of distinct kernels seen since the last
 * reset; then entry k (k < that number) is read with the three accessors.
 * Durations are in milliseconds.  Not thread-safe against concurrent calls. */
void dpfused_timing_reset(void);
int32_t dpfused_timing_collect(void);
const char* dpfused_timing_name(int32_t k);
double dpfused_timing_total_ms(int32_t k);
int64_t dpfused_timing_launches(int32_t k);

const char* dpfused_status_string(dpf_status s);
const char* dpfused_last_error(void);
int32_t dpfused_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DPFUSED_H */
