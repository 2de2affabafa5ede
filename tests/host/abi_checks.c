/* Host-side checks of the C ABI's argument validation, built with the host
 * sanitizers (address, undefined) together with a host-sanitized build of the
 * library.  Every call here fails its checks before anything is queued, so no
 * GPU is needed and no device memory is touched: the "device" pointers are
 * aligned host addresses that the library never dereferences. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dpfused.h"

static _Alignas(16) unsigned char g_fake[4096];
#define FAKE ((void*)g_fake)
static int g_failures = 0;

#define EXPECT(call, want)                                                             \
  do {                                                                                 \
    const int got_ = (int)(call);                                                      \
    if (got_ != (int)(want)) {                                                         \
      fprintf(stderr, "%s:%d: %s -> %d, expected %d (%s)\n", __FILE__, __LINE__, #call, \
              got_, (int)(want), dpfused_last_error());                                \
      ++g_failures;                                                                    \
    } else if ((want) != DPF_OK && dpfused_last_error()[0] == '\0') {                  \
      fprintf(stderr, "%s:%d: %s: empty error message\n", __FILE__, __LINE__, #call);  \
      ++g_failures;                                                                    \
    }                                                                                  \
  } while (0)

static dpf_act act(int64_t B, int64_t T, int64_t D, int32_t dtype) {
  dpf_act a;
  memset(&a, 0, sizeof a);
  a.data = FAKE;
  a.dtype = dtype;
  a.B = B;
  a.T = T;
  a.D = D;
  a.stride_t = D;
  a.stride_b = T * D;
  return a;
}

int main(void) {
  const dpf_act X = act(2, 3, 8, DPF_BF16), G = act(2, 3, 16, DPF_BF16);
  float* out = (float*)FAKE;

  if (dpfused_abi_version() != DPFUSED_ABI_VERSION) {
    fprintf(stderr, "ABI version %d != header %d\n", dpfused_abi_version(), DPFUSED_ABI_VERSION);
    ++g_failures;
  }
  for (int s = 0; s <= 4; ++s)
    if (strncmp(dpfused_status_string((dpf_status)s), "DPF_", 4) != 0) ++g_failures;

  /* the dense call */
  EXPECT(dpfused_linear_clip_accumulate(NULL, &G, NULL, 1.f, 1.f, 0, 0, out, NULL, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  dpf_act bad = X;
  bad.dtype = 7;
  EXPECT(dpfused_linear_clip_accumulate(&bad, &G, NULL, 1.f, 1.f, 0, 0, out, NULL, NULL),
         DPF_ERR_UNSUPPORTED);
  bad = X;
  bad.B = 3;
  bad.stride_b = 3 * 8;
  EXPECT(dpfused_linear_clip_accumulate(&bad, &G, NULL, 1.f, 1.f, 0, 0, out, NULL, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  bad = X;
  bad.stride_t = 4;
  EXPECT(dpfused_linear_clip_accumulate(&bad, &G, NULL, 1.f, 1.f, 0, 0, out, NULL, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  bad = X;
  bad.data = g_fake + 2;
  EXPECT(dpfused_linear_clip_accumulate(&bad, &G, NULL, 1.f, 1.f, 0, 0, out, NULL, NULL),
         DPF_ERR_UNSUPPORTED);
  bad = X;
  bad.reserved = 1;
  EXPECT(dpfused_linear_clip_accumulate(&bad, &G, NULL, 1.f, 1.f, 0, 0, out, NULL, NULL),
         DPF_ERR_UNSUPPORTED);
  EXPECT(dpfused_linear_clip_accumulate(&X, &G, NULL, 0.f, 1.f, 0, 0, out, NULL, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_linear_clip_accumulate(&X, &G, NULL, 1.f, NAN, 0, 0, out, NULL, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_linear_clip_accumulate(&X, &G, NULL, 1.f, -1.f, 0, 0, out, NULL, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_linear_clip_accumulate(&X, &G, NULL, 1.f, 1.f, 0, 0, NULL, NULL, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_linear_clip_accumulate(&X, &G, NULL, 1.f, 1.f, 0, 0, out + 1, NULL, NULL),
         DPF_ERR_UNSUPPORTED);

  /* explicit denominator / accumulation */
  EXPECT(dpfused_linear_clip_accumulate_ex(&X, &G, NULL, 1.f, 1.f, 0, 0, 0.f, 0, out, NULL, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_linear_clip_accumulate_ex(&X, &G, NULL, 1.f, 1.f, 0, 0, NAN, 0, out, NULL, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_linear_clip_accumulate_ex(&X, &G, NULL, 1.f, 1.f, 0, 0, 2.f, 2, out, NULL, NULL),
         DPF_ERR_INVALID_ARGUMENT);

  /* projected variants */
  EXPECT(dpfused_linear_clip_accumulate_projected(&X, &G, NULL, NULL, 8, 1.f, 1.f, 0, 0, out,
                                                  NULL, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_linear_clip_accumulate_projected(&X, &G, NULL, FAKE, 0, 1.f, 1.f, 0, 0, out,
                                                  NULL, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_linear_clip_accumulate_projected_seeded(&X, &G, NULL, 12, 7, 0, 0.25f, 1.f, 1.f,
                                                         0, 0, out, NULL, NULL),
         DPF_ERR_UNSUPPORTED);
  EXPECT(dpfused_linear_clip_accumulate_projected_seeded(&X, &G, NULL, 8, 7, 0, INFINITY, 1.f,
                                                         1.f, 0, 0, out, NULL, NULL),
         DPF_ERR_INVALID_ARGUMENT);

  /* the projection step alone */
  EXPECT(dpfused_project(&X, NULL, NULL, 8, out, NULL), DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_project(&X, NULL, FAKE, 8, NULL, NULL), DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_project(&X, NULL, FAKE, 0, out, NULL), DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_project(&X, NULL, (const char*)FAKE + 8, 8, out, NULL), DPF_ERR_UNSUPPORTED);
  EXPECT(dpfused_project(NULL, NULL, FAKE, 8, out, NULL), DPF_ERR_INVALID_ARGUMENT);

  /* building blocks */
  EXPECT(dpfused_per_sample_sqnorms(&X, &G, NULL, NULL, 0, NULL), DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_clip_factors((const double*)FAKE, 0, 1.f, out, NULL, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_scaled_accumulate(&X, &G, NULL, NULL, 0.f, 0, 0, out, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_scaled_accumulate(&X, &G, NULL, out, -1.f, 0, 0, out, NULL),
         DPF_ERR_INVALID_ARGUMENT);

  /* bias, group, projected Adam */
  EXPECT(dpfused_linear_clip_accumulate_bias(&X, &G, NULL, 1.f, 1.f, 0, 0, out, NULL, NULL, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  {
    const dpf_act xs[2] = {X, X};
    const dpf_act gs[2] = {G, act(2, 4, 16, DPF_BF16)};
    const uint64_t offs[2] = {0, 0};
    float* outs[2] = {out, out};
    EXPECT(dpfused_group_clip_accumulate(0, xs, gs, NULL, 1.f, 1.f, 0, offs, outs, NULL, NULL),
           DPF_ERR_INVALID_ARGUMENT);
    EXPECT(dpfused_group_clip_accumulate(2, xs, gs, NULL, 1.f, 1.f, 0, offs, outs, NULL, NULL),
           DPF_ERR_INVALID_ARGUMENT);
    EXPECT(dpfused_group_clip_accumulate(1, xs, gs, NULL, 1.f, 1.f, 0, NULL, outs, NULL, NULL),
           DPF_ERR_INVALID_ARGUMENT);
    const void* ps[2] = {FAKE, FAKE};
    EXPECT(dpfused_linear_clip_accumulate_projected_many(0, xs, gs, NULL, ps, 8, 1.f, 1.f, 0, offs,
                                                         outs, NULL, NULL),
           DPF_ERR_INVALID_ARGUMENT);
    EXPECT(dpfused_linear_clip_accumulate_projected_many(2, xs, gs, NULL, NULL, 8, 1.f, 1.f, 0, offs,
                                                         outs, NULL, NULL),
           DPF_ERR_INVALID_ARGUMENT);
    EXPECT(dpfused_linear_clip_accumulate_projected_many(2, xs, gs, NULL, ps, 8, 1.f, 1.f, 0, offs,
                                                         outs, NULL, NULL),
           DPF_ERR_INVALID_ARGUMENT);   /* the second G has another T */
  }
  EXPECT(dpfused_projected_adam_step(out, out, out, NULL, 8, 8, 8, 1, 1e-3f, 0.9f, 0.999f, 1e-8f,
                                     NULL, DPF_F32, 0, 0, 0.1f, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_projected_adam_step(out, out, out, out, 8, 8, 6, 1, 1e-3f, 0.9f, 0.999f, 1e-8f,
                                     NULL, DPF_F32, 0, 0, 0.1f, NULL),
         DPF_ERR_UNSUPPORTED);
  EXPECT(dpfused_projected_adam_step(out, out, out, out, 8, 8, 8, 0, 1e-3f, 0.9f, 0.999f, 1e-8f,
                                     NULL, DPF_F32, 0, 0, 0.1f, NULL),
         DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_projected_adam_step(out, out, out, out, 8, 8, 8, 1, 1e-3f, 1.0f, 0.999f, 1e-8f,
                                     NULL, DPF_F32, 0, 0, 0.1f, NULL),
         DPF_ERR_INVALID_ARGUMENT);

  /* fills */
  EXPECT(dpfused_philox4x32_10(0, 0, -1, (uint32_t*)FAKE, NULL), DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_philox4x32_10(0, 0, 4, NULL, NULL), DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_philox4x32_10(0, 0, 0, NULL, NULL), DPF_OK);
  EXPECT(dpfused_gaussian_fill(0, 0, 4, 1.f, 9, FAKE, NULL), DPF_ERR_UNSUPPORTED);
  EXPECT(dpfused_gaussian_fill(0, 0, 4, NAN, DPF_F32, FAKE, NULL), DPF_ERR_INVALID_ARGUMENT);
  if (dpfused_noise_blocks(5) != 2 || dpfused_noise_blocks(0) != 0 || dpfused_noise_blocks(-3) != 0)
    ++g_failures;

  /* options */
  EXPECT(dpfused_set_option("bogus", 1), DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_set_option(NULL, 1), DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_set_option("norm_path", 5), DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_set_option("norm_path", 4), DPF_OK);
  EXPECT(dpfused_set_option("onepass_never_ready", 2), DPF_ERR_INVALID_ARGUMENT);
  EXPECT(dpfused_set_option("norm_path", 3), DPF_OK);
  if (dpfused_get_option("norm_path") != 3) ++g_failures;
  EXPECT(dpfused_set_option("norm_path", 0), DPF_OK);
  if (dpfused_get_option("bogus") != -1) ++g_failures;

  if (g_failures != 0) {
    fprintf(stderr, "%d ABI check(s) failed\n", g_failures);
    return 1;
  }
  printf("abi checks passed\n");
  return 0;
}
