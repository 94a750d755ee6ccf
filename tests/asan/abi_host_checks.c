/* Host-side argument checks of every libmoe_mi355x entry point, built with AddressSanitizer on
 * the host code of the library (tests/test_host_asan.py compiles the library sources host-only
 * with the sanitizer and links this driver against them).
 *
 * Every call here must be rejected, or finish as a no-op, on the host: device pointers are
 * placeholders that are never dereferenced, so the driver runs on a machine without a GPU.
 * Host structs (the layout descriptor, the activation parameters) are heap blocks of exactly
 * their size, so a read past them in the library is reported by the sanitizer.  Exit status 0
 * when every status code matches, 1 otherwise. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_mi355x.h"

static void *const P = (void *)0x100000;   /* placeholder device pointer */
static int failures = 0;

#define EXPECT(call, want)                                                                   \
  do {                                                                                       \
    const int got_ = (int)(call);                                                            \
    if (got_ != (int)(want)) {                                                               \
      fprintf(stderr, "%s:%d: %s -> %d, expected %d\n", __FILE__, __LINE__, #call, got_,     \
              (int)(want));                                                                  \
      ++failures;                                                                            \
    }                                                                                        \
  } while (0)

static moe_layout_t *layout(int32_t cap, int32_t bm, int weights, int row_of) {
  moe_layout_t *L = (moe_layout_t *)malloc(sizeof(moe_layout_t));
  L->sorted_token_ids = (int32_t *)P;
  L->sorted_weights = weights ? (float *)P : NULL;
  L->expert_ids = (int32_t *)P;
  L->num_tiles = (int32_t *)P;
  L->row_of = row_of ? (int32_t *)P : NULL;
  L->sync = NULL;
  L->cap_tiles = cap;
  L->block_m = bm;
  return L;
}

static moe_act_params_t *act_params(int32_t act, float beta, float lb) {
  moe_act_params_t *a = (moe_act_params_t *)malloc(sizeof(moe_act_params_t));
  a->act = act;
  a->beta = beta;
  a->linear_beta = lb;
  return a;
}

static void sort_checks(void) {
  const int32_t T = 4, K = 2, E = 8;
  moe_layout_t *ok = layout(moe_cap_tiles(T, K, E, 16), 16, 1, 1);
  EXPECT(moe_sort(P, P, -1, K, 0, E, ok, P, 1 << 20, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_sort(P, P, T, 0, 0, E, ok, P, 1 << 20, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_sort(P, P, T, K, 0, 0, ok, P, 1 << 20, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_sort(P, P, T, K, 0, 4096, ok, P, 1 << 20, NULL), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_sort(NULL, P, T, K, 0, E, ok, P, 1 << 20, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_sort(P, NULL, T, K, 0, E, ok, P, 1 << 20, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_sort(P, P, T, K, 0, E, NULL, P, 1 << 20, NULL), MOE_ERR_INVALID_ARG);
  moe_layout_t *bm64 = layout(100, 64, 1, 1);
  EXPECT(moe_sort(P, P, T, K, 0, E, bm64, P, 1 << 20, NULL), MOE_ERR_UNSUPPORTED);
  moe_layout_t *small = layout(moe_cap_tiles(T, K, E, 16) - 1, 16, 1, 1);
  EXPECT(moe_sort(P, P, T, K, 0, E, small, P, 1 << 20, NULL), MOE_ERR_CAPACITY);
  moe_layout_t *no_ids = layout(100, 16, 0, 1);
  no_ids->sorted_token_ids = NULL;
  EXPECT(moe_sort(P, P, T, K, 0, E, no_ids, P, 1 << 20, NULL), MOE_ERR_INVALID_ARG);
  /* a multi-chunk sort needs its workspace */
  const int32_t TB = 2000, KB = 16;
  moe_layout_t *big = layout(moe_cap_tiles(TB, KB, E, 16), 16, 1, 1);
  EXPECT(moe_sort(P, P, TB, KB, 0, E, big, P, 16, NULL), MOE_ERR_WORKSPACE);
  EXPECT(moe_sort(P, P, TB, KB, 0, E, big, NULL, moe_sort_ws_bytes(TB, KB, E), NULL), MOE_ERR_INVALID_ARG);
  free(ok); free(bm64); free(small); free(no_ids); free(big);
}

/* moe_fused with the default valid arguments, each case changing one of them */
typedef struct {
  int32_t a_dtype, w_layout, T, K, E, D, I, stages;
  const void *x, *xs;
  uint16_t *out;
  moe_layout_t *L;
  moe_act_params_t *act;
  size_t ws_bytes;
} fused_args;

static fused_args fused_default(void) {
  fused_args a;
  memset(&a, 0, sizeof(a));
  a.a_dtype = MOE_DT_BF16; a.w_layout = MOE_W_PACKED;
  a.T = 4; a.K = 2; a.E = 8; a.D = 256; a.I = 128; a.stages = MOE_STAGE_ALL;
  a.x = P; a.xs = NULL; a.out = (uint16_t *)P;
  a.L = layout(moe_cap_tiles(a.T, a.K, a.E, 16), 16, 1, 1);
  a.act = act_params(MOE_ACT_SITUV2, 4.0f, 25.0f);
  a.ws_bytes = (size_t)1 << 30;
  return a;
}

static int fused(const fused_args *a) {
  return moe_fused(a->x, (const uint8_t *)a->xs, a->a_dtype, P, a->w_layout, P, P, P, P, a->L, a->T, a->K,
                   a->E, a->D, a->I, a->act, a->out, P, a->ws_bytes, a->stages, NULL);
}

static int fused_noalloc(const fused_args *a) {
  return moe_fused_noalloc(a->x, (const uint8_t *)a->xs, a->a_dtype, P, a->w_layout, P, P, P, P, a->L, a->T,
                           a->K, a->E, a->D, a->I, a->act, a->out, a->stages, NULL);
}

static void fused_checks(int noalloc) {
  int (*call)(const fused_args *) = noalloc ? fused_noalloc : fused;
  fused_args a;
#define CASE(edit, want)            \
  do {                              \
    a = fused_default();            \
    edit;                           \
    EXPECT(call(&a), want);         \
    free(a.L); free(a.act);         \
  } while (0)
  CASE(a.a_dtype = 7, MOE_ERR_INVALID_ARG);
  CASE(a.act->act = 5, MOE_ERR_UNSUPPORTED);
  CASE(a.act->beta = 0.0f, MOE_ERR_INVALID_ARG);
  CASE(a.act->linear_beta = -1.0f, MOE_ERR_INVALID_ARG);
  CASE((free(a.act), a.act = NULL), MOE_ERR_INVALID_ARG);
  CASE(a.D = 200, MOE_ERR_UNSUPPORTED);
  CASE(a.I = 96, MOE_ERR_UNSUPPORTED);
  CASE(a.T = -1, MOE_ERR_INVALID_ARG);
  CASE((a.a_dtype = MOE_DT_FP8_E4M3, a.xs = NULL), MOE_ERR_INVALID_ARG);
  CASE(a.xs = P, MOE_ERR_INVALID_ARG);
  CASE(a.x = NULL, MOE_ERR_INVALID_ARG);
  CASE(a.out = NULL, MOE_ERR_INVALID_ARG);
  CASE(a.L->cap_tiles = 1, MOE_ERR_CAPACITY);
  CASE(a.L->block_m = 8, MOE_ERR_UNSUPPORTED);
  CASE(a.L->row_of = NULL, MOE_ERR_INVALID_ARG);
  CASE((free(a.L), a.L = NULL), MOE_ERR_INVALID_ARG);
  CASE(a.stages = 0, MOE_ERR_INVALID_ARG);
  CASE(a.stages = 4, MOE_ERR_INVALID_ARG);
  CASE(a.w_layout = MOE_W_ROW_MAJOR, MOE_ERR_UNSUPPORTED);
  CASE(a.w_layout = MOE_W1_PACKED, MOE_ERR_UNSUPPORTED);
  CASE(a.w_layout = 3, MOE_ERR_INVALID_ARG);
  CASE(a.T = 0, MOE_OK);
  if (!noalloc) CASE(a.ws_bytes = 10, MOE_ERR_WORKSPACE);
  if (noalloc) {
    /* more than the fixed scratch: rejected before the scratch is looked up */
    CASE((a.a_dtype = MOE_DT_FP8_E4M3, a.xs = P, a.T = 1024, a.K = 16, a.E = 896, a.D = 3584, a.I = 384,
          free(a.L), a.L = layout(moe_cap_tiles(1024, 16, 896, 32), 32, 1, 1)),
         MOE_ERR_WORKSPACE);
  }
#undef CASE
}

static void quant_checks(void) {
  EXPECT(moe_quant_act(P, 4, 64, MOE_DT_BF16, P, P, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_quant_act(P, 4, 48, MOE_DT_FP8_E4M3, P, P, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_quant_act(P, -1, 64, MOE_DT_FP8_E4M3, P, P, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_quant_act(NULL, 4, 64, MOE_DT_FP8_E4M3, P, P, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_quant_act(P, 4, 64, MOE_DT_FP4_E2M1, P, NULL, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(moe_quant_act(P, 0, 64, MOE_DT_FP4_E2M1, P, P, NULL), MOE_OK);
}

typedef moe_status_t (*pack_fn)(const uint8_t *, int32_t, int32_t, int32_t, uint8_t *, void *);

static void pack_checks(pack_fn pack, size_t n /* bytes of the weights at E = 2, D = 256, I = 128 */) {
  uint8_t *w = (uint8_t *)P;
  uint8_t *other = (uint8_t *)0x4000000;
  EXPECT(pack(w, 2, 256, 128, w, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(pack(w, 2, 256, 128, w + n - 16, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(pack(w + 16, 2, 256, 128, w, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(pack(NULL, 2, 256, 128, other, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(pack(w, 2, 256, 128, NULL, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(pack(w, 0, 256, 128, other, NULL), MOE_ERR_INVALID_ARG);
  EXPECT(pack(w, 2, 192, 128, other, NULL), MOE_ERR_UNSUPPORTED);
  EXPECT(pack(w, 2, 256, 64, other, NULL), MOE_ERR_UNSUPPORTED);
}

int main(void) {
  sort_checks();
  fused_checks(0);
  fused_checks(1);
  quant_checks();
  pack_checks(moe_pack_w1, (size_t)2 * 256 * 128);   /* [E, 2I, D/2] */
  pack_checks(moe_pack_w2, (size_t)2 * 256 * 64);    /* [E, D, I/2] */
  EXPECT(moe_last_hip_error(), 0);   /* nothing above reached the HIP runtime */
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi host checks: all passed\n");
  return 0;
}
