/* Shows that the sanitizer build of the library's host code is live: the activation parameters
 * are handed over in a heap block one field short, so moe_fused's check of linear_beta reads 4
 * bytes past it, which AddressSanitizer must report (tests/test_host_asan.py expects the
 * report).  Device pointers are placeholders; the call never reaches the HIP runtime. */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "moe_mi355x.h"

int main(void) {
  void *const P = (void *)0x100000;
  moe_act_params_t *a = (moe_act_params_t *)malloc(offsetof(moe_act_params_t, linear_beta));
  a->act = MOE_ACT_SITUV2;
  a->beta = 4.0f;
  moe_layout_t *L = (moe_layout_t *)calloc(1, sizeof(moe_layout_t));
  L->sorted_token_ids = (int32_t *)P;
  L->expert_ids = (int32_t *)P;
  L->num_tiles = (int32_t *)P;
  L->row_of = (int32_t *)P;
  L->cap_tiles = 100;
  L->block_m = 16;
  const int st = moe_fused(P, NULL, MOE_DT_BF16, P, MOE_W_PACKED, P, P, P, P, L, 4, 2, 8, 256, 128, a,
                           (uint16_t *)P, P, (size_t)1 << 30, MOE_STAGE_ALL, NULL);
  printf("status %d\n", st);
  free(a);
  free(L);
  return 0;
}
