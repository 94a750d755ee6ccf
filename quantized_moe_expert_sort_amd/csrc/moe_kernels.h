// Internal interface between the C-ABI entry points (moe_api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_mi355x.h"

namespace moe {

struct SortLayout {
  int32_t* sorted_ids;
  float* sorted_w;        // may be null
  int32_t* expert_ids;
  int32_t* num_tiles;
  int64_t cap_tiles;
};

constexpr int MAX_SORT_EXPERTS = 2048;

hipError_t launch_sort(const int32_t* topk_ids, const float* topk_w, int64_t n, int expert_begin,
                       int E, int block_m, const SortLayout& L, void* ws, hipStream_t s);

hipError_t launch_quant_act(const uint16_t* x, int64_t rows, int64_t cols, int dt, void* q,
                            uint8_t* scale, hipStream_t s);

struct FusedArgs {
  const uint8_t* x;        // activations (bf16 / fp8 / fp4x2 bytes)
  const uint8_t* xs;       // activation scales or null
  const uint8_t* w1;
  const uint8_t* w1s;
  const uint8_t* w2;
  const uint8_t* w2s;
  const float* topk_w;
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* num_tiles;
  float* acc;              // [T, D] fp32 combine accumulator
  uint8_t* inter;          // [cap*bm, I] intermediate codes
  uint8_t* inter_s;        // [cap*bm, I/32] intermediate scales (fp8 / fp4)
  float* dbg;              // [cap*bm, 2I] raw gate/up sums (NONE_TEST) or null
  int* counters;           // [D/16] stage2 completion counters (cleared by stage1)
  int n_counters;          // counters stage1 clears (set by the launcher)
  uint16_t* out;           // [T, D] bf16
  int T, topk, E, D, I, cap_tiles, block_m, a_dtype, act;
  float beta, linear_beta;
  int stages;              // bit 0: stage1, bit 1: stage2 + finalize
};

hipError_t launch_fused(const FusedArgs& a, hipStream_t s);

}  // namespace moe
