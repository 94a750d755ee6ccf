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
  int32_t* row_of;        // may be null
  int32_t* sync;          // may be null; zeroed when given
  int64_t sync_words;
  int64_t cap_tiles;
};

constexpr int MAX_SORT_EXPERTS = MOE_SORT_MAX_EXPERTS;

// ---------------------------------------------------------------- debug checks
//
// Built with -DMOE_DEBUG_CHECKS (the separate library libmoe_mi355x_debug.so), the kernels check
// index invariants they otherwise take from the sort and the host checks: the positions the
// sort writes, the row ids and expert ids the stages read from the layout, the tile ranges of
// the grouped stages and the rows the combine gathers.  A failed check does not trap: it sets
// its bit in the violation word of its source file and the access it guards is skipped (a row
// id outside the layout reads as padding), so the launch ends normally.  Every entry point of
// the debug library then waits for the device, collects and clears the words and returns
// MOE_ERR_DEBUG_CHECK if a bit was set.  In the normal build MOE_DCHECK is `true` and adds no
// code.
enum : uint32_t {
  DBG_SORT_POS = 1u,      // a sorted position past cap_tiles * block_m
  DBG_LAYOUT_ROW = 2u,    // a layout row id outside [0, T*topk] (T*topk marks padding)
  DBG_EXPERT = 4u,        // a tile's expert id >= num_local_experts
  DBG_GROUP = 8u,         // a tile group outside [0, cap_tiles)
  DBG_COMBINE_ROW = 16u,  // a row_of entry outside [-1, cap_tiles * block_m)
};
#ifdef MOE_DEBUG_CHECKS
static __device__ uint32_t dbg_word;   // one per source file
#define MOE_DCHECK(cond, bit) ((cond) ? true : (atomicOr(&::moe::dbg_word, (uint32_t)(bit)), false))
// host side: the word of one source file, cleared after it is read
#define MOE_DEBUG_READER(name)                                                         \
  hipError_t debug_take_##name(uint32_t* v) {                                          \
    const uint32_t z = 0;                                                              \
    hipError_t e = hipMemcpyFromSymbol(v, HIP_SYMBOL(dbg_word), sizeof(uint32_t));     \
    return e != hipSuccess ? e : hipMemcpyToSymbol(HIP_SYMBOL(dbg_word), &z, sizeof(uint32_t)); \
  }
hipError_t debug_take_sort(uint32_t* v);
hipError_t debug_take_gemm(uint32_t* v);
hipError_t debug_take_grouped(uint32_t* v);
hipError_t debug_take_single(uint32_t* v);
#else
#define MOE_DCHECK(cond, bit) true
#define MOE_DEBUG_READER(name)
#endif
// a layout row id (T*topk marks padding; the stages read anything else as padding too)
__device__ __forceinline__ void dcheck_row_id(int v, int TK) { (void)MOE_DCHECK((unsigned)v <= (unsigned)TK, DBG_LAYOUT_ROW); }
// a tile's expert id for a weight address: -1 never reaches here; an id past E reads expert 0
__device__ __forceinline__ int dcheck_expert(int e, int E) { return MOE_DCHECK((unsigned)e < (unsigned)E, DBG_EXPERT) ? e : 0; }

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
  const int32_t* row_of;   // [T*topk] position of each routed row or -1
  uint8_t* rowout;         // [cap*bm, D] stage2 rows (bf16)
  uint8_t* inter;          // [cap*bm, I] intermediate codes
  uint8_t* inter_s;        // [cap*bm, I/32] intermediate scales (fp8 / fp4)
  int2* groups;            // [cap] tile groups (large-batch path)
  int32_t* num_groups;     // [1]
  int2* cgroups;           // [cap] the groups of experts not taken token-major by Stage2
  int32_t* num_cgroups;    // [1]
  int32_t* tile_hot;       // [cap] hot index of each tile's expert, or -1
  int32_t* hot_e;          // [MOE_HOT_MAX] hot experts, then their count at [MOE_HOT_MAX]
  int32_t* hotpos;         // [T, MOE_HOT_MAX] layout row of (token, hot expert) or the zero row
  float* hotw;             // [T, MOE_HOT_MAX] router weight of (token, hot expert) or 0
  uint32_t* hotmask;       // [T] slots whose expert is hot
  uint8_t* hot_out;        // [T, D] bf16 router-weighted sum of the token's hot-expert rows
  float* dbg;              // [cap*bm, 2I] raw gate/up sums (NONE_TEST) or null
  int32_t* sync;           // completion counters of the single-launch path or null
  uint16_t* out;           // [T, D] bf16
  int T, topk, E, D, I, cap_tiles, block_m, a_dtype, act;
  float beta, linear_beta;
  int stages;              // bit 0: stage1, bit 1: stage2 + finalize
};

hipError_t launch_fused(const FusedArgs& a, hipStream_t s);

// Large-batch stages (moe_gemm_grouped.hip): tile groups of one expert, LDS-tiled GEMMs.
// The tile groups are built with Stage1, so Stage2 takes the grouped path only where Stage1 does.
bool tiled_path_supported(const FusedArgs& a);
// Whether the large-batch Stage2 takes the hot experts token-major (then the combine adds hot_out).
bool hot_path(const FusedArgs& a);
hipError_t launch_tiled(const FusedArgs& a, int2* groups, int32_t* ngroups, hipStream_t s);
constexpr int TILED_MIN_TOKENS_S1 = 2048;   // Stage1 from this batch size
constexpr int TILED_MIN_TOKENS_S2 = 2048;   // Stage2 from this batch size
static_assert(TILED_MIN_TOKENS_S1 <= TILED_MIN_TOKENS_S2, "Stage2 reads Stage1's tile groups");

// Stage1 weights [E, 2I, D/2] and Stage2 weights [E, D, I/2] row-major -> the packed layout of
// moe_pack.hip (same size).
hipError_t launch_pack_w1(const uint8_t* w1, uint8_t* out, int E, int D, int I, hipStream_t s);
hipError_t launch_pack_w2(const uint8_t* w2, uint8_t* out, int E, int D, int I, hipStream_t s);

// Single-launch path (moe_single.hip): Stage1, Stage2 and the combine in one grid whose
// workgroups signal each other through the layout's sync words.
hipError_t launch_single(const FusedArgs& a, hipStream_t s);

// Word offsets inside the sync array.  Every counter has a 64-byte line of its own: device-scope
// atomics on one line are serialized (about 11 ns each on gfx950), whatever word they touch.
//   line 0               word 0: sticky timeout flag
//   lines 1 .. cap       Stage1 items finished, per tile
//   next cap lines       Stage2 items finished, per tile
//   next 16*T lines      (row, column block) pairs finished, per (token, column class)
constexpr int64_t SYNC_LINE = 16;
constexpr int64_t SYNC_ERR = 0;
__host__ __device__ inline int64_t sync_done1(int64_t cap, int64_t tile) { (void)cap; return SYNC_LINE * (1 + tile); }
__host__ __device__ inline int64_t sync_done2(int64_t cap, int64_t tile) { return SYNC_LINE * (1 + cap + tile); }
__host__ __device__ inline int64_t sync_token(int64_t cap, int64_t t, int cls) {
  return SYNC_LINE * (1 + 2 * cap + (int64_t)MOE_SYNC_CLASSES * t + cls);
}

}  // namespace moe
