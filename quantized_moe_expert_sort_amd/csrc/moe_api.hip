// extern "C" entry points of libmoe_mi355x.so: argument validation on the host, then the
// kernel launchers.  Nothing here allocates or synchronizes.  State kept between calls: the
// thread-local copy of the last HIP error, and for moe_fused_noalloc the per-device address of
// the library's fixed scratch array (taken once per device).
#include <cmath>
#include <cstdio>
#include <mutex>

#include "moe_kernels.h"

// Workspace of moe_fused_noalloc, for callers that cannot allocate: one copy per device, held
// until the process ends, shared by every call on that device.  In host code this name is only
// a stand-in for the symbol; kernels get the device address noalloc_scratch() takes for the
// current device with hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// Device address of the current device's scratch array (taken once per device, with that
// device current).  On failure returns null and sets *err.
void* noalloc_scratch(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= MAX_DEVICES) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !p) {
      if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

thread_local int32_t g_last_hip_error = 0;

moe_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = (int32_t)e;
  return MOE_ERR_HIP;
}

// The debug build (MOE_DEBUG_CHECKS) ends every launching call by waiting for the device and
// collecting the kernels' violation words; the normal build returns the launch status as is.
moe_status_t finish(moe_status_t st) {
#ifdef MOE_DEBUG_CHECKS
  if (st != MOE_OK) return st;
  hipError_t e = hipDeviceSynchronize();
  uint32_t bits = 0;
  hipError_t (*const take[])(uint32_t*) = {moe::debug_take_sort, moe::debug_take_gemm, moe::debug_take_grouped,
                                           moe::debug_take_single};
  for (auto f : take) {
    uint32_t v = 0;
    if (e == hipSuccess) e = f(&v);
    bits |= v;
  }
  if (e != hipSuccess) return hip_status(e);
  if (bits) {
    fprintf(stderr, "libmoe_mi355x_debug: device index check failed (bits 0x%x)\n", bits);
    return MOE_ERR_DEBUG_CHECK;
  }
#endif
  return st;
}

bool valid_dtype(int32_t dt) { return dt == MOE_DT_BF16 || dt == MOE_DT_FP8_E4M3 || dt == MOE_DT_FP4_E2M1; }

moe_status_t check_layout(const moe_layout_t* L, int32_t tokens, int32_t topk, int32_t E) {
  if (!L || !L->sorted_token_ids || !L->expert_ids || !L->num_tiles) return MOE_ERR_INVALID_ARG;
  if (L->block_m != 16 && L->block_m != 32) return MOE_ERR_UNSUPPORTED;
  if (L->cap_tiles < 0 || L->cap_tiles < moe_cap_tiles(tokens, topk, E, L->block_m)) return MOE_ERR_CAPACITY;
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_last_hip_error(void) { return g_last_hip_error; }

moe_status_t moe_sort(const int32_t* topk_ids, const float* topk_w, int32_t tokens, int32_t topk,
                      int32_t expert_begin, int32_t num_local_experts, const moe_layout_t* layout,
                      void* ws, size_t ws_bytes, void* stream) {
  if (tokens < 0 || topk < 1 || num_local_experts < 1) return MOE_ERR_INVALID_ARG;
  if ((int64_t)tokens * topk >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (num_local_experts > moe::MAX_SORT_EXPERTS) return MOE_ERR_UNSUPPORTED;
  if (tokens > 0 && !topk_ids) return MOE_ERR_INVALID_ARG;
  moe_status_t st = check_layout(layout, tokens, topk, num_local_experts);
  if (st != MOE_OK) return st;
  if (layout->sorted_weights && tokens > 0 && !topk_w) return MOE_ERR_INVALID_ARG;
  const int64_t n = (int64_t)tokens * topk;
  if (n > MOE_SORT_CHUNK) {
    if (!ws) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < moe_sort_ws_bytes(tokens, topk, num_local_experts)) return MOE_ERR_WORKSPACE;
  }
  moe::SortLayout L{layout->sorted_token_ids, layout->sorted_weights, layout->expert_ids,
                    layout->num_tiles, layout->row_of, layout->sync,
                    layout->sync ? (int64_t)moe_sync_words(tokens, layout->cap_tiles) : 0,
                    layout->cap_tiles};
  return finish(hip_status(moe::launch_sort(topk_ids, topk_w, n, expert_begin, num_local_experts,
                                            layout->block_m, L, ws, (hipStream_t)stream)));
}

}  // extern "C"

namespace {

// moe_pack_w1 and moe_pack_w2: the same checks on `rows_per_expert` rows of `k` fp4 values (w1:
// 2I rows of D, w2: D rows of I); the copy reads w and writes w_packed in a different order, so
// the two byte ranges must be disjoint.
moe_status_t check_pack(const uint8_t* w, int32_t num_experts, int32_t model_dim, int32_t inter_dim,
                        const uint8_t* w_packed, int64_t rows_per_expert, int64_t k) {
  if (!w || !w_packed) return MOE_ERR_INVALID_ARG;
  if (num_experts < 1 || model_dim <= 0 || inter_dim <= 0) return MOE_ERR_INVALID_ARG;
  if (model_dim % 128 != 0 || inter_dim % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)num_experts * rows_per_expert * (k / 2) / 16 >= ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
  const uintptr_t bytes = (uintptr_t)num_experts * (uintptr_t)rows_per_expert * (uintptr_t)(k / 2);
  const uintptr_t a = (uintptr_t)w, b = (uintptr_t)w_packed;
  if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_pack_w1(const uint8_t* w1, int32_t num_experts, int32_t model_dim, int32_t inter_dim,
                         uint8_t* w1_packed, void* stream) {
  const moe_status_t st = check_pack(w1, num_experts, model_dim, inter_dim, w1_packed, 2 * (int64_t)inter_dim, model_dim);
  if (st != MOE_OK) return st;
  return finish(hip_status(moe::launch_pack_w1(w1, w1_packed, num_experts, model_dim, inter_dim, (hipStream_t)stream)));
}

moe_status_t moe_pack_w2(const uint8_t* w2, int32_t num_experts, int32_t model_dim, int32_t inter_dim,
                         uint8_t* w2_packed, void* stream) {
  const moe_status_t st = check_pack(w2, num_experts, model_dim, inter_dim, w2_packed, model_dim, inter_dim);
  if (st != MOE_OK) return st;
  return finish(hip_status(moe::launch_pack_w2(w2, w2_packed, num_experts, model_dim, inter_dim, (hipStream_t)stream)));
}

moe_status_t moe_quant_act(const uint16_t* x_bf16, int64_t rows, int64_t cols, int32_t dt, void* q_out,
                           uint8_t* scale_out, void* stream) {
  if (dt != MOE_DT_FP8_E4M3 && dt != MOE_DT_FP4_E2M1) return MOE_ERR_INVALID_ARG;
  if (rows < 0 || cols <= 0 || cols % 32 != 0) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!x_bf16 || !q_out || !scale_out) return MOE_ERR_INVALID_ARG;
  return finish(hip_status(moe::launch_quant_act(x_bf16, rows, cols, dt, q_out, scale_out, (hipStream_t)stream)));
}

}  // extern "C"

namespace {

// moe_fused and moe_fused_noalloc: the same validation and launches; the no-alloc variant takes
// its workspace from the scratch array (scratch == true; ws and ws_bytes are ignored).
moe_status_t fused_call(const void* x, const uint8_t* x_scale, int32_t a_dtype, const uint8_t* w1,
                        int32_t w_layout, const uint8_t* w1_scale, const uint8_t* w2, const uint8_t* w2_scale,
                        const float* topk_w, const moe_layout_t* layout, int32_t tokens, int32_t topk,
                        int32_t num_local_experts, int32_t model_dim, int32_t inter_dim,
                        const moe_act_params_t* act, uint16_t* out_bf16, void* ws, size_t ws_bytes,
                        int32_t stages, void* stream, bool use_scratch) {
  if (!valid_dtype(a_dtype)) return MOE_ERR_INVALID_ARG;
  if (w_layout != MOE_W_PACKED && w_layout != MOE_W1_PACKED && w_layout != MOE_W_ROW_MAJOR) return MOE_ERR_INVALID_ARG;
  if (w_layout != MOE_W_PACKED) return MOE_ERR_UNSUPPORTED;   // the kernels stream packed blocks only
  if (stages != MOE_STAGE_1 && stages != MOE_STAGE_2 && stages != MOE_STAGE_ALL) return MOE_ERR_INVALID_ARG;
  if (!act) return MOE_ERR_INVALID_ARG;
  if (act->act != MOE_ACT_SITUV2 && act->act != MOE_ACT_SILU && act->act != MOE_ACT_NONE_TEST)
    return MOE_ERR_UNSUPPORTED;
  if (act->act == MOE_ACT_SITUV2 &&
      !(std::isfinite(act->beta) && act->beta > 0.f && std::isfinite(act->linear_beta) && act->linear_beta > 0.f))
    return MOE_ERR_INVALID_ARG;
  if (tokens < 0 || topk < 1 || num_local_experts < 1 || model_dim <= 0 || inter_dim <= 0)
    return MOE_ERR_INVALID_ARG;
  if (model_dim % 128 != 0 || inter_dim % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)tokens * topk >= ((int64_t)1 << 31) || (int64_t)tokens * model_dim >= ((int64_t)1 << 31))
    return MOE_ERR_UNSUPPORTED;
  moe_status_t st = check_layout(layout, tokens, topk, num_local_experts);
  if (st != MOE_OK) return st;
  if ((int64_t)layout->cap_tiles * layout->block_m >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (tokens == 0) return MOE_OK;
  if (!x || !w1 || !w1_scale || !w2 || !w2_scale || !topk_w || (!use_scratch && !ws)) return MOE_ERR_INVALID_ARG;
  if ((a_dtype == MOE_DT_BF16) != (x_scale == nullptr)) return MOE_ERR_INVALID_ARG;
  if (act->act != MOE_ACT_NONE_TEST && (stages & MOE_STAGE_2) && (!out_bf16 || !layout->row_of))
    return MOE_ERR_INVALID_ARG;
  const size_t need = moe_fused_ws_bytes(tokens, model_dim, inter_dim, layout->cap_tiles, layout->block_m,
                                         a_dtype, act->act);
  if (use_scratch) {
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    hipError_t err = hipSuccess;
    ws = noalloc_scratch(&err);
    if (!ws) return hip_status(err);
    ws_bytes = MOE_NOALLOC_SCRATCH_BYTES;
  }
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;

  uint8_t* base = (uint8_t*)ws;
  const moe_fused_ws_parts_t W = moe_fused_ws_parts(tokens, model_dim, inter_dim, layout->cap_tiles,
                                                    layout->block_m, a_dtype, act->act);
  const size_t groups_bytes = moe_align256((size_t)layout->cap_tiles * 8);
  moe::FusedArgs a;
  a.x = (const uint8_t*)x;
  a.xs = x_scale;
  a.w1 = w1;
  a.w1s = w1_scale;
  a.w2 = w2;
  a.w2s = w2_scale;
  a.topk_w = topk_w;
  a.sorted_ids = layout->sorted_token_ids;
  a.expert_ids = layout->expert_ids;
  a.num_tiles = layout->num_tiles;
  a.rowout = base + W.rowout;
  a.groups = (int2*)(base + W.groups);
  a.num_groups = (int32_t*)(base + W.groups + groups_bytes);
  a.cgroups = (int2*)(base + W.cgroups);
  a.num_cgroups = (int32_t*)(base + W.cgroups + groups_bytes);
  a.tile_hot = (int32_t*)(base + W.tile_hot);
  a.hot_e = (int32_t*)(base + W.hot_e);
  a.hotpos = (int32_t*)(base + W.hotpos);
  a.hotw = (float*)(base + W.hotw);
  a.hotmask = (uint32_t*)(base + W.hotmask);
  a.hot_out = base + W.hot_out;
  a.row_of = layout->row_of;
  a.inter = base + W.inter;
  a.inter_s = a_dtype == MOE_DT_BF16 ? nullptr : base + W.iscale;
  a.dbg = act->act == MOE_ACT_NONE_TEST ? (float*)(base + W.dbg) : nullptr;
  a.sync = layout->sync;
  a.out = out_bf16;
  a.T = tokens;
  a.topk = topk;
  a.E = num_local_experts;
  a.D = model_dim;
  a.I = inter_dim;
  a.cap_tiles = layout->cap_tiles;
  a.block_m = layout->block_m;
  a.a_dtype = a_dtype;
  a.act = act->act;
  a.beta = act->beta;
  a.linear_beta = act->linear_beta;
  a.stages = stages;
  if (layout->sync && tokens < MOE_SINGLE_LAUNCH_MAX_TOKENS && stages == MOE_STAGE_ALL &&
      act->act != MOE_ACT_NONE_TEST)
    return finish(hip_status(moe::launch_single(a, (hipStream_t)stream)));
  return finish(hip_status(moe::launch_fused(a, (hipStream_t)stream)));
}

}  // namespace

extern "C" {

moe_status_t moe_fused(const void* x, const uint8_t* x_scale, int32_t a_dtype, const uint8_t* w1,
                       int32_t w_layout, const uint8_t* w1_scale, const uint8_t* w2, const uint8_t* w2_scale,
                       const float* topk_w, const moe_layout_t* layout, int32_t tokens, int32_t topk,
                       int32_t num_local_experts, int32_t model_dim, int32_t inter_dim,
                       const moe_act_params_t* act, uint16_t* out_bf16, void* ws, size_t ws_bytes,
                       int32_t stages, void* stream) {
  return fused_call(x, x_scale, a_dtype, w1, w_layout, w1_scale, w2, w2_scale, topk_w, layout, tokens, topk,
                    num_local_experts, model_dim, inter_dim, act, out_bf16, ws, ws_bytes, stages, stream, false);
}

moe_status_t moe_fused_noalloc(const void* x, const uint8_t* x_scale, int32_t a_dtype, const uint8_t* w1,
                               int32_t w_layout, const uint8_t* w1_scale, const uint8_t* w2,
                               const uint8_t* w2_scale, const float* topk_w, const moe_layout_t* layout,
                               int32_t tokens, int32_t topk, int32_t num_local_experts, int32_t model_dim,
                               int32_t inter_dim, const moe_act_params_t* act, uint16_t* out_bf16,
                               int32_t stages, void* stream) {
  return fused_call(x, x_scale, a_dtype, w1, w_layout, w1_scale, w2, w2_scale, topk_w, layout, tokens, topk,
                    num_local_experts, model_dim, inter_dim, act, out_bf16, nullptr, 0, stages, stream, true);
}

}  // extern "C"
