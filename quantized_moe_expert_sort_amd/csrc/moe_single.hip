// Single-launch path of the fused MXFP4 MoE for batches below MOE_SINGLE_LAUNCH_MAX_TOKENS.
//
// Launch boundaries cost several microseconds each on gfx950 (dispatch, the end-of-kernel cache
// release, the next kernel's ramp), which at decode sizes is as long as streaming the touched
// expert weights.  Here one grid holds every work item, in this block order:
//   [zero items]    one per 16 tokens: writes the zero rows of tokens without a local expert;
//   [Stage1 items]  (tile, nb) tile-major, as in the per-stage kernel;
//   [Stage2 items]  (tile, nb) tile-major.
// A Stage2 item issues the loads of its first weight steps, then waits until every Stage1 item
// of its tile has finished, so the down-projection weights stream while Stage1 still runs.
// Workgroups are dispatched in block order, so every Stage1 item has been dispatched before any
// Stage2 item waits for it, and Stage1 items never wait: the waits always end.  Each wait is
// still bounded in time; on expiry it sets the layout's sticky error word and goes on.
//
// Cross-workgroup data (the intermediate rows and the per-row Stage2 outputs) is written with
// device-coherent stores and read with device-coherent loads (sc1: through to / from the
// device coherence point, past the per-XCD L2s), and each producer waits for its stores to
// complete before it bumps a counter with a device-scope atomic.  No device-wide cache
// writeback is needed.  The combine of a token's columns is done by the Stage2 item that
// completes the last of that token's rows for a column class (a last-arriver count per
// (token, class)), with the same arithmetic as the per-stage combine kernel.  Every counter is
// set back to zero by its last user, so the next call finds them cleared.
#include "moe_kernels.h"
#include "moe_stage_items.h"

namespace moe {

namespace {

constexpr int THREADS = ITEM_THREADS;
constexpr int ZERO_TOKENS = 16;                       // tokens per zero item
constexpr uint64_t SPIN_TICKS = 25000000ull;          // s_memrealtime runs at 100 MHz: 0.25 s

template <int ADT, int BM>
struct SCfg {
  static constexpr int NI = ADT == DT_BF16 ? 16 : 32;         // Stage1 intermediate columns / item
  static constexpr int KW = 4;                                // waves splitting K in Stage1
  static constexpr int PF1 = (ADT == DT_BF16 && BM == 16) ? 7 : 4;
  static constexpr int NF2 = ADT == DT_BF16 ? (BM == 16 ? 4 : 2) : (BM == 16 ? 8 : 4);   // Stage2 fragments / wave
  static constexpr int PF2 = 3;
  static constexpr int NO = ITEM_WAVES * NF2 * 16;            // Stage2 output columns / item
};

// Thread 0 waits until *ctr >= target (relaxed device-scope loads, which bypass the
// non-coherent caches); the workgroup then passes a barrier.
__device__ __forceinline__ void wait_count(const int32_t* ctr, int target, int32_t* err) {
  if (threadIdx.x == 0) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (__builtin_amdgcn_s_memrealtime() - t0 > SPIN_TICKS) {
        atomicOr(err, 1);
        break;
      }
    }
  }
  __syncthreads();
}

__device__ __forceinline__ int local_rows(const FusedArgs& p, int t) {
  int n = 0;
  for (int k = 0; k < p.topk; ++k) n += p.row_of[(int64_t)t * p.topk + k] >= 0;
  return n;
}

template <int ADT, int BM, int ACT>
__global__ __launch_bounds__(THREADS, 2) void single_kernel(FusedArgs p, int n1, int n2, int n_zero) {
  using C = SCfg<ADT, BM>;
  __shared__ float red[C::KW][BM][2 * C::NI + 1];
  __shared__ int todo[BM];
  __shared__ int n_todo;
  __shared__ int zflag[ZERO_TOKENS];

  const int64_t cap = p.cap_tiles;
  int32_t* err = p.sync + SYNC_ERR;
  int64_t b = blockIdx.x;

  // ---- zero items: rows of tokens whose every expert is non-local
  if (b < n_zero) {
    const int t0 = (int)b * ZERO_TOKENS;
    if (threadIdx.x < ZERO_TOKENS) {
      const int t = t0 + threadIdx.x;
      zflag[threadIdx.x] = t < p.T && local_rows(p, t) == 0;
    }
    __syncthreads();
    for (int i = 0; i < ZERO_TOKENS; ++i) {
      if (!zflag[i]) continue;
      uint4* row = reinterpret_cast<uint4*>(p.out + (size_t)(t0 + i) * p.D);
      for (int c = threadIdx.x; c < p.D / 8; c += THREADS) row[c] = uint4{0u, 0u, 0u, 0u};
    }
    return;
  }
  b -= n_zero;

  // ---- Stage1 items
  if (b < cap * n1) {
    const int tile = (int)(b / n1), nb = (int)(b - (int64_t)tile * n1);
    if (!stage1_item<ADT, BM, C::NI, C::KW, C::PF1, ACT, true>(p, tile, nb, red)) return;
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) atomicAdd(p.sync + sync_done1(cap, tile), 1);
    return;
  }
  b -= cap * n1;

  // ---- Stage2 items
  const int tile = (int)(b / n2), nb = (int)(b - (int64_t)tile * n2);
  if (threadIdx.x == 0) n_todo = 0;
  if (!stage2_item<ADT, BM, C::NF2, C::PF2, true>(p, tile, nb,
                                                  [&] { wait_count(p.sync + sync_done1(cap, tile), n1, err); }))
    return;
  wait_stores();
  __syncthreads();

  const int cls = nb % MOE_SYNC_CLASSES;
  const int blocks_in_cls = (n2 - cls + MOE_SYNC_CLASSES - 1) / MOE_SYNC_CLASSES;
  if (threadIdx.x < BM) {
    const int v = p.sorted_ids[tile * BM + threadIdx.x];
    if ((unsigned)v < (unsigned)(p.T * p.topk)) {
      const int t = v / p.topk;
      const int target = local_rows(p, t) * blocks_in_cls;
      int32_t* c = p.sync + sync_token(cap, t, cls);
      if (atomicAdd(c, 1) == target - 1) {
        __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        todo[atomicAdd(&n_todo, 1)] = t;
      }
    }
  } else if (threadIdx.x == BM) {
    int32_t* d2 = p.sync + sync_done2(cap, tile);
    if (atomicAdd(d2, 1) == n2 - 1) {
      __hip_atomic_store(p.sync + sync_done1(cap, tile), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(d2, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  const int nt = n_todo;
  for (int i = 0; i < nt; ++i) {
    const int t = todo[i];
    for (int blk = cls; blk < n2; blk += MOE_SYNC_CLASSES)
      combine_token_cols<true>(p, t, blk * C::NO, min((blk + 1) * C::NO, p.D));
  }
}

template <int ADT, int BM>
hipError_t run(const FusedArgs& a, hipStream_t s) {
  using C = SCfg<ADT, BM>;
  const int n1 = a.I / C::NI;
  const int n2 = (a.D + C::NO - 1) / C::NO;
  static_assert(C::NO % 64 == 0 && C::NI <= 128, "");
  const int n_zero = (a.T + ZERO_TOKENS - 1) / ZERO_TOKENS;
  const int64_t grid = n_zero + (int64_t)a.cap_tiles * (n1 + n2);
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (a.act == ACT_SITUV2)
    single_kernel<ADT, BM, ACT_SITUV2><<<(unsigned)grid, THREADS, 0, s>>>(a, n1, n2, n_zero);
  else
    single_kernel<ADT, BM, ACT_SILU><<<(unsigned)grid, THREADS, 0, s>>>(a, n1, n2, n_zero);
  return hipGetLastError();
}

template <int ADT>
hipError_t run_dtype(const FusedArgs& a, hipStream_t s) {
  return a.block_m == 16 ? run<ADT, 16>(a, s) : run<ADT, 32>(a, s);
}

}  // namespace

hipError_t launch_single(const FusedArgs& a, hipStream_t s) {
  if (a.act != ACT_SITUV2 && a.act != ACT_SILU) return hipErrorInvalidValue;
  return a.a_dtype == DT_BF16 ? run_dtype<DT_BF16>(a, s)
         : a.a_dtype == DT_FP8 ? run_dtype<DT_FP8>(a, s)
                               : run_dtype<DT_FP4>(a, s);
}

MOE_DEBUG_READER(single)

}  // namespace moe
