// Per-stage kernels of the fused MXFP4 MoE (one launch per stage) and the dispatch between
// them, the large-batch tiled stages and the single-launch kernel.  The work items themselves
// (Stage1 with the SiTUv2 / SiLU epilogue, Stage2 with the router-weight scaling, the combine)
// are the shared device functions of moe_stage_items.h.
//
// Combine kernel: thread = 8 consecutive columns of one token; it sums that token's routed-row
// outputs (found through the sort's inverse map row_of) in ascending k and rounds to bf16.
#include "moe_kernels.h"
#include "moe_stage_items.h"

namespace moe {

namespace {

constexpr int THREADS = ITEM_THREADS;
constexpr int NWAVES = ITEM_WAVES;

// ---------------------------------------------------------------- Stage1

template <int ADT, int BM, int NI, int KW, int PF, int MINW, int ACT>
__global__ __launch_bounds__(KW * WAVE, MINW) void stage1_kernel(FusedArgs p, int n_nblk) {
  __shared__ float red[KW][BM][2 * NI + 1];
  const int tile = blockIdx.x / n_nblk;
  const int nb = blockIdx.x - tile * n_nblk;
  stage1_item<ADT, BM, NI, KW, PF, ACT, false>(p, tile, nb, red);
}

// ---------------------------------------------------------------- Stage2
//
// Workgroup (tile, column block nb): blockIdx = nb * cap + tile, so the tiles of one column
// block run together.

template <int ADT, int BM, int NF, int PF, int MINW>
__global__ __launch_bounds__(THREADS, MINW) void stage2_kernel(FusedArgs p, int cap) {
  const int tile = blockIdx.x % cap;
  const int nb = blockIdx.x / cap;
  stage2_item<ADT, BM, NF, PF, false>(p, tile, nb, [] {});
}

// ---------------------------------------------------------------- combine
//
// out[t, c] = sum over k (ascending) of rowout[row_of[t*topk + k], c], in fp32, rounded to
// bf16.  Thread = 8 consecutive columns of one token; rows of non-local experts (-1) are skipped.

template <bool F32>
__global__ __launch_bounds__(THREADS) void combine_kernel(const uint8_t* __restrict__ rowout,
                                                          const int32_t* __restrict__ row_of,
                                                          uint16_t* __restrict__ out, int T, int topk,
                                                          int D) {
  const int groups = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * THREADS + threadIdx.x;
  if (idx >= (int64_t)T * groups) return;
  const int t = (int)(idx / groups), c = (int)(idx - (int64_t)t * groups) * 8;
  float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // all row indices of a group of KG slots first, then all their row loads, then the sums
  constexpr int KG = 8;
  for (int k0 = 0; k0 < topk; k0 += KG) {
    int r[KG];
#pragma unroll
    for (int u = 0; u < KG; ++u) r[u] = k0 + u < topk ? row_of[(int64_t)t * topk + k0 + u] : -1;
    if (F32) {
      float4 a[KG], b[KG];
#pragma unroll
      for (int u = 0; u < KG; ++u) {
        if (r[u] >= 0) {
          const float4* src = reinterpret_cast<const float4*>(rowout + ((size_t)r[u] * D + c) * 4);
          a[u] = src[0];
          b[u] = src[1];
        } else {
          a[u] = b[u] = float4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int u = 0; u < KG; ++u) {
        sum[0] += a[u].x; sum[1] += a[u].y; sum[2] += a[u].z; sum[3] += a[u].w;
        sum[4] += b[u].x; sum[5] += b[u].y; sum[6] += b[u].z; sum[7] += b[u].w;
      }
    } else {
      uint4 q[KG];
#pragma unroll
      for (int u = 0; u < KG; ++u)
        q[u] = r[u] >= 0 ? *reinterpret_cast<const uint4*>(rowout + ((size_t)r[u] * D + c) * 2)
                         : uint4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < KG; ++u) {
        const uint32_t w[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          sum[2 * h] += __uint_as_float(w[h] << 16);
          sum[2 * h + 1] += __uint_as_float(w[h] & 0xFFFF0000u);
        }
      }
    }
  }
  uint4 o;
  o.x = (uint32_t)f32_to_bf16_rne(sum[0]) | ((uint32_t)f32_to_bf16_rne(sum[1]) << 16);
  o.y = (uint32_t)f32_to_bf16_rne(sum[2]) | ((uint32_t)f32_to_bf16_rne(sum[3]) << 16);
  o.z = (uint32_t)f32_to_bf16_rne(sum[4]) | ((uint32_t)f32_to_bf16_rne(sum[5]) << 16);
  o.w = (uint32_t)f32_to_bf16_rne(sum[6]) | ((uint32_t)f32_to_bf16_rne(sum[7]) << 16);
  *reinterpret_cast<uint4*>(out + (size_t)t * D + c) = o;
}

// Stage tiling per activation dtype and block_m.
template <int ADT, int BM>
struct Cfg {
  static constexpr int NI = ADT == DT_BF16 ? 16 : 32;         // intermediate columns / workgroup
  static constexpr int KW = 4;                                // waves splitting K in stage1
  static constexpr int PF1 = (ADT == DT_BF16 && BM == 16) ? 7 : 4;   // K steps in flight per wave
  static constexpr int MINW1 = 2;                               // waves per SIMD kept
  static constexpr int NF2 = BM == 16 ? 4 : 2;                // stage2 16-column fragments / wave
  static constexpr int PF2 = 3;                               // K steps in flight (I = 384: all)
  static constexpr int MINW2 = 2;
};

template <int ADT, int BM>
hipError_t run_stages(FusedArgs a, hipStream_t s) {
  using C = Cfg<ADT, BM>;
  const int n1 = a.I / C::NI;
  const unsigned grid1 = (unsigned)((int64_t)a.cap_tiles * n1);
  const int n2 = (a.D + NWAVES * C::NF2 * 16 - 1) / (NWAVES * C::NF2 * 16);
  constexpr int T1 = C::KW * WAVE;
  if (ADT != DT_BF16 && a.T >= TILED_MIN_TOKENS && tiled_path_supported(a)) {
    hipError_t err = launch_tiled(a, a.groups, a.num_groups, s);
    if (err != hipSuccess || !(a.stages & 2)) return err;
  } else if (a.stages & 1) {
    if (a.act == ACT_SITUV2)
      stage1_kernel<ADT, BM, C::NI, C::KW, C::PF1, C::MINW1, ACT_SITUV2><<<grid1, T1, 0, s>>>(a, n1);
    else if (a.act == ACT_SILU)
      stage1_kernel<ADT, BM, C::NI, C::KW, C::PF1, C::MINW1, ACT_SILU><<<grid1, T1, 0, s>>>(a, n1);
    else
      stage1_kernel<ADT, BM, C::NI, C::KW, C::PF1, C::MINW1, ACT_NONE><<<grid1, T1, 0, s>>>(a, n1);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (!(a.stages & 2) || a.act == ACT_NONE) return hipSuccess;
  if (!(ADT != DT_BF16 && a.T >= TILED_MIN_TOKENS && tiled_path_supported(a))) {
    const unsigned grid2 = (unsigned)((int64_t)a.cap_tiles * n2);
    stage2_kernel<ADT, BM, C::NF2, C::PF2, C::MINW2><<<grid2, THREADS, 0, s>>>(a, a.cap_tiles);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int64_t nthreads = (int64_t)a.T * (a.D / 8);
  const unsigned gridc = (unsigned)((nthreads + THREADS - 1) / THREADS);
  if (ADT == DT_BF16)
    combine_kernel<true><<<gridc, THREADS, 0, s>>>(a.rowout, a.row_of, a.out, a.T, a.topk, a.D);
  else
    combine_kernel<false><<<gridc, THREADS, 0, s>>>(a.rowout, a.row_of, a.out, a.T, a.topk, a.D);
  return hipGetLastError();
}

template <int ADT>
hipError_t run_dtype(const FusedArgs& a, hipStream_t s) {
  return a.block_m == 16 ? run_stages<ADT, 16>(a, s) : run_stages<ADT, 32>(a, s);
}

}  // namespace

hipError_t launch_fused(const FusedArgs& a, hipStream_t s) {
  return a.a_dtype == DT_BF16 ? run_dtype<DT_BF16>(a, s)
         : a.a_dtype == DT_FP8 ? run_dtype<DT_FP8>(a, s)
                               : run_dtype<DT_FP4>(a, s);
}

}  // namespace moe
