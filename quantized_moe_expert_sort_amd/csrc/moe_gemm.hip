// Per-stage kernels of the fused MXFP4 MoE (one launch per stage) and the dispatch between
// them, the large-batch tiled stages and the single-launch kernel.  The work items themselves
// (Stage1 with the SiTUv2 / SiLU epilogue, Stage2 with the router-weight scaling, the combine)
// are the shared device functions of moe_stage_items.h.
//
// Combine kernel: thread = 8 consecutive columns of one token; it sums that token's routed-row
// outputs (found through the sort's inverse map row_of) in ascending k and rounds to bf16.
#include <type_traits>

#include "moe_kernels.h"

#pragma clang diagnostic ignored "-Winline-asm"   // m0 is written by the load-to-LDS copies
#include "moe_stage_items.h"

namespace moe {

namespace {

constexpr int THREADS = ITEM_THREADS;
constexpr int NWAVES = ITEM_WAVES;

// ---------------------------------------------------------------- Stage1

template <int ADT, int BM, int NI, int KW, int PF, int MINW, int ACT, bool LDSA>
__global__ __launch_bounds__(KW * WAVE, MINW) void stage1_kernel(FusedArgs p, int n_nblk) {
  __shared__ float red[KW][BM][2 * NI + 1];
  __shared__ __attribute__((aligned(16))) uint8_t astage[LDSA ? KW * AStage<ADT, PF>::BYTES : 16];
  const int tile = blockIdx.x / n_nblk;
  const int nb = blockIdx.x - tile * n_nblk;
  stage1_item<ADT, BM, NI, KW, PF, ACT, false, LDSA>(p, tile, nb, red, astage);
}

// ---------------------------------------------------------------- Stage2
//
// Workgroup (tile, column block nb): blockIdx = nb * cap + tile, so the tiles of one column
// block run together.

template <int ADT, int BM, int NF, int PF, int MINW, bool LDSA>
__global__ __launch_bounds__(THREADS, MINW) void stage2_kernel(FusedArgs p, int cap) {
  __shared__ __attribute__((aligned(16))) uint8_t astage[LDSA ? S2Stage<ADT, BM>::BYTES : 16];
  const int tile = blockIdx.x % cap;
  const int nb = blockIdx.x / cap;
  auto none = [] {};
  stage2_item<ADT, BM, NF, PF, false, decltype(none)&, LDSA>(p, tile, nb, none, astage);
}

// ---------------------------------------------------------------- combine
//
// out[t, c] = sum over k (ascending) of rowout[row_of[t*topk + k], c], in fp32, rounded to
// bf16.  Thread = 8 consecutive columns of one token; rows of non-local experts (-1) are skipped.
// W: the rows were stored without the router weight (grouped Stage2); each is multiplied by
// topk_w[t*topk + k] in fp32 before it is added.  hot_e (with W, may be null): when it lists hot
// experts, a token's slots in hotmask[t] were summed token-major into hot_out[t] (router weight
// applied); the sum then starts from that row and skips those slots.

template <bool W = false>
__global__ __launch_bounds__(THREADS) void combine_kernel(const uint8_t* __restrict__ rowout,
                                                          const int32_t* __restrict__ row_of,
                                                          uint16_t* __restrict__ out, int T, int topk,
                                                          int D, const float* __restrict__ topk_w = nullptr,
                                                          const int32_t* __restrict__ hot_e = nullptr,
                                                          const uint32_t* __restrict__ hotmask = nullptr,
                                                          const uint8_t* __restrict__ hot_out = nullptr) {
  const int groups = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * THREADS + threadIdx.x;
  if (idx >= (int64_t)T * groups) return;
  const int t = (int)(idx / groups), c = (int)(idx - (int64_t)t * groups) * 8;
  float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  uint32_t hmask = 0;
  if (W && hot_e && hot_e[MOE_HOT_MAX] > 0) {
    hmask = hotmask[t];
    if (hmask) {
      const uint4 q = *reinterpret_cast<const uint4*>(hot_out + ((size_t)t * D + c) * 2);
      const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        sum[2 * h] = __uint_as_float(w4[h] << 16);
        sum[2 * h + 1] = __uint_as_float(w4[h] & 0xFFFF0000u);
      }
    }
  }
  // all row indices of a group of KG slots first, then all their row loads, then the sums
  constexpr int KG = 8;
  for (int k0 = 0; k0 < topk; k0 += KG) {
    int r[KG];
#pragma unroll
    for (int u = 0; u < KG; ++u)
      r[u] = k0 + u < topk && !((hmask >> (k0 + u)) & 1u) ? row_of[(int64_t)t * topk + k0 + u] : -1;
    uint4 q[KG];
    float wk[KG];
#pragma unroll
    for (int u = 0; u < KG; ++u) {
      q[u] = r[u] >= 0 ? *reinterpret_cast<const uint4*>(rowout + ((size_t)r[u] * D + c) * 2)
                       : uint4{0u, 0u, 0u, 0u};
      if (W) wk[u] = r[u] >= 0 ? topk_w[(int64_t)t * topk + k0 + u] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < KG; ++u) {
      const uint32_t w[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (W) {
          sum[2 * h] += wk[u] * __uint_as_float(w[h] << 16);
          sum[2 * h + 1] += wk[u] * __uint_as_float(w[h] & 0xFFFF0000u);
        } else {
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

// ---------------------------------------------------------------- Stage2 + combine, small batches
//
// For at most SMALL_ROWS routed rows (decode), one kernel does Stage2 and the combine: workgroup
// nb owns output columns [16 nb, 16 nb + 16) of every token.  Its sixteen waves take the layout's
// tiles round robin (a non-empty expert has at least one row per tile, so at most SMALL_ROWS
// tiles are in use and a wave has at most two; their expert ids are read together, and the
// tiles past num_tiles carry expert -1, so num_tiles itself is never waited for); for each
// tile a wave computes the 16 x 16 block (tile rows x the block's
// columns) with exactly the MFMA sequence of stage2_item (same operands, K steps ascending),
// scales it by the router weight and rounds it to bf16 as stage2_item stores it, into slot
// [t*topk + k] of an LDS array.  The token sums then run
// over k ascending with 0 for non-local rows, as the combine kernel does: the output has the
// same bits as Stage2 + combine, without the per-row buffer or the extra launch.

// A wave walks its tiles one at a time, which loses to Stage2 + combine once it has several.
constexpr int SMALL_ROWS = 32;
constexpr int SMALL_THREADS = 1024;
constexpr int SMALL_WAVES = SMALL_THREADS / WAVE;
constexpr int SMALL_TPW = SMALL_ROWS / SMALL_WAVES;   // tiles per wave
static_assert(SMALL_ROWS % SMALL_WAVES == 0, "every tile in use belongs to one wave");

template <int ADT, int BM, int PF>
__global__ __launch_bounds__(SMALL_THREADS) void stage2_small_kernel(FusedArgs p) {
  constexpr int MF = BM / 16;
  __shared__ float vals[SMALL_ROWS][16];
  const int nb = blockIdx.x;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / WAVE);   // wave-uniform
  const int r16 = lane & 15, g = lane >> 4;
  const int TK = p.T * p.topk, D = p.D, I = p.I, S = I / 128;
  for (int i = threadIdx.x; i < TK * 16; i += SMALL_THREADS) (&vals[0][0])[i] = 0.f;
  __syncthreads();

  const size_t a_row = (size_t)I * row_bytes_num<ADT>() / row_bytes_den<ADT>();
  // expert ids and row ids of every tile of this wave, requested together
  int eid[SMALL_TPW], vrq[SMALL_TPW][MF], vrowq[SMALL_TPW][MF][4];
#pragma unroll
  for (int q = 0; q < SMALL_TPW; ++q) {   // unconditional loads (a tile past cap reads the last)
    const int tile = min(wave + SMALL_WAVES * q, p.cap_tiles - 1);
    eid[q] = p.expert_ids[tile];
#pragma unroll
    for (int f = 0; f < MF; ++f) {
      vrq[q][f] = p.sorted_ids[tile * BM + 16 * f + r16];
#pragma unroll
      for (int i = 0; i < 4; ++i) vrowq[q][f][i] = p.sorted_ids[tile * BM + 16 * f + 4 * g + i];
    }
  }
#pragma unroll
  for (int q = 0; q < SMALL_TPW; ++q)
    if (wave + SMALL_WAVES * q >= p.cap_tiles) eid[q] = -1;
#pragma unroll
  for (int q = 0; q < SMALL_TPW; ++q) {
    const int tile = wave + SMALL_WAVES * q;
    const int e = eid[q];
    if (e < 0 || e >= p.E) continue;
    int vr[MF], vrow[MF][4];
#pragma unroll
    for (int f = 0; f < MF; ++f) {
      vr[f] = vrq[q][f];
#pragma unroll
      for (int i = 0; i < 4; ++i) vrow[f][i] = vrowq[q][f][i];
    }
    // router weights of the accumulator rows, requested with the operands
    float wv[MF][4];
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[f][i] = (unsigned)vrow[f][i] < (unsigned)TK ? p.topk_w[vrow[f][i]] : 0.f;
    const uint8_t* arow[MF];
    const uint8_t* asrow[MF];
    bool aval[MF];
#pragma unroll
    for (int f = 0; f < MF; ++f) {
      const size_t R = (size_t)tile * BM + 16 * f + r16;
      aval[f] = (unsigned)vr[f] < (unsigned)TK;
      arow[f] = p.inter + R * a_row;
      asrow[f] = ADT == DT_BF16 ? nullptr : p.inter_s + R * (I / 32);
    }
    const size_t wr = (size_t)e * D + nb * 16 + r16;
    const uint8_t* brow = p.w2 + wr * (I / 2);
    const uint8_t* bsrow = p.w2s + wr * (I / 32);
    v4f acc[MF];
#pragma unroll
    for (int f = 0; f < MF; ++f) acc[f] = v4f{0.f, 0.f, 0.f, 0.f};
    // scales and intermediate rows first, weights last: the MFMAs of step i wait only for the
    // weights of steps <= i (loads complete in order)
    auto chunk = [&](int s0, auto full) {
      constexpr bool FULL = decltype(full)::value;
      uint4 bq[PF];
      ScaleQuads<PF> bsq;
      AOperand<ADT> A[PF][MF];
      ScaleQuads<PF> asq[MF];
      bsq.load(bsrow, s0, S, g, true);
#pragma unroll
      for (int f = 0; f < MF; ++f)
        if (ADT != DT_BF16) asq[f].load(asrow[f], s0, S, g, aval[f]);
#pragma unroll
      for (int i = 0; i < PF; ++i)
        if (FULL || s0 + i < S)
#pragma unroll
          for (int f = 0; f < MF; ++f) A[i][f].load(arow[f], s0 + i, g, aval[f]);
#pragma unroll
      for (int i = 0; i < PF; ++i)
        if (FULL || s0 + i < S) bq[i] = ld16(brow + (s0 + i) * 64 + 16 * g);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        if (FULL || s0 + i < S) {
          const uint32_t bs = bsq.get(i, r16, g);
#pragma unroll
          for (int f = 0; f < MF; ++f) {
            const uint32_t as = ADT == DT_BF16 ? 0u : asq[f].get(i, r16, g);
            acc[f] = A[i][f].mma(bq[i], bs, as, acc[f]);
          }
        }
      }
    };
    int s0 = 0;
    for (; s0 + PF <= S; s0 += PF) chunk(s0, std::true_type{});
    if (s0 < S) chunk(s0, std::false_type{});
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = vrow[f][i];
        if ((unsigned)v < (unsigned)TK) {
          const float o = acc[f][i] * wv[f][i];
          vals[v][r16] = __uint_as_float((uint32_t)f32_to_bf16_rne(o) << 16);
        }
      }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < p.T * 16; idx += SMALL_THREADS) {
    const int t = idx >> 4, c = idx & 15;
    float sum = 0.f;
    for (int k = 0; k < p.topk; ++k) sum += vals[t * p.topk + k][c];
    p.out[(size_t)t * D + nb * 16 + c] = f32_to_bf16_rne(sum);
  }
}

// Stage tiling per activation dtype and block_m.
template <int ADT, int BM>
struct Cfg {
  // intermediate columns / workgroup: wider at 32-row tiles, where the re-reads of the gathered
  // activation rows by the workgroups of one tile dominate (fp8/fp4: 64, 3% faster at 1024
  // tokens; bf16: 32, Stage1 30% faster at 8192 tokens); slower at 16-row tiles
  static constexpr int NI = BM == 32 ? (ADT == DT_BF16 ? 32 : 64) : (ADT == DT_BF16 ? 16 : 32);
  static constexpr int KW = 4;                                // waves splitting K in stage1
  // K steps in flight per wave (the bf16 operands are 4x the fp4 ones in registers; at 64
  // columns fp8 keeps 2 (3: 272 -> 409 us at 1024 tokens), fp4 takes 3 (468 -> 447 us fused))
  static constexpr int PF1 = BM == 16 ? 7 : (ADT == DT_FP4 && NI == 64 ? 3 : (ADT == DT_BF16 || NI == 64 ? 2 : 4));
  static constexpr int MINW1 = 2;                               // waves per SIMD kept
  // activation rows staged in LDS (fp8 measured faster with its rows in registers)
  static constexpr bool LDSA = BM == 16 && ADT != DT_FP8;
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
  const bool tiled = tiled_path_supported(a);
  const bool tiled1 = tiled && a.T >= TILED_MIN_TOKENS_S1, tiled2 = tiled && a.T >= TILED_MIN_TOKENS_S2;
  if (tiled1 || (tiled2 && !(a.stages & 1))) {
    FusedArgs t = a;
    t.stages = a.stages & ((tiled1 ? 1 : 0) | (tiled2 ? 2 : 0));
    hipError_t err = launch_tiled(t, a.groups, a.num_groups, s);
    if (err != hipSuccess || !(a.stages & 2)) return err;
  } else if (a.stages & 1) {
    // the staged copies address x with 32-bit offsets
    if (C::LDSA && (int64_t)a.T * a.D * 2 < ((int64_t)1 << 31)) {
      if (a.act == ACT_SITUV2)
        stage1_kernel<ADT, BM, C::NI, C::KW, C::PF1, C::MINW1, ACT_SITUV2, C::LDSA><<<grid1, T1, 0, s>>>(a, n1);
      else if (a.act == ACT_SILU)
        stage1_kernel<ADT, BM, C::NI, C::KW, C::PF1, C::MINW1, ACT_SILU, C::LDSA><<<grid1, T1, 0, s>>>(a, n1);
      else
        stage1_kernel<ADT, BM, C::NI, C::KW, C::PF1, C::MINW1, ACT_NONE, C::LDSA><<<grid1, T1, 0, s>>>(a, n1);
    } else {
      if (a.act == ACT_SITUV2)
        stage1_kernel<ADT, BM, C::NI, C::KW, C::PF1, C::MINW1, ACT_SITUV2, false><<<grid1, T1, 0, s>>>(a, n1);
      else if (a.act == ACT_SILU)
        stage1_kernel<ADT, BM, C::NI, C::KW, C::PF1, C::MINW1, ACT_SILU, false><<<grid1, T1, 0, s>>>(a, n1);
      else
        stage1_kernel<ADT, BM, C::NI, C::KW, C::PF1, C::MINW1, ACT_NONE, false><<<grid1, T1, 0, s>>>(a, n1);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (!(a.stages & 2) || a.act == ACT_NONE) return hipSuccess;
  if ((int64_t)a.T * a.topk <= SMALL_ROWS && a.D % 16 == 0) {
    stage2_small_kernel<ADT, BM, C::PF2><<<(unsigned)(a.D / 16), SMALL_THREADS, 0, s>>>(a);
    return hipGetLastError();
  }
  if (!tiled2) {
    const unsigned grid2 = (unsigned)((int64_t)a.cap_tiles * n2);
    // staged intermediate rows: the whole K in one chunk, 32-bit copy offsets
    const int64_t rb = (int64_t)a.I * row_bytes_num<ADT>() / row_bytes_den<ADT>();
    if (a.I <= S2_I_MAX && a.I <= 128 * C::PF2 && (int64_t)a.cap_tiles * BM * rb < ((int64_t)1 << 31))
      stage2_kernel<ADT, BM, C::NF2, C::PF2, C::MINW2, true><<<grid2, THREADS, 0, s>>>(a, a.cap_tiles);
    else
      stage2_kernel<ADT, BM, C::NF2, C::PF2, C::MINW2, false><<<grid2, THREADS, 0, s>>>(a, a.cap_tiles);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int64_t nthreads = (int64_t)a.T * (a.D / 8);
  const unsigned gridc = (unsigned)((nthreads + THREADS - 1) / THREADS);
  if (tiled2)   // grouped Stage2 rows carry no router weight
    combine_kernel<true><<<gridc, THREADS, 0, s>>>(a.rowout, a.row_of, a.out, a.T, a.topk, a.D, a.topk_w,
                                                   hot_path(a) ? a.hot_e : nullptr, a.hotmask, a.hot_out);
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
