// Per-stage kernels of the fused MXFP4 MoE (one launch per stage) and the dispatch between
// them, the large-batch tiled stages and the single-launch kernel.  The work items themselves
// (Stage1 with the SiTUv2 / SiLU epilogue, Stage2 with the router-weight scaling, the combine)
// are the shared device functions of moe_stage_items.h.
//
// Combine kernel: thread = 8 consecutive columns of one token; it sums that token's routed-row
// outputs (found through the sort's inverse map row_of) in ascending k and rounds to bf16.  Each
// per-row output is read once, a wave reading 1 KB of one row, with the non-temporal hint
// (ldw16): 16% faster at 8192 tokens.
#include <type_traits>

#include "moe_kernels.h"

#pragma clang diagnostic ignored "-Winline-asm"   // m0 is written by the load-to-LDS copies
#include "moe_stage_items.h"

namespace moe {

namespace {

constexpr int THREADS = ITEM_THREADS;
constexpr int NWAVES = ITEM_WAVES;

// ---------------------------------------------------------------- Stage1

// Workgroup b runs on XCD b % 8 (workgroups are dealt to the eight XCDs round robin).  With
// r = b / 8, it takes column block r % n_nblk of tile (r / n_nblk) * 8 + b % 8: the column blocks
// of a tile are consecutive workgroups of one XCD, so the tile's gathered activation rows are
// fetched into one L2 and re-read from there.  The grid covers cap_tiles rounded up to 8.
template <int ADT, int BM, int NI, int KW, int PF, int MINW, int ACT, bool LDSA>
__global__ __launch_bounds__(KW * WAVE, MINW) void stage1_kernel(FusedArgs p, int n_nblk) {
  __shared__ float red[KW][BM][2 * NI + 1];
  __shared__ __attribute__((aligned(16))) uint8_t astage[LDSA ? KW * AStage<ADT, PF>::BYTES : 16];
  const int xcd = blockIdx.x & 7, r = blockIdx.x >> 3;
  const int tq = r / n_nblk;
  const int tile = tq * 8 + xcd, nb = r - tq * n_nblk;
  if (tile >= p.cap_tiles) return;
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
                                                          int D, int64_t n_rows,
                                                          const float* __restrict__ topk_w = nullptr,
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
      const uint4 q = ldw16(hot_out + ((size_t)t * D + c) * 2);
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
#pragma unroll
    for (int u = 0; u < KG; ++u)
      if (!MOE_DCHECK(r[u] >= -1 && r[u] < n_rows, DBG_COMBINE_ROW)) r[u] = -1;
    uint4 q[KG];
    float wk[KG];
#pragma unroll
    for (int u = 0; u < KG; ++u) {
      q[u] = r[u] >= 0 ? ldw16(rowout + ((size_t)r[u] * D + c) * 2) : uint4{0u, 0u, 0u, 0u};
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
// tiles round robin, TPW tiles each (a non-empty expert has at least one routed row per tile, so
// at most T*topk tiles are in use; tiles past num_tiles carry expert -1, so num_tiles itself is
// never read).  A wave issues all of its memory traffic before its first MFMA: it copies the
// intermediate rows of its tiles' routed rows into LDS (one slot per flat row index t*topk + k,
// written and read by this wave only) and loads the weight bytes and scales of all its tiles into
// registers, for SMALL_PS K steps at a time.  For each tile it then computes the 16 x 16 block
// (tile rows x the block's columns) with the MFMA sequence of stage2_item (same operands, K steps
// ascending) and keeps the fp32 sums in LDS.  The token sums run over k ascending: each routed
// row's sum times its router weight, rounded to bf16 as stage2_item stores it, and nothing for
// rows of non-local experts, as the combine kernel adds them: the output has the same bits as
// Stage2 + combine, without the per-row buffer or the extra launch.

constexpr int SMALL_ROWS = 32;
constexpr int SMALL_PS = 3;                           // K steps per pass (inter_dim 384: one pass)

// wait_vm<STEP * n> for a wave-uniform n in [0, 1] (the loads of n later tiles still in flight)
template <int STEP>
__device__ __forceinline__ void wait_vm_n(int n) {
  if (n == 0) wait_vm<0>();
  else wait_vm<STEP>();
}

// s_barrier without the vector-memory wait that __syncthreads adds (loads stay in flight)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
}

// NW waves of TPW tiles each (16 x 1 or 16 x 2).  More rows per workgroup measured slower than
// the per-tile Stage2 + combine: at 64 routed rows (dec-4) 16 x 4 took 17.8 us and 8 x 8 20.6 us
// against 15.9 (each workgroup then streams 16-column slices of 64 experts' weights).
template <int ADT, int BM, int NW, int TPW>
__global__ __launch_bounds__(NW * WAVE) void stage2_small_kernel(FusedArgs p) {
  static_assert(TPW <= 2, "wait_vm_n covers two tiles per wave");
  constexpr int MF = BM / 16;
  constexpr int SMALL_WAVES = NW, SMALL_THREADS = NW * WAVE;
  constexpr int NR = SMALL_WAVES * TPW;                                    // rows handled
  constexpr int SB = 128 * row_bytes_num<ADT>() / row_bytes_den<ADT>();   // bytes of one K step
  constexpr int SLOT = SMALL_PS * SB;
  static_assert(SLOT % 16 == 0 && SLOT <= 16 * WAVE, "a row's pass is one copy instruction");
  __shared__ float vals[NR][16];
  __shared__ float wsh[NR];
  __shared__ int written[NR];
  __shared__ __attribute__((aligned(16))) uint8_t arows[NR * SLOT + SB];   // + one zero step
  const int nb = blockIdx.x;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / WAVE);   // wave-uniform
  const int r16 = lane & 15, g = lane >> 4;
  const int TK = p.T * p.topk, D = p.D, I = p.I, S = I / 128;
  uint8_t* const zero_step = arows + NR * SLOT;

  // router weight of routed row threadIdx.x: requested first, needed only for the token sums
  const float wmine = (int)threadIdx.x < TK ? p.topk_w[threadIdx.x] : 0.f;
  // expert ids and row ids of every tile of this wave, requested together
  int eid[TPW], vr[TPW][MF];
#pragma unroll
  for (int q = 0; q < TPW; ++q) {   // unconditional loads (a tile past cap reads the last)
    const int tile = min(wave + SMALL_WAVES * q, p.cap_tiles - 1);
    eid[q] = p.expert_ids[tile];
#pragma unroll
    for (int f = 0; f < MF; ++f) {
      vr[q][f] = p.sorted_ids[tile * BM + 16 * f + r16];
      dcheck_row_id(vr[q][f], TK);
    }
  }
  if ((int)threadIdx.x < NR) written[threadIdx.x] = 0;
  if ((int)threadIdx.x < SB / 4) reinterpret_cast<uint32_t*>(zero_step)[threadIdx.x] = 0u;
  lds_barrier();

  bool tv[TPW];   // wave-uniform: the tile has a local expert
  int ew[TPW];    // its expert, or expert 0 (whose rows then serve as in-bounds stand-ins)
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int tile = wave + SMALL_WAVES * q;
    const int e = __builtin_amdgcn_readfirstlane(eid[q]);
    tv[q] = tile < p.cap_tiles && e >= 0 && e < p.E;
    ew[q] = tv[q] ? e : 0;
  }
  const size_t a_row = (size_t)I * row_bytes_num<ADT>() / row_bytes_den<ADT>();
  const uint32_t lds_rows = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)arows);
  v4f acc[TPW][MF];
#pragma unroll
  for (int q = 0; q < TPW; ++q)
#pragma unroll
    for (int f = 0; f < MF; ++f) acc[q][f] = v4f{0.f, 0.f, 0.f, 0.f};

  auto pass = [&](int s0, auto full) {
    constexpr bool FULL = decltype(full)::value;
    const int n_s = FULL ? SMALL_PS : S - s0;
    // intermediate rows: one copy per routed row, lanes [0, n_s * SB / 16) of the wave
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      if (!tv[q]) continue;
      const int tile = wave + SMALL_WAVES * q;
#pragma unroll
      for (int f = 0; f < MF; ++f) {
        uint64_t m = __ballot((unsigned)vr[q][f] < (unsigned)TK) & 0xFFFFull;   // lanes 0..15: rows 0..15
        while (m) {
          const int l = __ffsll((unsigned long long)m) - 1;
          m &= m - 1ull;
          const int v = __builtin_amdgcn_readlane(vr[q][f], l);
          const uint32_t off = (uint32_t)((size_t)(tile * BM + 16 * f + l) * a_row) + (uint32_t)(s0 * SB + 16 * lane);
          if (lane < n_s * SB / 16) dma16_lds(p.inter, off, lds_rows + (uint32_t)(v * SLOT));
        }
      }
    }
    // scales, then the weights of every tile slot and step, tile after tile; a slot without a
    // local expert loads expert 0's bytes (the same lines for every such slot, served by the L2)
    // so that every wave issues the same loads and a tile's wait below is a fixed count
    ScaleQuads<SMALL_PS> bsq[TPW];
    ScaleQuads<SMALL_PS> asq[TPW][MF];
    uint4 bq[TPW][SMALL_PS];
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      const size_t wr = (size_t)ew[q] * D + nb * 16 + r16;
      bsq[q].load(p.w2s + wr * (I / 32), s0, s0 + n_s, g, tv[q]);
#pragma unroll
      for (int f = 0; f < MF; ++f)
        if (ADT != DT_BF16) {
          const size_t R = (size_t)(wave + SMALL_WAVES * q) * BM + 16 * f + r16;
          asq[q][f].load(p.inter_s + R * (I / 32), s0, s0 + n_s, g, tv[q] && (unsigned)vr[q][f] < (unsigned)TK);
        }
    }
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      const uint8_t* brow = p.w2 + ((size_t)ew[q] * D + nb * 16) * (I / 2) + 16 * lane;   // packed w2
#pragma unroll
      for (int i = 0; i < SMALL_PS; ++i)
        if (FULL || i < n_s) bq[q][i] = ldw16(brow + (s0 + i) * 1024);
    }
    __builtin_amdgcn_sched_barrier(0);
    auto tile_mfmas = [&](int q) {
      const uint8_t* abase[MF];
      int astep[MF];
#pragma unroll
      for (int f = 0; f < MF; ++f) {
        const int v = vr[q][f];
        const bool in = (unsigned)v < (unsigned)TK;
        abase[f] = in ? arows + v * SLOT : zero_step;
        astep[f] = in ? SB : 0;
      }
#pragma unroll
      for (int i = 0; i < SMALL_PS; ++i) {
        if (FULL || i < n_s) {
          const uint32_t bs = bsq[q].get(i, r16, g);
#pragma unroll
          for (int f = 0; f < MF; ++f) {
            AOperand<ADT> A;
            A.load_lds(abase[f] + i * astep[f], g);
            const uint32_t as = ADT == DT_BF16 ? 0u : asq[q][f].get(i, r16, g);
            acc[q][f] = A.mma(bq[q][i], bs, as, acc[q][f]);
          }
        }
      }
    };
    // loads complete in order: once at most the later tiles' weight loads are outstanding, the
    // copies, the scales and this tile's weights have arrived
    if constexpr (FULL) {
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        wait_vm_n<SMALL_PS>(TPW - 1 - q);
        if (tv[q]) tile_mfmas(q);
      }
    } else {
      wait_vm<0>();
#pragma unroll
      for (int q = 0; q < TPW; ++q)
        if (tv[q]) tile_mfmas(q);
    }
    // every LDS read of this pass is done before the next pass's copies replace the rows
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  int s0 = 0;
  for (; s0 + SMALL_PS <= S; s0 += SMALL_PS) pass(s0, std::true_type{});
  if (s0 < S) pass(s0, std::false_type{});

  // fp32 sums of the routed rows: element i of lane (r16, g) is row 4 g + i of the fragment
#pragma unroll
  for (int q = 0; q < TPW; ++q)
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = __shfl(vr[q][f], 4 * g + i, WAVE);
        if (tv[q] && (unsigned)v < (unsigned)TK) {
          vals[v][r16] = acc[q][f][i];
          if (r16 == 0) written[v] = 1;
        }
      }
  if ((int)threadIdx.x < TK) wsh[threadIdx.x] = wmine;
  __syncthreads();
  for (int idx = threadIdx.x; idx < p.T * 16; idx += SMALL_THREADS) {
    const int t = idx >> 4, c = idx & 15;
    float sum = 0.f;
    for (int k = 0; k < p.topk; ++k) {
      const int v = t * p.topk + k;
      if (written[v]) sum += __uint_as_float((uint32_t)f32_to_bf16_rne(vals[v][c] * wsh[v]) << 16);
    }
    p.out[(size_t)t * D + nb * 16 + c] = f32_to_bf16_rne(sum);
  }
}

template <int ADT, int BM>
hipError_t launch_stage2_small(const FusedArgs& a, hipStream_t s) {
  const int rows = a.T * a.topk;
  const dim3 grid((unsigned)(a.D / 16));
  if (rows <= 16) stage2_small_kernel<ADT, BM, 16, 1><<<grid, 16 * WAVE, 0, s>>>(a);
  else if (rows <= SMALL_ROWS) stage2_small_kernel<ADT, BM, 16, 2><<<grid, 16 * WAVE, 0, s>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
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
  // stage2 16-column fragments / wave (32-row tiles: 4 measured 3% faster than 2 at 1024 tokens
  // with the packed w2)
  static constexpr int NF2 = 4;
  static constexpr int PF2 = 3;                               // K steps in flight (I = 384: all)
  static constexpr int MINW2 = 2;
};

template <int ADT, int BM>
hipError_t run_stages(FusedArgs a, hipStream_t s) {
  using C = Cfg<ADT, BM>;
  const int n1 = a.I / C::NI;
  const unsigned grid1 = (unsigned)((int64_t)(a.cap_tiles + 7) / 8 * 8 * n1);
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
  // the small kernel's copies address the intermediate with 32-bit offsets
  if ((int64_t)a.T * a.topk <= SMALL_ROWS && a.D % 16 == 0 &&
      (int64_t)a.cap_tiles * BM * a.I * 2 < ((int64_t)1 << 31))
    return launch_stage2_small<ADT, BM>(a, s);
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
  const int64_t n_rows = (int64_t)a.cap_tiles * a.block_m;
  const unsigned gridc = (unsigned)((nthreads + THREADS - 1) / THREADS);
  if (tiled2)   // grouped Stage2 rows carry no router weight
    combine_kernel<true><<<gridc, THREADS, 0, s>>>(a.rowout, a.row_of, a.out, a.T, a.topk, a.D, n_rows, a.topk_w,
                                                   hot_path(a) ? a.hot_e : nullptr, a.hotmask, a.hot_out);
  else
    combine_kernel<false><<<gridc, THREADS, 0, s>>>(a.rowout, a.row_of, a.out, a.T, a.topk, a.D, n_rows);
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

MOE_DEBUG_READER(gemm)

}  // namespace moe
