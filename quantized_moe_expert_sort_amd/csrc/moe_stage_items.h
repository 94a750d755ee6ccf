// One work item of each stage of the fused MXFP4 MoE, as device functions shared by the
// per-stage kernels (moe_gemm.hip) and the single-launch kernel (moe_single.hip), so both
// paths compute every output with the same instructions in the same order.
//
// Stage1 item (tile, nb) (github ROCm/aiter PR 6259 "Technical Details": SiTUv2 in the stage1
//   epilogue): block_m sorted rows x NI intermediate columns.  The gate columns [n0, n0+NI)
//   and the matching up columns [I+n0, I+n0+NI) are computed together (NI a multiple of 16, so
//   every 16-row weight fragment is one packed block of gate or of up rows), and g and u of one
//   output element meet in the LDS reduction.  KW waves split the K = model_dim reduction into
//   contiguous ranges of 128-deep steps; each lane streams its weight bytes and its gathered
//   activation row straight from memory into matrix-core operands (every byte is loaded once
//   per item), issuing the loads of PF steps before the first MFMA that uses them; the partial
//   sums meet in LDS.
//   The epilogue applies SiTUv2 or SiLU and re-encodes the intermediate: bf16, or fp8 / fp4 with
//   one e8m0 scale per 32 columns (the 32 columns of a block are 32 lanes of one wave).
// Stage2 item (tile, nb) (PR 5118 review items 9-10: bf16 x MXFP4 stage2 with a per-token
//   scatter of the weighted rows): block_m rows x 64*NF output columns (the last block of a row
//   may be partial); each wave owns 16*NF columns over the whole K = inter_dim.  The fp32 result
//   row is scaled by the router weight of its routed row and stored, rounded to bf16, as that
//   routed row's output.
// Combine: each token's routed-row outputs summed in ascending k in fp32, rounded to bf16.
#pragma once

#include <stdint.h>
#include <type_traits>

#include "moe_kernels.h"
#include "moe_operands.h"

namespace moe {

constexpr int ITEM_THREADS = 256;
constexpr int ITEM_WAVES = ITEM_THREADS / WAVE;

// 16 bytes per lane copied from global (base + off) straight to LDS (lds + 16 * lane); base and
// lds are wave-uniform.  The copy is counted by vmcnt like any vector load.
__device__ __forceinline__ void dma16_lds(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}

// Wait until at most N of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Activations of a 16-row tile with few routed rows (decode and mid batches): instead of every
// lane group loading its 16-byte pieces of the gathered rows into registers (partial-wave loads:
// 28 per bf16 row and K range), each wave copies the K range of up to NV routed rows into LDS
// with whole-wave load-to-LDS copies and reads each step's operand from there just before its
// MFMAs.  Rows without a routed row (and rows of another group when a tile has more than NV)
// read a zero block.
template <int ADT, int PF>
struct AStage {
  static constexpr int SB = 128 * row_bytes_num<ADT>() / row_bytes_den<ADT>();   // bytes per step
  static constexpr int SLOT = PF * SB;               // bytes of one row's K range (PF steps)
  static constexpr int NV = 7168 / SLOT < 16 ? 7168 / SLOT : 16;   // rows staged at once
  static constexpr int ZERO = NV * SLOT;             // zero block of one step (SB bytes)
  static constexpr int BYTES = NV * SLOT + 256;      // per wave
  static constexpr int COPIES = (NV * SLOT + 1023) / 1024;
};

// Stage1 K split: wave w of KW takes the 128-deep steps [k_lo, k_hi) of K = D.
__device__ __forceinline__ int k_lo_of(int D, int w, int KW) { return w * ((D / 128 + KW - 1) / KW); }
__device__ __forceinline__ int k_hi_of(int D, int w, int KW) {
  return min(D / 128, (w + 1) * ((D / 128 + KW - 1) / KW));
}

// ---------------------------------------------------------------- Stage1

// Both items return false without doing anything for a tile with no expert (past num_tiles:
// the sort writes expert id -1 there), so they can be launched over all cap_tiles tiles.  The
// tile's row ids and its expert id are loaded together: one memory latency before the weight
// addresses are known, instead of a chain of dependent loads.
template <int ADT, int BM, int NI, int KW, int PF, int ACT, bool COH, bool LDSA = false>
__device__ __forceinline__ bool stage1_item(const FusedArgs& p, int tile, int nb,
                                            float (*red)[BM][2 * NI + 1], uint8_t* astage = nullptr) {
  static_assert(!LDSA || BM == 16, "LDS staging is for 16-row tiles");
  constexpr int NT = KW * WAVE;
  constexpr int MF = BM / 16;
  constexpr int NB = 2 * NI / 16;
  // the packed-w1 addressing below takes fragment j's 16 weight rows as one packed block
  // (row n of the block at n % 16 == r16): the gate and the up rows of a fragment never mix
  static_assert(NI % 16 == 0, "gate and up columns fill whole 16-row packed blocks");
  static_assert((BM * NI) % NT == 0 || (BM * NI) % WAVE == 0 && BM * NI < NT,
                "every wave of the epilogue runs the same trip count on all of its lanes");
  static_assert(ADT == DT_BF16 || NI % 32 == 0, "a quantized intermediate needs whole 32-column blocks");

  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / WAVE);   // wave-uniform
  const int r16 = lane & 15, g = lane >> 4;
  const int TK = p.T * p.topk, D = p.D, I = p.I;

  int vr[MF];
#pragma unroll
  for (int f = 0; f < MF; ++f) vr[f] = p.sorted_ids[tile * BM + 16 * f + r16];
  const int e = p.expert_ids[tile];
  if (e < 0 || e >= p.E) {
    (void)MOE_DCHECK(e < p.E, DBG_EXPERT);   // -1 marks an unused tile
    return false;
  }
#pragma unroll
  for (int f = 0; f < MF; ++f) dcheck_row_id(vr[f], TK);

  const size_t a_row = (size_t)D * row_bytes_num<ADT>() / row_bytes_den<ADT>();
  const uint8_t* arow[MF];
  const uint8_t* asrow[MF];
  bool aval[MF];
#pragma unroll
  for (int f = 0; f < MF; ++f) {
    const int v = vr[f];
    aval[f] = (unsigned)v < (unsigned)TK;
    const int t = aval[f] ? v / p.topk : 0;
    arow[f] = p.x + (size_t)t * a_row;
    asrow[f] = ADT == DT_BF16 ? nullptr : p.xs + (size_t)t * (D / 32);
  }
  // Operand column c = 16 j + r16 of fragment j: gate column nb*NI + c for c < NI, else up
  // column I + nb*NI + c - NI.
  const uint8_t* brow[NB];
  const uint8_t* bsrow[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int c = 16 * j + r16;
    const int n = (c < NI) ? nb * NI + c : I + nb * NI + c - NI;
    const size_t wr = (size_t)e * 2 * I + n;
    // packed w1 (moe_pack.hip): the 1 KB block of row group n / 16 and K step s holds the 16 rows
    // x 64 bytes in lane order, lane (r16, g) at bytes 16 (16 g + r16); consecutive steps are
    // consecutive blocks
    brow[j] = p.w1 + ((size_t)e * (2 * I / 16) + n / 16) * (size_t)(D / 128) * 1024 + 16 * (16 * g + r16);
    bsrow[j] = p.w1s + wr * (D / 32);
  }

  v4f acc[MF][NB];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // A chunk of up to PF steps: the scale words and the activation rows are requested first and
  // the weights last, step by step.  Loads complete in order, so the MFMAs of step i wait only
  // for the weights of steps <= i and overlap the arrival of the later steps.  A chunk of PF
  // whole steps has no per-step condition, so its loads and waits are straight-line code.
  auto chunk = [&](int s0, auto full) {
    constexpr bool FULL = decltype(full)::value;
    const int s_end = FULL ? s0 + PF : k_hi_of(D, wave, KW);
    uint4 bq[PF][NB];
    ScaleQuads<PF> bsq[NB];
    ScaleQuads<PF> asq[MF];
    AOperand<ADT> A[PF][MF];
#pragma unroll
    for (int j = 0; j < NB; ++j) bsq[j].load(bsrow[j], s0, s_end, g, true);
#pragma unroll
    for (int f = 0; f < MF; ++f)
      if (ADT != DT_BF16) asq[f].load(asrow[f], s0, s_end, g, aval[f]);
#pragma unroll
    for (int i = 0; i < PF; ++i)
      if (FULL || s0 + i < s_end)
#pragma unroll
        for (int f = 0; f < MF; ++f) A[i][f].load(arow[f], s0 + i, g, aval[f]);
    // one base address per fragment; the steps are immediate offsets of the loads
    const uint8_t* bbase[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) bbase[j] = brow[j] + s0 * 1024;
#pragma unroll
    for (int i = 0; i < PF; ++i)
      if (FULL || s0 + i < s_end)
#pragma unroll
        for (int j = 0; j < NB; ++j) bq[i][j] = ldw16(bbase[j] + i * 1024);
    // every load of the chunk is issued before the first wait (the scheduler would otherwise
    // sink the later steps' loads below the first MFMAs, a second memory round trip)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (FULL || s0 + i < s_end) {
        uint32_t bs[NB], as[MF];
#pragma unroll
        for (int j = 0; j < NB; ++j) bs[j] = bsq[j].get(i, r16, g);
#pragma unroll
        for (int f = 0; f < MF; ++f) as[f] = ADT == DT_BF16 ? 0u : asq[f].get(i, r16, g);
#pragma unroll
        for (int f = 0; f < MF; ++f)
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[f][j] = A[i][f].mma(bq[i][j], bs[j], as[f], acc[f][j]);
      }
    }
  };
  // The LDS-staged variant of a chunk (16-row tiles).
  using AS = AStage<ADT, PF>;
  uint8_t* const xs = astage + wave * AS::BYTES;
  uint32_t mask16 = 0, my_j = 0, tok = 0;
  int ngroups = 0;
  if constexpr (LDSA) {
    reinterpret_cast<uint32_t*>(xs + AS::ZERO)[lane] = 0u;
    mask16 = (uint32_t)__ballot(aval[0]) & 0xFFFFu;        // lanes 0..15 hold rows 0..15
    my_j = __popc(mask16 & ((1u << r16) - 1u));
    tok = aval[0] ? (uint32_t)(vr[0] / p.topk) : 0u;
    ngroups = (__popc(mask16) + AS::NV - 1) / AS::NV;
  }
  // copy the K range [s0, s0 + n_s) of routed rows q*NV .. q*NV + NV - 1 of the tile into LDS
  auto stage_group = [&](int q, int s0, int n_s) {
    uint32_t m = mask16;
    for (int k = 0; k < q * AS::NV; ++k) m &= m - 1u;
    const int nrows = min(AS::NV, __popc(m));
    uint32_t tk[AS::NV];                                     // tokens of the group's rows
#pragma unroll
    for (int k = 0; k < AS::NV; ++k) {
      const int row = m ? __ffs(m) - 1 : 0;
      tk[k] = (uint32_t)__builtin_amdgcn_readlane((int)tok, row);
      m &= m - 1u;
    }
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)xs);
    const int ncopy = (nrows * AS::SLOT + 1023) / 1024;
#pragma unroll
    for (int c = 0; c < AS::COPIES; ++c) {
      if (c >= ncopy) break;
      int o = c * 1024 + lane * 16;
      asm volatile("" : "+v"(o));   // computed here, not kept live across the chunk loop
      const int k = o / AS::SLOT, rem = o - k * AS::SLOT, i = rem / AS::SB;
      uint32_t t = tk[0];
#pragma unroll
      for (int kk = 1; kk < AS::NV; ++kk) t = k == kk ? tk[kk] : t;
      const bool ok = k < nrows && i < n_s;
      const uint32_t off =
          ok ? t * (uint32_t)a_row + (uint32_t)(s0 + i) * AS::SB + (uint32_t)(rem % AS::SB) : 0u;
      dma16_lds(p.x, off, lds0 + c * 1024);
    }
  };
  auto chunk_lds = [&](int s0, auto full) {
    constexpr bool FULL = decltype(full)::value;
    const int s_end = FULL ? s0 + PF : k_hi_of(D, wave, KW);
    const int n_s = s_end - s0;
    uint4 bq[PF][NB];
    ScaleQuads<PF> bsq[NB];
    ScaleQuads<PF> asq;
#pragma unroll
    for (int j = 0; j < NB; ++j) bsq[j].load(bsrow[j], s0, s_end, g, true);
    if (ADT != DT_BF16) asq.load(asrow[0], s0, s_end, g, aval[0]);
    stage_group(0, s0, n_s);
    const uint8_t* bbase[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) bbase[j] = brow[j] + s0 * 1024;
#pragma unroll
    for (int i = 0; i < PF; ++i)
      if (FULL || i < n_s)
#pragma unroll
        for (int j = 0; j < NB; ++j) bq[i][j] = ldw16(bbase[j] + i * 1024);
    __builtin_amdgcn_sched_barrier(0);
    // the copies were issued before the PF*NB weight loads: once at most that many loads are
    // outstanding, the staged rows are in LDS
    if (FULL) wait_vm<PF * NB>();
    else wait_vm<0>();
    int q = 0;
    do {   // at least one pass, so every weight load is consumed on every path
      if (q > 0) {   // every operand read of the previous group is done before its rows are replaced
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        stage_group(q, s0, n_s);
        wait_vm<0>();
      }
      // a row of this group reads its slot, any other row the zero block (step stride 0)
      const bool in = ((mask16 >> r16) & 1u) && (int)my_j / AS::NV == q;
      const uint8_t* abase = xs + (in ? ((int)my_j % AS::NV) * AS::SLOT : AS::ZERO);
      const int astep = in ? AS::SB : 0;
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        if (FULL || i < n_s) {
          AOperand<ADT> A;
          A.load_lds(abase + i * astep, g);
          uint32_t bs[NB];
#pragma unroll
          for (int j = 0; j < NB; ++j) bs[j] = bsq[j].get(i, r16, g);
          const uint32_t as = ADT == DT_BF16 ? 0u : asq.get(i, r16, g);
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[0][j] = A.mma(bq[i][j], bs[j], as, acc[0][j]);
        }
      }
    } while (++q < ngroups);
  };

  const int k_lo = k_lo_of(D, wave, KW), k_hi = k_hi_of(D, wave, KW);
  int s0 = k_lo;
  if constexpr (LDSA) {
    for (; s0 + PF <= k_hi; s0 += PF) chunk_lds(s0, std::true_type{});
    if (s0 < k_hi) chunk_lds(s0, std::false_type{});
  } else {
    for (; s0 + PF <= k_hi; s0 += PF) chunk(s0, std::true_type{});
    if (s0 < k_hi) chunk(s0, std::false_type{});
  }

#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][16 * f + 4 * g + i][16 * j + r16] = acc[f][j][i];
  __syncthreads();

  // Epilogue: thread idx owns column idx % NI of row idx / NI, so the columns of one row sit on
  // consecutive lanes and are packed into 4-byte stores with lane shuffles.
  const float inv_beta = 1.0f / p.beta, inv_lb = 1.0f / p.linear_beta;
  for (int idx = threadIdx.x; idx < BM * NI; idx += NT) {
    const int row = idx / NI, col = idx - row * NI;
    float gs = 0.f, us = 0.f;
#pragma unroll
    for (int w = 0; w < KW; ++w) { gs += red[w][row][col]; us += red[w][row][NI + col]; }
    const int R = tile * BM + row;
    // the row's sorted id, read from the lanes that loaded it
    int rv = __shfl(vr[0], row & 15, WAVE);
#pragma unroll
    for (int f = 1; f < MF; ++f) {
      const int o = __shfl(vr[f], row & 15, WAVE);
      rv = (row >> 4) == f ? o : rv;
    }
    const bool valid = (unsigned)rv < (unsigned)TK;
    const int ocol = nb * NI + col;
    if (ACT == ACT_NONE) {
      if (valid) {
        p.dbg[(size_t)R * 2 * I + ocol] = gs;
        p.dbg[(size_t)R * 2 * I + I + ocol] = us;
      }
      continue;
    }
    const float y = ACT == ACT_SITUV2 ? situv2(gs, us, p.beta, inv_beta, p.linear_beta, inv_lb) : silu_mul(gs, us);
    if (ADT == DT_BF16) {
      const uint32_t h = f32_to_bf16_rne(y);
      const uint32_t h1 = (uint32_t)__shfl_down((int)h, 1, WAVE);
      if (valid && (col & 1) == 0)
        st<COH>(reinterpret_cast<uint32_t*>(p.inter + ((size_t)R * I + ocol) * 2), h | (h1 << 16));
    } else {
      // the 1x32 rule over the 32 lanes of a block with the hardware converts: an even lane
      // encodes its column and the next (the odd lane's value comes over DPP), then the pairs
      // are gathered into 4-byte stores
      const uint32_t bits = __float_as_uint(y);
      const uint32_t amax = halfwave_max_u32(bits & 0x7FFFFFFFu);
      const bool bad = amax >= 0x7F800000u;                // Inf / NaN: scale 255, zero codes
      const int sexp = block_sexp_any(bad ? 0u : amax, ADT == DT_FP8 ? Fp8Fmt::EMAX : Fp4Fmt::EMAX);
      const float yn = __uint_as_float(lane_xor1(bits));
      if (ADT == DT_FP8) {
        const uint32_t pr = bad ? 0u : encode_pair_fp8_hw(y, yn, sexp);
        const uint32_t word = pr | ((uint32_t)__shfl_down((int)pr, 2, WAVE) << 16);
        if (valid && (col & 3) == 0) st<COH>(reinterpret_cast<uint32_t*>(p.inter + (size_t)R * I + ocol), word);
      } else {
        const uint32_t pb = bad ? 0u : encode_pair_fp4_hw(y, yn, e8m0_scale_float(sexp));
        const uint32_t p2 = pb | ((uint32_t)__shfl_down((int)pb, 2, WAVE) << 8);
        const uint32_t word = p2 | ((uint32_t)__shfl_down((int)p2, 4, WAVE) << 16);
        if (valid && (col & 7) == 0)
          st<COH>(reinterpret_cast<uint32_t*>(p.inter + (size_t)R * (I / 2) + ocol / 2), word);
      }
      if (valid && (col & 31) == 0)
        st<COH>(p.inter_s + (size_t)R * (I / 32) + ocol / 32, (uint8_t)(bad ? 255u : (uint32_t)(sexp + 127)));
    }
  }
  return true;
}

// ---------------------------------------------------------------- Stage2
//
// wait() runs after the weight loads of the first PF steps are issued and before the first
// intermediate row is read (the single-launch kernel waits there for the tile's Stage1).

// Stage2 with the tile's intermediate rows staged in LDS (inter_dim up to S2_I_MAX, so the
// whole K fits one chunk of PF steps): the four waves of an item need the same rows, so they
// are copied once per workgroup with whole-wave load-to-LDS copies instead of being loaded by
// every wave.  Rows are S2Stage::pitch bytes apart so the 16 rows of an operand read fall in
// distinct banks.
constexpr int S2_I_MAX = 384;
template <int ADT, int BM>
struct S2Stage {
  static constexpr int RB_MAX = S2_I_MAX * row_bytes_num<ADT>() / row_bytes_den<ADT>();
  __host__ __device__ static constexpr int pitch(int rb) { return ((rb >> 4) | 1) << 4; }
  static constexpr int COPIES = (BM * pitch(RB_MAX) + 1023) / 1024;
  static constexpr int BYTES = COPIES * 1024;
};

template <int ADT, int BM, int NF, int PF, bool COH, class Wait, bool LDSA = false>
__device__ __forceinline__ bool stage2_item(const FusedArgs& p, int tile, int nb, Wait&& wait,
                                            uint8_t* astage = nullptr) {
  static_assert(!LDSA || !COH, "the staged rows come from a previous launch");
  constexpr int MF = BM / 16;
  constexpr int NO = ITEM_WAVES * NF * 16;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / WAVE);   // wave-uniform
  const int r16 = lane & 15, g = lane >> 4;
  const int TK = p.T * p.topk, D = p.D, I = p.I;

  int vr[MF];
#pragma unroll
  for (int f = 0; f < MF; ++f) vr[f] = p.sorted_ids[tile * BM + 16 * f + r16];
  // rows of this lane's accumulator elements, used by the epilogue
  int vrow[MF][4];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) vrow[f][i] = p.sorted_ids[tile * BM + 16 * f + 4 * g + i];
  const int e = p.expert_ids[tile];
  if (e < 0 || e >= p.E) {
    (void)MOE_DCHECK(e < p.E, DBG_EXPERT);
    return false;
  }
#pragma unroll
  for (int f = 0; f < MF; ++f) dcheck_row_id(vr[f], TK);
  // router weights of the accumulator rows, requested before the operands
  float wrow[MF][4];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = vrow[f][i];
      wrow[f][i] = (unsigned)v < (unsigned)TK ? p.topk_w[v] : 0.f;
    }

  const size_t a_row = (size_t)I * row_bytes_num<ADT>() / row_bytes_den<ADT>();
  const uint8_t* arow[MF];
  const uint8_t* asrow[MF];
  bool aval[MF];
#pragma unroll
  for (int f = 0; f < MF; ++f) {
    const int R = tile * BM + 16 * f + r16;
    aval[f] = (unsigned)vr[f] < (unsigned)TK;
    arow[f] = p.inter + (size_t)R * a_row;
    asrow[f] = ADT == DT_BF16 ? nullptr : p.inter_s + (size_t)R * (I / 32);
  }
  const uint8_t* brow[NF];
  const uint8_t* bsrow[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) {
    const int n = nb * NO + wave * NF * 16 + 16 * j + r16;
    const size_t wr = (size_t)e * D + n;
    // packed w2 (moe_pack.hip): the 16 rows of fragment j at K step s are the 1 KB block at
    // (fragment's first row) * I/2 + 1024 s, lane l's 16 bytes at 16 l
    brow[j] = p.w2 + (wr - r16) * (I / 2) + 16 * lane;
    bsrow[j] = p.w2s + wr * (I / 32);
  }
  v4f acc[MF][NF];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // the last column block may be partial (D is a multiple of 64, NO of 64 or more): waves whose
  // columns start at or past D load, compute and store nothing (a wave-uniform condition)
  const bool wave_on = nb * NO + wave * NF * 16 < D;
  const int S = wave_on ? I / 128 : 0;
  if constexpr (LDSA) {
    // scales, then this wave's share of the row copies, then the weights; every wave takes part
    // in the copies and the barrier (also a wave whose columns are past D).  With the whole K
    // in PF steps (FULL) the loads are straight-line code, so each MFMA waits for its own step.
    const int RB = (int)a_row, RBP = S2Stage<ADT, BM>::pitch(RB);
    const int ncopy = (BM * RBP + 1023) / 1024;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)astage);
    const int wv = wave;
    constexpr int CPW = (S2Stage<ADT, BM>::COPIES + ITEM_WAVES - 1) / ITEM_WAVES;
    // source offsets of this wave's copies; a row's validity comes from the lanes holding its id
    uint32_t coff[CPW];
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const int o = (wv + ITEM_WAVES * u) * 1024 + 16 * lane;
      const int row = min(o / RBP, BM - 1), col = o - (o / RBP) * RBP;
      int v = __shfl(vr[0], row & 15, WAVE);
#pragma unroll
      for (int f = 1; f < MF; ++f) {
        const int vf = __shfl(vr[f], row & 15, WAVE);
        v = (row >> 4) == f ? vf : v;
      }
      const bool ok = o / RBP < BM && col < RB && (unsigned)v < (unsigned)TK;
      coff[u] = ok ? (uint32_t)((tile * BM + row) * RB + col) : 0u;
    }
    auto run = [&](auto full) {
      constexpr bool FULL = decltype(full)::value;
      uint4 bq[PF][NF];
      ScaleQuads<PF> bsq[NF];
      ScaleQuads<PF> asq[MF];
#pragma unroll
      for (int j = 0; j < NF; ++j) bsq[j].load(bsrow[j], 0, S, g, true);
#pragma unroll
      for (int f = 0; f < MF; ++f)
        if (ADT != DT_BF16) asq[f].load(asrow[f], 0, S, g, aval[f]);
#pragma unroll
      for (int u = 0; u < CPW; ++u) {
        const int c = wv + ITEM_WAVES * u;
        if (c < ncopy) dma16_lds(p.inter, coff[u], lds0 + c * 1024);
      }
#pragma unroll
      for (int i = 0; i < PF; ++i)
        if (FULL || i < S)
#pragma unroll
          for (int j = 0; j < NF; ++j) bq[i][j] = ldw16(brow[j] + i * 1024);
      __builtin_amdgcn_sched_barrier(0);
      // the copies were issued before this wave's weight loads; the barrier makes every wave's
      // copies visible
      if (FULL) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(PF * NF) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        if (FULL || i < S) {
          uint32_t bs[NF], as[MF];
          AOperand<ADT> A[MF];
#pragma unroll
          for (int f = 0; f < MF; ++f) A[f].load(astage + (16 * f + r16) * RBP, i, g, aval[f]);
#pragma unroll
          for (int j = 0; j < NF; ++j) bs[j] = bsq[j].get(i, r16, g);
#pragma unroll
          for (int f = 0; f < MF; ++f) as[f] = ADT == DT_BF16 ? 0u : asq[f].get(i, r16, g);
#pragma unroll
          for (int f = 0; f < MF; ++f)
#pragma unroll
            for (int j = 0; j < NF; ++j) acc[f][j] = A[f].mma(bq[i][j], bs[j], as[f], acc[f][j]);
        }
      }
    };
    if (S == PF) run(std::true_type{});
    else run(std::false_type{});
  } else {
  uint4 bq[PF][NF];
  ScaleQuads<PF> bsq[NF];
  auto load_weights = [&](int s0) {
#pragma unroll
    for (int j = 0; j < NF; ++j) {
#pragma unroll
      for (int i = 0; i < PF; ++i)
        if (s0 + i < S) bq[i][j] = ldw16(brow[j] + (s0 + i) * 1024);
      bsq[j].load(bsrow[j], s0, S, g, true);
    }
  };
  load_weights(0);
  wait();
  for (int s0 = 0; s0 < S; s0 += PF) {
    if (s0 > 0) load_weights(s0);
    AOperand<ADT> A[PF][MF];
    ScaleQuads<PF, COH> asq[MF];
#pragma unroll
    for (int f = 0; f < MF; ++f) {
#pragma unroll
      for (int i = 0; i < PF; ++i)
        if (s0 + i < S) A[i][f].template load<COH>(arow[f], s0 + i, g, aval[f]);
      if (ADT != DT_BF16) asq[f].load(asrow[f], s0, S, g, aval[f]);
    }
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (s0 + i < S) {
        uint32_t bs[NF], as[MF];
#pragma unroll
        for (int j = 0; j < NF; ++j) bs[j] = bsq[j].get(i, r16, g);
#pragma unroll
        for (int f = 0; f < MF; ++f) as[f] = ADT == DT_BF16 ? 0u : asq[f].get(i, r16, g);
#pragma unroll
        for (int f = 0; f < MF; ++f)
#pragma unroll
          for (int j = 0; j < NF; ++j) acc[f][j] = A[i][f].mma(bq[i][j], bs[j], as[f], acc[f][j]);
      }
    }
  }
  }

  // each routed row's weighted output goes to its own row of rowout; padding rows are not
  // written and never read.  bf16 pairs of neighbouring columns are packed into one store.
#pragma unroll
  for (int f = 0; f < MF; ++f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = wave_on && (unsigned)vrow[f][i] < (unsigned)TK;
      const size_t R = (size_t)tile * BM + 16 * f + 4 * g + i;
      const size_t c0 = (size_t)nb * NO + wave * NF * 16 + r16;
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const float o = acc[f][j][i] * wrow[f][i];
        const uint32_t h = f32_to_bf16_rne(o);
        const uint32_t h1 = (uint32_t)__shfl_down((int)h, 1, WAVE);
        if (valid && (r16 & 1) == 0)
          st<COH>(reinterpret_cast<uint32_t*>(p.rowout + (R * D + c0 + 16 * j) * 2), h | (h1 << 16));
      }
    }
  }
  return true;
}

// ---------------------------------------------------------------- combine
//
// out[t, c] = bf16(sum over k = 0 .. topk-1 of rowout[row_of[t*topk + k], c]), the sum taken in
// fp32 in ascending k with 0 for rows of non-local experts.

// Row positions of KG consecutive slots of token t (-1 past topk).
template <int KG>
__device__ __forceinline__ void token_rows(const FusedArgs& p, int t, int k0, int (&r)[KG]) {
#pragma unroll
  for (int u = 0; u < KG; ++u) {
    r[u] = k0 + u < p.topk ? p.row_of[(int64_t)t * p.topk + k0 + u] : -1;
    if (!MOE_DCHECK(r[u] >= -1 && (int64_t)r[u] < (int64_t)p.cap_tiles * p.block_m, DBG_COMBINE_ROW)) r[u] = -1;
  }
}

// Two neighbouring columns c, c+1 of routed row r (0 where r < 0).
template <bool COH>
__device__ __forceinline__ float2 rowout_pair(const FusedArgs& p, int r, int c) {
  if (r < 0) return float2{0.f, 0.f};
  const uint32_t q = ld<COH>(reinterpret_cast<const uint32_t*>(p.rowout + ((size_t)r * p.D + c) * 2));
  return float2{__uint_as_float(q << 16), __uint_as_float(q & 0xFFFF0000u)};
}

// Columns [c_begin, c_end) of token t, two per thread of the workgroup.
template <bool COH>
__device__ __forceinline__ void combine_token_cols(const FusedArgs& p, int t, int c_begin, int c_end) {
  constexpr int KG = 8;
  for (int c = c_begin + 2 * (int)threadIdx.x; c < c_end; c += 2 * (int)blockDim.x) {
    float s0 = 0.f, s1 = 0.f;
    for (int k0 = 0; k0 < p.topk; k0 += KG) {
      int r[KG];
      token_rows<KG>(p, t, k0, r);
      float2 v[KG];
#pragma unroll
      for (int u = 0; u < KG; ++u) v[u] = rowout_pair<COH>(p, r[u], c);
#pragma unroll
      for (int u = 0; u < KG; ++u) { s0 += v[u].x; s1 += v[u].y; }
    }
    const uint32_t o = (uint32_t)f32_to_bf16_rne(s0) | ((uint32_t)f32_to_bf16_rne(s1) << 16);
    *reinterpret_cast<uint32_t*>(p.out + (size_t)t * p.D + c) = o;
  }
}

}  // namespace moe
