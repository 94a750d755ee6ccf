// One work item of each stage of the fused MXFP4 MoE, as device functions shared by the
// per-stage kernels (moe_gemm.hip) and the single-launch kernel (moe_single.hip), so both
// paths compute every output with the same instructions in the same order.
//
// Stage1 item (tile, nb) (github ROCm/aiter PR 6259 "Technical Details": SiTUv2 in the stage1
//   epilogue): block_m sorted rows x NI intermediate columns.  The gate columns [n0, n0+NI)
//   and the matching up columns [I+n0, I+n0+NI) are computed together, so a lane holds g and u
//   of the same output element.  KW waves split the K = model_dim reduction into contiguous
//   ranges of 128-deep steps; each lane streams its weight bytes and its gathered activation row
//   straight from memory into matrix-core operands (every byte is loaded once per item), issuing
//   the loads of PF steps before the first MFMA that uses them; the partial sums meet in LDS.
//   The epilogue applies SiTUv2 or SiLU and re-encodes the intermediate: bf16, or fp8 / fp4 with
//   one e8m0 scale per 32 columns (the 32 columns of a block are 32 lanes of one wave).
// Stage2 item (tile, nb) (PR 5118 review items 9-10: bf16 x MXFP4 stage2 with a per-token
//   scatter of the weighted rows): block_m rows x 64*NF output columns (the last block of a row
//   may be partial); each wave owns 16*NF columns over the whole K = inter_dim.  The fp32 result row is scaled by the router weight
//   of its routed row and stored as that routed row's output (fp32 for bf16 activations, bf16
//   otherwise).
// Combine: each token's routed-row outputs summed in ascending k in fp32, rounded to bf16.
#pragma once

#include "moe_kernels.h"
#include "moe_operands.h"

namespace moe {

constexpr int ITEM_THREADS = 256;
constexpr int ITEM_WAVES = ITEM_THREADS / WAVE;

// ---------------------------------------------------------------- Stage1

// Both items return false without doing anything for a tile with no expert (past num_tiles:
// the sort writes expert id -1 there), so they can be launched over all cap_tiles tiles.  The
// tile's row ids and its expert id are loaded together: one memory latency before the weight
// addresses are known, instead of a chain of dependent loads.
template <int ADT, int BM, int NI, int KW, int PF, int ACT, bool COH>
__device__ __forceinline__ bool stage1_item(const FusedArgs& p, int tile, int nb,
                                            float (*red)[BM][2 * NI + 1]) {
  constexpr int NT = KW * WAVE;
  constexpr int MF = BM / 16;
  constexpr int NF = NI / 16;
  constexpr int NB = 2 * NF;
  static_assert((BM * NI) % NT == 0, "the epilogue loop runs the same trip count on every lane");
  static_assert(ADT == DT_BF16 || NI % 32 == 0, "a quantized intermediate needs whole 32-column blocks");

  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int r16 = lane & 15, g = lane >> 4;
  const int TK = p.T * p.topk, D = p.D, I = p.I;

  int vr[MF];
#pragma unroll
  for (int f = 0; f < MF; ++f) vr[f] = p.sorted_ids[tile * BM + 16 * f + r16];
  const int e = p.expert_ids[tile];
  if (e < 0 || e >= p.E) return false;

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
  const uint8_t* brow[NB];
  const uint8_t* bsrow[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int n = (j < NF) ? nb * NI + 16 * j + r16 : I + nb * NI + 16 * (j - NF) + r16;
    const size_t wr = (size_t)e * 2 * I + n;
    brow[j] = p.w1 + wr * (D / 2);
    bsrow[j] = p.w1s + wr * (D / 32);
  }

  v4f acc[MF][NB];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int S = D / 128;
  const int spw = (S + KW - 1) / KW;
  const int k_lo = wave * spw, k_hi = min(S, k_lo + spw);
  for (int s0 = k_lo; s0 < k_hi; s0 += PF) {
    uint4 bq[PF][NB];
    ScaleQuads<PF> bsq[NB];
    ScaleQuads<PF> asq[MF];
    AOperand<ADT> A[PF][MF];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int i = 0; i < PF; ++i)
        if (s0 + i < k_hi) bq[i][j] = ld16(brow[j] + (s0 + i) * 64 + 16 * g);
      bsq[j].load(bsrow[j], s0, k_hi, g, true);
    }
#pragma unroll
    for (int f = 0; f < MF; ++f) {
#pragma unroll
      for (int i = 0; i < PF; ++i)
        if (s0 + i < k_hi) A[i][f].load(arow[f], s0 + i, g, aval[f]);
      if (ADT != DT_BF16) asq[f].load(asrow[f], s0, k_hi, g, aval[f]);
    }
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (s0 + i < k_hi) {
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
    const bool valid = (unsigned)p.sorted_ids[R] < (unsigned)TK;
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
      uint32_t sb, word;
      if (ADT == DT_FP8) {
        const uint32_t c = block_encode_lane<Fp8Fmt>(y, &sb);
        const uint32_t c1 = (uint32_t)__shfl_down((int)c, 1, WAVE);
        const uint32_t c2 = (uint32_t)__shfl_down((int)c, 2, WAVE);
        const uint32_t c3 = (uint32_t)__shfl_down((int)c, 3, WAVE);
        word = c | (c1 << 8) | (c2 << 16) | (c3 << 24);
        if (valid && (col & 3) == 0) st<COH>(reinterpret_cast<uint32_t*>(p.inter + (size_t)R * I + ocol), word);
      } else {
        const uint32_t c = block_encode_lane<Fp4Fmt>(y, &sb);
        const uint32_t p2 = c | ((uint32_t)__shfl_down((int)c, 1, WAVE) << 4);
        const uint32_t p4 = p2 | ((uint32_t)__shfl_down((int)p2, 2, WAVE) << 8);
        word = p4 | ((uint32_t)__shfl_down((int)p4, 4, WAVE) << 16);
        if (valid && (col & 7) == 0)
          st<COH>(reinterpret_cast<uint32_t*>(p.inter + (size_t)R * (I / 2) + ocol / 2), word);
      }
      if (valid && (col & 31) == 0) st<COH>(p.inter_s + (size_t)R * (I / 32) + ocol / 32, (uint8_t)sb);
    }
  }
  return true;
}

// ---------------------------------------------------------------- Stage2
//
// wait() runs after the weight loads of the first PF steps are issued and before the first
// intermediate row is read (the single-launch kernel waits there for the tile's Stage1).

template <int ADT, int BM, int NF, int PF, bool COH, class Wait>
__device__ __forceinline__ bool stage2_item(const FusedArgs& p, int tile, int nb, Wait&& wait) {
  constexpr int MF = BM / 16;
  constexpr int NO = ITEM_WAVES * NF * 16;
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
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
  if (e < 0 || e >= p.E) return false;

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
    brow[j] = p.w2 + wr * (I / 2);
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
  uint4 bq[PF][NF];
  ScaleQuads<PF> bsq[NF];
  auto load_weights = [&](int s0) {
#pragma unroll
    for (int j = 0; j < NF; ++j) {
#pragma unroll
      for (int i = 0; i < PF; ++i)
        if (s0 + i < S) bq[i][j] = ld16(brow[j] + (s0 + i) * 64 + 16 * g);
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

  float wrow[MF][4];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = vrow[f][i];
      wrow[f][i] = (unsigned)v < (unsigned)TK ? p.topk_w[v] : 0.f;
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
        if (ADT == DT_BF16) {
          if (valid) st<COH>(reinterpret_cast<float*>(p.rowout) + R * D + c0 + 16 * j, o);
        } else {
          const uint32_t h = f32_to_bf16_rne(o);
          const uint32_t h1 = (uint32_t)__shfl_down((int)h, 1, WAVE);
          if (valid && (r16 & 1) == 0)
            st<COH>(reinterpret_cast<uint32_t*>(p.rowout + (R * D + c0 + 16 * j) * 2), h | (h1 << 16));
        }
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
  for (int u = 0; u < KG; ++u) r[u] = k0 + u < p.topk ? p.row_of[(int64_t)t * p.topk + k0 + u] : -1;
}

// Two neighbouring columns c, c+1 of routed row r (0 where r < 0).
template <bool F32, bool COH>
__device__ __forceinline__ float2 rowout_pair(const FusedArgs& p, int r, int c) {
  if (r < 0) return float2{0.f, 0.f};
  if (F32) {
    const uint64_t q = ld<COH>(reinterpret_cast<const uint64_t*>(p.rowout + ((size_t)r * p.D + c) * 4));
    return float2{__uint_as_float((uint32_t)q), __uint_as_float((uint32_t)(q >> 32))};
  }
  const uint32_t q = ld<COH>(reinterpret_cast<const uint32_t*>(p.rowout + ((size_t)r * p.D + c) * 2));
  return float2{__uint_as_float(q << 16), __uint_as_float(q & 0xFFFF0000u)};
}

// Columns [c_begin, c_end) of token t, two per thread of the workgroup.
template <bool F32, bool COH>
__device__ __forceinline__ void combine_token_cols(const FusedArgs& p, int t, int c_begin, int c_end) {
  constexpr int KG = 8;
  for (int c = c_begin + 2 * (int)threadIdx.x; c < c_end; c += 2 * (int)blockDim.x) {
    float s0 = 0.f, s1 = 0.f;
    for (int k0 = 0; k0 < p.topk; k0 += KG) {
      int r[KG];
      token_rows<KG>(p, t, k0, r);
      float2 v[KG];
#pragma unroll
      for (int u = 0; u < KG; ++u) v[u] = rowout_pair<F32, COH>(p, r[u], c);
#pragma unroll
      for (int u = 0; u < KG; ++u) { s0 += v[u].x; s1 += v[u].y; }
    }
    const uint32_t o = (uint32_t)f32_to_bf16_rne(s0) | ((uint32_t)f32_to_bf16_rne(s1) << 16);
    *reinterpret_cast<uint32_t*>(p.out + (size_t)t * p.D + c) = o;
  }
}

}  // namespace moe
