// Stage1 and Stage2 of the fused MXFP4 MoE on gfx950 block-scaled matrix cores.
//
// Stage1 (github ROCm/aiter PR 6259 "Technical Details": SiTUv2 in the stage1 epilogue):
//   one workgroup = one tile of block_m sorted rows x NI intermediate columns.  It computes
//   the gate columns [n0, n0+NI) and the matching up columns [I+n0, I+n0+NI) together, so a
//   lane holds g and u of the same output element.  The four waves split the K = model_dim
//   reduction (K steps of 128, step s on wave s % 4); each lane streams its weight bytes and
//   its gathered activation row straight from memory into matrix-core operands (every byte
//   is loaded once per workgroup), and the partial sums meet in LDS.  The epilogue applies
//   SiTUv2 or SiLU and re-encodes the intermediate: bf16, or fp8 / fp4 with one e8m0 scale per
//   32 columns (the 32 columns of a block are 32 lanes of one wave).
// Stage2 (PR 5118 review items 9-10 and commit notes: bf16 x MXFP4 stage2, atomic scatter):
//   one workgroup = one tile x 64 * NF output columns; each wave owns 16 * NF columns over the
//   whole K = inter_dim.  The fp32 result row is scaled by the router weight of its routed row
//   and stored as that routed row's output (fp32 for bf16 activations, bf16 otherwise).
// Combine sums each token's routed-row outputs (via the sort's inverse map) and rounds to bf16.
#include "moe_kernels.h"
#include "moe_device.h"

namespace moe {

namespace {

constexpr int THREADS = 256;
constexpr int NWAVES = THREADS / WAVE;

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ v8i fp4_operand(const uint4& q) {
  v8i r = {(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
  return r;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// One 16-row activation operand for one 128-deep K step (lane holds row r16, group g).
template <int ADT>
struct AOperand;

template <>
struct AOperand<DT_FP8> {
  v8i a;
  uint32_t s;
  __device__ __forceinline__ void load(const uint8_t* row, const uint8_t* srow, int step, int g, bool valid) {
    if (valid) {
      const uint4 lo = ld16(row + step * 128 + 16 * g);
      const uint4 hi = ld16(row + step * 128 + 64 + 16 * g);
      a = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      s = srow[step * 4 + g];
    } else {
      a = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      s = 127u;
    }
  }
  __device__ __forceinline__ v4f mma(const uint4& bq, uint32_t bs, const v4f& c) const {
    return mfma_fp8_fp4(a, fp4_operand(bq), c, s, bs);
  }
};

template <>
struct AOperand<DT_FP4> {
  v8i a;
  uint32_t s;
  __device__ __forceinline__ void load(const uint8_t* row, const uint8_t* srow, int step, int g, bool valid) {
    if (valid) {
      a = fp4_operand(ld16(row + step * 64 + 16 * g));
      s = srow[step * 4 + g];
    } else {
      a = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      s = 127u;
    }
  }
  __device__ __forceinline__ v4f mma(const uint4& bq, uint32_t bs, const v4f& c) const {
    return mfma_fp4_fp4(a, fp4_operand(bq), c, s, bs);
  }
};

// bf16 activations: the 128-deep step is four 32-deep bf16 MFMAs.  Sub-step jj takes K
// elements [32g + 8jj, 32g + 8jj + 8) of the step on lane group g for both operands, so a lane
// reads 32 consecutive bf16 of its row and the 32 fp4 weights of one scale block.
template <>
struct AOperand<DT_BF16> {
  v8bf a[4];
  __device__ __forceinline__ void load(const uint8_t* row, const uint8_t*, int step, int g, bool valid) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if (valid) {
        const uint4 q = ld16(row + step * 256 + 64 * g + 16 * jj);
        a[jj] = as_bf16x8(q.x, q.y, q.z, q.w);
      } else {
        a[jj] = as_bf16x8(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ v4f mma(const uint4& bq, uint32_t bs, const v4f& c) const {
    const float sc = e8m0_to_float(bs);
    v4f r = c;
    r = mfma_bf16(a[0], fp4x8_to_bf16(bq.x, sc), r);
    r = mfma_bf16(a[1], fp4x8_to_bf16(bq.y, sc), r);
    r = mfma_bf16(a[2], fp4x8_to_bf16(bq.z, sc), r);
    r = mfma_bf16(a[3], fp4x8_to_bf16(bq.w, sc), r);
    return r;
  }
};

template <int ADT>
__host__ __device__ constexpr int row_bytes_num() { return ADT == DT_BF16 ? 2 : 1; }
template <int ADT>
__host__ __device__ constexpr int row_bytes_den() { return ADT == DT_FP4 ? 2 : 1; }

// ---------------------------------------------------------------- Stage1
//
// KW waves split the K steps (each wave a contiguous range); each wave issues the weight and
// activation loads of PF of its steps before the first MFMA that uses them, so every lane has
// PF * (2*NF + MF) loads in flight and waits once per PF steps.

template <int ADT, int BM, int NI, int KW, int PF, int MINW, int ACT>
__global__ __launch_bounds__(KW * WAVE, MINW) void stage1_kernel(FusedArgs p, int n_nblk) {
  constexpr int NT = KW * WAVE;
  constexpr int MF = BM / 16;
  constexpr int NF = NI / 16;
  constexpr int NB = 2 * NF;
  static_assert(ADT == DT_BF16 || (NI % 32 == 0 && (BM * NI) % NT == 0),
                "a quantized intermediate needs whole 32-column blocks on full waves");
  __shared__ float red[KW][BM][2 * NI + 1];

  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int r16 = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x / n_nblk;
  const int nb = blockIdx.x - tile * n_nblk;
  if (tile >= *p.num_tiles) return;
  const int e = p.expert_ids[tile];
  if (e < 0 || e >= p.E) return;
  const int TK = p.T * p.topk, D = p.D, I = p.I;

  const size_t a_row = (size_t)D * row_bytes_num<ADT>() / row_bytes_den<ADT>();
  const uint8_t* arow[MF];
  const uint8_t* asrow[MF];
  bool aval[MF];
#pragma unroll
  for (int f = 0; f < MF; ++f) {
    const int v = p.sorted_ids[tile * BM + 16 * f + r16];
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

  // wave `wave` owns the contiguous K steps [k_lo, k_hi); all loads of PF steps are issued
  // before the first MFMA that uses them
  const int S = D / 128;
  const int spw = (S + KW - 1) / KW;
  const int k_lo = wave * spw, k_hi = min(S, k_lo + spw);
  for (int s0 = k_lo; s0 < k_hi; s0 += PF) {
    uint4 bq[PF][NB];
    uint32_t bs[PF][NB];
    AOperand<ADT> A[PF][MF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (s0 + i < k_hi) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          bq[i][j] = ld16(brow[j] + (s0 + i) * 64 + 16 * g);
          bs[i][j] = bsrow[j][(s0 + i) * 4 + g];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < PF; ++i)
      if (s0 + i < k_hi) {
#pragma unroll
        for (int f = 0; f < MF; ++f) A[i][f].load(arow[f], asrow[f], s0 + i, g, aval[f]);
      }
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (s0 + i < k_hi) {
#pragma unroll
        for (int f = 0; f < MF; ++f)
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[f][j] = A[i][f].mma(bq[i][j], bs[i][j], acc[f][j]);
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
      if (valid) reinterpret_cast<uint16_t*>(p.inter)[(size_t)R * I + ocol] = f32_to_bf16_rne(y);
    } else {
      uint32_t sb;
      if (ADT == DT_FP8) {
        const uint32_t c = block_encode_lane<Fp8Fmt>(y, &sb);
        if (valid) p.inter[(size_t)R * I + ocol] = (uint8_t)c;
      } else {
        const uint32_t c = block_encode_lane<Fp4Fmt>(y, &sb);
        const uint32_t c_hi = (uint32_t)__shfl_down((int)c, 1, WAVE);
        if (valid && (col & 1) == 0) p.inter[(size_t)R * (I / 2) + ocol / 2] = (uint8_t)(c | (c_hi << 4));
      }
      if (valid && (col & 31) == 0) p.inter_s[(size_t)R * (I / 32) + ocol / 32] = (uint8_t)sb;
    }
  }
}

// ---------------------------------------------------------------- Stage2
//
// Workgroup (tile, column block nb): blockIdx = nb * cap + tile, so the tiles of one column
// block run together and share that block's slice of the accumulator rows in L2.

template <int ADT, int BM, int NF, int PF, int MINW>
__global__ __launch_bounds__(THREADS, MINW) void stage2_kernel(FusedArgs p, int cap) {
  constexpr int MF = BM / 16;
  constexpr int NO = NWAVES * NF * 16;
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int r16 = lane & 15, g = lane >> 4;
  const int tile = blockIdx.x % cap;
  const int nb = blockIdx.x / cap;
  if (tile >= *p.num_tiles) return;
  const int e = p.expert_ids[tile];
  if (e < 0 || e >= p.E) return;
  const int TK = p.T * p.topk, D = p.D, I = p.I;

  const size_t a_row = (size_t)I * row_bytes_num<ADT>() / row_bytes_den<ADT>();
  const uint8_t* arow[MF];
  const uint8_t* asrow[MF];
  bool aval[MF];
#pragma unroll
  for (int f = 0; f < MF; ++f) {
    const int R = tile * BM + 16 * f + r16;
    aval[f] = (unsigned)p.sorted_ids[R] < (unsigned)TK;
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
  // rows of this lane's accumulator elements: loaded early, used by the epilogue
  int vrow[MF][4];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) vrow[f][i] = p.sorted_ids[tile * BM + 16 * f + 4 * g + i];

  v4f acc[MF][NF];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int S = I / 128;
  for (int s0 = 0; s0 < S; s0 += PF) {
    uint4 bq[PF][NF];
    uint32_t bs[PF][NF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (s0 + i < S) {
#pragma unroll
        for (int j = 0; j < NF; ++j) {
          bq[i][j] = ld16(brow[j] + (s0 + i) * 64 + 16 * g);
          bs[i][j] = bsrow[j][(s0 + i) * 4 + g];
        }
      }
    }
    AOperand<ADT> A[PF][MF];
#pragma unroll
    for (int i = 0; i < PF; ++i)
      if (s0 + i < S) {
#pragma unroll
        for (int f = 0; f < MF; ++f) A[i][f].load(arow[f], asrow[f], s0 + i, g, aval[f]);
      }
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      if (s0 + i < S) {
#pragma unroll
        for (int f = 0; f < MF; ++f)
#pragma unroll
          for (int j = 0; j < NF; ++j) acc[f][j] = A[i][f].mma(bq[i][j], bs[i][j], acc[f][j]);
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
  // each routed row's weighted output goes to its own row of rowout (no atomics); padding rows
  // are not written and never read
#pragma unroll
  for (int f = 0; f < MF; ++f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if ((unsigned)vrow[f][i] >= (unsigned)TK) continue;
      const size_t R = (size_t)tile * BM + 16 * f + 4 * g + i;
      const size_t c0 = (size_t)nb * NO + wave * NF * 16 + r16;
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const float o = acc[f][j][i] * wrow[f][i];
        if (ADT == DT_BF16) reinterpret_cast<float*>(p.rowout)[R * D + c0 + 16 * j] = o;
        else reinterpret_cast<uint16_t*>(p.rowout)[R * D + c0 + 16 * j] = f32_to_bf16_rne(o);
      }
    }
  }
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

unsigned stream_blocks(int64_t n) {
  int64_t b = (n + THREADS - 1) / THREADS;
  if (b > 256 * 16) b = 256 * 16;
  return (unsigned)(b < 1 ? 1 : b);
}

// Stage tiling per activation dtype and block_m.
template <int ADT, int BM>
struct Cfg {
  static constexpr int NI = ADT == DT_BF16 ? 16 : 32;         // intermediate columns / workgroup
  static constexpr int KW = 4;                                // waves splitting K in stage1
  static constexpr int PF1 = (ADT == DT_BF16 && BM == 16) ? 7 : 4;   // K steps in flight per wave
  static constexpr int MINW1 = 2;                               // waves per SIMD kept
  static constexpr int NF2 = 1;                               // stage2 16-column fragments / wave
  static constexpr int PF2 = 4;
  static constexpr int MINW2 = BM == 16 ? 4 : 2;
};

template <int ADT, int BM>
hipError_t run_stages(FusedArgs a, hipStream_t s) {
  using C = Cfg<ADT, BM>;
  const int n1 = a.I / C::NI;
  const unsigned grid1 = (unsigned)((int64_t)a.cap_tiles * n1);
  const int n2 = a.D / (NWAVES * C::NF2 * 16);
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
