// Large-batch Stage1 / Stage2: LDS-tiled block-scaled GEMMs over groups of sort tiles.
//
// With many routed rows per expert (prefill, expert-parallel shards) the per-tile kernels of
// moe_gemm.hip re-stream an expert's weights for every 16/32-row tile.  Here a workgroup owns a
// group of up to GT consecutive tiles of the same expert (GT*32 rows) and BNW weight rows, so
// each weight byte fetched serves GT*32 rows.  Both operands are staged through LDS per 128-deep
// K step (double buffered, one barrier per step; rows padded by 16 bytes so the 16-lane row
// reads of a matrix-core operand hit distinct banks).  Four waves each compute all GT*32 rows
// times BNW/4 weight rows with v_mfma_scale_f32_16x16x128_f8f6f4 (fp8 x fp4 or fp4 x fp4).
//
// Stage1 epilogue (github ROCm/aiter PR 6259 "Technical Details": SiTUv2 in the stage1
// epilogue): a wave's B rows are [gate block | matching up block], so g and u of one output sit
// in the same lane; y = act(g, u) is re-encoded per 32-column block (PR 4463 "Three tuner
// defects" item 2: fused fp4 stage1 output) with the block maximum reduced over 16 lanes.
// Stage2 epilogue: the row result times the router weight, stored as bf16 per routed row for the
// gather combine (no atomics).
#include "moe_kernels.h"
#include "moe_device.h"

namespace moe {

namespace {

constexpr int THREADS = 256;
constexpr int WAVES = THREADS / WAVE;

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------- tile groups
//
// groups[g] = (first tile, tile count): maximal runs of GT consecutive tiles of one expert,
// cut at expert boundaries and every GT tiles within an expert.  One workgroup of 1024 threads.

constexpr int GROUP_THREADS = 1024;

template <int GT>
__global__ __launch_bounds__(GROUP_THREADS) void group_kernel(const int32_t* __restrict__ expert_ids,
                                                              const int32_t* __restrict__ num_tiles_p,
                                                              int cap, int2* __restrict__ groups,
                                                              int32_t* __restrict__ num_groups) {
  __shared__ int tmp[GROUP_THREADS / WAVE + 1];
  const int n = *num_tiles_p;
  const int per = (cap + GROUP_THREADS - 1) / GROUP_THREADS;
  const int t0 = threadIdx.x * per;
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  // 1. last run start at or before each tile: inclusive max-scan of (run start ? tile : -1)
  int local_max = -1;
  for (int i = 0; i < per; ++i) {
    const int t = t0 + i;
    if (t < n && (t == 0 || expert_ids[t] != expert_ids[t - 1])) local_max = t;
  }
  int incl = local_max;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const int o = __shfl_up(incl, d, WAVE);
    if (lane >= d) incl = max(incl, o);
  }
  if (lane == WAVE - 1) tmp[w] = incl;
  __syncthreads();
  int before = -1;
  for (int i = 0; i < w; ++i) before = max(before, tmp[i]);
  int excl = __shfl_up(incl, 1, WAVE);
  if (lane == 0) excl = -1;
  int run_start = max(before, excl);            // last run start before this thread's chunk
  __syncthreads();
  // 2. group starts and their count
  int starts = 0;
  for (int i = 0; i < per; ++i) {
    const int t = t0 + i;
    if (t >= n) break;
    if (t == 0 || expert_ids[t] != expert_ids[t - 1]) run_start = t;
    starts += ((t - run_start) % GT) == 0;
  }
  int scan = starts;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const int o = __shfl_up(scan, d, WAVE);
    if (lane >= d) scan += o;
  }
  if (lane == WAVE - 1) tmp[w] = scan;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < GROUP_THREADS / WAVE; ++i) { const int c = tmp[i]; tmp[i] = run; run += c; }
    tmp[GROUP_THREADS / WAVE] = run;
  }
  __syncthreads();
  int gidx = tmp[w] + scan - starts;
  // 3. write the groups (the run start is recomputed the same way as above)
  run_start = max(before, excl);
  for (int i = 0; i < per; ++i) {
    const int t = t0 + i;
    if (t >= n) break;
    if (t == 0 || expert_ids[t] != expert_ids[t - 1]) run_start = t;
    if (((t - run_start) % GT) == 0) {
      int c = 1;
      while (c < GT && t + c < n && expert_ids[t + c] == expert_ids[t]) ++c;
      groups[gidx++] = int2{t, c};
    }
  }
  if (threadIdx.x == 0) *num_groups = tmp[GROUP_THREADS / WAVE];
}

// ---------------------------------------------------------------- tiled GEMM

// A operand: fp8 or fp4 activations (stage1: gathered x rows; stage2: intermediate rows).
// B operand: fp4 weight rows.  K step = 128 elements: A row slice KA bytes, B row slice 64 bytes.
template <int ADT>
struct AFmt {
  static constexpr int KA = ADT == DT_FP8 ? 128 : 64;
};

template <int ADT, int GT, int BNW, int STAGE, int ACT>
__global__ __launch_bounds__(THREADS, ADT == DT_FP4 ? 2 : 1) void gemm_tiled_kernel(FusedArgs p, const int2* __restrict__ groups,
                                                                const int32_t* __restrict__ num_groups,
                                                                int n_nblk) {
  constexpr int BMW = GT * 32;                  // rows per workgroup
  constexpr int KA = AFmt<ADT>::KA;
  constexpr int KB = 64;
  constexpr int SA = KA + 16, SB = KB + 16;     // padded LDS row strides (bytes)
  constexpr int MF = BMW / 16;                  // 16-row A fragments (all waves use all rows)
  constexpr int NFW = BNW / WAVES / 16;         // 16-row B fragments per wave
  constexpr int CA = BMW * KA / 16;             // 16-byte A chunks per K step
  constexpr int CB = BNW * KB / 16;
  static_assert(CA % THREADS == 0 && CB % THREADS == 0, "chunks per thread");
  constexpr int CAT = CA / THREADS, CBT = CB / THREADS;
  constexpr int A_CHUNKS_PER_ROW = KA / 16;
  static_assert(STAGE == 2 || (NFW % 4 == 0), "stage1: whole 32-column gate/up blocks per wave");

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BMW * SA];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BNW * SB];
  __shared__ uint32_t lds_as[2][BMW];
  __shared__ uint32_t lds_bs[2][BNW];
  __shared__ int lds_v[BMW];

  // XCD-aware work id: the active items (groups x column blocks, known on the device) are cut
  // into 8 contiguous chunks, one per XCD (blockIdx % 8 selects the XCD), so the column blocks
  // of a group and the groups of an expert run on one XCD and share its L2.
  const int n_act = *num_groups * n_nblk;
  const int chunk = (n_act + 7) / 8;
  const int local = blockIdx.x >> 3;
  if (local >= chunk) return;
  const int work = (blockIdx.x & 7) * chunk + local;
  if (work >= n_act) return;
  const int gi = work / n_nblk, nb = work - gi * n_nblk;
  const int2 grp = groups[gi];
  const int tile0 = grp.x, ntile = grp.y;
  const int e = p.expert_ids[tile0];
  if (e < 0 || e >= p.E) return;
  const int TK = p.T * p.topk, D = p.D, I = p.I;
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  const int r16 = lane & 15, g = lane >> 4;
  const int row_base = tile0 * 32;              // first layout row of the group
  const int rows_used = ntile * 32;

  for (int r = threadIdx.x; r < BMW; r += THREADS)
    lds_v[r] = r < rows_used ? p.sorted_ids[row_base + r] : TK;
  __syncthreads();

  // ---- per-thread global sources of its A and B chunks
  const int K = STAGE == 1 ? D : I;
  const int S = K / 128;
  const size_t a_rowbytes = STAGE == 1 ? (size_t)D * KA / 128 : (size_t)I * KA / 128;
  const uint8_t* a_src[CAT];
  const uint8_t* as_src = nullptr;              // A scales (threads < BMW)
  bool a_ok[CAT];
#pragma unroll
  for (int c = 0; c < CAT; ++c) {
    const int chunk = threadIdx.x + c * THREADS;
    const int row = chunk / A_CHUNKS_PER_ROW, part = chunk - row * A_CHUNKS_PER_ROW;
    const int v = lds_v[row];
    a_ok[c] = (unsigned)v < (unsigned)TK;
    const size_t srow = STAGE == 1 ? (size_t)(a_ok[c] ? v / p.topk : 0) : (size_t)(row_base + row);
    a_src[c] = (STAGE == 1 ? p.x : p.inter) + srow * a_rowbytes + part * 16;
  }
  bool as_ok = false;
  if (threadIdx.x < BMW) {
    const int v = lds_v[threadIdx.x];
    as_ok = (unsigned)v < (unsigned)TK;
    const size_t srow = STAGE == 1 ? (size_t)(as_ok ? v / p.topk : 0) : (size_t)(row_base + threadIdx.x);
    as_src = (STAGE == 1 ? p.xs : p.inter_s) + srow * (K / 32);
  }
  // B rows of this workgroup: stage1 [gate NI | up NI] with NI = BNW/2, stage2 BNW output rows
  auto b_row = [&](int r) -> size_t {
    if (STAGE == 1) {
      const int ni = BNW / 2;
      const int n = r < ni ? nb * ni + r : I + nb * ni + (r - ni);
      return (size_t)e * 2 * I + n;
    }
    return (size_t)e * D + nb * BNW + r;
  };
  const uint8_t* wq = STAGE == 1 ? p.w1 : p.w2;
  const uint8_t* ws = STAGE == 1 ? p.w1s : p.w2s;
  const uint8_t* b_src[CBT];
#pragma unroll
  for (int c = 0; c < CBT; ++c) {
    const int chunk = threadIdx.x + c * THREADS;
    const int row = chunk / (KB / 16), part = chunk - row * (KB / 16);
    b_src[c] = wq + b_row(row) * (size_t)(K / 2) + part * 16;
  }
  const uint8_t* bs_src = ws + b_row(threadIdx.x < BNW ? threadIdx.x : 0) * (size_t)(K / 32);

  uint4 ra[CAT], rb[CBT];
  uint32_t ras = 0, rbs = 0;
  auto gload = [&](int s) {
#pragma unroll
    for (int c = 0; c < CAT; ++c) ra[c] = a_ok[c] ? ld16(a_src[c] + (size_t)s * KA) : uint4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < CBT; ++c) rb[c] = ld16(b_src[c] + (size_t)s * KB);
    if (threadIdx.x < BMW) ras = as_ok ? *reinterpret_cast<const uint32_t*>(as_src + s * 4) : 0x7F7F7F7Fu;
    if (threadIdx.x < BNW) rbs = *reinterpret_cast<const uint32_t*>(bs_src + s * 4);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CAT; ++c) {
      const int chunk = threadIdx.x + c * THREADS;
      const int row = chunk / A_CHUNKS_PER_ROW, part = chunk - row * A_CHUNKS_PER_ROW;
      *reinterpret_cast<uint4*>(&lds_a[buf][row * SA + part * 16]) = ra[c];
    }
#pragma unroll
    for (int c = 0; c < CBT; ++c) {
      const int chunk = threadIdx.x + c * THREADS;
      const int row = chunk / (KB / 16), part = chunk - row * (KB / 16);
      *reinterpret_cast<uint4*>(&lds_b[buf][row * SB + part * 16]) = rb[c];
    }
    if (threadIdx.x < BMW) lds_as[buf][threadIdx.x] = ras;
    if (threadIdx.x < BNW) lds_bs[buf][threadIdx.x] = rbs;
  };

  // wave's B fragments: stage1 -> gate frags [wave*NFW/2, ...) of the gate block and the same
  // frags of the up block; stage2 -> frags [wave*NFW, (wave+1)*NFW)
  auto b_frag_row = [&](int j) -> int {
    if (STAGE == 1) {
      constexpr int H = NFW / 2;
      return j < H ? (wave * H + j) * 16 : BNW / 2 + (wave * H + (j - H)) * 16;
    }
    return (wave * NFW + j) * 16;
  };

  v4f acc[MF][NFW];
#pragma unroll
  for (int f = 0; f < MF; ++f)
#pragma unroll
    for (int j = 0; j < NFW; ++j) acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < S; ++s) {
    const int buf = s & 1;
    if (s + 1 < S) gload(s + 1);
    v8i bop[NFW];
    uint32_t bsc[NFW];
#pragma unroll
    for (int j = 0; j < NFW; ++j) {
      const int br = b_frag_row(j) + r16;
      const uint4 q = *reinterpret_cast<const uint4*>(&lds_b[buf][br * SB + 16 * g]);
      bop[j] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      bsc[j] = (lds_bs[buf][br] >> (8 * g)) & 0xFFu;
    }
#pragma unroll
    for (int f = 0; f < MF; ++f) {
      const int ar = 16 * f + r16;
      v8i aop;
      if (ADT == DT_FP8) {
        const uint4 lo = *reinterpret_cast<const uint4*>(&lds_a[buf][ar * SA + 16 * g]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&lds_a[buf][ar * SA + 64 + 16 * g]);
        aop = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      } else {
        const uint4 q = *reinterpret_cast<const uint4*>(&lds_a[buf][ar * SA + 16 * g]);
        aop = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      }
      const uint32_t asc = (lds_as[buf][ar] >> (8 * g)) & 0xFFu;
#pragma unroll
      for (int j = 0; j < NFW; ++j) {
        if (ADT == DT_FP8) acc[f][j] = mfma_fp8_fp4(aop, bop[j], acc[f][j], asc, bsc[j]);
        else acc[f][j] = mfma_fp4_fp4(aop, bop[j], acc[f][j], asc, bsc[j]);
      }
    }
    if (s + 1 < S) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogues
  if (STAGE == 1) {
    constexpr int H = NFW / 2;                  // gate fragments per wave (pairs with up)
    const float inv_beta = 1.0f / p.beta, inv_lb = 1.0f / p.linear_beta;
#pragma unroll
    for (int f = 0; f < MF; ++f) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * f + 4 * g + i;
        const bool valid = (unsigned)lds_v[row] < (unsigned)TK;
        const size_t R = (size_t)row_base + row;
#pragma unroll
        for (int jb = 0; jb < H; jb += 2) {      // one 32-column block = gate frags jb, jb+1
          float y[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float gs = acc[f][jb + h][i], us = acc[f][H + jb + h][i];
            y[h] = ACT == ACT_SITUV2 ? situv2(gs, us, p.beta, inv_beta, p.linear_beta, inv_lb) : silu_mul(gs, us);
          }
          uint32_t amax = max(__float_as_uint(y[0]) & 0x7FFFFFFFu, __float_as_uint(y[1]) & 0x7FFFFFFFu);
#pragma unroll
          for (int m = 8; m >= 1; m >>= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)amax, m, WAVE);
            amax = o > amax ? o : amax;
          }
          const int col0 = nb * (BNW / 2) + (wave * H + jb) * 16;   // intermediate column of the block
          uint32_t code[2], sbyte;
          if (amax >= 0x7F800000u) {
            sbyte = 255u; code[0] = code[1] = 0u;
          } else if (amax == 0u) {
            sbyte = 0u;
#pragma unroll
            for (int h = 0; h < 2; ++h)
              code[h] = (__float_as_uint(y[h]) >> 31) ? (ADT == DT_FP8 ? 0x80u : 0x8u) : 0u;
          } else if (ADT == DT_FP8) {
            const int sx = block_sexp<Fp8Fmt>(amax);
            sbyte = (uint32_t)(sx + 127);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t b = __float_as_uint(y[h]);
              code[h] = encode_mag<Fp8Fmt>(b & 0x7FFFFFFFu, sx) | ((b >> 31) ? 0x80u : 0u);
            }
          } else {
            const int sx = block_sexp<Fp4Fmt>(amax);
            sbyte = (uint32_t)(sx + 127);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t b = __float_as_uint(y[h]);
              code[h] = encode_mag<Fp4Fmt>(b & 0x7FFFFFFFu, sx) | ((b >> 31) ? 0x8u : 0u);
            }
          }
          if (ADT == DT_FP8) {
            if (valid) {
              p.inter[R * I + col0 + r16] = (uint8_t)code[0];
              p.inter[R * I + col0 + 16 + r16] = (uint8_t)code[1];
            }
          } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t partner = (uint32_t)__shfl_xor((int)code[h], 1, WAVE);
              if (valid && (r16 & 1) == 0)
                p.inter[R * (I / 2) + (col0 + 16 * h + r16) / 2] = (uint8_t)(code[h] | (partner << 4));
            }
          }
          if (valid && r16 == 0) p.inter_s[R * (I / 32) + col0 / 32] = (uint8_t)sbyte;
        }
      }
    }
  } else {
#pragma unroll
    for (int f = 0; f < MF; ++f) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * f + 4 * g + i;
        const int v = lds_v[row];
        if ((unsigned)v >= (unsigned)TK) continue;
        const float w = p.topk_w[v];
        const size_t R = (size_t)row_base + row;
        uint16_t* orow = reinterpret_cast<uint16_t*>(p.rowout) + R * D + nb * BNW + wave * NFW * 16 + r16;
#pragma unroll
        for (int j = 0; j < NFW; ++j) orow[16 * j] = bf16_rne(acc[f][j][i] * w);
      }
    }
  }
}

template <int ADT, int STAGE>
hipError_t launch_tiled_stage(const FusedArgs& a, const int2* groups, const int32_t* ngroups, hipStream_t s) {
  constexpr int GT = 4, BNW = 256;
  const int n_nblk = STAGE == 1 ? (2 * a.I) / BNW : a.D / BNW;
  const int64_t n_work = (int64_t)a.cap_tiles * n_nblk;   // groups <= tiles
  const unsigned grid = (unsigned)((n_work + 7) / 8 * 8);
  if (STAGE == 2)
    gemm_tiled_kernel<ADT, GT, BNW, 2, ACT_SITUV2><<<grid, THREADS, 0, s>>>(a, groups, ngroups, n_nblk);
  else if (a.act == ACT_SITUV2)
    gemm_tiled_kernel<ADT, GT, BNW, 1, ACT_SITUV2><<<grid, THREADS, 0, s>>>(a, groups, ngroups, n_nblk);
  else
    gemm_tiled_kernel<ADT, GT, BNW, 1, ACT_SILU><<<grid, THREADS, 0, s>>>(a, groups, ngroups, n_nblk);
  return hipGetLastError();
}

}  // namespace

bool tiled_path_supported(const FusedArgs& a) {
  return a.a_dtype != DT_BF16 && a.block_m == 32 && a.act != ACT_NONE && (2 * a.I) % 256 == 0 &&
         a.D % 256 == 0;
}

hipError_t launch_tiled(const FusedArgs& a, int2* groups, int32_t* ngroups, hipStream_t s) {
  hipError_t err;
  if (a.stages & 1) {
    group_kernel<4><<<1, GROUP_THREADS, 0, s>>>(a.expert_ids, a.num_tiles, a.cap_tiles, groups, ngroups);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    err = a.a_dtype == DT_FP8 ? launch_tiled_stage<DT_FP8, 1>(a, groups, ngroups, s)
                              : launch_tiled_stage<DT_FP4, 1>(a, groups, ngroups, s);
    if (err != hipSuccess) return err;
  }
  if (a.stages & 2) {
    err = a.a_dtype == DT_FP8 ? launch_tiled_stage<DT_FP8, 2>(a, groups, ngroups, s)
                              : launch_tiled_stage<DT_FP4, 2>(a, groups, ngroups, s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
