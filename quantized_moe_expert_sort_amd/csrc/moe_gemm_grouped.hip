// Large-batch Stage1 / Stage2: LDS-tiled block-scaled grouped GEMMs over groups of sort tiles.
//
// With many routed rows per expert (prefill, expert-parallel shards) the per-tile items of
// moe_stage_items.h re-stream an expert's weights for every 16/32-row tile.  Here a work item
// is (group, column block): a group is up to GT consecutive sort tiles of one expert (an
// expert's tiles are split into groups of balanced size), so each weight byte fetched serves
// up to GT*32 rows, and a column block is BNW weight rows.  Eight waves in a 2 (rows) x 4
// (weight rows) grid each compute a 128 x 64 sub-tile with v_mfma_scale_f32_16x16x128_f8f6f4
// (fp8 x fp4 or fp4 x fp4); 16-row fragments past the group's rows are skipped.  bf16
// activations take items of at most 128 rows (64 x 64 per wave) and v_mfma_f32_16x16x32_bf16 on
// weights widened to bf16 in registers.  Waves w and
// w + 4 share a SIMD and own the two row halves, so every SIMD does the same work whatever
// the group's row count.
//
// Operand staging: per 128-deep K step the A rows (gathered activations or intermediate rows)
// and the B rows (fp4 weights) are copied global -> LDS by the load-to-LDS instructions
// (global_load_lds_dwordx4 / _dword: lane l of a wave instruction writes bytes [16l, 16l+16)
// (or [4l, 4l+4)) after the wave's LDS address in m0), P steps in flight (P LDS buffers), one
// barrier per step; Stage1 copies the e8m0 scales of a row 16 bytes (four K steps) at a time.  The copies are issued from inline assembly,
// so the only waits on them are the explicit vmcnt waits of the pipeline.  The 16-byte chunks
// of an activation / intermediate row and of a Stage2 weight row are stored XOR-swizzled (chunk
// p of row r at position p ^ swz(r)), so the 16 lanes that read one chunk column of 16 rows for
// a matrix-core operand hit distinct LDS banks.  The weights arrive packed (moe_pack.hip): one
// copy instruction moves a whole 1 KB block (16 rows x one K step); Stage1 keeps the block in
// lane order, so a lane group's operand read is 256 consecutive bytes, and Stage2 has each lane
// fetch the 16-byte piece of the block that its swizzled LDS position holds.
//
// The grid is persistent: one workgroup per CU, each looping over work items.  Groups are
// dealt to the 8 XCDs round robin (workgroup b runs on XCD b % 8) and the column blocks of a
// group stay on one XCD, so its activation rows are fetched into one L2 and every XCD gets a
// similar mix of group sizes.
//
// Stage1 epilogue (github ROCm/aiter PR 6259 "Technical Details": SiTUv2 in the stage1
// epilogue): a wave's B rows are [32 gate rows | the matching 32 up rows], so g and u of one
// output sit in the same lane; y = act(g, u) is re-encoded per 32-column block (PR 4463 "Three
// tuner defects" item 2: fused fp4 stage1 output) with the block maximum reduced over 16 lanes.
// Stage2 (grouped_stage2_kernel below) stores bf16 rows without the router weight; the combine
// applies it.
#include "moe_kernels.h"
#include "moe_operands.h"

#include <type_traits>

#pragma clang diagnostic ignored "-Winline-asm"   // m0 is written by the load-to-LDS copies

namespace moe {

namespace {

constexpr int GT = 8;                         // sort tiles (of 32 rows) per group, at most
constexpr int GTHREADS = 512;
constexpr int GWAVES = GTHREADS / WAVE;       // 8
constexpr int WM = 2, WN = 4;                 // wave grid: rows x weight rows
constexpr int BNW = 256;                      // weight rows per column block
constexpr int NFW = BNW / WN / 16;            // 16-row B fragments per wave: 4
static_assert(WM * WN == GWAVES, "wave grid");

// ---------------------------------------------------------------- tile groups
//
// groups[g] = (first tile, tile count).  The tiles of an expert (a maximal run of equal
// expert_ids; the sort writes them in ascending expert order, so there are at most
// MOE_SORT_MAX_EXPERTS runs) are cut into groups of gs = ceil(n / ceil(n / GT)) tiles (the last
// one shorter).  One workgroup of 1024 threads, in three passes with a workgroup scan after each
// of the first two: (1) each thread counts the run starts (a tile whose expert differs from the
// previous tile's) in its contiguous chunk of tiles and records their positions in LDS; (2) each
// thread takes a contiguous chunk of runs and derives their group and hot counts, which the
// scans turn into output positions; (3) each thread writes the hot index of every tile of its
// tile chunk.  The tile -> expert map is staged in LDS (up to GROUP_LDS_TILES tiles, else read
// from global memory).

constexpr int GROUP_THREADS = 1024;
constexpr int GROUP_LDS_TILES = 16384;
constexpr int GROUP_MAX_RUNS = MOE_SORT_MAX_EXPERTS;
constexpr int HOT_MAX_G = MOE_HOT_MAX;

static_assert(GROUP_LDS_TILES % GROUP_THREADS == 0, "whole loads per thread");
static_assert(GROUP_MAX_RUNS % GROUP_THREADS == 0, "whole runs per thread");
// Besides the groups, the same passes pick the hot experts of the token-major Stage2 (below): an
// expert whose run has at least hot_min_tiles tiles is hot, hot indices follow the expert order
// up to MOE_HOT_MAX; every tile gets its expert's hot index (or -1) in tile_hot, the hot experts
// go to hot_e (their count at hot_e[MOE_HOT_MAX]) and the groups of the other experts, in order,
// to cgroups.
__global__ __launch_bounds__(GROUP_THREADS) void group_kernel(const int32_t* __restrict__ expert_ids,
                                                              const int32_t* __restrict__ num_tiles_p,
                                                              int cap, int2* __restrict__ groups,
                                                              int32_t* __restrict__ num_groups, int hot_min_tiles,
                                                              int2* __restrict__ cgroups,
                                                              int32_t* __restrict__ num_cgroups,
                                                              int32_t* __restrict__ tile_hot,
                                                              int32_t* __restrict__ hot_e) {
  __shared__ int lds_e[GROUP_LDS_TILES];
  __shared__ int run_start[GROUP_MAX_RUNS + 1];
  __shared__ int run_hot[GROUP_MAX_RUNS];
  __shared__ int tmp[2][GROUP_THREADS / WAVE + 1];
  const int n = min(*num_tiles_p, cap);
  const bool in_lds = n <= GROUP_LDS_TILES;
  if (in_lds) {   // GROUP_LDS_TILES / GROUP_THREADS loads per thread, all issued before the stores
    constexpr int PER = GROUP_LDS_TILES / GROUP_THREADS;
    int v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = threadIdx.x + u * GROUP_THREADS;
      v[u] = i < n ? expert_ids[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = threadIdx.x + u * GROUP_THREADS;
      if (i < n) lds_e[i] = v[u];
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  // exclusive scans of two per-thread counts over the workgroup; also the totals
  auto scan2 = [&](int v0, int v1, int (&ex)[2], int (&tot)[2]) {
    int vv[2] = {v0, v1};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      int sc = vv[q];
#pragma unroll
      for (int d = 1; d < WAVE; d <<= 1) {
        const int o = __shfl_up(sc, d, WAVE);
        if (lane >= d) sc += o;
      }
      if (lane == WAVE - 1) tmp[q][w] = sc;
      vv[q] = sc;
    }
    __syncthreads();
    if (threadIdx.x < 2) {
      int run = 0;
      for (int i = 0; i < GROUP_THREADS / WAVE; ++i) { const int c = tmp[threadIdx.x][i]; tmp[threadIdx.x][i] = run; run += c; }
      tmp[threadIdx.x][GROUP_THREADS / WAVE] = run;
    }
    __syncthreads();
    ex[0] = tmp[0][w] + vv[0] - v0;
    ex[1] = tmp[1][w] + vv[1] - v1;
    tot[0] = tmp[0][GROUP_THREADS / WAVE];
    tot[1] = tmp[1][GROUP_THREADS / WAVE];
    __syncthreads();
  };
  // the tile -> expert reads: one instantiation reads LDS, the other global memory (a select
  // between the two would become a generic-address load on every read)
  auto work = [&](auto E) {
    const int per = (n + GROUP_THREADS - 1) / GROUP_THREADS;
    const int t0 = min(n, (int)threadIdx.x * per), t1 = min(n, t0 + per);
    auto is_start = [&](int t) { return t == 0 || E(t) != E(t - 1); };
    // (1) run starts: positions in tile order
    int starts = 0;
    for (int t = t0; t < t1; ++t) starts += is_start(t);
    int ex[2], tot[2];
    scan2(starts, 0, ex, tot);
    const int rbase = ex[0];
    const int nruns = min(tot[0], GROUP_MAX_RUNS);      // ascending expert ids: at most that many
    {
      int r = rbase;
      for (int t = t0; t < t1; ++t)
        if (is_start(t)) {
          if (r < GROUP_MAX_RUNS) run_start[r] = t;
          ++r;
        }
    }
    if (threadIdx.x == 0) run_start[nruns] = n;
    __syncthreads();
    // (2) runs [r0, r1) of this thread: group counts and hot runs, then the cold group counts
    constexpr int RPT = GROUP_MAX_RUNS / GROUP_THREADS;
    const int rper = (nruns + GROUP_THREADS - 1) / GROUP_THREADS;   // <= RPT
    const int r0 = min(nruns, (int)threadIdx.x * rper), r1 = min(nruns, r0 + rper);
    int rs[RPT], len[RPT], gs[RPT], ng[RPT];
    int my_groups = 0, my_hot = 0;
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
      const int r = r0 + q;
      rs[q] = r < r1 ? run_start[r] : 0;
      len[q] = r < r1 ? run_start[r + 1] - rs[q] : 0;
      const int parts = (len[q] + GT - 1) / GT;
      gs[q] = parts > 0 ? (len[q] + parts - 1) / parts : 1;
      ng[q] = (len[q] + gs[q] - 1) / gs[q];
      my_groups += ng[q];
      my_hot += len[q] > 0 && len[q] >= hot_min_tiles;
    }
    scan2(my_groups, my_hot, ex, tot);
    const int nh = min(tot[1], HOT_MAX_G);
    int hq[RPT], my_cold = 0;
    {
      int h = ex[1];
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        const bool hot = len[q] > 0 && len[q] >= hot_min_tiles;
        hq[q] = hot && h < HOT_MAX_G ? h : -1;
        h += hot;
        my_cold += hq[q] < 0 ? ng[q] : 0;
      }
    }
    int exc[2], totc[2];
    scan2(my_cold, 0, exc, totc);
    {
      int gidx = ex[0], cidx = exc[0];
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        const int r = r0 + q;
        if (r >= r1) break;
        run_hot[r] = hq[q];
        if (hq[q] >= 0) hot_e[hq[q]] = E(rs[q]);
        for (int j = 0; j < ng[q]; ++j) {
          const int2 gr = int2{rs[q] + j * gs[q], min(gs[q], len[q] - j * gs[q])};
          groups[gidx++] = gr;
          if (hq[q] < 0) cgroups[cidx++] = gr;
        }
      }
    }
    __syncthreads();
    // (3) the hot index of every tile: its run is the last run starting at or before it
    {
      int r = rbase - 1;
      for (int t = t0; t < t1; ++t) {
        r += is_start(t);
        tile_hot[t] = r >= 0 && r < nruns ? run_hot[r] : -1;
      }
    }
    if (threadIdx.x == 0) {
      *num_groups = tot[0];
      *num_cgroups = totc[0];
      hot_e[HOT_MAX_G] = nh;
    }
    if (threadIdx.x < 8) num_groups[1 + threadIdx.x] = 0;   // the grouped Stage1's work counters
  };
  if (in_lds)
    work([&](int i) { return lds_e[i]; });
  else
    work([&](int i) { return expert_ids[i]; });
}

// ---------------------------------------------------------------- load-to-LDS copies

// 16 bytes per lane: global (base + off) -> LDS (lds + 16 * lane).  base and lds are
// wave-uniform.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base) : "memory", "m0");
}

// The same copy with the non-temporal hint, for the packed Stage1 weights: each instruction
// copies whole 128-byte lines, which in most groups no other item reads (ldw16 has the
// measurements).
__device__ __forceinline__ void dma16nt(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(lds), "v"(off), "s"(base) : "memory", "m0");
}

// 4 bytes per lane: global (base + off) -> LDS (lds + 4 * lane).
__device__ __forceinline__ void dma4(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(off), "s"(base) : "memory", "m0");
}

// Wait until at most n of this wave's vector memory operations are outstanding (they complete
// in issue order), then meet the other waves.  lgkmcnt(0): this wave's LDS accesses are done,
// so a buffer may be refilled once every wave has passed.  n = 63 waits for nothing; n > 63
// waits for everything.
__device__ __forceinline__ void wait_and_barrier(int n) {
  switch (n) {
#define MOE_WB(k) case k: asm volatile("s_waitcnt vmcnt(" #k ") lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    MOE_WB(1) MOE_WB(2) MOE_WB(3) MOE_WB(4) MOE_WB(5) MOE_WB(6) MOE_WB(7) MOE_WB(8) MOE_WB(9)
    MOE_WB(10) MOE_WB(11) MOE_WB(12) MOE_WB(13) MOE_WB(14) MOE_WB(15) MOE_WB(16) MOE_WB(17)
    MOE_WB(18) MOE_WB(19) MOE_WB(20) MOE_WB(21) MOE_WB(22) MOE_WB(23) MOE_WB(24) MOE_WB(25)
    MOE_WB(26) MOE_WB(27) MOE_WB(28) MOE_WB(29) MOE_WB(30) MOE_WB(31) MOE_WB(32) MOE_WB(33)
    MOE_WB(34) MOE_WB(35) MOE_WB(36) MOE_WB(37) MOE_WB(38) MOE_WB(39) MOE_WB(40) MOE_WB(41)
    MOE_WB(42) MOE_WB(43) MOE_WB(44) MOE_WB(45) MOE_WB(46) MOE_WB(47) MOE_WB(48) MOE_WB(49)
    MOE_WB(50) MOE_WB(51) MOE_WB(52) MOE_WB(53) MOE_WB(54) MOE_WB(55) MOE_WB(56) MOE_WB(57)
    MOE_WB(58) MOE_WB(59) MOE_WB(60) MOE_WB(61) MOE_WB(62)
#undef MOE_WB
    case 63: asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
  }
}

// Barrier for LDS data only: pending global stores of this wave are not waited for.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

// Position of 16-byte chunk `part` of row `row` in a row-major LDS tile with CPR chunks per row.
// A matrix-core operand read has the 16 lanes of a group read chunk `part` of 16 rows (16
// consecutive rows, or for the interleaved Stage2 weight rows rows {0-3, 8-11, 16-19, 24-27} of
// a 32-row block, plus 4); the XOR term (a function of the row only, so the fragments of a
// wave differ by constant offsets) spreads those reads over the banks.  For 64-byte rows it
// flips chunk bit 1 in rows with bit 3 set: on gfx950 a 16-byte read of chunk c from rows r and
// r + 8 costs a second LDS cycle (bank-conflict counter, microbenchmark over every XOR key of
// row bits 0-4: this key reads all three row sets conflict-free; the 128-byte key reads 16
// consecutive rows conflict-free).
template <int CPR>
__device__ __forceinline__ int swz_slot(int row, int part) {
  if constexpr (CPR == 16) return row * 16 + (part ^ (row & 15));
  else if constexpr (CPR == 8) return row * 8 + (part ^ (((row >> 1) ^ (row << 2)) & 7));
  else return row * 4 + (part ^ ((row >> 2) & 2));
}

// ---------------------------------------------------------------- grouped GEMM
//
// Wave roles.  On gfx9 a wave's loads and stores share one in-order completion counter
// (vmcnt), so a wave that waits for a load also waits for every store it issued before it.
// Waves 0..3 (the loaders) therefore issue every global load of the kernel (the operand
// copies, the row ids and router weights of an item) and never store; waves 4..7 (the
// storers) issue every global store (the item's output tile, staged in LDS) and never wait on
// vmcnt, so the output of one item drains while the next item's operands stream in.  All
// eight waves run the MFMAs.

constexpr int NLOAD = 4;                      // loader waves

// scalar (constant-cache) load of a wave-uniform address: counted by lgkmcnt, not vmcnt
__device__ __forceinline__ int ld_const(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)(uintptr_t)p;
}

// The grouped GEMMs take the fp4 weight rows as the MFMA's first operand and the activation /
// intermediate rows as its second: lane (r, g) of a 16 x 16 accumulator then holds the four
// consecutive weight rows (output columns) 4 g .. 4 g + 3 of activation row r.
template <int ADT>
__device__ __forceinline__ v4f mfma_w_x(const v8i& w, const v8i& x, const v4f& c, uint32_t sw, uint32_t sx) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x, c, MFMA_FMT_FP4,
                                                          ADT == DT_FP8 ? MFMA_FMT_FP8 : MFMA_FMT_FP4, 0, sw, 0, sx);
}

// bf16 activations / intermediate rows: an item takes one part of a group (up to 4 tiles, 128
// rows), so the 256-byte A row pieces of a K step leave room for three buffers; the B side
// (fp4 rows and their scales) is that of fp8 / fp4.
template <int ADT>
struct GFmt {
  static constexpr int GTA = ADT == DT_BF16 ? GT / 2 : GT;   // sort tiles per item, at most
  static constexpr int BM = GTA * 32;                     // rows per group
  static constexpr int MF = BM / WM / 16;                 // 16-row A fragments per wave
  static constexpr int KA = ADT == DT_FP8 ? 128 : ADT == DT_FP4 ? 64 : 256;   // A bytes per row per K step
  static constexpr int ACPR = KA / 16;                    // 16-byte chunks per A row
  static constexpr int P = ADT == DT_FP4 ? 4 : 3;         // LDS buffers = K steps in flight + 1
  // A fragments read ahead of the MFMAs (fp8: 1 measured 1.2% faster than 2 in the Stage1)
  static constexpr int AD = ADT == DT_FP4 ? 3 : 1;
  static constexpr int A_BYTES = BM * KA;
  static constexpr int B_BYTES = BNW * 64;
  static constexpr int BUF = A_BYTES + B_BYTES + (BM + BNW) * 4;   // Stage2: + per-step scale dwords
  static constexpr int A_IPL = A_BYTES / 1024 / NLOAD;    // A copy instructions per loader per step
  static constexpr int B_IPL = B_BYTES / 1024 / NLOAD;
  static constexpr int ROWS_PER_AI = 1024 / KA;           // A rows covered by one instruction
  static constexpr int OB = ADT == DT_FP8 ? BNW / 2 : ADT == DT_FP4 ? BNW / 4 : BNW;   // Stage1 output bytes per row
  static constexpr int OBS = OB + 16;                     // their LDS row stride
};

// Stage1 LDS: P operand buffers [A tile | B tile | A scale dwords (fp8)], then two slots of
// per-row scale chunks.  16 bytes of a row's e8m0 scales cover four K steps (512 columns), so a
// row's scales arrive with one 16-byte copy per four steps instead of a 4-byte copy per step
// (a copy instruction whose 64 lanes touch 64 different cache lines costs the memory pipeline
// as much as one that moves a kilobyte).  fp4 activations take A and B scales in chunks; the
// fp8 A tile leaves room for the B chunks only (its A scale dwords travel with each step); bf16
// activations have no scales.
template <int ADT>
struct S1Fmt {
  using F = GFmt<ADT>;
  static constexpr bool AW = ADT == DT_FP4;               // A scales in chunks
  static constexpr bool AS1 = ADT == DT_FP8;              // A scale dwords per step
  static constexpr int BUF = F::A_BYTES + F::B_BYTES + (AS1 ? F::BM * 4 : 0);
  static constexpr int A_SLOT = AW ? F::BM * 16 : 0;
  static constexpr int SLOT = A_SLOT + BNW * 16;
  static constexpr int BYTES = F::P * BUF + 2 * SLOT;
};

template <int ADT, int ACT>
__global__ __launch_bounds__(GTHREADS, 1) void grouped_stage1_kernel(FusedArgs p, const int2* __restrict__ groups,
                                                                    const int32_t* __restrict__ num_groups,
                                                                    int n_nblk) {
  using F = GFmt<ADT>;
  using L1 = S1Fmt<ADT>;
  constexpr int KA = F::KA, ACPR = F::ACPR, P = F::P, BM = F::BM, MF = F::MF;
  constexpr bool AW = L1::AW, AS1 = L1::AS1, HAS_AS = AW || AS1;
  static_assert(F::A_IPL * NLOAD * 1024 == F::A_BYTES && F::B_IPL * NLOAD * 1024 == F::B_BYTES, "copy split");
  static_assert(BM <= NLOAD * WAVE && BNW == NLOAD * WAVE, "at most one scale copy of each operand per loader");
  static_assert(BM * (F::OBS + 4) <= L1::BUF, "the staging tile fits one operand buffer");
  static_assert(P <= 5, "a chunk slot is refilled only after the four steps of its previous chunk");

  __shared__ __attribute__((aligned(1024))) uint8_t lds[L1::BYTES];
  __shared__ int lds_v[2][BM];                             // row ids of this item and the next
  __shared__ int s_claim;                                  // the item after the next one

  const int TK = p.T * p.topk, D = p.D, I = p.I;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);   // wave-uniform
  const bool loader = wave < NLOAD;
  const int lw = wave & (NLOAD - 1);
  const int r16 = lane & 15, g = lane >> 4;
  const int wm = wave / WN, wn = wave % WN;
  const int K = D;                                        // a multiple of 512: whole chunks
  const int S = K / 128;
  const uint32_t lds0 = lds_addr(lds);
  const uint32_t slot0 = lds0 + P * L1::BUF;

  // groups gi = xcd, xcd + 8, ... run on XCD xcd; item (part, group, column block), where a
  // bf16 group of more than GTA tiles is taken in two parts.  The column blocks of a group are
  // consecutive items, so they run at the same time on CUs of one XCD and fetch the group's
  // activation rows into its L2 once; second parts (empty for most small groups) come last.
  constexpr int PARTS = GT / F::GTA;
  const int ng = ld_const(num_groups);
  const int xcd = blockIdx.x & 7, stride = gridDim.x >> 3, local0 = blockIdx.x >> 3;
  const int per_part = (ng > xcd ? (ng - xcd + 7) / 8 : 0) * n_nblk;
  const int items_here = PARTS * per_part;
  const size_t a_rowbytes = (size_t)K * KA / 128;

  // item `local`: its column block and the first tile and tile count of its rows (bf16: a group
  // of up to GTA tiles is one part, a larger one two parts of ceil(n/2) and floor(n/2) tiles)
  auto item_tiles = [&](int local, int& tile0, int& ntile, int& nb) {
    const int part = local >= per_part ? 1 : 0, rem = local - part * per_part;
    const int gl = rem / n_nblk;
    nb = rem - gl * n_nblk;
    const int32_t* gp = reinterpret_cast<const int32_t*>(groups + gl * 8 + xcd);
    tile0 = ld_const(gp);
    ntile = ld_const(gp + 1);
    if (!MOE_DCHECK(tile0 >= 0 && ntile >= 0 && tile0 + ntile <= p.cap_tiles, DBG_GROUP)) tile0 = ntile = 0;
    if (PARTS == 2) {
      const int h0 = ntile <= F::GTA ? ntile : (ntile + 1) >> 1;
      tile0 += part ? h0 : 0;
      ntile = part ? ntile - h0 : h0;
    }
  };
  // this workgroup's first item at or after `local` that has rows (only a bf16 second part can
  // be empty), or items_here
  auto next_item = [&](int local) {
    if constexpr (PARTS == 2) {
      for (; local < items_here; local += stride) {
        int t0, nt, cb;
        item_tiles(local, t0, nt, cb);
        if (nt > 0) break;
      }
    }
    return local < items_here ? local : items_here;
  };

  // Copy sources of an item.  A: the gathered x rows (padding rows read token 0, their results
  // are never stored).  B: [gate NI | up NI] rows of column block nb (NI = BNW/2), one 1 KB block
  // of packed w1 per 16 rows and step.  Loader lw issues tile instructions j = i * NLOAD + lw
  // (A rows [j * ROWS_PER_AI, ...), instructions wholly past the group's rows are not issued;
  // B rows [16 j, 16 j + 16)) and the scales of A rows and B rows [64 lw, 64 lw + 64).
  struct Src {
    const uint8_t *b, *bs;
    uint32_t a_off[F::A_IPL], b_off[F::B_IPL], as_off, bs_off;
    int n_ai, n_data, n_chunk, rows_used, row_base, nb;
    bool as_on;
  };
  // every wave: the item's rows and column block; the loaders also the copy offsets (their
  // rows' token ids read from the sorted layout) and the item's row ids in lds_v[vb]
  auto make = [&](int local, Src& q, int vb) {
    int tile0, ntile;
    item_tiles(local, tile0, ntile, q.nb);
    q.rows_used = ntile * 32;
    q.row_base = tile0 * 32;
    if (!loader) return;
    const int e = dcheck_expert(ld_const(p.expert_ids + tile0), p.E);
    q.b = p.w1 + (size_t)e * 2 * I * (D / 2);
    q.bs = p.w1s + (size_t)e * 2 * I * (D / 32);
    auto b_row = [&](int r) -> int {                      // weight row within the expert
      constexpr int NI = BNW / 2;
      return r < NI ? q.nb * NI + r : I + q.nb * NI + (r - NI);
    };
    // the row ids of the loader's A rows and of its scale row (= its lds_v row), loaded together
    // (indices clamped into the group; rows past it are padding); the lane index is re-derived
    // here so that nothing computed from it stays live across the item loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int sc_row = lw * WAVE + ln;
    int rid[F::A_IPL + 1];
#pragma unroll
    for (int i = 0; i < F::A_IPL; ++i)
      rid[i] = p.sorted_ids[q.row_base + min(((i * NLOAD + lw) * WAVE + ln) / ACPR, q.rows_used - 1)];
    rid[F::A_IPL] = p.sorted_ids[q.row_base + min(sc_row, q.rows_used - 1)];
#pragma unroll
    for (int i = 0; i <= F::A_IPL; ++i) dcheck_row_id(rid[i], TK);
    auto tok = [&](int row, int v) -> uint32_t {          // token row of A row `row`
      return (uint32_t)(row < q.rows_used && (unsigned)v < (unsigned)TK ? v / p.topk : 0);
    };
    int n_ai = 0;
#pragma unroll
    for (int i = 0; i < F::A_IPL; ++i) {
      const int j = i * NLOAD + lw;
      const int qq = j * WAVE + ln;
      const int row = qq / ACPR, part = swz_slot<ACPR>(row, qq % ACPR) - row * ACPR;   // the XOR is an involution
      q.a_off[i] = tok(row, rid[i]) * (uint32_t)a_rowbytes + part * 16;
      n_ai += j * F::ROWS_PER_AI < q.rows_used;
    }
#pragma unroll
    for (int i = 0; i < F::B_IPL; ++i) {
      const int j = i * NLOAD + lw;
      q.b_off[i] = (uint32_t)(b_row(16 * j) / 16) * (uint32_t)(S * 1024) + 16 * ln;
    }
    q.as_on = HAS_AS && lw * WAVE < q.rows_used;          // rows_used <= BM
    q.as_off = HAS_AS && sc_row < BM ? tok(sc_row, rid[F::A_IPL]) * (uint32_t)(K / 32) : 0u;
    q.bs_off = (uint32_t)b_row(sc_row) * (uint32_t)(K / 32);
    q.n_ai = n_ai;
    // copy instructions a loader issues for step s: the chunks travel with steps 0, 4, 8, ...
    q.n_data = n_ai + F::B_IPL + (AS1 && q.as_on ? 1 : 0);
    q.n_chunk = 1 + (AW && q.as_on ? 1 : 0);
    if (sc_row < BM) lds_v[vb][sc_row] = sc_row < q.rows_used ? rid[F::A_IPL] : TK;
  };
  // per step the K advance goes into the (scalar) global base; lane offsets stay fixed.  The
  // chunk copies are issued first, so the wait for a step's tiles covers them.
  auto issue = [&](const Src& q, int s, int buf) {
    if ((s & 3) == 0) {
      const uint32_t C = __builtin_amdgcn_readfirstlane(slot0 + ((s >> 2) & 1) * L1::SLOT);
      const int cb = (s >> 2) * 16;
      if (AW && q.as_on) dma16(p.xs + cb, q.as_off, C + lw * 1024);
      dma16(q.bs + cb, q.bs_off, C + L1::A_SLOT + lw * 1024);
    }
    const uint32_t L = __builtin_amdgcn_readfirstlane(lds0 + buf * L1::BUF);
    const uint8_t* ab = p.x + s * KA;
    const uint8_t* bb = q.b + s * 1024;
#pragma unroll
    for (int i = 0; i < F::A_IPL; ++i)
      if (i < q.n_ai) dma16(ab, q.a_off[i], L + (i * NLOAD + lw) * 1024);
#pragma unroll
    for (int i = 0; i < F::B_IPL; ++i)
      dma16nt(bb, q.b_off[i], L + F::A_BYTES + (i * NLOAD + lw) * 1024);
    if (AS1 && q.as_on) dma4(p.xs + s * 4, q.as_off, L + F::A_BYTES + F::B_BYTES + lw * 256);
  };

  // Items are taken two ahead: the first two of a workgroup are local0 and local0 + stride; with
  // fp8 / fp4 rows every later one is claimed from the XCD's work counter (zeroed by the group
  // kernel) during the epilogue of the item before the next, so workgroups that drew smaller
  // groups take more items; bf16 items (whose second parts may be empty) keep the fixed stride.
  constexpr bool DYN = PARTS == 1;
  int32_t* const ctr = const_cast<int32_t*>(num_groups) + 1 + xcd;

  // The first P-1 steps of an item are issued before its K loop: for the first item here, for
  // every later one during the epilogue of the item before (its staging tile sits in buffer
  // P-1, the copies go to buffers 0 .. P-2), so an item's first operands are in flight while the
  // previous item's activation, re-encode and stores run.
  Src cur, nxt;
  int local = next_item(local0), vb = 0;
  int nl = local < items_here ? next_item(local + stride) : items_here;
  if (local < items_here) {
    make(local, cur, 0);
    if (loader) {
#pragma unroll
      for (int q = 0; q < P - 1; ++q)
        if (q < S) issue(cur, q, q);
    }
  }
  lds_barrier();                                          // lds_v[0] is complete

  while (local < items_here) {
    const int rows_used = cur.rows_used, row_base = cur.row_base, nb = cur.nb;

    // the wave's B fragment rows: gate rows [32wn, 32wn+32) and the same up rows
    auto b_frag_row = [&](int j) -> int { return j < 2 ? 32 * wn + 16 * j : BNW / 2 + 32 * wn + 16 * (j - 2); };
    // A fragments of a wave: with fp8 / fp4 rows they alternate between the two wave rows
    // (fragment f of wave row wm holds rows 16 (2 f + wm) .. + 15), so the two waves of a SIMD
    // (w and w + 4) get the same count, rows_used / 32, for any group size (ep-8192 Stage1
    // 501 -> 481 us, pre-a8-8192 504 -> 485); bf16 keeps contiguous row halves (measured 1%
    // faster there), 0, 2 or 4 fragments.  The MFMA loop is instantiated per count (no
    // per-fragment branches inside it).
    constexpr bool ALT = ADT != DT_BF16;
    constexpr int FS = ALT ? 32 : 16;                      // row step between a wave's fragments
    const int arow0 = ALT ? 16 * wm : (BM / WM) * wm;      // the wave's first A row
    const int n_af = max(0, min(MF, ALT ? (rows_used - arow0 + 31) / 32 : (rows_used - arow0) / 16));

    auto run = [&](auto na_c) {
      constexpr int NA = decltype(na_c)::value;
      v4f acc[NA > 0 ? NA : 1][NFW];
#pragma unroll
      for (int f = 0; f < NA; ++f)
#pragma unroll
        for (int j = 0; j < NFW; ++j) acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};

      auto compute_bf16 = [&](int s) {
        const uint8_t* la = lds + (s % P) * L1::BUF;
        const uint8_t* lb = la + F::A_BYTES;
        const uint8_t* slot = lds + P * L1::BUF + ((s >> 2) & 1) * L1::SLOT;
        const int kq = (s & 3) * 4;
        // lane group g takes K [32 g, 32 g + 32) of the step (one scale block) for both
        // operands: four 32-deep bf16 MFMAs, sub-step jj on K [32 g + 8 jj, 32 g + 8 jj + 8);
        // the fp4 weights are widened to bf16 once per step with the scaled converts
        v8bf bop[NFW][4];
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
          const int br = b_frag_row(j) + r16;
          // packed B block of rows b_frag_row(j) .. + 15: lane (r16, g) at 16 (16 g + r16)
          const uint4 q = *reinterpret_cast<const uint4*>(lb + b_frag_row(j) * 64 + lane * 16);
          const uint32_t bs = (*reinterpret_cast<const uint32_t*>(slot + L1::A_SLOT + br * 16 + kq) >> (8 * g)) & 0xFFu;
          const float sc = e8m0_to_float(bs);
          bop[j][0] = fp4x8_to_bf16(q.x, sc);
          bop[j][1] = fp4x8_to_bf16(q.y, sc);
          bop[j][2] = fp4x8_to_bf16(q.z, sc);
          bop[j][3] = fp4x8_to_bf16(q.w, sc);
        }
        auto load_a = [&](int f, v8bf* a) {
          const int ar = arow0 + FS * f + r16;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const uint4 q = *reinterpret_cast<const uint4*>(la + swz_slot<16>(ar, 4 * g + jj) * 16);
            a[jj] = as_bf16x8(q.x, q.y, q.z, q.w);
          }
        };
        constexpr int AD = F::AD;
        v8bf aq[AD + 1][4];
#pragma unroll
        for (int d = 0; d < AD; ++d)
          if (d < NA) load_a(d, aq[d]);
#pragma unroll
        for (int f = 0; f < NA; ++f) {
          if (f + AD < NA) load_a(f + AD, aq[(f + AD) % (AD + 1)]);
          const v8bf* a_cur = aq[f % (AD + 1)];
          // sub-step outer: consecutive MFMAs write different accumulators, so none waits for
          // the one before it (a wave alone on its SIMD would stall on a dependent chain)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int j = 0; j < NFW; ++j) acc[f][j] = mfma_bf16(bop[j][jj], a_cur[jj], acc[f][j]);
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      auto compute_q = [&](int s) {
        const uint8_t* la = lds + (s % P) * L1::BUF;
        const uint8_t* lb = la + F::A_BYTES;
        const uint32_t* las = reinterpret_cast<const uint32_t*>(lb + F::B_BYTES);
        // this step's scale dword of row r in the chunk slot: bytes [16 r + kq, 16 r + kq + 4)
        const uint8_t* slot = lds + P * L1::BUF + ((s >> 2) & 1) * L1::SLOT;
        const int kq = (s & 3) * 4;
        v8i bop[NFW];
        uint32_t bsc[NFW];
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
          const int br = b_frag_row(j) + r16;
          bop[j] = fp4_operand_lo(*reinterpret_cast<const uint4*>(lb + b_frag_row(j) * 64 + lane * 16));
          bsc[j] = (*reinterpret_cast<const uint32_t*>(slot + L1::A_SLOT + br * 16 + kq) >> (8 * g)) & 0xFFu;
        }
        // A fragment f+AD is read from LDS while the MFMAs of fragment f run (an LDS read
        // takes longer than the four MFMAs of one fragment); the scheduling barrier keeps the
        // compiler from hoisting every fragment read (register pressure)
        auto load_a = [&](int f, v8i& aop, uint32_t& asc) {
          const int ar = arow0 + FS * f + r16;
          if (ADT == DT_FP8) {
            const uint4 lo = *reinterpret_cast<const uint4*>(la + swz_slot<8>(ar, g) * 16);
            const uint4 hi = *reinterpret_cast<const uint4*>(la + swz_slot<8>(ar, 4 + g) * 16);
            aop = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          } else {
            aop = fp4_operand_lo(*reinterpret_cast<const uint4*>(la + swz_slot<4>(ar, g) * 16));
          }
          const uint32_t sw = AW ? *reinterpret_cast<const uint32_t*>(slot + ar * 16 + kq) : AS1 ? las[ar] : 0u;
          asc = sw;                                     // the byte is taken where it is used
        };
        constexpr int AD = F::AD;
        v8i aq[AD + 1];
        uint32_t asq[AD + 1];
#pragma unroll
        for (int d = 0; d < AD; ++d)
          if (d < NA) load_a(d, aq[d], asq[d]);
#pragma unroll
        for (int f = 0; f < NA; ++f) {
          if (f + AD < NA) load_a(f + AD, aq[(f + AD) % (AD + 1)], asq[(f + AD) % (AD + 1)]);
          const v8i& a_cur = aq[f % (AD + 1)];
          const uint32_t as_cur = (asq[f % (AD + 1)] >> (8 * g)) & 0xFFu;
#pragma unroll
          for (int j = 0; j < NFW; ++j) acc[f][j] = mfma_w_x<ADT>(bop[j], a_cur, acc[f][j], bsc[j], as_cur);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      auto compute = [&](int s) {
        if constexpr (ADT == DT_BF16) compute_bf16(s);
        else compute_q(s);
      };

      // ---- K loop: steps s+1 .. s+P-2 in flight while step s is computed
      for (int s = 0; s < S; ++s) {
        // a loader's copies of step s are done once at most those of the later steps in
        // flight remain
        int later = 0;
#pragma unroll
        for (int t = 1; t <= P - 2; ++t)
          if (s + t < S) later += cur.n_data + (((s + t) & 3) == 0 ? cur.n_chunk : 0);
        wait_and_barrier(loader ? later : 63);
        if (loader && s + P - 1 < S) issue(cur, s + P - 1, (s + P - 1) % P);   // refills the buffer of step s-1
        if (NA > 0) compute(s);
      }
      lds_barrier();                                      // every operand read of the item is done
      if (nl < items_here) {                              // the next item's first steps
        make(nl, nxt, vb ^ 1);
        if (loader) {
#pragma unroll
          for (int q = 0; q < P - 1; ++q)
            if (q < S) issue(nxt, q, q);
        }
      }

      // ---- epilogue: the item's output tile is staged in LDS buffer P-1 by every wave
      {
        // the first storer wave claims the item after the next one (its result is read after
        // the activation math; this wave waits on no copies)
        int claim = 0;
        if (DYN && wave == NLOAD && lane == 0 && nl < items_here) claim = atomicAdd(ctr, 1);
        uint8_t* st_codes = lds + (P - 1) * L1::BUF;      // [BM][OBS]
        uint8_t* st_scales = st_codes + BM * F::OBS;      // [BM][4]: one byte per 32-column block
        const float inv_beta = 1.0f / p.beta, inv_lb = 1.0f / p.linear_beta;
        // lane (r16, g) holds, for row arow0 + FS f + r16, the gate sums (fragments 0, 1) and
        // the up sums (fragments 2, 3) of the four consecutive columns 32 wn + 16 h + 4 g + i:
        // one 1x32 block per row and wave, its 32 values in the four lanes r16 + 16 g
#pragma unroll
        for (int f = 0; f < NA; ++f) {
          const int row = arow0 + FS * f + r16;
          float y[2][4];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float gs = acc[f][h][i], us = acc[f][2 + h][i];
              y[h][i] = ACT == ACT_SITUV2 ? situv2(gs, us, p.beta, inv_beta, p.linear_beta, inv_lb) : silu_mul(gs, us);
            }
          if constexpr (ADT == DT_BF16) {   // bf16 intermediate: four columns in one 8-byte write
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint2 v = {(uint32_t)f32_to_bf16_rne(y[h][0]) | ((uint32_t)f32_to_bf16_rne(y[h][1]) << 16),
                               (uint32_t)f32_to_bf16_rne(y[h][2]) | ((uint32_t)f32_to_bf16_rne(y[h][3]) << 16)};
              *reinterpret_cast<uint2*>(st_codes + row * F::OBS + 2 * (32 * wn + 16 * h + 4 * g)) = v;
            }
            continue;
          }
          uint32_t m = 0;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = max(m, __float_as_uint(y[h][i]) & 0x7FFFFFFFu);
          const uint32_t amax = cross_row_max_u32(m);
          // the 1x32 rule with the hardware converts, two columns per convert; an Inf / NaN
          // block gets scale 255 and zero codes
          const bool bad = amax >= 0x7F800000u;
          const int sexp = block_sexp_any(bad ? 0u : amax, ADT == DT_FP8 ? Fp8Fmt::EMAX : Fp4Fmt::EMAX);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int c = 32 * wn + 16 * h + 4 * g;
            if (ADT == DT_FP8) {
              const uint32_t lo = bad ? 0u : encode_pair_fp8_hw(y[h][0], y[h][1], sexp);
              const uint32_t hi = bad ? 0u : encode_pair_fp8_hw(y[h][2], y[h][3], sexp);
              *reinterpret_cast<uint32_t*>(st_codes + row * F::OBS + c) = lo | (hi << 16);
            } else {
              const float scale = e8m0_scale_float(sexp);
              const uint32_t lo = bad ? 0u : encode_pair_fp4_hw(y[h][0], y[h][1], scale);
              const uint32_t hi = bad ? 0u : encode_pair_fp4_hw(y[h][2], y[h][3], scale);
              *reinterpret_cast<uint16_t*>(st_codes + row * F::OBS + c / 2) = (uint16_t)(lo | (hi << 8));
            }
          }
          st_scales[row * 4 + wn] = (uint8_t)(bad ? 255u : (uint32_t)(sexp + 127));
        }
        if (DYN && wave == NLOAD && lane == 0) s_claim = nl < items_here ? min(2 * stride + claim, items_here) : items_here;
        lds_barrier();
        if (!loader) {
          const int t = threadIdx.x - NLOAD * WAVE;
          constexpr int CPRO = F::OB / 16;
          const size_t irow = ADT == DT_FP8 ? (size_t)I : ADT == DT_FP4 ? (size_t)I / 2 : (size_t)I * 2;   // intermediate row bytes
          for (int c = t; c < rows_used * CPRO; c += (GWAVES - NLOAD) * WAVE) {
            const int row = c / CPRO, part = c - row * CPRO;
            if ((unsigned)lds_v[vb][row] < (unsigned)TK) {
              const size_t R = (size_t)row_base + row;
              *reinterpret_cast<uint4*>(p.inter + R * irow + (size_t)nb * F::OB + part * 16) =
                  *reinterpret_cast<const uint4*>(st_codes + row * F::OBS + part * 16);
            }
          }
          for (int row = t; ADT != DT_BF16 && row < rows_used; row += (GWAVES - NLOAD) * WAVE) {
            if ((unsigned)lds_v[vb][row] < (unsigned)TK) {
              const size_t R = (size_t)row_base + row;
              *reinterpret_cast<uint32_t*>(p.inter_s + R * (I / 32) + (size_t)nb * 4) =
                  *reinterpret_cast<const uint32_t*>(st_scales + row * 4);
            }
          }
        }
      }
    };
    if constexpr (MF == 4) {
      switch (n_af) {
        case 0: run(std::integral_constant<int, 0>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        default: run(std::integral_constant<int, 4>{}); break;
      }
    } else {
      static_assert(MF == 8 && ALT, "fragment counts");
      switch (n_af) {
        case 0: run(std::integral_constant<int, 0>{}); break;
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        case 4: run(std::integral_constant<int, 4>{}); break;
        case 5: run(std::integral_constant<int, 5>{}); break;
        case 6: run(std::integral_constant<int, 6>{}); break;
        case 7: run(std::integral_constant<int, 7>{}); break;
        default: run(std::integral_constant<int, 8>{}); break;
      }
    }
    lds_barrier();                                        // the staging tile and lds_v[vb] are reused
    const int nn = DYN ? __builtin_amdgcn_readfirstlane(s_claim) : (nl < items_here ? next_item(nl + stride) : items_here);
    cur = nxt;
    local = nl;
    nl = nn;
    vb ^= 1;
  }
}

// ---------------------------------------------------------------- grouped Stage2
//
// Stage2 items stage nothing in LDS.  The MFMA takes the weight rows as its first operand and
// the intermediate rows as its second, so lane (r, g) of a 16 x 16 accumulator holds four
// consecutive output columns of row r; the weight rows of a wave's four fragments are
// interleaved (row m of fragment j is output column 32 (j / 2) + 8 (m / 4) + 4 (j % 2) + m % 4 of
// the wave's 64), so a lane ends up with two runs of 8 consecutive columns of one row, written
// as two 16-byte stores that cover 64 contiguous bytes per row across the lane groups.  The operand buffers are free as soon as the K loop ends: the loader waves issue the
// next item's first P-1 steps before storing, and one item's output drains while the next
// item's operands arrive (the loaders' waits count the stores issued after those copies).  The
// rows are stored without the router weight; the combine applies it.

template <int ADT>
__global__ __launch_bounds__(GTHREADS, 1) void grouped_stage2_kernel(FusedArgs p, const int2* __restrict__ groups,
                                                                     const int32_t* __restrict__ num_groups,
                                                                     int n_nblk) {
  using F = GFmt<ADT>;
  constexpr int KA = F::KA, ACPR = F::ACPR, P = F::P, BM = F::BM, MF = F::MF;
  constexpr bool HAS_AS = ADT != DT_BF16;
  constexpr int PARTS = GT / F::GTA;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[P * F::BUF];

  const int D = p.D, I = p.I;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);   // wave-uniform
  const bool loader = wave < NLOAD;
  const int lw = wave & (NLOAD - 1);
  const int r16 = lane & 15, g = lane >> 4;
  const int wm = wave / WN, wn = wave % WN;
  const int S = I / 128;
  const uint32_t lds0 = lds_addr(lds);
  const size_t a_rowbytes = (size_t)I * KA / 128;

  const int ng = ld_const(num_groups);
  const int xcd = blockIdx.x & 7, stride = gridDim.x >> 3, local0 = blockIdx.x >> 3;
  const int per_part = (ng > xcd ? (ng - xcd + 7) / 8 : 0) * n_nblk;   // items (part, group, column block)
  const int items_here = PARTS * per_part;

  struct Src {
    const uint8_t *a, *as, *b, *bs;
    uint32_t a_off[F::A_IPL], b_off[F::B_IPL], as_off, bs_off;
    int n_ai, rows_used, row_base, nb, per_step;
    bool as_on, b_on;
  };
  // copy sources of item `local`: A the group's intermediate rows (rows past the group read its
  // first row; their results are not stored), B output rows [nb*BNW, nb*BNW + BNW) of packed
  // w2 (16 rows x one K step per 1 KB block: piece (row r, chunk p) at 16 (16 p + r % 16))
  // (bf16: a group of up to GTA tiles is one part, a larger one two parts of ceil(n/2) and
  // floor(n/2) tiles; the empty second part of a small group copies nothing)
  auto make = [&](int local, Src& q) {
    const int part = local >= per_part ? 1 : 0, rem = local - part * per_part;
    const int gl = rem / n_nblk;
    q.nb = rem - gl * n_nblk;
    const int32_t* gp = reinterpret_cast<const int32_t*>(groups + gl * 8 + xcd);
    int tile0 = ld_const(gp), ntiles = ld_const(gp + 1);
    if (!MOE_DCHECK(tile0 >= 0 && ntiles >= 0 && tile0 + ntiles <= p.cap_tiles, DBG_GROUP)) tile0 = ntiles = 0;
    if (PARTS == 2) {
      const int h0 = ntiles <= F::GTA ? ntiles : (ntiles + 1) >> 1;
      tile0 += part ? h0 : 0;
      ntiles = part ? ntiles - h0 : h0;
    }
    q.rows_used = ntiles * 32;
    q.row_base = tile0 * 32;
    const int e = dcheck_expert(ld_const(p.expert_ids + tile0), p.E);
    q.a = p.inter + (size_t)q.row_base * a_rowbytes;
    q.as = p.inter_s + (size_t)q.row_base * (I / 32);
    q.b = p.w2 + (size_t)e * D * (I / 2);
    q.bs = p.w2s + (size_t)e * D * (I / 32);
    int n_ai = 0;
#pragma unroll
    for (int i = 0; i < F::A_IPL; ++i) {
      const int j = i * NLOAD + lw;
      const int qq = j * WAVE + lane;
      const int row = qq / ACPR, part = swz_slot<ACPR>(row, qq % ACPR) - row * ACPR;
      q.a_off[i] = (uint32_t)(row < q.rows_used ? row : 0) * (uint32_t)a_rowbytes + part * 16;
      n_ai += j * F::ROWS_PER_AI < q.rows_used;
    }
#pragma unroll
    for (int i = 0; i < F::B_IPL; ++i) {
      const int j = i * NLOAD + lw;
      const int qq = j * WAVE + lane;
      const int row = qq / 4, part = swz_slot<4>(row, qq % 4) - row * 4;
      q.b_off[i] = (uint32_t)((q.nb * BNW + row) / 16) * (uint32_t)(8 * I) + 16 * (16 * part + row % 16);
    }
    const int sc_row = lw * WAVE + lane;
    q.as_on = HAS_AS && lw * WAVE < q.rows_used;
    q.b_on = q.rows_used > 0;
    q.as_off = (uint32_t)(sc_row < q.rows_used ? sc_row : 0) * (uint32_t)(I / 32);
    q.bs_off = (uint32_t)(q.nb * BNW + sc_row) * (uint32_t)(I / 32);
    q.n_ai = n_ai;
    q.per_step = n_ai + (q.b_on ? F::B_IPL + 1 : 0) + (q.as_on ? 1 : 0);
  };
  auto issue = [&](const Src& q, int s, int buf) {
    const uint32_t L = __builtin_amdgcn_readfirstlane(lds0 + buf * F::BUF);
    const uint8_t* ab = q.a + s * KA;
    const uint8_t* bb = q.b + s * 1024;
#pragma unroll
    for (int i = 0; i < F::A_IPL; ++i)
      if (i < q.n_ai) dma16(ab, q.a_off[i], L + (i * NLOAD + lw) * 1024);
    if (!q.b_on) return;
#pragma unroll
    for (int i = 0; i < F::B_IPL; ++i)
      dma16nt(bb, q.b_off[i], L + F::A_BYTES + (i * NLOAD + lw) * 1024);
    if (q.as_on) dma4(q.as + s * 4, q.as_off, L + F::A_BYTES + F::B_BYTES + lw * 256);
    dma4(q.bs + s * 4, q.bs_off, L + F::A_BYTES + F::B_BYTES + BM * 4 + lw * 256);
  };

  // A fragments alternate between the two wave rows: fragment f of wave row wm holds rows
  // 16 (2 f + wm) .. + 15, so the waves sharing a SIMD (w and w + 4) have the same number of
  // fragments for any group size (4% faster at 8192 tokens than contiguous row halves)
  const int arow0 = 16 * wm;
  Src cur, nxt;
  int local = local0;
  if (local < items_here) {
    make(local, cur);
    if (loader) {
#pragma unroll
      for (int q = 0; q < P - 1; ++q)
        if (q < S) issue(cur, q, q);
    }
  }
  int n_st = 0;   // stores this wave issued after the current item's first copies
  for (; local < items_here; local += stride) {
    const bool has_next = local + stride < items_here;
    if (has_next) make(local + stride, nxt);
    const int n_af = max(0, min(MF, (cur.rows_used - arow0 + 2 * 16 - 1) / (2 * 16)));

    auto run = [&](auto na_c) {
      constexpr int NA = decltype(na_c)::value;
      v4f acc[NA > 0 ? NA : 1][NFW];
#pragma unroll
      for (int f = 0; f < NA; ++f)
#pragma unroll
        for (int j = 0; j < NFW; ++j) acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};

      // bf16 intermediate rows: lane group g takes K [32 g, 32 g + 32) of the step for both
      // operands (one weight scale block), four 32-deep bf16 MFMAs per 16 x 16 block, the fp4
      // weight rows widened to bf16 with the scaled converts
      auto compute_bf16 = [&](int buf) {
        const uint8_t* la = lds + buf * F::BUF;
        const uint8_t* lb = la + F::A_BYTES;
        const uint32_t* lbs = reinterpret_cast<const uint32_t*>(lb + F::B_BYTES) + BM;
        v8bf wop[NFW][4];
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
          const int br = 64 * wn + (j >> 1) * 32 + 8 * (r16 >> 2) + 4 * (j & 1) + (r16 & 3);
          const uint4 q = *reinterpret_cast<const uint4*>(lb + swz_slot<4>(br, g) * 16);
          const float sc = e8m0_to_float((lbs[br] >> (8 * g)) & 0xFFu);
          wop[j][0] = fp4x8_to_bf16(q.x, sc);
          wop[j][1] = fp4x8_to_bf16(q.y, sc);
          wop[j][2] = fp4x8_to_bf16(q.z, sc);
          wop[j][3] = fp4x8_to_bf16(q.w, sc);
        }
        auto load_x = [&](int f, v8bf* x) {
          const int ar = arow0 + 32 * f + r16;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const uint4 q = *reinterpret_cast<const uint4*>(la + swz_slot<16>(ar, 4 * g + jj) * 16);
            x[jj] = as_bf16x8(q.x, q.y, q.z, q.w);
          }
        };
        v8bf x_cur[4];
        load_x(0, x_cur);
#pragma unroll
        for (int f = 0; f < NA; ++f) {
          v8bf x_nxt[4] = {x_cur[0], x_cur[1], x_cur[2], x_cur[3]};
          if (f + 1 < NA) load_x(f + 1, x_nxt);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int j = 0; j < NFW; ++j) acc[f][j] = mfma_bf16(wop[j][jj], x_cur[jj], acc[f][j]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) x_cur[jj] = x_nxt[jj];
        }
      };

      auto compute_q = [&](int buf) {
        const uint8_t* la = lds + buf * F::BUF;
        const uint8_t* lb = la + F::A_BYTES;
        const uint32_t* las = reinterpret_cast<const uint32_t*>(lb + F::B_BYTES);
        const uint32_t* lbs = las + BM;
        v8i wop[NFW];
        uint32_t wsc[NFW];
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
          const int br = 64 * wn + (j >> 1) * 32 + 8 * (r16 >> 2) + 4 * (j & 1) + (r16 & 3);
          wop[j] = fp4_operand_lo(*reinterpret_cast<const uint4*>(lb + swz_slot<4>(br, g) * 16));
          wsc[j] = (lbs[br] >> (8 * g)) & 0xFFu;
        }
        auto load_x = [&](int f, v8i& xop, uint32_t& xsc) {
          const int ar = arow0 + 32 * f + r16;
          if (ADT == DT_FP8) {
            const uint4 lo = *reinterpret_cast<const uint4*>(la + swz_slot<8>(ar, g) * 16);
            const uint4 hi = *reinterpret_cast<const uint4*>(la + swz_slot<8>(ar, 4 + g) * 16);
            xop = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          } else {
            xop = fp4_operand_lo(*reinterpret_cast<const uint4*>(la + swz_slot<4>(ar, g) * 16));
          }
          xsc = las[ar];                                // the byte is taken where it is used
        };
        v8i x_cur;
        uint32_t xs_cur;
        load_x(0, x_cur, xs_cur);
#pragma unroll
        for (int f = 0; f < NA; ++f) {
          v8i x_nxt = x_cur;
          uint32_t xs_nxt = xs_cur;
          if (f + 1 < NA) load_x(f + 1, x_nxt, xs_nxt);
          const uint32_t xb = (xs_cur >> (8 * g)) & 0xFFu;
#pragma unroll
          for (int j = 0; j < NFW; ++j) acc[f][j] = mfma_w_x<ADT>(wop[j], x_cur, acc[f][j], wsc[j], xb);
          __builtin_amdgcn_sched_barrier(0);
          x_cur = x_nxt;
          xs_cur = xs_nxt;
        }
      };
      auto compute = [&](int buf) {
        if constexpr (ADT == DT_BF16) compute_bf16(buf);
        else compute_q(buf);
      };

      for (int s = 0; s < S; ++s) {
        // a loader's copies of step s are done once at most (those issued after them) remain:
        // the later steps' copies, and for the first P-1 steps also the previous item's stores
        wait_and_barrier(loader ? cur.per_step * min(S - 1 - s, P - 2) + (s < P - 1 ? n_st : 0) : 63);
        if (loader && s + P - 1 < S) issue(cur, s + P - 1, (s + P - 1) % P);
        if (NA > 0) compute(s % P);
      }
      lds_barrier();                                      // every operand read of the item is done
      if (loader && has_next) {
#pragma unroll
        for (int q = 0; q < P - 1; ++q)
          if (q < S) issue(nxt, q, q);
      }
      // row arow0 + 32 f + r16, output columns 64 wn + 8 g .. + 7 and 64 wn + 32 + 8 g .. + 7 of
      // column block nb: each store instruction covers 64 contiguous bytes of 16 rows
      uint8_t* obase = p.rowout + (((size_t)cur.row_base + arow0 + r16) * D + (size_t)cur.nb * BNW + 64 * wn + 8 * g) * 2;
#pragma unroll
      for (int f = 0; f < NA; ++f) {
        uint32_t d[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          d[k] = (uint32_t)f32_to_bf16_rne(acc[f][k >> 1][2 * (k & 1)]) |
                 ((uint32_t)f32_to_bf16_rne(acc[f][k >> 1][2 * (k & 1) + 1]) << 16);
        uint8_t* o = obase + (size_t)32 * f * D * 2;
        *reinterpret_cast<uint4*>(o) = uint4{d[0], d[1], d[2], d[3]};
        *reinterpret_cast<uint4*>(o + 64) = uint4{d[4], d[5], d[6], d[7]};
      }
      n_st = 2 * NA;
    };
    if constexpr (MF == 4) {
      switch (n_af) {
        case 0: run(std::integral_constant<int, 0>{}); break;
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        default: run(std::integral_constant<int, 4>{}); break;
      }
    } else {
      switch (n_af) {
        case 0: run(std::integral_constant<int, 0>{}); break;
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        case 4: run(std::integral_constant<int, 4>{}); break;
        case 5: run(std::integral_constant<int, 5>{}); break;
        case 6: run(std::integral_constant<int, 6>{}); break;
        case 7: run(std::integral_constant<int, 7>{}); break;
        default: run(std::integral_constant<int, 8>{}); break;
      }
    }
    cur = nxt;
  }
}

// ---------------------------------------------------------------- grouped Stage2, resident rows
//
// With the short K of a tensor-parallel shard (I = 384) a group's whole intermediate tile fits
// in LDS (at most 96 KB: 256 rows x 384 fp8 or fp4 codes, 128 rows x 384 bf16), so an item takes
// a range of up to RB consecutive column blocks instead of one: the loaders copy the A tile (every
// K step, with its scale dwords) once, then stream the weight rows of the range through a ring of
// P2 buffers, K step after K step and column block after column block without a break, and each
// column block's output rows are stored as soon as its last K step is done.  Against one column
// block per item this reads the group's intermediate rows RB times less often and keeps the copy
// pipeline running between column blocks.  The arithmetic of an output element (operands, MFMA
// order over K, rounding) is that of grouped_stage2_kernel.

template <int ADT>
struct RFmt {
  using F = GFmt<ADT>;
  static constexpr int S_MAX = 3;                                   // K steps of 128 kept in LDS
  static constexpr int P2 = ADT == DT_FP4 ? 4 : 3;                  // weight buffers
  static constexpr int AS_BYTES = ADT == DT_BF16 ? 0 : F::BM * 4;   // A scale dwords of a step
  static constexpr int A_STEP = F::A_BYTES + AS_BYTES;
  static constexpr int A_REGION = S_MAX * A_STEP;
  static constexpr int B_BUF = F::B_BYTES + BNW * 4;                // weight rows + scale dwords
  static constexpr int BYTES = A_REGION + P2 * B_BUF;
  static constexpr int RB = 7;                                      // column blocks per item, at most
  static constexpr int NB_STEP = F::B_IPL + 1;                      // copies per weight step per loader
};

bool resident_stage2(const FusedArgs& a) { return a.I % 128 == 0 && a.I / 128 <= RFmt<DT_FP8>::S_MAX; }

template <int ADT>
__global__ __launch_bounds__(GTHREADS, 1) void grouped_stage2_res_kernel(FusedArgs p, const int2* __restrict__ groups,
                                                                         const int32_t* __restrict__ num_groups,
                                                                         int n_nblk, int n_rng) {
  using F = GFmt<ADT>;
  using R = RFmt<ADT>;
  constexpr int KA = F::KA, ACPR = F::ACPR, BM = F::BM, MF = F::MF, P2 = R::P2;
  constexpr bool HAS_AS = ADT != DT_BF16;
  constexpr int PARTS = GT / F::GTA;
  static_assert(R::BYTES <= 160 * 1024, "LDS");
  static_assert((P2 - 2) * R::NB_STEP + (P2 - 1) * 2 * MF <= 62, "vmcnt wait counts fit");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[R::BYTES];

  const int D = p.D, I = p.I;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);   // wave-uniform
  const bool loader = wave < NLOAD;
  const int lw = wave & (NLOAD - 1);
  const int r16 = lane & 15, g = lane >> 4;
  const int wm = wave / WN, wn = wave % WN;
  const int S = I / 128;                                  // <= S_MAX (resident_stage2)
  const uint32_t lds0 = lds_addr(lds);
  const size_t a_rowbytes = (size_t)I * KA / 128;

  const int ng = ld_const(num_groups);
  const int xcd = blockIdx.x & 7, stride = gridDim.x >> 3, local0 = blockIdx.x >> 3;
  const int per_part = (ng > xcd ? (ng - xcd + 7) / 8 : 0) * n_rng;   // items (part, group, column range)
  const int items_here = PARTS * per_part;

  // weight copies: loader lw's instruction i moves rows 16 j .. 16 j + 15 (j = i * NLOAD + lw) of a
  // column block's K step, chunks XOR-swizzled as grouped_stage2_kernel reads them
  uint32_t b_off[F::B_IPL];
#pragma unroll
  for (int i = 0; i < F::B_IPL; ++i) {
    const int j = i * NLOAD + lw;
    const int qq = j * WAVE + lane;
    const int row = qq / 4, part = swz_slot<4>(row, qq % 4) - row * 4;
    b_off[i] = (uint32_t)(row / 16) * (uint32_t)(8 * I) + 16 * (16 * part + row % 16);
  }
  const int sc_row = lw * WAVE + lane;
  const uint32_t bs_off = (uint32_t)sc_row * (uint32_t)(I / 32);
  const int arow0 = 16 * wm;                              // fragments alternate between the wave rows

  for (int local = local0; local < items_here; local += stride) {
    const int part = local >= per_part ? 1 : 0, rem = local - part * per_part;
    const int gl = rem / n_rng, rg = rem - gl * n_rng;
    const int32_t* gp = reinterpret_cast<const int32_t*>(groups + gl * 8 + xcd);
    int tile0 = ld_const(gp), ntiles = ld_const(gp + 1);
    if (!MOE_DCHECK(tile0 >= 0 && ntiles >= 0 && tile0 + ntiles <= p.cap_tiles, DBG_GROUP)) tile0 = ntiles = 0;
    if (PARTS == 2) {
      const int h0 = ntiles <= F::GTA ? ntiles : (ntiles + 1) >> 1;
      tile0 += part ? h0 : 0;
      ntiles = part ? ntiles - h0 : h0;
    }
    const int cb0 = rg * n_nblk / n_rng, cb1 = (rg + 1) * n_nblk / n_rng;
    if (ntiles == 0 || cb0 == cb1) continue;             // the empty second part of a small group
    const int rows_used = ntiles * 32, row_base = tile0 * 32;
    const int e = dcheck_expert(ld_const(p.expert_ids + tile0), p.E);
    const uint8_t* qa = p.inter + (size_t)row_base * a_rowbytes;
    const uint8_t* qas = p.inter_s + (size_t)row_base * (I / 32);
    const uint8_t* qb = p.w2 + (size_t)e * D * (I / 2);
    const uint8_t* qbs = p.w2s + (size_t)e * D * (I / 32);
    uint32_t a_off[F::A_IPL];
    int n_ai = 0;
#pragma unroll
    for (int i = 0; i < F::A_IPL; ++i) {
      const int j = i * NLOAD + lw;
      const int qq = j * WAVE + lane;
      const int row = qq / ACPR, pt = swz_slot<ACPR>(row, qq % ACPR) - row * ACPR;
      a_off[i] = (uint32_t)(row < rows_used ? row : 0) * (uint32_t)a_rowbytes + pt * 16;
      n_ai += j * F::ROWS_PER_AI < rows_used;
    }
    const bool as_on = HAS_AS && lw * WAVE < rows_used;
    const uint32_t as_off = (uint32_t)(sc_row < rows_used ? sc_row : 0) * (uint32_t)(I / 32);
    const int NT = (cb1 - cb0) * S;                       // weight steps of the item

    // weight step t = (column block cb0 + t / S, K step t % S) into ring buffer t % P2
    auto issue_b = [&](int t) {
      const int c = t / S, s = t - c * S;
      const uint32_t L = __builtin_amdgcn_readfirstlane(lds0 + R::A_REGION + (t % P2) * R::B_BUF);
      const uint8_t* bb = qb + (size_t)(cb0 + c) * BNW * (I / 2) + s * 1024;
#pragma unroll
      for (int i = 0; i < F::B_IPL; ++i) dma16nt(bb, b_off[i], L + (i * NLOAD + lw) * 1024);
      dma4(qbs + (size_t)(cb0 + c) * BNW * (I / 32) + s * 4, bs_off, L + F::B_BYTES + lw * 256);
    };

    lds_barrier();                                        // every read of the previous item's tiles is done
    if (loader) {
      for (int s = 0; s < S; ++s) {
        const uint32_t L = __builtin_amdgcn_readfirstlane(lds0 + s * R::A_STEP);
        const uint8_t* ab = qa + s * KA;
#pragma unroll
        for (int i = 0; i < F::A_IPL; ++i)
          if (i < n_ai) dma16(ab, a_off[i], L + (i * NLOAD + lw) * 1024);
        if (as_on) dma4(qas + s * 4, as_off, L + F::A_BYTES + lw * 256);
      }
#pragma unroll
      for (int t = 0; t < P2 - 1; ++t)
        if (t < NT) issue_b(t);
    }
    const int n_af = max(0, min(MF, (rows_used - arow0 + 2 * 16 - 1) / (2 * 16)));

    auto run = [&](auto na_c) {
      constexpr int NA = decltype(na_c)::value;
      v4f acc[NA > 0 ? NA : 1][NFW];

      auto compute_bf16 = [&](const uint8_t* la, const uint8_t* lb) {
        const uint32_t* lbs = reinterpret_cast<const uint32_t*>(lb + F::B_BYTES);
        v8bf wop[NFW][4];
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
          const int br = 64 * wn + (j >> 1) * 32 + 8 * (r16 >> 2) + 4 * (j & 1) + (r16 & 3);
          const uint4 q = *reinterpret_cast<const uint4*>(lb + swz_slot<4>(br, g) * 16);
          const float sc = e8m0_to_float((lbs[br] >> (8 * g)) & 0xFFu);
          wop[j][0] = fp4x8_to_bf16(q.x, sc);
          wop[j][1] = fp4x8_to_bf16(q.y, sc);
          wop[j][2] = fp4x8_to_bf16(q.z, sc);
          wop[j][3] = fp4x8_to_bf16(q.w, sc);
        }
        auto load_x = [&](int f, v8bf* x) {
          const int ar = arow0 + 32 * f + r16;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const uint4 q = *reinterpret_cast<const uint4*>(la + swz_slot<16>(ar, 4 * g + jj) * 16);
            x[jj] = as_bf16x8(q.x, q.y, q.z, q.w);
          }
        };
        v8bf x_cur[4];
        load_x(0, x_cur);
#pragma unroll
        for (int f = 0; f < NA; ++f) {
          v8bf x_nxt[4] = {x_cur[0], x_cur[1], x_cur[2], x_cur[3]};
          if (f + 1 < NA) load_x(f + 1, x_nxt);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int j = 0; j < NFW; ++j) acc[f][j] = mfma_bf16(wop[j][jj], x_cur[jj], acc[f][j]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) x_cur[jj] = x_nxt[jj];
        }
      };

      auto compute_q = [&](const uint8_t* la, const uint8_t* lb) {
        const uint32_t* las = reinterpret_cast<const uint32_t*>(la + F::A_BYTES);
        const uint32_t* lbs = reinterpret_cast<const uint32_t*>(lb + F::B_BYTES);
        v8i wop[NFW];
        uint32_t wsc[NFW];
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
          const int br = 64 * wn + (j >> 1) * 32 + 8 * (r16 >> 2) + 4 * (j & 1) + (r16 & 3);
          wop[j] = fp4_operand_lo(*reinterpret_cast<const uint4*>(lb + swz_slot<4>(br, g) * 16));
          wsc[j] = (lbs[br] >> (8 * g)) & 0xFFu;
        }
        auto load_x = [&](int f, v8i& xop, uint32_t& xsc) {
          const int ar = arow0 + 32 * f + r16;
          if (ADT == DT_FP8) {
            const uint4 lo = *reinterpret_cast<const uint4*>(la + swz_slot<8>(ar, g) * 16);
            const uint4 hi = *reinterpret_cast<const uint4*>(la + swz_slot<8>(ar, 4 + g) * 16);
            xop = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          } else {
            xop = fp4_operand_lo(*reinterpret_cast<const uint4*>(la + swz_slot<4>(ar, g) * 16));
          }
          xsc = las[ar];                                // the byte is taken where it is used
        };
        v8i x_cur;
        uint32_t xs_cur;
        load_x(0, x_cur, xs_cur);
#pragma unroll
        for (int f = 0; f < NA; ++f) {
          v8i x_nxt = x_cur;
          uint32_t xs_nxt = xs_cur;
          if (f + 1 < NA) load_x(f + 1, x_nxt, xs_nxt);
          const uint32_t xb = (xs_cur >> (8 * g)) & 0xFFu;
#pragma unroll
          for (int j = 0; j < NFW; ++j) acc[f][j] = mfma_w_x<ADT>(wop[j], x_cur, acc[f][j], wsc[j], xb);
          __builtin_amdgcn_sched_barrier(0);
          x_cur = x_nxt;
          xs_cur = xs_nxt;
        }
      };

      for (int t = 0; t < NT; ++t) {
        const int c = t / S, s = t - c * S;
        // a loader's copies of step t are done once at most those issued after them remain: the
        // copies of steps t+1 .. t+P2-2 and the stores of the column blocks that ended after
        // step t's copies were issued (at iteration t-P2+1, or at the item's start)
        int later = 0;
        if (loader) {
          const int hi = min(t + P2 - 2, NT - 1);
          later = (hi > t ? hi - t : 0) * R::NB_STEP;
          for (int i = max(0, t - P2 + 1); i < t; ++i)
            if (i % S == S - 1) later += 2 * NA;
        }
        wait_and_barrier(loader ? later : 63);
        if (loader && t + P2 - 1 < NT) issue_b(t + P2 - 1);   // refills the buffer of step t-1
        if (s == 0) {
#pragma unroll
          for (int f = 0; f < NA; ++f)
#pragma unroll
            for (int j = 0; j < NFW; ++j) acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};
        }
        if (NA > 0) {
          const uint8_t* la = lds + s * R::A_STEP;
          const uint8_t* lb = lds + R::A_REGION + (t % P2) * R::B_BUF;
          if constexpr (ADT == DT_BF16) compute_bf16(la, lb);
          else compute_q(la, lb);
        }
        if (s == S - 1) {
          // row arow0 + 32 f + r16, output columns 64 wn + 8 g .. + 7 and 64 wn + 32 + 8 g .. + 7
          // of column block cb0 + c
          uint8_t* obase =
              p.rowout + (((size_t)row_base + arow0 + r16) * D + (size_t)(cb0 + c) * BNW + 64 * wn + 8 * g) * 2;
#pragma unroll
          for (int f = 0; f < NA; ++f) {
            uint32_t d[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
              d[k] = (uint32_t)f32_to_bf16_rne(acc[f][k >> 1][2 * (k & 1)]) |
                     ((uint32_t)f32_to_bf16_rne(acc[f][k >> 1][2 * (k & 1) + 1]) << 16);
            uint8_t* o = obase + (size_t)32 * f * D * 2;
            *reinterpret_cast<uint4*>(o) = uint4{d[0], d[1], d[2], d[3]};
            *reinterpret_cast<uint4*>(o + 64) = uint4{d[4], d[5], d[6], d[7]};
          }
        }
      }
    };
    if constexpr (MF == 4) {
      switch (n_af) {
        case 0: run(std::integral_constant<int, 0>{}); break;
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        default: run(std::integral_constant<int, 4>{}); break;
      }
    } else {
      switch (n_af) {
        case 0: run(std::integral_constant<int, 0>{}); break;
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        case 4: run(std::integral_constant<int, 4>{}); break;
        case 5: run(std::integral_constant<int, 5>{}); break;
        case 6: run(std::integral_constant<int, 6>{}); break;
        case 7: run(std::integral_constant<int, 7>{}); break;
        default: run(std::integral_constant<int, 8>{}); break;
      }
    }
  }
}

// ---------------------------------------------------------------- token-major Stage2 of hot experts
//
// With a skewed routing a few experts are chosen by a large share of the tokens (the prefill
// workload's Zipf prior: the top 16 experts hold ~64% of the routed rows).  Their Stage2 rows are
// taken token-major: an item is 256 (fp4) or 128 (fp8) consecutive tokens x 256 output columns
// and loops over the hot experts, gathering for each the intermediate rows of the item's tokens
// (the workspace's zero row for a token that does not route to it), so the router-weighted
// contributions of all hot experts to a token add up in registers and one bf16 partial row per
// token is stored, instead of one row per (token, hot expert) that the combine would read back.  The other experts' groups take the
// grouped Stage2 as before, and the combine adds the token's partial row to its other rows.
// The router weights enter without a second set of accumulators: a token row's accumulator is
// kept divided by s, the weight of the last hot expert the token routes to, so at the first K
// step of expert e (weight w != 0) the accumulator is multiplied by s / w before the matrix
// cores add W2[e] y, s becomes w, and the stored row is s times the accumulator.  A token that
// does not route to e reads the zero row (adding exact zeros) and keeps its s.
// An expert is hot when its rows are at least a quarter of the tokens (so at most a quarter of an
// item's MFMA rows are zero rows), up to MOE_HOT_MAX experts in ascending expert order.

constexpr int HOT_MAX = MOE_HOT_MAX;
// Thread = token: its layout row and router weight for each hot expert (the zero row and 0 for a
// hot expert it does not route to; the sum of the weights when it routes to one twice) and the
// mask of its slots whose expert is hot; workgroup 0 also clears the zero row of the
// intermediate.  Nothing is written when no expert is hot.
constexpr int TABLE_THREADS = 256;
static_assert(HOT_MAX % 4 == 0, "the tables are written 16 bytes at a time");
__global__ __launch_bounds__(TABLE_THREADS) void hot_table_kernel(FusedArgs p, int zrow, int row_bytes) {
  const int nh = p.hot_e[HOT_MAX];
  if (nh == 0) return;
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < row_bytes; i += TABLE_THREADS) p.inter[(size_t)zrow * row_bytes + i] = 0;
    if (p.inter_s)
      for (int i = threadIdx.x; i < p.I / 32; i += TABLE_THREADS) p.inter_s[(size_t)zrow * (p.I / 32) + i] = 0;
  }
  const int t = blockIdx.x * TABLE_THREADS + threadIdx.x;
  if (t >= p.T) return;
  const int K = p.topk;
  int pos[HOT_MAX];
  float wt[HOT_MAX];
#pragma unroll
  for (int h = 0; h < HOT_MAX; ++h) {
    pos[h] = zrow;
    wt[h] = 0.f;
  }
  uint32_t mask = 0;
  // a batch of slots: row positions and router weights loaded together (indices clamped into the
  // token's slots), then their tiles' hot indices, then the slots taken in ascending k.  Two slots
  // of one token on the same hot expert hold the same intermediate row: their weights add up.
  constexpr int KB = 16;
  for (int k0 = 0; k0 < K; k0 += KB) {
    int r[KB], hk[KB];
    float w[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int64_t v = (int64_t)t * K + min(k0 + u, K - 1);
      r[u] = p.row_of[v];
      w[u] = p.topk_w[v];
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) hk[u] = p.tile_hot[max(r[u], 0) / 32];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const bool on = k0 + u < K && r[u] >= 0 && hk[u] >= 0;
#pragma unroll
      for (int h = 0; h < HOT_MAX; ++h) {
        const bool m = on && hk[u] == h;
        pos[h] = m ? r[u] : pos[h];
        wt[h] += m ? w[u] : 0.f;
      }
      mask |= on ? 1u << (k0 + u) : 0u;
    }
  }
  int4* pv = reinterpret_cast<int4*>(p.hotpos + (size_t)t * HOT_MAX);
  float4* wv = reinterpret_cast<float4*>(p.hotw + (size_t)t * HOT_MAX);
#pragma unroll
  for (int q = 0; q < HOT_MAX / 4; ++q) {
    pv[q] = int4{pos[4 * q], pos[4 * q + 1], pos[4 * q + 2], pos[4 * q + 3]};
    wv[q] = float4{wt[4 * q], wt[4 * q + 1], wt[4 * q + 2], wt[4 * q + 3]};
  }
  p.hotmask[t] = mask;
}

// LDS operand staging of the token-major items: P buffers [A tile 128 rows | B tile 256 weight
// rows | A scale dwords | B scale dwords], then the item's tables of layout rows and router
// weights (128 tokens x MOE_HOT_MAX each) and the hot experts.
template <int ADT>
struct HFmt {
  // tokens per item: 256 with fp4 intermediates (each copied weight row serves twice the
  // tokens), 128 with fp8 (the 256-row fp8 tile would leave LDS for one step in flight)
  static constexpr int BM = ADT == DT_FP4 ? 256 : 128;
  static constexpr int MF = BM / WM / 16;                 // 16-row fragments per wave: 8 or 4
  static constexpr int KA = ADT == DT_FP8 ? 128 : 64;     // A bytes per row per K step
  static constexpr int ACPR = KA / 16;
  static constexpr int P = ADT == DT_FP4 ? 3 : 4;         // LDS buffers
  static constexpr int A_BYTES = BM * KA;
  static constexpr int B_BYTES = BNW * 64;
  static constexpr int BUF = A_BYTES + B_BYTES + (BM + BNW) * 4;
  static constexpr int A_IPL = A_BYTES / 1024 / NLOAD;    // A copy instructions per loader per step
  static constexpr int B_IPL = B_BYTES / 1024 / NLOAD;
  static constexpr int TAB = BM * HOT_MAX;                // entries per table
  static constexpr int BYTES = P * BUF + 2 * TAB * 4;
};

template <int ADT>
__global__ __launch_bounds__(GTHREADS, 1) void hot_stage2_kernel(FusedArgs p, int zrow) {
  using F = HFmt<ADT>;
  constexpr int KA = F::KA, ACPR = F::ACPR, P = F::P, BM = F::BM, MF = F::MF;
  static_assert(F::A_IPL * NLOAD * 1024 == F::A_BYTES && F::B_IPL * NLOAD * 1024 == F::B_BYTES, "copy split");
  static_assert(F::BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[F::BYTES];
  __shared__ int s_hot[HOT_MAX];
  int32_t* tpos = reinterpret_cast<int32_t*>(lds + P * F::BUF);
  float* tw = reinterpret_cast<float*>(lds + P * F::BUF + F::TAB * 4);

  const int nh = ld_const(p.hot_e + HOT_MAX);
  if (nh == 0) return;
  const int D = p.D, I = p.I, T = p.T;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);   // wave-uniform
  const bool loader = wave < NLOAD;
  const int lw = wave & (NLOAD - 1);
  const int r16 = lane & 15, g = lane >> 4;
  const int wm = wave / WN, wn = wave % WN;
  const int S = I / 128, SS = nh * S;                     // K steps per expert, per item
  const uint32_t lds0 = lds_addr(lds);
  const uint32_t a_rowbytes = (uint32_t)(I * KA / 128);
  if (threadIdx.x < HOT_MAX) s_hot[threadIdx.x] = p.hot_e[threadIdx.x];

  // items in column-block-major order, cut into 8 contiguous ranges, one per XCD: an XCD touches
  // the weight rows of at most a few column blocks (they stay in its L2) while every token tile's
  // gathered rows come from the memory-side cache
  const int ntl = (T + BM - 1) / BM, n_nblk = D / BNW, n_items = ntl * n_nblk;
  const int xcd = blockIdx.x & 7, stride = gridDim.x >> 3, local0 = blockIdx.x >> 3;
  const int it_lo = (int)((int64_t)n_items * xcd / 8), it_hi = (int)((int64_t)n_items * (xcd + 1) / 8);

  // the item's tables: layout row of (token, hot expert) and its router weight; tokens past T
  // read the zero row with weight 0 (loaded by the loader waves, whose only stores still in flight
  // are those of the item before)
  auto load_tables = [&](int item) {
    const int tl = item % ntl;
    const int tok0 = tl * BM;
    constexpr int PER = F::TAB / (NLOAD * WAVE);          // entries per loader lane: 8
    int vp[PER];
    float vw[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = (u * NLOAD + lw) * WAVE + lane;
      const int tok = tok0 + i / HOT_MAX;
      vp[u] = tok < T ? p.hotpos[(size_t)tok * HOT_MAX + (i % HOT_MAX)] : zrow;
      vw[u] = tok < T ? p.hotw[(size_t)tok * HOT_MAX + (i % HOT_MAX)] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = (u * NLOAD + lw) * WAVE + lane;
      tpos[i] = vp[u];
      tw[i] = vw[u];
    }
  };
  // copies of step ss (expert ss / S, K step ss % S) of item `item` into buffer buf
  auto issue = [&](int item, int ss, int buf) {
    const int hh = ss / S, s = ss - hh * S;
    const int nb = item / ntl;
    const int e = s_hot[hh];
    const uint32_t L = __builtin_amdgcn_readfirstlane(lds0 + buf * F::BUF);
    const uint8_t* ab = p.inter + s * KA;
    const uint8_t* bb = p.w2 + (size_t)e * D * (I / 2) + s * 1024;
#pragma unroll
    for (int i = 0; i < F::A_IPL; ++i) {
      const int j = i * NLOAD + lw;
      const int q = j * WAVE + lane;
      const int row = q / ACPR, part = swz_slot<ACPR>(row, q % ACPR) - row * ACPR;
      const int r = tpos[row * HOT_MAX + hh];
      dma16(ab, (uint32_t)r * a_rowbytes + part * 16, L + j * 1024);
    }
#pragma unroll
    for (int i = 0; i < F::B_IPL; ++i) {
      const int j = i * NLOAD + lw;
      const int q = j * WAVE + lane;
      const int row = q / 4, part = swz_slot<4>(row, q % 4) - row * 4;
      dma16(bb, (uint32_t)((nb * BNW + row) / 16) * (uint32_t)(8 * I) + 16 * (16 * part + row % 16),
            L + F::A_BYTES + j * 1024);
    }
    const int sc = lw * WAVE + lane;
    if (lw * WAVE < BM) {
      const int r = tpos[min(sc, BM - 1) * HOT_MAX + hh];
      dma4(p.inter_s + s * 4, (uint32_t)r * (uint32_t)(I / 32), L + F::A_BYTES + F::B_BYTES + lw * 256);
    }
    dma4(p.w2s + (size_t)e * D * (I / 32) + s * 4, (uint32_t)(nb * BNW + sc) * (uint32_t)(I / 32),
         L + F::A_BYTES + F::B_BYTES + BM * 4 + lw * 256);
  };
  // copy instructions a loader issues per step
  const int per_step = F::A_IPL + F::B_IPL + 1 + (lw * WAVE < BM ? 1 : 0);

  const int arow0 = (BM / WM) * wm;
  int item = it_lo + local0;
  if (item < it_hi && loader) {
    load_tables(item);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  lds_barrier();                                          // tables and hot experts are in LDS
  if (item < it_hi && loader) {
#pragma unroll
    for (int q = 0; q < P - 1; ++q)
      if (q < SS) issue(item, q, q);
  }
  int n_st = 0;
  for (; item < it_hi; item += stride) {
    const int nxt = item + stride;
    v4f acc[MF][NFW];
    float sc[MF];                                         // the divisor of each row's accumulator
#pragma unroll
    for (int f = 0; f < MF; ++f) {
      sc[f] = 1.f;
#pragma unroll
      for (int j = 0; j < NFW; ++j) acc[f][j] = v4f{0.f, 0.f, 0.f, 0.f};
    }

    auto compute = [&](int buf) {
      const uint8_t* la = lds + buf * F::BUF;
      const uint8_t* lb = la + F::A_BYTES;
      const uint32_t* las = reinterpret_cast<const uint32_t*>(lb + F::B_BYTES);
      const uint32_t* lbs = las + BM;
      v8i wop[NFW];
      uint32_t wsc[NFW];
#pragma unroll
      for (int j = 0; j < NFW; ++j) {
        const int br = 64 * wn + (j >> 1) * 32 + 8 * (r16 >> 2) + 4 * (j & 1) + (r16 & 3);
        wop[j] = fp4_operand_lo(*reinterpret_cast<const uint4*>(lb + swz_slot<4>(br, g) * 16));
        wsc[j] = (lbs[br] >> (8 * g)) & 0xFFu;
      }
      auto load_x = [&](int f, v8i& xop, uint32_t& xsc) {
        const int ar = arow0 + 16 * f + r16;
        if (ADT == DT_FP8) {
          const uint4 lo = *reinterpret_cast<const uint4*>(la + swz_slot<8>(ar, g) * 16);
          const uint4 hi = *reinterpret_cast<const uint4*>(la + swz_slot<8>(ar, 4 + g) * 16);
          xop = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        } else {
          xop = fp4_operand_lo(*reinterpret_cast<const uint4*>(la + swz_slot<4>(ar, g) * 16));
        }
        xsc = las[ar];                                  // the byte is taken where it is used
      };
      v8i x_cur;
      uint32_t xs_cur;
      load_x(0, x_cur, xs_cur);
#pragma unroll
      for (int f = 0; f < MF; ++f) {
        v8i x_nxt = x_cur;
        uint32_t xs_nxt = xs_cur;
        if (f + 1 < MF) load_x(f + 1, x_nxt, xs_nxt);
        const uint32_t xb = (xs_cur >> (8 * g)) & 0xFFu;
#pragma unroll
        for (int j = 0; j < NFW; ++j) acc[f][j] = mfma_w_x<ADT>(wop[j], x_cur, acc[f][j], wsc[j], xb);
        __builtin_amdgcn_sched_barrier(0);
        x_cur = x_nxt;
        xs_cur = xs_nxt;
      }
    };

    for (int ss = 0; ss < SS; ++ss) {
      wait_and_barrier(loader ? per_step * min(SS - 1 - ss, P - 2) + (ss < P - 1 ? n_st : 0) : 63);
      if (loader && ss + P - 1 < SS) issue(item, ss + P - 1, (ss + P - 1) % P);
      if (ss % S == 0) {                                   // the expert's first K step: rescale
        const int hh = ss / S;
#pragma unroll
        for (int f = 0; f < MF; ++f) {
          const float wv = tw[(arow0 + 16 * f + r16) * HOT_MAX + hh];
          if (wv != 0.f) {
            const float r = sc[f] / wv;
#pragma unroll
            for (int j = 0; j < NFW; ++j)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[f][j][i] *= r;
            sc[f] = wv;
          }
        }
      }
      compute(ss % P);
    }
    lds_barrier();                                        // every operand and table read is done
    const int tok_base = (item % ntl) * BM;
    const int nb = item / ntl;
    if (nxt < it_hi && loader) {
      load_tables(nxt);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    lds_barrier();                                        // the next item's tables are in LDS
    if (nxt < it_hi && loader) {
#pragma unroll
      for (int q = 0; q < P - 1; ++q)
        if (q < SS) issue(nxt, q, q);
    }
    // token arow0 + 16 f + r16, output columns 64 wn + 8 g .. + 7 and 64 wn + 32 + 8 g .. + 7.
    // The loaders' first waits of the next item let these stores stay in flight: counted only
    // when every one of them is issued (a tile wholly below T), else none (the wait is stricter)
    const bool full_tile = tok_base + BM <= T;
#pragma unroll
    for (int f = 0; f < MF; ++f) {
      const int tok = tok_base + arow0 + 16 * f + r16;
      uint32_t d[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        d[k] = (uint32_t)f32_to_bf16_rne(sc[f] * acc[f][k >> 1][2 * (k & 1)]) |
               ((uint32_t)f32_to_bf16_rne(sc[f] * acc[f][k >> 1][2 * (k & 1) + 1]) << 16);
      if (tok < T) {
        uint8_t* o = p.hot_out + ((size_t)tok * D + (size_t)nb * BNW + 64 * wn + 8 * g) * 2;
        *reinterpret_cast<uint4*>(o) = uint4{d[0], d[1], d[2], d[3]};
        *reinterpret_cast<uint4*>(o + 64) = uint4{d[4], d[5], d[6], d[7]};
      }
    }
    n_st = full_tile ? 2 * MF : 0;
  }
}

// Compute units of the current device, queried at each launch (a host call of about a
// microsecond next to kernels of hundreds): no state shared between threads or devices.
int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n >= 8)
    return n;
  return 256;
}

template <int ADT, int STAGE>
hipError_t launch_grouped_stage(const FusedArgs& a, const int2* groups, const int32_t* ngroups, hipStream_t s) {
  const int n_nblk = STAGE == 1 ? (2 * a.I) / BNW : a.D / BNW;
  const unsigned grid = (unsigned)(num_cus() / 8 * 8);    // one workgroup per CU, a multiple of 8
  if constexpr (STAGE == 2) {
    if constexpr (ADT != DT_BF16) {
      if (hot_path(a)) {   // hot experts token-major, the other experts' groups below
        const int zrow = a.cap_tiles * a.block_m;
        const int row_bytes = ADT == DT_FP8 ? a.I : a.I / 2;
        hot_table_kernel<<<(unsigned)((a.T + TABLE_THREADS - 1) / TABLE_THREADS), TABLE_THREADS, 0, s>>>(a, zrow,
                                                                                                      row_bytes);
        hot_stage2_kernel<ADT><<<grid, GTHREADS, 0, s>>>(a, zrow);
        groups = a.cgroups;
        ngroups = a.num_cgroups;
      }
    }
    if (resident_stage2(a)) {
      const int n_rng = (n_nblk + RFmt<ADT>::RB - 1) / RFmt<ADT>::RB;
      grouped_stage2_res_kernel<ADT><<<grid, GTHREADS, 0, s>>>(a, groups, ngroups, n_nblk, n_rng);
    } else {
      grouped_stage2_kernel<ADT><<<grid, GTHREADS, 0, s>>>(a, groups, ngroups, n_nblk);
    }
  } else if (a.act == ACT_SITUV2)
    grouped_stage1_kernel<ADT, ACT_SITUV2><<<grid, GTHREADS, 0, s>>>(a, groups, ngroups, n_nblk);
  else
    grouped_stage1_kernel<ADT, ACT_SILU><<<grid, GTHREADS, 0, s>>>(a, groups, ngroups, n_nblk);
  return hipGetLastError();
}

}  // namespace

bool hot_path(const FusedArgs& a) {
  // fp8 / fp4 intermediates, slots fit the 32-bit mask, the large-batch Stage2
  return a.a_dtype != DT_BF16 && a.topk <= 32 && tiled_path_supported(a) && a.T >= TILED_MIN_TOKENS_S2;
}

bool tiled_path_supported(const FusedArgs& a) {
  // the A copies address the activation rows with 32-bit offsets
  const int64_t x_bytes = (int64_t)a.T * a.D * (a.a_dtype == DT_BF16 ? 4 : a.a_dtype == DT_FP8 ? 2 : 1) / 2;
  return a.block_m == 32 && a.act != ACT_NONE && (2 * a.I) % BNW == 0 && x_bytes < ((int64_t)1 << 32) &&
         a.D % 512 == 0;   // Stage1 takes whole 16-byte scale chunks; Stage2 needs D % BNW == 0
}

hipError_t launch_tiled(const FusedArgs& a, int2* groups, int32_t* ngroups, hipStream_t s) {
  hipError_t err;
  if (a.stages & 1) {
    // hot experts: rows at least a quarter of the tokens (tiles of 32 rows)
    const int hot_min_tiles = hot_path(a) ? (a.T + 4 * 32 - 1) / (4 * 32) : INT32_MAX;
    group_kernel<<<1, GROUP_THREADS, 0, s>>>(a.expert_ids, a.num_tiles, a.cap_tiles, groups, ngroups, hot_min_tiles,
                                             a.cgroups, a.num_cgroups, a.tile_hot, a.hot_e);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    err = a.a_dtype == DT_FP8   ? launch_grouped_stage<DT_FP8, 1>(a, groups, ngroups, s)
          : a.a_dtype == DT_FP4 ? launch_grouped_stage<DT_FP4, 1>(a, groups, ngroups, s)
                                : launch_grouped_stage<DT_BF16, 1>(a, groups, ngroups, s);
    if (err != hipSuccess) return err;
  }
  if (a.stages & 2) {
    err = a.a_dtype == DT_FP8   ? launch_grouped_stage<DT_FP8, 2>(a, groups, ngroups, s)
          : a.a_dtype == DT_FP4 ? launch_grouped_stage<DT_FP4, 2>(a, groups, ngroups, s)
                                : launch_grouped_stage<DT_BF16, 2>(a, groups, ngroups, s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

MOE_DEBUG_READER(grouped)

}  // namespace moe
