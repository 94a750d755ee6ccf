// Routing sort: groups routed rows by local expert and pads each expert to a whole tile
// (github ROCm/aiter PR 5118, "Summary": moe_sorting pads every expert up to a full block_m).
//
// The layout is unique (experts ascending, rows ascending in v = t*topk + k, sentinel T*topk on
// padding), so the kernels rank rows without atomics.  A chunk of rows is split into
// contiguous per-wave sub-chunks; inside a wave the rank of a row among the lanes holding the
// same expert comes from per-bit ballots (a match-any), each wave keeps its own 16-bit counters
// in LDS, and an exclusive scan over waves, chunks and experts (in index order) turns the
// counts into positions.
//
//   rows <= 64    : one wave, ranks and offsets from ballots and cross-lane reads only.
//   rows <= 4096  : eight workgroups each rank every row and scan the experts, then write one
//                   round of rows each.
//   larger        : count (one workgroup per chunk of 1024 to 4096 rows) -> scan (one
//                   workgroup) -> scatter (one workgroup per 1024 rows).
// The layout's optional sync words are zeroed by the single-wave / single-workgroup kernel or,
// on the multi-chunk path, by the counting kernel.
#include "moe_kernels.h"
#include "moe_device.h"

namespace moe {

namespace {

constexpr int SORT_THREADS = 512;
constexpr int SORT_WAVES = SORT_THREADS / WAVE;              // 8
constexpr int SUB = MOE_SORT_CHUNK / SORT_WAVES;             // rows per wave: 512
constexpr int ROUNDS = SUB / WAVE;                           // 8
static_assert(SUB <= 65535, "16-bit per-wave counters");

// Lanes of this wave with the same key (valid lanes only); key_bits distinguishes all keys.
__device__ __forceinline__ uint64_t match_any(int key, bool valid, int key_bits) {
  uint64_t mask = __ballot(valid);
  for (int b = 0; b < key_bits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t ones = __ballot(valid && bit);
    mask &= bit ? ones : ~ones;
  }
  return valid ? mask : 0ull;
}

__device__ __forceinline__ int bits_for(int n) {   // bits needed to write 0 .. n-1
  int b = 1;
  while ((1 << b) < n) ++b;
  return b;
}

// Rows of one wave's sub-chunk: a chunk of n_in rows is split evenly over the waves in whole
// rounds of 64 rows, so a short chunk still spreads over every wave (a 256-row chunk was
// ranked by one wave when each wave took a fixed 512).
__device__ __forceinline__ int sub_rows(int n_in) {
  return min(SUB, (n_in + SORT_WAVES * WAVE - 1) / (SORT_WAVES * WAVE) * WAVE);
}

// Rank the rows [base, base + n_in) of one chunk (wave w takes rows [w*sub, w*sub + sub),
// sub = sub_rows(n_in)).  On return (after a barrier):
//   wc[w*E + e]  exclusive prefix over waves of the rows of expert e (per wave sub-chunk),
//   tot[e]       rows of expert e in the chunk (if tot != nullptr),
//   key[r]       local expert of this lane's row in round r (-1 if skipped),
//   rank[r]      its rank among earlier same-expert rows of the chunk.
__device__ __forceinline__ void rank_chunk(const int32_t* __restrict__ ids, int64_t base, int n_in,
                                           int expert_begin, int E, uint16_t* wc, int* tot,
                                           int key[ROUNDS], int rank[ROUNDS]) {
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  for (int i = threadIdx.x; i < SORT_WAVES * E; i += SORT_THREADS) wc[i] = 0;
  const int sub = sub_rows(n_in), first = w * sub;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {                 // issue every load before using any
    const int idx = first + r * WAVE + lane;
    key[r] = r * WAVE < sub && idx < n_in ? ids[base + idx] - expert_begin : -1;
  }
  __syncthreads();
  const int kb = bits_for(E);
  const uint64_t lt = (1ull << lane) - 1ull;
  uint16_t* my = wc + w * E;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    int k = key[r];
    k = (k >= 0 && k < E) ? k : -1;
    key[r] = k;
    rank[r] = 0;
    if (r * WAVE >= sub || first + r * WAVE >= n_in) continue;   // uniform: nothing left in this wave
    const bool valid = k >= 0;
    const uint64_t same = match_any(k, valid, kb);
    if (valid) {
      const int prev = my[k];
      rank[r] = prev + __popcll(same & lt);
      if ((same & lt) == 0ull) my[k] = (uint16_t)(prev + __popcll(same));   // group leader
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += SORT_THREADS) {
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < SORT_WAVES; ++ww) {
      const int c = wc[ww * E + e];
      wc[ww * E + e] = (uint16_t)run;
      run += c;
    }
    if (tot) tot[e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r)
    if (key[r] >= 0) rank[r] += wc[w * E + key[r]];
}

// Exclusive scan over the NT threads of a block; returns this thread's prefix, *total = sum.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  int incl = v;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const int o = __shfl_up(incl, d, WAVE);
    if (lane >= d) incl += o;
  }
  if (lane == WAVE - 1) tmp[w] = incl;
  __syncthreads();
  if (threadIdx.x < WAVE) {
    const int nw = NT / WAVE;
    int t = threadIdx.x < nw ? tmp[threadIdx.x] : 0;
    int s = t;
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
      const int o = __shfl_up(s, d, WAVE);
      if ((int)threadIdx.x >= d) s += o;
    }
    if (threadIdx.x < nw) tmp[threadIdx.x] = s - t;
    if (threadIdx.x == nw - 1) tmp[nw] = s;
  }
  __syncthreads();
  const int res = tmp[w] + incl - v;
  *total = tmp[NT / WAVE];
  __syncthreads();
  return res;
}


// The layout's sync words (a multiple of 4, 16-byte aligned) set to zero by threads
// first, first + stride, ...
__device__ __forceinline__ void zero_sync(const SortLayout& L, int64_t first, int64_t stride) {
  uint4* p = reinterpret_cast<uint4*>(L.sync);
  for (int64_t i = first; i < L.sync_words / 4; i += stride) p[i] = uint4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------- one-wave path (rows <= 64)
//
// Lane i holds row v = i.  One pass over the key bits from the top, with a ballot per bit,
// gives every lane both the set of lanes with its own expert (its rank is the number of lower
// lanes in it) and the set of lanes with a smaller expert; the tile offset of its expert is
// the sum of the tile counts held by the group leaders (lowest lane of each expert) in that
// set, summed bit by bit over ballots of the tile counts.

__global__ __launch_bounds__(WAVE) void sort_wave_kernel(const int32_t* __restrict__ ids,
                                                         const float* __restrict__ topk_w, int n,
                                                         int expert_begin, int E, int block_m,
                                                         SortLayout L) {
  const int lane = threadIdx.x;
  int k = -1;
  float w = 0.0f;
  if (n > 0) {   // both loads issued together (lanes past n re-read row n-1): one memory latency
    const int src = min(lane, n - 1);
    const int id = ids[src] - expert_begin;
    if (L.sorted_w) w = topk_w[src];
    k = (lane < n && id >= 0 && id < E) ? id : -1;
  }
  const bool valid = k >= 0;
  uint64_t same = __ballot(valid), less = 0ull;
  for (int b = bits_for(E) - 1; b >= 0; --b) {
    const bool bit = (k >> b) & 1;
    const uint64_t ones = __ballot(valid && bit);
    if (bit) less |= same & ~ones;
    same &= bit ? ones : ~ones;
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  const int rank = __popcll(same & lt);
  const int cnt = __popcll(same);
  const bool leader = valid && (same & lt) == 0ull;
  const int tiles = leader ? (cnt + block_m - 1) / block_m : 0;
  int off = 0, total = 0;
  for (int t = 0; (1 << t) <= (WAVE + block_m - 1) / block_m; ++t) {   // bits of a tile count
    const uint64_t tb = __ballot((tiles >> t) & 1);
    off += __popcll(less & tb) << t;
    total += __popcll(tb) << t;
  }
  const int sentinel = n;
  const int p = off * block_m + rank;
  if (valid && MOE_DCHECK((int64_t)p < L.cap_tiles * block_m, DBG_SORT_POS)) {
    L.sorted_ids[p] = lane;
    if (L.sorted_w) L.sorted_w[p] = w;
  }
  if (L.row_of && lane < n) L.row_of[lane] = valid ? p : -1;
  if (leader) {
    for (int t = 0; t < tiles; ++t) L.expert_ids[off + t] = k;
    for (int p = cnt; p < tiles * block_m; ++p) {
      L.sorted_ids[off * block_m + p] = sentinel;
      if (L.sorted_w) L.sorted_w[off * block_m + p] = 0.0f;
    }
  }
  for (int64_t t = total + lane; t < L.cap_tiles; t += WAVE) L.expert_ids[t] = -1;
  for (int64_t p = (int64_t)total * block_m + lane; p < (int64_t)L.cap_tiles * block_m; p += WAVE) {
    L.sorted_ids[p] = sentinel;
    if (L.sorted_w) L.sorted_w[p] = 0.0f;
  }
  zero_sync(L, lane, WAVE);
  if (lane == 0) *L.num_tiles = total;
}

// ---------------------------------------------------------------- one-chunk path
//
// Rows <= MOE_SORT_CHUNK: SMALL_SORT_WGS workgroups each rank every row and scan the experts
// (the input is at most 16 KB), then write a share of the layout: workgroup g the rows of round
// g of every wave (with the tile expert ids from each tile's first row and the padding from
// each expert's last row) and a slice of the unused tail.  One workgroup writing everything
// was bound by its CU's address unit.

constexpr int SMALL_SORT_WGS = ROUNDS;

__global__ __launch_bounds__(SORT_THREADS) void sort_small_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ topk_w, int n, int expert_begin,
    int E, int block_m, SortLayout L) {
  extern __shared__ int smem[];
  int* cnt = smem;                                             // [E] rows per expert
  int* tmp = cnt + E;                                          // [SORT_WAVES + 1]
  uint16_t* wc = reinterpret_cast<uint16_t*>(tmp + SORT_WAVES + 1);   // [SORT_WAVES][E]
  int key[ROUNDS], rank[ROUNDS];
  rank_chunk(ids, 0, n, expert_begin, E, wc, cnt, key, rank);
  zero_sync(L, (int64_t)blockIdx.x * SORT_THREADS + threadIdx.x, (int64_t)gridDim.x * SORT_THREADS);
  // first row of every expert (into the consumed per-wave counters; the scan's barriers order
  // these writes after every counter read)
  int* first = reinterpret_cast<int*>(wc);
  const int per = (E + SORT_THREADS - 1) / SORT_THREADS;
  const int e0 = threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (e0 + i < E) local += (cnt[e0 + i] + block_m - 1) / block_m;
  int total = 0;
  int off = block_exclusive_scan<SORT_THREADS>(local, tmp, &total);
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    first[e] = off * block_m;
    off += (cnt[e] + block_m - 1) / block_m;
  }
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x == 0) *L.num_tiles = total;
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  const int sentinel = n, sub = sub_rows(n);
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    if (r % (int)gridDim.x != (int)blockIdx.x) continue;
    const int v = w * sub + r * WAVE + lane;
    if (r * WAVE >= sub || v >= n) continue;
    const int k = key[r];
    if (k < 0) {
      if (L.row_of) L.row_of[v] = -1;
      continue;
    }
    const int q = rank[r];                                     // rank within the expert
    const int f = first[k], p = f + q;
    if (!MOE_DCHECK((int64_t)p < L.cap_tiles * block_m, DBG_SORT_POS)) continue;
    L.sorted_ids[p] = v;
    if (L.sorted_w) L.sorted_w[p] = topk_w[v];
    if (L.row_of) L.row_of[v] = p;
    if ((q & (block_m - 1)) == 0) L.expert_ids[p / block_m] = k;   // f is a multiple of block_m
    const int c = cnt[k];
    if (q == c - 1) {
      const int end = f + (c + block_m - 1) / block_m * block_m;
      for (int pp = p + 1; pp < end; ++pp) {
        L.sorted_ids[pp] = sentinel;
        if (L.sorted_w) L.sorted_w[pp] = 0.0f;
      }
    }
  }
  const int64_t tid = (int64_t)blockIdx.x * SORT_THREADS + threadIdx.x;
  const int64_t nth = (int64_t)gridDim.x * SORT_THREADS;
  for (int64_t t = total + tid; t < L.cap_tiles; t += nth) L.expert_ids[t] = -1;
  for (int64_t pp = (int64_t)total * block_m + tid; pp < (int64_t)L.cap_tiles * block_m; pp += nth) {
    L.sorted_ids[pp] = sentinel;
    if (L.sorted_w) L.sorted_w[pp] = 0.0f;
  }
}

// ---------------------------------------------------------------- multi-chunk path

__global__ __launch_bounds__(SORT_THREADS) void sort_count_kernel(
    const int32_t* __restrict__ ids, int64_t n, int chunk, int expert_begin, int E, int* __restrict__ hist,
    int* __restrict__ ranks, SortLayout L) {
  extern __shared__ int smem[];
  int* tot = smem;                                             // [E]
  uint16_t* wc = reinterpret_cast<uint16_t*>(tot + E);         // [SORT_WAVES][E]
  const int64_t base = (int64_t)blockIdx.x * chunk;
  const int n_in = (int)(n - base < chunk ? n - base : chunk);
  int key[ROUNDS], rank[ROUNDS];
  rank_chunk(ids, base, n_in, expert_begin, E, wc, tot, key, rank);
  zero_sync(L, (int64_t)blockIdx.x * SORT_THREADS + threadIdx.x, (int64_t)gridDim.x * SORT_THREADS);
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r)
    if (key[r] >= 0) ranks[base + w * sub_rows(n_in) + r * WAVE + lane] = rank[r];
  for (int e = threadIdx.x; e < E; e += SORT_THREADS) hist[(int64_t)blockIdx.x * E + e] = tot[e];
}

constexpr int SCAN_THREADS = 1024;

// One workgroup: per expert, the chunk counts become exclusive offsets within the expert
// (hist[c*E + e]); the expert's first row goes to first[e] and its row count to cnt[e]
// (first = hist + nchunks*E, cnt = first + E), the tile total to num_tiles.  The layout itself
// is written by the scatter's many workgroups (a single workgroup's scattered stores are bound
// by its one CU's address unit).
__global__ __launch_bounds__(SCAN_THREADS) void sort_scan_kernel(int* __restrict__ hist, int nchunks,
                                                                 int E, int block_m, SortLayout L) {
  extern __shared__ int smem[];
  int* pos = smem;                       // [E]
  int* tmp = pos + E;                    // [SCAN_THREADS / WAVE + 1]
  // the counts of SB chunks are loaded together, then turned into exclusive offsets: a memory
  // latency per SB chunks instead of one per chunk
  constexpr int SB = 32;
  for (int e = threadIdx.x; e < E; e += SCAN_THREADS) {
    int run = 0;
    for (int c0 = 0; c0 < nchunks; c0 += SB) {
      int h[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u) h[u] = c0 + u < nchunks ? hist[(int64_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        if (c0 + u < nchunks) hist[(int64_t)(c0 + u) * E + e] = run;
        run += h[u];
      }
    }
    pos[e] = run;
  }
  __syncthreads();
  int* first = hist + (int64_t)nchunks * E;
  int* cnt = first + E;
  const int per = (E + SCAN_THREADS - 1) / SCAN_THREADS;
  const int e0 = threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (e0 + i < E) local += (pos[e0 + i] + block_m - 1) / block_m;
  int total = 0;
  int off = block_exclusive_scan<SCAN_THREADS>(local, tmp, &total);
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    const int c = pos[e];
    first[e] = off * block_m;
    cnt[e] = c;
    off += (c + block_m - 1) / block_m;
  }
  if (threadIdx.x == 0) *L.num_tiles = total;
}

// Rows to their positions: chunk / SCATTER_ROWS workgroups per chunk, each thread SCATTER_RPT
// rows with all their loads issued together.  The row that opens a tile writes the tile's expert id, an
// expert's last row writes the padding of its last tile, and all workgroups share the unused
// tail (expert -1, sentinel rows).
constexpr int SCATTER_THREADS = 256;
constexpr int SCATTER_RPT = 4;
constexpr int SCATTER_ROWS = SCATTER_THREADS * SCATTER_RPT;   // rows per workgroup
static_assert(MOE_SORT_MIN_CHUNK % SCATTER_ROWS == 0 && MOE_SORT_CHUNK % MOE_SORT_MIN_CHUNK == 0, "whole chunks");

__global__ __launch_bounds__(SCATTER_THREADS) void sort_scatter_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ topk_w, int64_t n, int expert_begin,
    int E, int block_m, int nchunks, int chunk_rows, const int* __restrict__ hist, const int* __restrict__ ranks,
    SortLayout L) {
  const int split = chunk_rows / SCATTER_ROWS;
  const int chunk = blockIdx.x / split;
  const int64_t base = (int64_t)chunk * chunk_rows + (int64_t)(blockIdx.x % split) * SCATTER_ROWS;
  const int* first = hist + (int64_t)nchunks * E;
  const int* cnt = first + E;
  const int sentinel = (int)n;
  int k[SCATTER_RPT];
#pragma unroll
  for (int u = 0; u < SCATTER_RPT; ++u) {
    const int64_t v = base + u * SCATTER_THREADS + threadIdx.x;
    k[u] = v < n ? ids[v] - expert_begin : -1;
  }
  int f[SCATTER_RPT], h[SCATTER_RPT], r[SCATTER_RPT], c[SCATTER_RPT];
  float w[SCATTER_RPT];
#pragma unroll
  for (int u = 0; u < SCATTER_RPT; ++u) {
    const int64_t v = base + u * SCATTER_THREADS + threadIdx.x;
    const bool ok = k[u] >= 0 && k[u] < E;
    const int kk = ok ? k[u] : 0;
    f[u] = first[kk];
    c[u] = cnt[kk];
    h[u] = hist[(int64_t)chunk * E + kk];
    r[u] = ok ? ranks[v] : 0;
    w[u] = ok && L.sorted_w ? topk_w[v] : 0.0f;
  }
#pragma unroll
  for (int u = 0; u < SCATTER_RPT; ++u) {
    const int64_t v = base + u * SCATTER_THREADS + threadIdx.x;
    if (v >= n) continue;
    if (k[u] < 0 || k[u] >= E) {
      if (L.row_of) L.row_of[v] = -1;
      continue;
    }
    const int q = h[u] + r[u];                            // rank within the expert
    const int p = f[u] + q;
    if (!MOE_DCHECK((int64_t)p < L.cap_tiles * block_m, DBG_SORT_POS)) continue;
    L.sorted_ids[p] = (int32_t)v;
    if (L.sorted_w) L.sorted_w[p] = w[u];
    if (L.row_of) L.row_of[v] = p;
    if ((q & (block_m - 1)) == 0) L.expert_ids[p / block_m] = k[u];   // f is a multiple of block_m
    if (q == c[u] - 1) {
      const int end = f[u] + (c[u] + block_m - 1) / block_m * block_m;
      for (int pp = p + 1; pp < end; ++pp) {
        L.sorted_ids[pp] = sentinel;
        if (L.sorted_w) L.sorted_w[pp] = 0.0f;
      }
    }
  }
  const int64_t total = *L.num_tiles;
  const int64_t tid = (int64_t)blockIdx.x * SCATTER_THREADS + threadIdx.x;
  const int64_t nth = (int64_t)gridDim.x * SCATTER_THREADS;
  for (int64_t t = total + tid; t < L.cap_tiles; t += nth) L.expert_ids[t] = -1;
  for (int64_t pp = total * block_m + tid; pp < (int64_t)L.cap_tiles * block_m; pp += nth) {
    L.sorted_ids[pp] = sentinel;
    if (L.sorted_w) L.sorted_w[pp] = 0.0f;
  }
}

}  // namespace

hipError_t launch_sort(const int32_t* topk_ids, const float* topk_w, int64_t n, int expert_begin,
                       int E, int block_m, const SortLayout& L, void* ws, hipStream_t s) {
  const int sentinel = (int)n;
  const size_t wc_bytes = (size_t)SORT_WAVES * E * sizeof(uint16_t);
  if (n <= WAVE) {
    sort_wave_kernel<<<1, WAVE, 0, s>>>(topk_ids, topk_w, (int)n, expert_begin, E, block_m, L);
    return hipGetLastError();
  }
  if (n <= MOE_SORT_CHUNK) {
    const size_t lds = (size_t)(E + SORT_WAVES + 1) * sizeof(int) + wc_bytes;
    sort_small_kernel<<<SMALL_SORT_WGS, SORT_THREADS, lds, s>>>(topk_ids, topk_w, (int)n, expert_begin, E,
                                                              block_m, L);
    return hipGetLastError();
  }
  // about 64 chunks: enough counting workgroups at 16k rows, few enough chunk offsets for the
  // one-workgroup scan at 256k (sort µs at 16384 / 131072 / 262144 rows: 22.6 / 20.0 / 26.5 with
  // 4096-row chunks, 18.0 / 20.0 / 37.4 with 1024, 19.4 / 18.6 / 28.3 with 2048)
  const int chunk = n <= 64 * MOE_SORT_MIN_CHUNK ? MOE_SORT_MIN_CHUNK
                    : n <= 64 * 2 * MOE_SORT_MIN_CHUNK ? 2 * MOE_SORT_MIN_CHUNK : MOE_SORT_CHUNK;
  const int nchunks = (int)((n + chunk - 1) / chunk);
  int* hist = (int*)ws;
  int* ranks = (int*)((char*)ws + moe_align256((size_t)(nchunks + 2) * E * sizeof(int)));
  sort_count_kernel<<<nchunks, SORT_THREADS, (size_t)E * sizeof(int) + wc_bytes, s>>>(
      topk_ids, n, chunk, expert_begin, E, hist, ranks, L);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  sort_scan_kernel<<<1, SCAN_THREADS, (size_t)(E + SCAN_THREADS / WAVE + 1) * sizeof(int), s>>>(
      hist, nchunks, E, block_m, L);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  sort_scatter_kernel<<<nchunks * (chunk / SCATTER_ROWS), SCATTER_THREADS, 0, s>>>(
      topk_ids, topk_w, n, expert_begin, E, block_m, nchunks, chunk, hist, ranks, L);
  return hipGetLastError();
}

MOE_DEBUG_READER(sort)

}  // namespace moe
