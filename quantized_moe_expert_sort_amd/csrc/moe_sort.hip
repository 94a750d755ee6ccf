// Routing sort: groups routed rows by local expert and pads each expert to a whole tile
// (github ROCm/aiter PR 5118, "Summary": moe_sorting pads every expert up to a full block_m).
//
// The layout is unique (experts ascending, rows ascending in v = t*topk + k, sentinel T*topk on
// padding), so the kernels rank rows without atomics: inside a wave the rank of a row among
// the lanes holding the same expert comes from per-bit ballots (a match-any), and waves,
// chunks and experts are combined in index order by exclusive scans.
//
//   rows <= MOE_SORT_CHUNK : one workgroup does counting, scan, padding and scatter.
//   larger                 : count (one workgroup per chunk) -> scan (one workgroup)
//                            -> scatter (one workgroup per chunk).
#include "moe_kernels.h"
#include "moe_device.h"

namespace moe {

namespace {

constexpr int SORT_THREADS = 256;
constexpr int SORT_WAVES = SORT_THREADS / WAVE;
constexpr int ROWS_PER_WAVE = MOE_SORT_CHUNK / SORT_WAVES;   // 1024
constexpr int ROUNDS = ROWS_PER_WAVE / WAVE;                  // 16

struct WaveMatch {
  uint64_t same;   // lanes holding the same key (valid lanes only)
};

// Lanes of this wave with the same key; key_bits = number of bits that distinguish keys.
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

// Counts the rows of one chunk per (wave, expert) in cnt[w*E + e] and returns, for each of
// this lane's ROUNDS rows, its rank among the same-expert rows of its wave's sub-chunk.
__device__ __forceinline__ void count_chunk(const int32_t* __restrict__ ids, int64_t base, int n_in,
                                            int expert_begin, int E, int* cnt, int key[ROUNDS],
                                            int rank[ROUNDS]) {
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  const int kb = bits_for(E);
  const uint64_t lt = (1ull << lane) - 1ull;
  int* my = cnt + w * E;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int idx = w * ROWS_PER_WAVE + r * WAVE + lane;
    int k = -1;
    if (idx < n_in) {
      const int id = ids[base + idx] - expert_begin;
      k = (id >= 0 && id < E) ? id : -1;
    }
    const bool valid = k >= 0;
    const uint64_t same = match_any(k, valid, kb);
    int rk = -1;
    if (valid) {
      const int prev = my[k];
      rk = prev + __popcll(same & lt);
      if ((same & lt) == 0ull) my[k] = prev + __popcll(same);   // lowest lane of the group
    }
    key[r] = k;
    rank[r] = rk;
  }
}

// Exclusive scan over a block of SORT_THREADS (or 1024) threads; returns this thread's
// exclusive prefix and writes the total to *total.
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
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < NT / WAVE; ++i) { const int t = tmp[i]; tmp[i] = run; run += t; }
    tmp[NT / WAVE] = run;
  }
  __syncthreads();
  const int res = tmp[w] + incl - v;
  *total = tmp[NT / WAVE];
  __syncthreads();
  return res;
}

// Per-expert tile counts -> tile offsets, expert_ids, padding sentinels, tail, num_tiles.
// counts[e] holds c_e on entry and the first row position of expert e on exit.
template <int NT>
__device__ void layout_from_counts(int* counts, int E, int block_m, int sentinel,
                                   const SortLayout& L, int* tmp) {
  const int per = (E + NT - 1) / NT;
  const int e0 = threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) local += (counts[e] + block_m - 1) / block_m;
  }
  int total = 0;
  int off = block_exclusive_scan<NT>(local, tmp, &total);
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    const int c = counts[e];
    const int nt = (c + block_m - 1) / block_m;
    for (int t = 0; t < nt; ++t) L.expert_ids[off + t] = e;
    const int64_t first = (int64_t)off * block_m;
    for (int p = c; p < nt * block_m; ++p) {          // padding of this expert's last tile
      L.sorted_ids[first + p] = sentinel;
      if (L.sorted_w) L.sorted_w[first + p] = 0.0f;
    }
    counts[e] = (int)first;
    off += nt;
  }
  for (int64_t t = total + threadIdx.x; t < L.cap_tiles; t += NT) L.expert_ids[t] = -1;
  for (int64_t p = (int64_t)total * block_m + threadIdx.x; p < (int64_t)L.cap_tiles * block_m; p += NT) {
    L.sorted_ids[p] = sentinel;
    if (L.sorted_w) L.sorted_w[p] = 0.0f;
  }
  if (threadIdx.x == 0) *L.num_tiles = total;
}

// ---------------------------------------------------------------- one-workgroup path

__global__ __launch_bounds__(SORT_THREADS) void sort_small_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ topk_w, int n, int expert_begin,
    int E, int block_m, SortLayout L) {
  extern __shared__ int smem[];
  int* cnt = smem;                       // [SORT_WAVES][E]
  int* pos = cnt + SORT_WAVES * E;       // [E]
  int* tmp = pos + E;                    // [SORT_WAVES + 1]
  for (int i = threadIdx.x; i < SORT_WAVES * E; i += SORT_THREADS) cnt[i] = 0;
  __syncthreads();
  int key[ROUNDS], rank[ROUNDS];
  count_chunk(ids, 0, n, expert_begin, E, cnt, key, rank);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += SORT_THREADS) {
    int run = 0;
    for (int w = 0; w < SORT_WAVES; ++w) { const int c = cnt[w * E + e]; cnt[w * E + e] = run; run += c; }
    pos[e] = run;
  }
  __syncthreads();
  layout_from_counts<SORT_THREADS>(pos, E, block_m, n, L, tmp);
  __syncthreads();
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    if (key[r] < 0) continue;
    const int v = w * ROWS_PER_WAVE + r * WAVE + lane;
    const int p = pos[key[r]] + cnt[w * E + key[r]] + rank[r];
    L.sorted_ids[p] = v;
    if (L.sorted_w) L.sorted_w[p] = topk_w[v];
  }
}

// ---------------------------------------------------------------- multi-chunk path

__global__ __launch_bounds__(SORT_THREADS) void sort_count_kernel(
    const int32_t* __restrict__ ids, int64_t n, int expert_begin, int E, int* __restrict__ hist,
    int* __restrict__ ranks) {
  extern __shared__ int cnt[];           // [SORT_WAVES][E]
  for (int i = threadIdx.x; i < SORT_WAVES * E; i += SORT_THREADS) cnt[i] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * MOE_SORT_CHUNK;
  const int n_in = (int)(n - base < MOE_SORT_CHUNK ? n - base : MOE_SORT_CHUNK);
  int key[ROUNDS], rank[ROUNDS];
  count_chunk(ids, base, n_in, expert_begin, E, cnt, key, rank);
  __syncthreads();
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    if (key[r] < 0) continue;
    int before = 0;
    for (int ww = 0; ww < w; ++ww) before += cnt[ww * E + key[r]];
    ranks[base + w * ROWS_PER_WAVE + r * WAVE + lane] = before + rank[r];
  }
  for (int e = threadIdx.x; e < E; e += SORT_THREADS) {
    int s = 0;
    for (int ww = 0; ww < SORT_WAVES; ++ww) s += cnt[ww * E + e];
    hist[(int64_t)blockIdx.x * E + e] = s;
  }
}

constexpr int SCAN_THREADS = 1024;

__global__ __launch_bounds__(SCAN_THREADS) void sort_scan_kernel(int* __restrict__ hist, int nchunks,
                                                                 int E, int block_m, int sentinel,
                                                                 SortLayout L) {
  extern __shared__ int smem[];
  int* pos = smem;                       // [E]
  int* tmp = pos + E;                    // [SCAN_THREADS / WAVE + 1]
  for (int e = threadIdx.x; e < E; e += SCAN_THREADS) {
    int run = 0;
    for (int c = 0; c < nchunks; ++c) {
      const int h = hist[(int64_t)c * E + e];
      hist[(int64_t)c * E + e] = run;
      run += h;
    }
    pos[e] = run;
  }
  __syncthreads();
  layout_from_counts<SCAN_THREADS>(pos, E, block_m, sentinel, L, tmp);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += SCAN_THREADS) {
    const int first = pos[e];
    for (int c = 0; c < nchunks; ++c) hist[(int64_t)c * E + e] += first;
  }
}

__global__ __launch_bounds__(SORT_THREADS) void sort_scatter_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ topk_w, int64_t n, int expert_begin,
    int E, const int* __restrict__ hist, const int* __restrict__ ranks, SortLayout L) {
  const int64_t base = (int64_t)blockIdx.x * MOE_SORT_CHUNK;
  for (int i = threadIdx.x; i < MOE_SORT_CHUNK; i += SORT_THREADS) {
    const int64_t v = base + i;
    if (v >= n) break;
    const int k = ids[v] - expert_begin;
    if (k < 0 || k >= E) continue;
    const int p = hist[(int64_t)blockIdx.x * E + k] + ranks[v];
    L.sorted_ids[p] = (int32_t)v;
    if (L.sorted_w) L.sorted_w[p] = topk_w[v];
  }
}

}  // namespace

hipError_t launch_sort(const int32_t* topk_ids, const float* topk_w, int64_t n, int expert_begin,
                       int E, int block_m, const SortLayout& L, void* ws, hipStream_t s) {
  const int sentinel = (int)n;
  if (n <= MOE_SORT_CHUNK) {
    const size_t lds = (size_t)(SORT_WAVES * E + E + SORT_WAVES + 1) * sizeof(int);
    sort_small_kernel<<<1, SORT_THREADS, lds, s>>>(topk_ids, topk_w, (int)n, expert_begin, E, block_m, L);
    return hipGetLastError();
  }
  const int nchunks = (int)((n + MOE_SORT_CHUNK - 1) / MOE_SORT_CHUNK);
  int* hist = (int*)ws;
  int* ranks = (int*)((char*)ws + moe_align256((size_t)nchunks * E * sizeof(int)));
  sort_count_kernel<<<nchunks, SORT_THREADS, (size_t)SORT_WAVES * E * sizeof(int), s>>>(
      topk_ids, n, expert_begin, E, hist, ranks);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  sort_scan_kernel<<<1, SCAN_THREADS, (size_t)(E + SCAN_THREADS / WAVE + 1) * sizeof(int), s>>>(
      hist, nchunks, E, block_m, sentinel, L);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  sort_scatter_kernel<<<nchunks, SORT_THREADS, 0, s>>>(topk_ids, topk_w, n, expert_begin, E, hist, ranks, L);
  return hipGetLastError();
}

}  // namespace moe
