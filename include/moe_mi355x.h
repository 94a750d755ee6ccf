/*
 * moe_mi355x.h -- C ABI of the fused two-stage MXFP4 mixture-of-experts FFN for MI355X
 * (gfx950), library libmoe_mi355x.so.
 *
 * The operator (github ROCm/aiter PR 6259 "Motivation"/"Technical Details", PR 5118
 * "Summary", PR 4463 "What", PR 4471 "Technical Details"):
 *   1. moe_sort      groups routed rows (token t, slot k) by expert and pads each expert to a
 *                    whole tile of block_m rows (PR 5118, "Summary": moe_sorting);
 *   2. moe_quant_act encodes bf16 activations as fp8 e4m3 or fp4 e2m1 codes with one e8m0
 *                    scale per 32 elements (PR 6259 "Test Result": fp8_blockwise_1x32;
 *                    PR 4463 "What": the fp4x2 activation dtype);
 *   3. moe_fused     Stage1: gathered rows x [gate|up] MXFP4 weights with the SiTUv2 epilogue
 *                    y = beta*tanh(g/beta)*sigmoid(g) * lb*tanh(u/lb) (PR 6259 "Motivation"),
 *                    tanh evaluated as 2*sigmoid(2x)-1 (PR 4471 "Technical Details");
 *                    the intermediate re-encoded in the activation dtype; Stage2: MXFP4
 *                    down-projection, times the router weight, summed into each token's row.
 *   moe_pack_w1 and moe_pack_w2 reorder the Stage1 and Stage2 weights once into the layout
 *   moe_fused streams; moe_fused takes a w_layout tag and accepts only those packed layouts.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  No call allocates or frees
 *     device memory, and none keeps a caller's pointer after it returns.  Host-side state: the
 *     thread-local last HIP error (moe_last_hip_error) and, for moe_fused_noalloc only, the
 *     device address of its fixed scratch array on each device (taken once, under a lock), so
 *     calls from several host threads are safe.  Launch shapes that depend on the device (the
 *     compute unit count of the large-batch kernels) are queried at each call.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only enqueues work on
 *     it and never synchronizes; results are ready when the stream reaches that point.
 *   - Arguments are validated on the host before anything is enqueued.  On a validation error
 *     nothing is launched and the output buffers are untouched.  MOE_ERR_HIP means a launch
 *     failed; hipGetLastError() was cleared and its value is returned by moe_last_hip_error().
 *   - Layouts are row-major and densely packed.  fp4x2 packs two e2m1 codes per byte, the
 *     element with the even index in the low nibble.  e8m0 scale byte s means 2^(s-127).
 *   - fp8 is OCP E4M3FN (bias 7, max 448, no infinities).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, bad enum value */
  MOE_ERR_UNSUPPORTED = 2,   /* a shape or option the kernels do not implement */
  MOE_ERR_CAPACITY = 3,      /* layout capacity smaller than moe_cap_tiles() */
  MOE_ERR_HIP = 4,           /* a HIP launch failed */
  MOE_ERR_WORKSPACE = 5,     /* workspace smaller than the *_ws_bytes() helper requires */
  MOE_ERR_DEBUG_CHECK = 6    /* debug build only (libmoe_mi355x_debug.so, compiled with
                                MOE_DEBUG_CHECKS): a device-side index check failed; the
                                guarded accesses were skipped and the outputs are not valid.
                                That build waits for the device at the end of every call. */
} moe_status_t;

typedef enum { MOE_DT_BF16 = 0, MOE_DT_FP8_E4M3 = 1, MOE_DT_FP4_E2M1 = 2 } moe_dtype_t;

/* Activation of the stage1 epilogue.  SITUV2 and SILU take act(g) * up as described above
 * (SILU: y = silu(g) * u, PR 4471 "Motivation").  NONE_TEST is a test hook: moe_fused runs
 * Stage1 only and writes the raw fp32 gate and up sums of every routed row to the workspace
 * (see moe_fused_debug_offset); `out` is not written.  Any other value -> MOE_ERR_UNSUPPORTED
 * (PR 4471 "Technical Details": reject activations other than silu and situv2). */
typedef enum { MOE_ACT_SITUV2 = 0, MOE_ACT_SILU = 1, MOE_ACT_NONE_TEST = 2 } moe_act_t;

/* Which stages moe_fused runs (see `stages` there). */
typedef enum { MOE_STAGE_1 = 1, MOE_STAGE_2 = 2, MOE_STAGE_ALL = 3 } moe_stages_t;

/* Byte layout of the weights handed to moe_fused.  ROW_MAJOR: w1 [E, 2I, D/2] and w2
 * [E, D, I/2] fp4x2 as stored by a checkpoint; W1_PACKED: w1 as moe_pack_w1 writes it, w2
 * row-major; PACKED: w1 from moe_pack_w1 and w2 from moe_pack_w2.  moe_fused streams only
 * PACKED (ROW_MAJOR and W1_PACKED -> MOE_ERR_UNSUPPORTED, any other value ->
 * MOE_ERR_INVALID_ARG): the tag makes the caller state which bytes it passes, since every
 * layout has the same size. */
typedef enum { MOE_W_ROW_MAJOR = 0, MOE_W1_PACKED = 1, MOE_W_PACKED = 2 } moe_w_layout_t;

/* There are no default betas: PR 4463 "Three tuner defects" item 1 shows two sides silently
 * using different defaults.  beta and linear_beta must be finite and > 0 for SITUV2. */
typedef struct {
  int32_t act;          /* moe_act_t */
  float beta;           /* SiTUv2 beta (4.0 on the pages) */
  float linear_beta;    /* SiTUv2 linear_beta (25.0 on the pages) */
} moe_act_params_t;

/* Padded expert-major layout written by moe_sort and read by moe_fused.
 * Routed row (t, k) is named by its flat index v = t*topk + k.  For each local expert e in
 * ascending order, its rows are listed in ascending v and padded with the sentinel T*topk to a
 * multiple of block_m; experts without rows get no tile.  Tile i holds rows
 * [i*block_m, (i+1)*block_m) of sorted_token_ids and belongs to expert expert_ids[i].
 * row_of is the inverse: the position of routed row v in sorted_token_ids, or -1 when v's
 * expert is not local.
 * sync is optional scratch of moe_sync_words(T, cap_tiles) int32 words, 16-byte aligned:
 * moe_sort sets it to zero; moe_fused, when it is given and T < MOE_SINGLE_LAUNCH_MAX_TOKENS,
 * runs Stage1, Stage2 and the combine as ONE launch whose workgroups count finished work items
 * in these words (and sets them back to zero before it ends, so the layout can be reused
 * without sorting again).  Calls that use the same sync words must not overlap in time.
 * Word 0 is a sticky error flag: nonzero after a wait for another workgroup timed out (about
 * 0.25 s; the outputs of that call are then invalid); only moe_sort clears it.  sync == NULL
 * selects one launch per stage, which measured faster on MI355X at every batch size tried (the single grid must hold Stage1's
 * register footprint, which lowers Stage2's occupancy); the single launch halves the number of
 * kernel launches per call, for callers bound by launch overhead. */
typedef struct {
  int32_t *sorted_token_ids; /* [cap_tiles*block_m] v, or T*topk on padding and unused tiles */
  float *sorted_weights;     /* [cap_tiles*block_m] topk_w[v], 0 on padding; may be NULL */
  int32_t *expert_ids;       /* [cap_tiles] local expert of each tile, -1 past num_tiles */
  int32_t *num_tiles;        /* [1] number of used tiles; written on the device only */
  int32_t *row_of;           /* [T*topk] position of each routed row, -1 if not local */
  int32_t *sync;             /* [moe_sync_words(T, cap_tiles)] or NULL, see above */
  int32_t cap_tiles;         /* tiles the buffers hold, >= moe_cap_tiles(...) */
  int32_t block_m;           /* rows per tile: 16 or 32 */
} moe_layout_t;

/* Rows per tile the library's kernels are tuned for: 16 up to 512 tokens, 32 above (PR 5118
 * "Summary" and "Optimizations Applied": block_m 16 for the decode batches, 32 for prefill;
 * the crossover measured on MI355X with the packed weights lies between 512 and 768 tokens).
 * Either value is accepted by every entry point; this is the default a caller should size its
 * layout with. */
static inline int32_t moe_block_m(int32_t tokens) { return tokens <= 512 ? 16 : 32; }

/* Largest batch (exclusive) that moe_fused runs as one launch when layout->sync is given. */
#define MOE_SINGLE_LAUNCH_MAX_TOKENS 2048
/* Column classes per token of the single-launch combine counters. */
#define MOE_SYNC_CLASSES 16

/* One 64-byte line per counter: a header line, two per tile, MOE_SYNC_CLASSES per token. */
static inline size_t moe_sync_words(int32_t tokens, int32_t cap_tiles) {
  return 16 * (1 + 2 * (size_t)cap_tiles + (size_t)MOE_SYNC_CLASSES * (size_t)tokens);
}

/* Tiles needed in the worst case: sum_e ceil(c_e/bm) <= ceil(T*topk/bm) + min(E, T*topk). */
static inline int32_t moe_cap_tiles(int32_t tokens, int32_t topk, int32_t num_local_experts,
                                    int32_t block_m) {
  int64_t n = (int64_t)tokens * topk;
  int64_t e = num_local_experts < n ? num_local_experts : n;
  return (int32_t)((n + block_m - 1) / block_m + e);
}

/* Most local experts moe_sort handles. */
#define MOE_SORT_MAX_EXPERTS 2048

/* Routed rows are counted in chunks of MOE_SORT_MIN_CHUNK to MOE_SORT_CHUNK flat indices (the
 * sort takes the size from the number of rows: about 64 chunks). */
#define MOE_SORT_CHUNK 4096
#define MOE_SORT_MIN_CHUNK 1024

static inline size_t moe_align256(size_t b) { return (b + 255) & ~(size_t)255; }

/* Workspace of moe_sort: per-chunk expert offsets plus each expert's first row and row count,
 * and per-row ranks (int32). */
static inline size_t moe_sort_ws_bytes(int32_t tokens, int32_t topk, int32_t num_local_experts) {
  int64_t n = (int64_t)tokens * topk;
  int64_t chunks = (n + MOE_SORT_MIN_CHUNK - 1) / MOE_SORT_MIN_CHUNK;
  return moe_align256((size_t)(chunks + 2) * (size_t)num_local_experts * 4) + moe_align256((size_t)n * 4);
}

/* Bytes of one intermediate row of inter_dim elements in dtype dt (codes only). */
static inline size_t moe_row_bytes(int32_t cols, int32_t dt) {
  return dt == MOE_DT_BF16 ? (size_t)cols * 2 : dt == MOE_DT_FP8_E4M3 ? (size_t)cols : (size_t)cols / 2;
}

/* Bytes per element of the per-row Stage2 outputs (bf16 for every activation dtype). */
static inline size_t moe_rowout_elem_bytes(int32_t a_dtype) { (void)a_dtype; return 2; }

/* Most experts the large-batch Stage2 takes token-major (see moe_fused: experts with at least a
 * quarter of the tokens' rows). */
#define MOE_HOT_MAX 16

/* Workspace of moe_fused: byte offsets of its parts (each 256-byte aligned) and the total.
 *   rowout    [cap*bm, D] bf16 per-row Stage2 outputs (router weight applied on the per-tile
 *             path, by the combine after the large-batch Stage2);
 *   inter     [cap*bm + 1, I] Stage1 intermediate in a_dtype (codes), in layout-row order; the
 *             extra last row is a zero row the token-major Stage2 reads for absent (token, expert)
 *             pairs;  iscale: its [cap*bm + 1, I/32] e8m0 scales (fp8 / fp4);
 *   groups    [cap] (first tile, tile count) groups of one expert's tiles, then their count and
 *             eight work counters of the large-batch Stage1;
 *   cgroups   the same list without the token-major (hot) experts' groups, then its count;
 *   tile_hot  [cap] hot index of each tile's expert or -1;  hot_e: [MOE_HOT_MAX] hot experts and
 *             their count;
 *   hotpos, hotw [T, MOE_HOT_MAX] each token's layout row and router weight per hot expert;
 *   hotmask   [T] the token's slots k whose expert is hot (bit k);
 *   hot_out   [T, D] bf16 sum over the token's hot experts of the router-weighted Stage2 rows;
 *   dbg       (NONE_TEST only) fp32 [cap*bm, 2I] raw gate (cols 0..I-1) and up (I..2I-1) sums of
 *             each layout row. */
typedef struct {
  size_t rowout, inter, iscale, groups, cgroups, tile_hot, hot_e, hotpos, hotw, hotmask, hot_out, dbg, total;
} moe_fused_ws_parts_t;

static inline moe_fused_ws_parts_t moe_fused_ws_parts(int32_t tokens, int32_t model_dim, int32_t inter_dim,
                                                      int32_t cap_tiles, int32_t block_m, int32_t a_dtype,
                                                      int32_t act) {
  moe_fused_ws_parts_t w;
  size_t rows = (size_t)cap_tiles * block_m, o = 0;
  size_t t = tokens > 0 ? (size_t)tokens : 0;
  w.rowout = o;   o += moe_align256(rows * (size_t)model_dim * moe_rowout_elem_bytes(a_dtype));
  w.inter = o;    o += moe_align256((rows + 1) * moe_row_bytes(inter_dim, a_dtype));
  w.iscale = o;   o += moe_align256(a_dtype == MOE_DT_BF16 ? 0 : (rows + 1) * (size_t)(inter_dim / 32));
  w.groups = o;   o += moe_align256((size_t)cap_tiles * 8) + 256;
  w.cgroups = o;  o += moe_align256((size_t)cap_tiles * 8) + 256;
  w.tile_hot = o; o += moe_align256((size_t)cap_tiles * 4);
  w.hot_e = o;    o += 256;
  w.hotpos = o;   o += moe_align256(t * MOE_HOT_MAX * 4);
  w.hotw = o;     o += moe_align256(t * MOE_HOT_MAX * 4);
  w.hotmask = o;  o += moe_align256(t * 4);
  w.hot_out = o;  o += moe_align256(t * (size_t)model_dim * 2);
  w.dbg = o;      o += act == MOE_ACT_NONE_TEST ? moe_align256(rows * (size_t)inter_dim * 2 * 4) : 0;
  w.total = o;
  return w;
}

/* Offset of the NONE_TEST debug area in the workspace. */
static inline size_t moe_fused_debug_offset(int32_t tokens, int32_t model_dim, int32_t inter_dim,
                                            int32_t cap_tiles, int32_t block_m, int32_t a_dtype) {
  return moe_fused_ws_parts(tokens, model_dim, inter_dim, cap_tiles, block_m, a_dtype, MOE_ACT_NONE_TEST).dbg;
}

static inline size_t moe_fused_ws_bytes(int32_t tokens, int32_t model_dim, int32_t inter_dim,
                                        int32_t cap_tiles, int32_t block_m, int32_t a_dtype,
                                        int32_t act) {
  return moe_fused_ws_parts(tokens, model_dim, inter_dim, cap_tiles, block_m, a_dtype, act).total;
}

/* moe_sort -- build the padded expert-major layout (PR 5118 "Summary"; PR 6259 Stage1 input).
 *   topk_ids  [tokens, topk] int32 global expert ids; ids outside
 *             [expert_begin, expert_begin + num_local_experts) (including -1) are skipped.
 *   topk_w    [tokens, topk] fp32 router weights, or NULL; required iff
 *             layout->sorted_weights is non-NULL.
 *   layout    buffers to fill; cap_tiles >= moe_cap_tiles(tokens, topk, num_local_experts,
 *             block_m), block_m in {16, 32}.  Every entry of all buffers is written (row_of may
 *             be NULL here; moe_fused needs it; sync, when given, is set to zero).
 *   ws        device scratch of ws_bytes >= moe_sort_ws_bytes(tokens, topk, num_local_experts).
 * The result is unique and bit-exact: it does not depend on launch order or timing.
 * Limits: tokens*topk < 2^31 (tokens == 0 writes an empty layout), 1 <= num_local_experts <= 2048
 * (MOE_SORT_MAX_EXPERTS: the per-expert counters live in LDS); larger values ->
 * MOE_ERR_UNSUPPORTED. */
moe_status_t moe_sort(const int32_t *topk_ids, const float *topk_w, int32_t tokens, int32_t topk,
                      int32_t expert_begin, int32_t num_local_experts, const moe_layout_t *layout,
                      void *ws, size_t ws_bytes, void *stream);

/* moe_quant_act -- 1x32 block quantization of bf16 rows (PR 6259 "Test Result"; PR 4463).
 *   x_bf16    [rows, cols] bf16 bit patterns, cols % 32 == 0.
 *   dt        MOE_DT_FP8_E4M3 -> q_out [rows, cols] bytes; MOE_DT_FP4_E2M1 -> q_out
 *             [rows, cols/2] fp4x2 bytes.  MOE_DT_BF16 -> MOE_ERR_INVALID_ARG.
 *   scale_out [rows, cols/32] e8m0 bytes.
 * Rule per block of 32 (OCP MX shared scale): amax = max|x|; amax == 0 -> scale byte 0 and
 * every element +-0; else sexp = clamp(floor(log2 amax) - emax, -127, 127) (emax 8 for e4m3, 2
 * for e2m1), scale byte sexp + 127, each element x / 2^sexp rounded to nearest, ties to even,
 * saturating at +-448 / +-6; the sign bit is kept.  A block holding Inf or NaN gets scale byte
 * 255 (NaN) and element codes 0. */
moe_status_t moe_quant_act(const uint16_t *x_bf16, int64_t rows, int64_t cols, int32_t dt,
                           void *q_out, uint8_t *scale_out, void *stream);

/* moe_pack_w1 -- reorder the Stage1 weights once into the layout moe_fused reads (a one-time
 * weight preparation, not a step of the pages' operator).  A matrix-core operand of 16 weight
 * rows at one 128-deep K step is then 1 KB of consecutive bytes in lane order instead of 16
 * separate 64-byte pieces; on MI355X this made Stage1 12-18% faster from 1 to 1024 tokens
 * (per-tile Stage1 9.1 -> 8.0 us at 1 token, 339 -> 278 us at 1024 tokens).
 *   w1         [E, 2I, D/2] fp4x2, row-major (rows 0..I-1 gate, I..2I-1 up).
 *   w1_packed  E*2I*D/2 bytes, caller-owned; the byte ranges of w1 and w1_packed must not
 *              overlap (else MOE_ERR_INVALID_ARG): 1 KB blocks (e, f, s) for row
 *              group f < 2I/16 and K step s < D/128, in that order (s fastest); byte
 *              16*(16*g + r) + b of a block is byte 64*s + 16*g + b of row 16*f + r of expert e
 *              (g < 4, r < 16, b < 16).  The e8m0 scales keep their layout.
 * Shapes as moe_fused: D % 128 == 0, I % 128 == 0 (else MOE_ERR_UNSUPPORTED); E >= 1.
 * Asynchronous on `stream`; a pure copy, bit-exact. */
moe_status_t moe_pack_w1(const uint8_t *w1, int32_t num_experts, int32_t model_dim, int32_t inter_dim,
                         uint8_t *w1_packed, void *stream);

/* moe_pack_w2 -- the same one-time reordering for the Stage2 weights.  Row-major, a 16-row
 * operand of w2 at one K step takes 64 of each row's I/2 bytes, so the 128-byte lines of the
 * rows are split between the loads of two steps; packed, each operand is one 1 KB block, read
 * whole with the non-temporal hint.  Measured on MI355X (moe_fused, 896 experts, 3584 x 384):
 * 4.6% faster at 1 token, 8.5% at 64, 7.5% at 256, 4.7% at 1024, 0.5-2.2% at 2048-16384.
 *   w2         [E, D, I/2] fp4x2, row-major.
 *   w2_packed  E*D*I/2 bytes, caller-owned; the byte ranges of w2 and w2_packed must not overlap
 *              (else MOE_ERR_INVALID_ARG): 1 KB blocks (e, f, s) for row group f < D/16 and K
 *              step s < I/128, in that order (s fastest); byte 16*(16*g + r) + b of a block is
 *              byte 64*s + 16*g + b of row 16*f + r of expert e (g < 4, r < 16, b < 16).  The
 *              e8m0 scales keep their layout.
 * Shapes as moe_fused: D % 128 == 0, I % 128 == 0 (else MOE_ERR_UNSUPPORTED); E >= 1.
 * Asynchronous on `stream`; a pure copy, bit-exact. */
moe_status_t moe_pack_w2(const uint8_t *w2, int32_t num_experts, int32_t model_dim, int32_t inter_dim,
                         uint8_t *w2_packed, void *stream);

/* moe_fused -- Stage1 + Stage2 over a layout from moe_sort.
 *   x         activations [tokens, D]: bf16 (a_dtype BF16), fp8 bytes (FP8) or fp4x2 bytes
 *             [tokens, D/2] (FP4), as moe_quant_act writes them.
 *   x_scale   [tokens, D/32] e8m0 for FP8 / FP4; must be NULL for BF16.
 *   w1        Stage1 weights [E, 2I, D/2] fp4x2 (rows 0..I-1 gate, I..2I-1 up) in the packed
 *             layout moe_pack_w1 writes.
 *   w_layout  MOE_W_PACKED (the only layout moe_fused reads; MOE_W_ROW_MAJOR and
 *             MOE_W1_PACKED -> MOE_ERR_UNSUPPORTED: pack both weights once with moe_pack_w1 and
 *             moe_pack_w2 first).
 *   w1_scale  [E, 2I, D/32] e8m0, row-major.
 *   w2        Stage2 weights [E, D, I/2] fp4x2 in the packed layout moe_pack_w2 writes.
 *   w2_scale  [E, D, I/32] e8m0, row-major.
 *   topk_w    [tokens, topk] fp32 router weights; row v of the layout is scaled by topk_w[v].
 *   layout    from moe_sort with the same tokens/topk/E; cap_tiles and block_m as there.
 *   act       activation and betas (no defaults).
 *   out_bf16  [tokens, D] bf16, overwritten; tokens with no local expert get zeros.
 *   ws        scratch of ws_bytes >= moe_fused_ws_bytes(...).
 *   stages    MOE_STAGE_ALL (both), MOE_STAGE_1 (Stage1 only: leaves the intermediate in
 *             ws; `out` untouched) or MOE_STAGE_2 (Stage2 + combine only, reading the
 *             intermediate a MOE_STAGE_1 call with the same layout and shapes left in the same
 *             ws).  Any other value -> MOE_ERR_INVALID_ARG.  The split calls always use one
 *             launch per stage.
 * Shapes: D % 128 == 0 and I % 128 == 0 (else MOE_ERR_UNSUPPORTED: every K step is one
 * 128-deep block-scaled MFMA); E >= 1.  Stage1 uses fp32 accumulation; the intermediate is
 * stored as bf16 (BF16) or re-encoded with the moe_quant_act rule (FP8, FP4); Stage2
 * accumulates in fp32, stores each routed row's output in bf16 (scaled by its router weight
 * in Stage2, or in the combine after the large-batch Stage2), and the combine sums each token's
 * rows in ascending k in fp32 and rounds to bf16: the result is deterministic, and the single-launch and per-stage paths give the same
 * bits.  layout->row_of must be set. */
moe_status_t moe_fused(const void *x, const uint8_t *x_scale, int32_t a_dtype,
                       const uint8_t *w1, int32_t w_layout, const uint8_t *w1_scale,
                       const uint8_t *w2, const uint8_t *w2_scale,
                       const float *topk_w, const moe_layout_t *layout,
                       int32_t tokens, int32_t topk, int32_t num_local_experts,
                       int32_t model_dim, int32_t inter_dim, const moe_act_params_t *act,
                       uint16_t *out_bf16, void *ws, size_t ws_bytes, int32_t stages,
                       void *stream);

/* Bytes of the fixed device scratch moe_fused_noalloc works in (128 MiB per device). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* moe_fused_noalloc -- moe_fused for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments,
 * kernels and results as moe_fused, without ws / ws_bytes.  Its workspace is a scratch array of
 * MOE_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on, from the first
 * call on that device until the process ends; the call itself allocates nothing (no hipMalloc,
 * hipFree or allocating library routine).
 *   - A call whose moe_fused_ws_bytes(...) exceeds MOE_NOALLOC_SCRATCH_BYTES returns
 *     MOE_ERR_WORKSPACE before anything is launched (at model_dim 3584 and inter_dim 384 the
 *     scratch holds batches up to 128 tokens of any activation dtype at top-16 over 896 experts;
 *     use moe_fused with a caller workspace above that).
 *   - Every call on a device shares that device's scratch, which keeps the last call's
 *     contents: calls that overlap in time on one device (other streams or other threads) race,
 *     and a MOE_STAGE_2 call reads the intermediate the last MOE_STAGE_1 call on that device left.
 *     No part of the scratch needs to start at zero: a call writes every byte it reads there.
 *   - The first call on a device takes the scratch's device address (hipGetSymbolAddress, not an
 *     allocation); a failure there returns MOE_ERR_HIP. */
moe_status_t moe_fused_noalloc(const void *x, const uint8_t *x_scale, int32_t a_dtype,
                               const uint8_t *w1, int32_t w_layout, const uint8_t *w1_scale,
                               const uint8_t *w2, const uint8_t *w2_scale,
                               const float *topk_w, const moe_layout_t *layout,
                               int32_t tokens, int32_t topk, int32_t num_local_experts,
                               int32_t model_dim, int32_t inter_dim, const moe_act_params_t *act,
                               uint16_t *out_bf16, int32_t stages, void *stream);

/* The hipError_t value behind the last MOE_ERR_HIP returned on this thread (0 if none). */
int32_t moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
