// One-time reordering of the Stage1 and Stage2 weights into the layout the kernels stream.
//
// A matrix-core operand of 16 weight rows at one 128-deep K step is 16 rows x 64 bytes of fp4:
// in the row-major layout a wave's load of it touches 16 separate 64-byte pieces.  Packed,
// block (e, f, s) = rows 16 f .. 16 f + 15 of expert e, bytes [64 s, 64 s + 64) of each, is
// 1 KB of consecutive bytes in the order the lanes read it: byte 16 (16 g + r) + b is row
// 16 f + r, byte 64 s + 16 g + b (lane 16 g + r of the wave holds row r, K [32 g, 32 g + 32) of
// the step).  The grouped stages copy the same blocks to LDS whole.  w1 ([E, 2I, D/2], K = D)
// and w2 ([E, D, I/2], K = I) are packed the same way.  This is a weight-load time preparation
// of this library, not a step of the operator: measured on MI355X, the per-tile Stage1 ran
// 12-18% faster on the packed blocks from 1 to 1024 tokens.
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int PACK_THREADS = 256;

// thread = one 16-byte piece of the packed output
// The weights as one [E * R, K/2] matrix (R rows per expert, a multiple of 16).
__global__ __launch_bounds__(PACK_THREADS) void pack_kernel(const uint8_t* __restrict__ w,
                                                            uint8_t* __restrict__ out, int64_t pieces, int K) {
  const int64_t o = (int64_t)blockIdx.x * PACK_THREADS + threadIdx.x;
  if (o >= pieces) return;
  const int S = K / 128;
  const int64_t blk = o >> 6;
  const int l = (int)(o & 63), r = l & 15, g = l >> 4;
  const int s = (int)(blk % S);
  const int64_t ef = blk / S;                             // e * (R / 16) + f
  const int64_t row = ef * 16 + r;                        // row e * R + 16 f + r of the [E * R, K/2] matrix
  const uint4 v = *reinterpret_cast<const uint4*>(w + row * (K / 2) + 64 * s + 16 * g);
  *reinterpret_cast<uint4*>(out + o * 16) = v;
}

hipError_t launch_pack(const uint8_t* w, uint8_t* out, int64_t rows, int K, hipStream_t s) {
  const int64_t pieces = rows * (K / 2) / 16;
  const int64_t grid = (pieces + PACK_THREADS - 1) / PACK_THREADS;
  pack_kernel<<<(unsigned)grid, PACK_THREADS, 0, s>>>(w, out, pieces, K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_w1(const uint8_t* w1, uint8_t* out, int E, int D, int I, hipStream_t s) {
  return launch_pack(w1, out, (int64_t)E * 2 * I, D, s);
}

hipError_t launch_pack_w2(const uint8_t* w2, uint8_t* out, int E, int D, int I, hipStream_t s) {
  return launch_pack(w2, out, (int64_t)E * D, I, s);
}

}  // namespace moe
