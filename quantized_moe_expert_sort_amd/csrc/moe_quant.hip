// 1x32 e8m0 block quantization of bf16 activations to fp8 e4m3 or fp4 e2m1
// (github ROCm/aiter PR 6259 "Test Result": fp8_blockwise_1x32; PR 4463 "What": fp4x2).
// Four lanes share a block of 32: each lane loads 8 bf16 (16 bytes, so a wave reads 1 KB of
// contiguous bytes per load), the block maximum is reduced over the 4 lanes, and each lane
// encodes its 8 values with the hardware scaled converts (two per instruction; the same codes
// as the integer encoder of moe_device.h) and writes 8 bytes (fp8) or 4 bytes (fp4x2); the
// first lane of a block writes the scale byte.
#include "moe_kernels.h"
#include "moe_device.h"
#include "moe_operands.h"

namespace moe {

namespace {

template <class F>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x, int64_t nocts,
                                                        uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nocts; i += stride) {
    const uint4 raw = ldw16(reinterpret_cast<const uint8_t*>(x + i * 8));   // read once: non-temporal
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = w[j] << 16, hi = w[j] & 0xFFFF0000u;
      v[2 * j] = __uint_as_float(lo);
      v[2 * j + 1] = __uint_as_float(hi);
      amax = max(amax, max(lo & 0x7FFFFFFFu, hi & 0x7FFFFFFFu));
    }
#pragma unroll
    for (int m = 2; m >= 1; m >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)amax, m, WAVE);
      amax = o > amax ? o : amax;
    }
    const bool bad = amax >= 0x7F800000u;                  // Inf / NaN: scale 255, zero codes
    const int sexp = block_sexp_any(bad ? 0u : amax, F::EMAX);
    if (F::SIGN == 0x80) {
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = bad ? 0u : encode_pair_fp8_hw(v[2 * j], v[2 * j + 1], sexp);
      *reinterpret_cast<uint2*>(q + i * 8) = uint2{c[0] | (c[1] << 16), c[2] | (c[3] << 16)};
    } else {
      const float scale = e8m0_scale_float(sexp);
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) word |= encode_pair_fp4_hw(v[2 * j], v[2 * j + 1], scale) << (8 * j);
      *reinterpret_cast<uint32_t*>(q + i * 4) = bad ? 0u : word;
    }
    if ((i & 3) == 0) sc[i >> 2] = (uint8_t)(bad ? 255u : (uint32_t)(sexp + 127));
  }
}

}  // namespace

hipError_t launch_quant_act(const uint16_t* x, int64_t rows, int64_t cols, int dt, void* q,
                            uint8_t* scale, hipStream_t s) {
  const int64_t nocts = rows * cols / 8;                 // cols % 32 == 0
  if (nocts == 0) return hipSuccess;
  int64_t blocks = (nocts + 255) / 256;
  if (blocks > 256 * 32) blocks = 256 * 32;
  if (dt == DT_FP8)
    quant_act_kernel<Fp8Fmt><<<(unsigned)blocks, 256, 0, s>>>(x, nocts, (uint8_t*)q, scale);
  else
    quant_act_kernel<Fp4Fmt><<<(unsigned)blocks, 256, 0, s>>>(x, nocts, (uint8_t*)q, scale);
  return hipGetLastError();
}

}  // namespace moe
