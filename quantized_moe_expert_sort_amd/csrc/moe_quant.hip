// 1x32 e8m0 block quantization of bf16 activations to fp8 e4m3 or fp4 e2m1
// (github ROCm/aiter PR 6259 "Test Result": fp8_blockwise_1x32; PR 4463 "What": fp4x2).
// Eight lanes share a block of 32: each lane loads 4 bf16 (8 bytes, so a wave reads 512
// contiguous bytes per load), the block maximum is reduced over the 8 lanes, and each lane
// writes its 4 codes (4 bytes fp8 or 2 bytes fp4x2); the first lane writes the scale byte.
#include "moe_kernels.h"
#include "moe_device.h"

namespace moe {

namespace {

template <class F>
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x, int64_t nquads,
                                                        uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nquads; i += stride) {
    const uint2 raw = *reinterpret_cast<const uint2*>(x + i * 4);
    uint32_t b[4] = {raw.x << 16, raw.x & 0xFFFF0000u, raw.y << 16, raw.y & 0xFFFF0000u};
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) { const uint32_t a = b[j] & 0x7FFFFFFFu; amax = a > amax ? a : amax; }
#pragma unroll
    for (int m = 4; m >= 1; m >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)amax, m, WAVE);
      amax = o > amax ? o : amax;
    }
    uint32_t code[4];
    uint32_t sbyte;
#pragma unroll
    for (int j = 0; j < 4; ++j) code[j] = encode_in_block<F>(b[j], amax, &sbyte);
    if (F::SIGN == 0x80) {
      *reinterpret_cast<uint32_t*>(q + i * 4) = code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24);
    } else {
      *reinterpret_cast<uint16_t*>(q + i * 2) = (uint16_t)(code[0] | (code[1] << 4) | (code[2] << 8) | (code[3] << 12));
    }
    if ((i & 7) == 0) sc[i >> 3] = (uint8_t)sbyte;
  }
}

}  // namespace

hipError_t launch_quant_act(const uint16_t* x, int64_t rows, int64_t cols, int dt, void* q,
                            uint8_t* scale, hipStream_t s) {
  const int64_t nquads = rows * cols / 4;
  if (nquads == 0) return hipSuccess;
  int64_t blocks = (nquads + 255) / 256;
  if (blocks > 256 * 32) blocks = 256 * 32;
  if (dt == DT_FP8)
    quant_act_kernel<Fp8Fmt><<<(unsigned)blocks, 256, 0, s>>>(x, nquads, (uint8_t*)q, scale);
  else
    quant_act_kernel<Fp4Fmt><<<(unsigned)blocks, 256, 0, s>>>(x, nquads, (uint8_t*)q, scale);
  return hipGetLastError();
}

}  // namespace moe
