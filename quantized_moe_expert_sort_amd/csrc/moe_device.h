// Device-side building blocks for the gfx950 MoE kernels: matrix-core operand types, the
// block-scaled MFMA wrappers, the fp4 -> bf16 dequantizer, SiTUv2 / SiLU, and the 1x32
// e8m0 block encoder.  Everything here is written for CDNA4 wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

enum : int { DT_BF16 = 0, DT_FP8 = 1, DT_FP4 = 2 };
enum : int { ACT_SITUV2 = 0, ACT_SILU = 1, ACT_NONE = 2 };

// Operand format codes of v_mfma_scale_f32_16x16x128_f8f6f4 (cbsz / blgp fields).
enum : int { MFMA_FMT_FP8 = 0, MFMA_FMT_FP4 = 4 };

constexpr int WAVE = 64;

// ------------------------------------------------------------------ matrix-core operand layout
//
// v_mfma_scale_f32_16x16x128_f8f6f4, lane l = 16*g + r (r = l % 16, g = l / 16):
//   fp4 operand: dwords 0..3 hold K elements [32g, 32g+32) of row r, element 2i in the low
//                nibble of byte i; dwords 4..7 are ignored.
//   fp8 operand: dwords 0..3 hold K [16g, 16g+16), dwords 4..7 hold K [64+16g, 64+16g+16).
//   scale byte (selected by opsel) of lane l scales row r, K block [32g, 32g+32).
// v_mfma_f32_16x16x32_bf16: lane l holds K [8g, 8g+8) of row r.
// Both: accumulator element i of lane l is C[4g + i][r].

__device__ __forceinline__ v4f mfma_fp8_fp4(const v8i& a, const v8i& b, const v4f& c,
                                            uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, MFMA_FMT_FP8, MFMA_FMT_FP4, 0, sa, 0, sb);
}

__device__ __forceinline__ v4f mfma_fp4_fp4(const v8i& a, const v8i& b, const v4f& c,
                                            uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, MFMA_FMT_FP4, MFMA_FMT_FP4, 0, sa, 0, sb);
}

__device__ __forceinline__ v4f mfma_bf16(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// e8m0 byte -> the float 2^(s-127) (only its exponent is read by the scaled converts).
__device__ __forceinline__ float e8m0_to_float(uint32_t s) {
  return s == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(s << 23);
}

// Eight e2m1 codes (one dword, element 2i in the low nibble of byte i) -> eight bf16 values
// times 2^(s-127), exact for every finite scale that keeps the result a bf16 normal.
__device__ __forceinline__ v8bf fp4x8_to_bf16(uint32_t q, float scale) {
  v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 0);
  v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 1);
  v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 2);
  v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 3);
  v8bf r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ v8bf as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  u4 t = {a, b, c, d};
  return __builtin_bit_cast(v8bf, t);
}

// ------------------------------------------------------------------ activations
//
// sigmoid over the exp2 / reciprocal fast path; tanh(x) = 2*sigmoid(2x) - 1, which saturates to
// +-1 without clamping (github ROCm/aiter PR 4471, "Technical Details").

__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

// SiTUv2 (github ROCm/aiter PR 6259, "Motivation"):
//   y = beta*tanh(g/beta)*sigmoid(g) * lb*tanh(u/lb); inv_* are 1/beta and 1/lb.
// Evaluated with tanh(x) = sign(x) * (2*sigmoid(2|x|) - 1) = sign(x) * (1 - a) / (1 + a),
// a = e^(-2|x|), and sigmoid(g) = (g < 0 ? b : 1) / (1 + b), b = e^(-|g|): three exponentials
// of non-positive arguments (no overflow) and one reciprocal of a product in [1, 8].
__device__ __forceinline__ float situv2(float g, float u, float beta, float inv_beta, float lb,
                                        float inv_lb) {
  constexpr float LOG2E = 1.4426950408889634f;
  const float ag = __builtin_fabsf(g), au = __builtin_fabsf(u);
  const float a = __builtin_amdgcn_exp2f(ag * (-2.0f * LOG2E * inv_beta));
  const float b = __builtin_amdgcn_exp2f(ag * -LOG2E);
  const float c = __builtin_amdgcn_exp2f(au * (-2.0f * LOG2E * inv_lb));
  const float num = (1.0f - a) * (1.0f - c) * (g < 0.0f ? b : 1.0f);
  const float den = (1.0f + a) * (1.0f + b) * (1.0f + c);
  const float y = (beta * lb) * num * __builtin_amdgcn_rcpf(den);
  return __uint_as_float(__float_as_uint(y) ^ ((__float_as_uint(g) ^ __float_as_uint(u)) & 0x80000000u));
}

// SiLU epilogue (github ROCm/aiter PR 4471, "Motivation"): silu(g) * u.
__device__ __forceinline__ float silu_mul(float g, float u) { return g * fast_sigmoid(g) * u; }

// ------------------------------------------------------------------ lane exchanges (DPP)
//
// Inside each row of 16 lanes, without an LDS round trip: the value of lane l ^ 1, and the
// maximum over the row (quad butterflies, then rotations by 4 and 8 lanes).

__device__ __forceinline__ uint32_t lane_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
}

__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  uint32_t o;
  o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);      // quad_perm [1,0,3,2]
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);      // quad_perm [2,3,0,1]
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false);     // row_ror:4
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);     // row_ror:8
  v = o > v ? o : v;
  return v;
}

// ------------------------------------------------------------------ 1x32 block encoder
//
// OCP MX shared-scale rule: the block exponent is floor(log2 amax) - emax clamped to
// [-127, 127] (read from the bits of amax, never from log2f), each element is v / 2^sexp
// rounded to nearest (ties to the even code) and saturated at the largest finite code, the sign
// kept; an all-zero block has scale byte 0, a block with Inf / NaN scale byte 255 and zero
// codes.  The elements are encoded with the gfx950 scaled converts (v_cvt_scalef32_pk_fp4_f32 /
// _fp8_f32), two per instruction; their scale operand is the float whose exponent field holds
// the e8m0 byte sexp + 127 (byte 0: the denormal 2^-127), and only that field is read.  On an
// MI355X the converts gave exactly the rule's codes (checked against an integer evaluation of
// the rule) for every finite bf16 value and 400k random fp32 values at 19 block exponents from
// -127 to 126, grid mid-points and their neighbours included, once fp8 inputs are clamped to
// +-448 * 2^sexp: above 464 * 2^sexp the fp8 convert returns NaN where the rule saturates.
// The activation-quant tests compare every code and scale byte with the oracle.

struct Fp8Fmt { static constexpr int EMAX = 8, SIGN = 0x80; };
struct Fp4Fmt { static constexpr int EMAX = 2, SIGN = 0x8; };

// Block exponent of a block whose largest magnitude has the (finite) bit pattern amax.
__device__ __forceinline__ int block_sexp_any(uint32_t amax, int emax) {   // amax finite
  if (amax == 0u) return -127;
  int e = amax >= 0x00800000u ? (int)(amax >> 23) - 127 : (31 - __clz(amax)) - 149;
  e -= emax;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
__device__ __forceinline__ float e8m0_scale_float(int sexp) {
  return sexp == -127 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)(sexp + 127) << 23);
}
// fp4: a in the low nibble, b in the high nibble of the returned byte
__device__ __forceinline__ uint32_t encode_pair_fp4_hw(float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, scale, 0) & 0xFFu;
}
// fp8: a in the low byte, b in the high byte of the returned 16 bits
__device__ __forceinline__ uint32_t encode_pair_fp8_hw(float a, float b, int sexp) {
  typedef short v2s_ __attribute__((ext_vector_type(2)));
  const float scale = e8m0_scale_float(sexp);
  const float lim = 448.0f * (sexp == -127 ? __uint_as_float(0x00400000u) : scale);
  const v2s_ old = {0, 0};
  const v2s_ r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, __builtin_amdgcn_fmed3f(a, -lim, lim),
                                                          __builtin_amdgcn_fmed3f(b, -lim, lim), scale, false);
  return (uint32_t)(uint16_t)r[0];
}

// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one lane of each 16-lane row), with the
// gfx950 row swaps: permlane32_swap of a value with itself leaves lanes l and l ^ 32 holding
// the two halves' values in its two results, permlane16_swap does the same for rows l and l ^ 16.
__device__ __forceinline__ uint32_t cross_row_max_u32(uint32_t v) {
  const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = h[0] > h[1] ? h[0] : h[1];
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return r[0] > r[1] ? r[0] : r[1];
}

// Reduce |v| bit patterns over the 32 lanes of a half-wave (xor shuffles stay inside it).
__device__ __forceinline__ uint32_t halfwave_max_u32(uint32_t v) {
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, m, WAVE);
    v = o > v ? o : v;
  }
  return v;
}

}  // namespace moe
