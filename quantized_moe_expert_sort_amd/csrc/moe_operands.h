// Matrix-core operand loaders and element stores shared by the per-stage kernels and the
// single-launch kernel.  COH selects device-coherent accesses for data that another workgroup
// of the same launch writes or reads: agent-scope relaxed atomic loads and stores, which gfx950
// issues with the sc1 cache-control bit (the store is written through to the device coherence
// point, the load misses every non-coherent cache level).
#pragma once

#include "moe_device.h"

namespace moe {

template <bool COH = false>
__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
  if constexpr (COH) {
    const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
    const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return uint4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}

// 16 bytes of a stream that is read once per launch in whole 128-byte lines (one load
// instruction of a wave covers a contiguous 1 KB: the packed Stage1 weights, the per-row Stage2
// outputs the combine sums), with the non-temporal hint.  On an MI355X a plain streaming read of
// 2 GiB ran at 7.0-7.2 TB/s with the hint and 6.1-6.2 TB/s without it.  Not for data whose lines
// are split between two load instructions (the 192-byte row-major Stage2 weight rows): there the
// hint made Stage2 slower.
__device__ __forceinline__ uint4 ldw16(const uint8_t* p) {
  typedef uint32_t u4v_ __attribute__((ext_vector_type(4)));
  const u4v_ v = __builtin_nontemporal_load(reinterpret_cast<const u4v_*>(p));
  return uint4{v[0], v[1], v[2], v[3]};
}

template <bool COH, class T>
__device__ __forceinline__ T ld(const T* p) {
  if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}

template <bool COH, class T>
__device__ __forceinline__ void st(T* p, T v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

// Wait until every store this lane issued has completed (for COH stores: reached the device
// coherence point).
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ v8i fp4_operand(const uint4& q) {
  v8i r = {(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
  return r;
}

// The same operand with dwords 4..7 left undefined: an fp4 operand of the block-scaled MFMA
// reads only dwords 0..3, so the upper registers of the tuple need not hold anything.
__device__ __forceinline__ v8i fp4_operand_lo(const uint4& q) {
  typedef int v4i_ __attribute__((ext_vector_type(4)));
  const v4i_ lo = {(int)q.x, (int)q.y, (int)q.z, (int)q.w};
  return __builtin_shufflevector(lo, lo, 0, 1, 2, 3, -1, -1, -1, -1);
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
  template <bool COH = false>
  __device__ __forceinline__ void load(const uint8_t* row, int step, int g, bool valid) {
    if (valid) {
      const uint4 lo = ld16<COH>(row + step * 128 + 16 * g);
      const uint4 hi = ld16<COH>(row + step * 128 + 64 + 16 * g);
      a = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    } else {
      a = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  // the step's operand from a row staged in LDS (base = the step's first byte)
  __device__ __forceinline__ void load_lds(const uint8_t* base, int g) {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + 16 * g);
    const uint4 hi = *reinterpret_cast<const uint4*>(base + 64 + 16 * g);
    a = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  __device__ __forceinline__ v4f mma(const uint4& bq, uint32_t bs, uint32_t as, const v4f& c) const {
    return mfma_fp8_fp4(a, fp4_operand(bq), c, as, bs);
  }
};

template <>
struct AOperand<DT_FP4> {
  v8i a;
  template <bool COH = false>
  __device__ __forceinline__ void load(const uint8_t* row, int step, int g, bool valid) {
    a = valid ? fp4_operand(ld16<COH>(row + step * 64 + 16 * g)) : v8i{0, 0, 0, 0, 0, 0, 0, 0};
  }
  __device__ __forceinline__ void load_lds(const uint8_t* base, int g) {
    a = fp4_operand(*reinterpret_cast<const uint4*>(base + 16 * g));
  }
  __device__ __forceinline__ v4f mma(const uint4& bq, uint32_t bs, uint32_t as, const v4f& c) const {
    return mfma_fp4_fp4(a, fp4_operand(bq), c, as, bs);
  }
};

// bf16 activations: the 128-deep step is four 32-deep bf16 MFMAs.  Sub-step jj takes K
// elements [32g + 8jj, 32g + 8jj + 8) of the step on lane group g for both operands, so a lane
// reads 32 consecutive bf16 of its row and the 32 fp4 weights of one scale block.
template <>
struct AOperand<DT_BF16> {
  v8bf a[4];
  template <bool COH = false>
  __device__ __forceinline__ void load(const uint8_t* row, int step, int g, bool valid) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if (valid) {
        const uint4 q = ld16<COH>(row + step * 256 + 64 * g + 16 * jj);
        a[jj] = as_bf16x8(q.x, q.y, q.z, q.w);
      } else {
        a[jj] = as_bf16x8(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void load_lds(const uint8_t* base, int g) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint4 q = *reinterpret_cast<const uint4*>(base + 64 * g + 16 * jj);
      a[jj] = as_bf16x8(q.x, q.y, q.z, q.w);
    }
  }
  __device__ __forceinline__ v4f mma(const uint4& bq, uint32_t bs, uint32_t, const v4f& c) const {
    const float sc = e8m0_to_float(bs);
    v4f r = c;
    r = mfma_bf16(a[0], fp4x8_to_bf16(bq.x, sc), r);
    r = mfma_bf16(a[1], fp4x8_to_bf16(bq.y, sc), r);
    r = mfma_bf16(a[2], fp4x8_to_bf16(bq.z, sc), r);
    r = mfma_bf16(a[3], fp4x8_to_bf16(bq.w, sc), r);
    return r;
  }
};

// e8m0 scale bytes of one matrix row for a batch of up to PF consecutive 128-deep K steps
// s0 .. s0+PF-1.  Lane (r16, g) consumes byte 4*s + g of its row for step s, so the four lane
// groups of a row need the four bytes of one dword per step.  Lane group g loads the dword of
// step s0 + 4q + g (one load instruction per four steps instead of one per step); the byte of
// step s0 + i is then taken from lane group i % 4 with a cross-lane read.  Rows whose operand
// is zero (padding) skip the load and use the scale 2^0.
template <int PF, bool COH = false>
struct ScaleQuads {
  static constexpr int NQ = (PF + 3) / 4;
  uint32_t d[NQ];
  __device__ __forceinline__ void load(const uint8_t* srow, int s0, int s_end, int g, bool valid) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int st_ = s0 + 4 * q + g;
      d[q] = (valid && st_ < s_end) ? ld<COH>(reinterpret_cast<const uint32_t*>(srow + 4 * st_)) : 0x7F7F7F7Fu;
    }
  }
  // byte of step s0 + i for this lane; wave-uniform i, executed by every lane
  __device__ __forceinline__ uint32_t get(int i, int r16, int g) const {
    const uint32_t w = (uint32_t)__shfl((int)d[i >> 2], 16 * (i & 3) + r16, WAVE);
    return (w >> (8 * g)) & 0xFFu;
  }
};

template <int ADT>
__host__ __device__ constexpr int row_bytes_num() { return ADT == DT_BF16 ? 2 : 1; }
template <int ADT>
__host__ __device__ constexpr int row_bytes_den() { return ADT == DT_FP4 ? 2 : 1; }

}  // namespace moe
