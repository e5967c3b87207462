// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, MFMA wrappers for the two half-precision input types,
// round-to-nearest-even packing and cross-half wave exchange.
//
// MFMA register layout used throughout (v_mfma_f32_32x32x16_{bf16,f16} and
// v_mfma_f32_32x32x2_f32, wave64):
//   result  C[i][j] sits in lane (j + 32*g), register r, where
//           i = 8*(r/4) + 4*g + (r%4), g = lane/32, r = 0..15;
//   inputs  A[i][k] in lane (i + 32*g), element e; B[k][j] in lane
//           (j + 32*g), element e, with the same (g, e) -> k assignment for A
//           and B. Only that sameness is relied on: the kernels pick which
//           (g, e) slot carries which key, and load both operands to match.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bfloat16 inputs: 32x32x16 MFMA, fp32 accumulate; RNE packing.
struct Bf16 {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float lo(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
  static __device__ __forceinline__ float hi(uint32_t x) {
    return __builtin_bit_cast(float, x & 0xffff0000u);
  }
};

// IEEE half inputs: same shape of MFMA, RNE packing.
struct F16 {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f16x2 r;
    r[0] = (_Float16)lo;
    r[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
  // Scalar half extraction (a bit_cast of a vector element to a 2 x half
  // vector was folded to the first element by the compiler).
  static __device__ __forceinline__ float lo(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
  }
};

// Combine a per-lane value with the value held by the lane 32 positions
// away (the other half of the wave). v_permlane32_swap exchanges the two
// halves between its two operands; feeding it the value twice leaves each
// lane holding {own, other} in its two results, in some order, so a
// symmetric combine of the two results is independent of that order.
__device__ __forceinline__ float half_swap_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ __forceinline__ float half_swap_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Map a linear workgroup id to a logical one so that runs of consecutive
// logical ids land on one XCD. Workgroups are dealt to the 8 XCDs round
// robin by linear id; when the grid is a multiple of 8, logical id
// (x * total/8 + s) is given to the s-th workgroup of XCD x.
__device__ __forceinline__ int xcd_logical_id(int lin, int total) {
  if ((total & 7) != 0) return lin;
  return (lin & 7) * (total >> 3) + (lin >> 3);
}

}  // namespace fa
