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

#include "fa_internal.h"

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
  static __device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
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
  static __device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f16x2 r;
    r[0] = (_Float16)lo;
    r[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, r);
  }
  // Scalar half extraction from a scalar word: this compiler evaluates
  // __builtin_bit_cast of a vector element (v[i]) as a bit_cast of element
  // 0, so callers pass the word itself, never a vector element.
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

// Combine over the four 16-lane rows of the wave (lanes l, l ^ 16, l ^ 32,
// l ^ 48): the 32-lane swap above, then v_permlane16_swap, which exchanges
// rows 0 <-> 1 and 2 <-> 3 between its operands the same way.
__device__ __forceinline__ float quad_max(float v) {
  v = half_swap_max(v);
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ __forceinline__ float quad_sum(float v) {
  v = half_swap_sum(v);
  auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Store one wave's 32 x D tile of fp32 MFMA results (lane (row lq, half hi),
// block db, register r -> column 32 db + 8 (r / 4) + 4 hi + r % 4), times the
// lane's factor sc and rounded to TT, as whole rows. Straight from that
// layout a store instruction would write 16 bytes into each of 32 rows; the
// tile goes through `stage` instead (32 * 2D bytes of LDS that only this wave
// uses, 16-byte chunks XOR-swizzled by row so that both the writes and the
// row-wise reads spread over the banks) and each lane then stores 16
// contiguous bytes, D / 8 lanes per row. Row r goes to out + r * stride
// (elements) when r < nrows.
template <typename TT, int D>
__device__ __forceinline__ void store_tile_rows(const f32x16 (&acc)[D / 32], float sc, char* stage,
                                                uint16_t* out, size_t stride, int nrows,
                                                int lane) {
  constexpr int CH = D / 8;     // 16-byte chunks per row
  constexpr int ROWB = 2 * D;   // bytes per row
  constexpr int RPS = 64 / CH;  // rows per store instruction
  const int lq = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      u32x2 v;
      v[0] = TT::pack2(acc[db][4 * g4 + 0] * sc, acc[db][4 * g4 + 1] * sc);
      v[1] = TT::pack2(acc[db][4 * g4 + 2] * sc, acc[db][4 * g4 + 3] * sc);
      const int chunk = (4 * db + g4) ^ (lq % CH);
      *(u32x2*)(stage + lq * ROWB + 16 * chunk + 8 * hi) = v;
    }
  // LDS operations of one wave complete in order: the reads below see the
  // writes above.
#pragma unroll
  for (int i = 0; i < 32 / RPS; ++i) {
    const int r = i * RPS + lane / CH, cpos = lane % CH;
    const u32x4 v = *(const u32x4*)(stage + r * ROWB + 16 * (cpos ^ (r % CH)));
    if (r < nrows) *(u32x4*)(out + (size_t)r * stride + 8 * cpos) = v;
  }
}

// ---- dropout bits -----------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds on a 128-bit counter with a 64-bit
// key; each round multiplies counter words 0 and 2 by two fixed constants,
// crosses the high halves into words 1 and 3 with the key, and the key is
// bumped by two Weyl constants.
// Each 32 x 32 -> 64-bit product is one multiply that gives both halves
// (v_mad_u64_u32), not a low and a high multiply.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    // Three-input XOR (bitop3 truth table 0x96): one instruction, not two.
    c = u32x4{(uint32_t)__builtin_amdgcn_bitop3_b32(hi1, c[1], k0, 0x96), lo1,
              (uint32_t)__builtin_amdgcn_bitop3_b32(hi0, c[3], k1, 0x96), lo0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Dropout of element (i, j) of head bh: byte j % 4 of word i % 4 of the
// Philox call with counter (j / 4, i / 4, bh, offset); dropped when the byte
// is below thr (thr = floor(256 p + 0.5)).
// (DropParams, the per-call constants, is declared in fa_internal.h.)

// 4x4 transpose of 32-bit words across the four lanes of a quad: lane s
// holds row s (x[0..3]) on entry and column s (rows 0..3 of column s) on
// return. It goes through LDS, one wave's own area of kQuadXWords words
// (16-byte aligned): word e of lane L is stored at word 80 e + L, and lane
// 4 q + s reads words 80 s + 4 q .. 80 s + 4 q + 3, word s of its quad's four
// lanes (three LDS instructions; the same with DPP lane exchanges took about
// twenty vector instructions). A wave's LDS accesses complete in order, so
// the area needs no barrier between uses; rows 80 words apart keep the word
// stores and the 16-byte reads free of bank conflicts.
constexpr int kQuadXWords = 3 * 80 + 64;
__device__ __forceinline__ u32x4 quad_transpose_lds(u32x4 x, uint32_t* area, int lane) {
#pragma unroll
  for (int e = 0; e < 4; ++e) area[80 * e + lane] = x[e];
  __builtin_amdgcn_wave_barrier();
  return *(const u32x4*)(area + 80 * (lane & 3) + 4 * (lane >> 2));
}

// 4x4 transpose of the bytes of four words: byte t of word w becomes byte w
// of word t. Two rounds of byte selects (v_perm: selector bytes 0 .. 3 pick
// from the second source, 4 .. 7 from the first): first the words pair up
// into (w0, w1) and (w2, w3) interleaves, then the interleaves into rows.
__device__ __forceinline__ u32x4 byte_transpose(u32x4 x) {
  const uint32_t a = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);  // x0.b0 x1.b0 x0.b1 x1.b1
  const uint32_t b = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);  // x0.b2 x1.b2 x0.b3 x1.b3
  const uint32_t c = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
  const uint32_t d = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
  return u32x4{(uint32_t)__builtin_amdgcn_perm(c, a, 0x05040100u),
               (uint32_t)__builtin_amdgcn_perm(c, a, 0x07060302u),
               (uint32_t)__builtin_amdgcn_perm(d, b, 0x05040100u),
               (uint32_t)__builtin_amdgcn_perm(d, b, 0x07060302u)};
}

// Keep flags of four bytes at once: bit 7 of byte k of the result is set
// when byte k of x, read as an unsigned number, is at least thr (0 <= thr <=
// 255; thr4 = thr in every byte, c4 = 0x80808080 - (thr4 & 0x7f7f7f7f), both
// precomputed on the host); the other bits are undefined. (x & 0x7f7f7f7f) + c4 carries into no other
// byte, and its bit 7 in byte k says whether the low seven bits of x reach
// those of thr there; where the top bits of x and thr differ, they decide.
// Both together: the top bit of the majority of x, NOT thr4 and that sum
// (bitop3 truth table 0xB2).
__device__ __forceinline__ uint32_t keep_flags4(uint32_t x, uint32_t thr4, uint32_t c4) {
  return (uint32_t)__builtin_amdgcn_bitop3_b32(x, thr4, (x & 0x7f7f7f7fu) + c4, 0xB2);
}

// From a word of keep flags g: 0xffff in the low half when the element of
// byte 2q is kept, and in the high half when that of byte 2q + 1 is. v_perm
// selectors 8 .. 11 copy bit 15 or bit 31 of either source into a whole
// byte: g holds the flags of bytes 1 and 3 there, g << 8 those of 0 and 2.
__device__ __forceinline__ uint32_t keep_mask_pair(uint32_t g, int q) {
  return (uint32_t)__builtin_amdgcn_perm(g << 8, g, q ? 0x09090b0bu : 0x08080a0au);
}

// The random bytes of the 16 scores a lane holds in the transposed-score
// layout (lane = one row, register r = key 8 (r / 4) + 4 hi + r % 4 of a
// 32-key block starting at key0; the four lanes of a quad hold rows 4a ..
// 4a + 3): byte r % 4 of word r / 4 belongs to element r, which is kept when
// that byte is at least thr. Each lane of the quad computes one of the four
// calls its rows need, and the quad transposes them through xa, the wave's
// kQuadXWords-word LDS area.
__device__ __forceinline__ u32x4 keep_bytes_rows(const DropParams& dp, int bh, int row,
                                                 int key0, int hi, int lane, uint32_t* xa) {
  const int s = lane & 3;
  const u32x4 w = philox4x32_10(
      u32x4{(uint32_t)((key0 >> 2) + 2 * s + hi), (uint32_t)(row >> 2), (uint32_t)bh, dp.offset},
      dp.k0, dp.k1);
  return quad_transpose_lds(w, xa, lane);  // word m = word (row % 4) of call m
}

// The same for the layout with rows in the registers: lane = one key,
// register r = row 8 (r / 4) + 4 hi + r % 4 of a 32-row block starting at
// row0; the four lanes of a quad hold keys 4b .. 4b + 3.
__device__ __forceinline__ u32x4 keep_bytes_keys(const DropParams& dp, int bh, int key,
                                                 int row0, int hi, int lane, uint32_t* xa) {
  const int s = lane & 3;
  const u32x4 w = philox4x32_10(
      u32x4{(uint32_t)(key >> 2), (uint32_t)((row0 >> 2) + 2 * s + hi), (uint32_t)bh, dp.offset},
      dp.k0, dp.k1);
  return quad_transpose_lds(byte_transpose(w), xa, lane);  // word m byte e: row 4 m' + e, this key
}

// Whether element r of a keep_bytes_* result is kept.
__device__ __forceinline__ bool byte_kept(const u32x4& v, int r, uint32_t thr) {
  return ((v[r >> 2] >> (8 * (r & 3))) & 0xffu) >= thr;
}

// 0xffffffff when the element of byte k (a compile-time 0 .. 3) of flag word
// g is kept, else 0 (keep_mask_pair's selectors, one byte's flag in all four).
__device__ __forceinline__ uint32_t keep_mask_elem(uint32_t g, int k) {
  const uint32_t sel = k == 0 ? 0x0a0a0a0au : k == 1 ? 0x08080808u : k == 2 ? 0x0b0b0b0bu : 0x09090909u;
  return (uint32_t)__builtin_amdgcn_perm(g << 8, g, sel);
}

// keep_bytes_keys as keep flags (keep_flags4 on each word).
__device__ __forceinline__ u32x4 keep_flags_keys(const DropParams& dp, int bh, int key,
                                                 int row0, int hi, int lane, uint32_t* xa) {
  const u32x4 v = keep_bytes_keys(dp, bh, key, row0, hi, lane, xa);
  u32x4 g;
#pragma unroll
  for (int m = 0; m < 4; ++m) g[m] = keep_flags4(v[m], dp.thr4, dp.bias4);
  return g;
}

// keep_bytes_rows as keep flags (keep_flags4 on each word).
__device__ __forceinline__ u32x4 keep_flags_rows(const DropParams& dp, int bh, int row,
                                                 int key0, int hi, int lane, uint32_t* xa) {
  const u32x4 v = keep_bytes_rows(dp, bh, row, key0, hi, lane, xa);
  u32x4 g;
#pragma unroll
  for (int m = 0; m < 4; ++m) g[m] = keep_flags4(v[m], dp.thr4, dp.bias4);
  return g;
}

}  // namespace fa
