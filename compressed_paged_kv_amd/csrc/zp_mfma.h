// 16x16 MFMA tiles of dot products between two sets of 16 rows (gfx950),
// shared by the scoring kernel (window logits, in-block Gram) and the
// all-pairs redundancy kernel.
//
// A lane holds operand row (lane % 16) and, per 16-byte fragment, a slice
// of the row chosen by lane / 16; step() adds the products of one fragment
// pair to the 16x16 accumulator, whose lane holds rows 4*(lane/16)+i,
// column lane % 16.  Both operands use the same slicing, so the sum over
// the row is exact whatever order the hardware adds the slices in.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "zp.h"

namespace zp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT>
struct Mma;

template <>
struct Mma<ZP_BF16> {
  static constexpr int kElemBytes = 2;
  __device__ static inline f32x4_t step(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ static inline float sumsq(uint4 a) {
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const float lo = __uint_as_float(w[k] << 16);
      const float hi = __uint_as_float(w[k] & 0xFFFF0000u);
      s = fmaf(lo, lo, s);
      s = fmaf(hi, hi, s);
    }
    return s;
  }
};

template <>
struct Mma<ZP_F32> {
  static constexpr int kElemBytes = 4;
  __device__ static inline f32x4_t step(uint4 a, uint4 b, f32x4_t c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
  __device__ static inline float sumsq(uint4 a) {
    const float x = __uint_as_float(a.x), y = __uint_as_float(a.y);
    const float z = __uint_as_float(a.z), w = __uint_as_float(a.w);
    return fmaf(w, w, fmaf(z, z, fmaf(y, y, x * x)));
  }
};

}  // namespace zp
