// Device helpers shared by the aggregation and accumulation kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace attnres {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two bf16 lanes of a 32-bit word: element 2i in the low half, 2i+1 in the high.
__device__ __forceinline__ float bf16_lo(unsigned u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(unsigned u) { return __uint_as_float(u & 0xFFFF0000u); }

// float32 pair -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(unsigned, p);
}

// Partial-sum update of one 16-byte vector: per element one float32 addition,
// then (bf16) one rounding to nearest even.
__device__ __forceinline__ u32x4 add_rows(u32x4 p, u32x4 f, bool bf16) {
  u32x4 r;
  if (bf16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = pack_bf16(bf16_lo(p[k]) + bf16_lo(f[k]), bf16_hi(p[k]) + bf16_hi(f[k]));
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = __float_as_uint(__uint_as_float(p[k]) + __uint_as_float(f[k]));
  }
  return r;
}

}  // namespace attnres
