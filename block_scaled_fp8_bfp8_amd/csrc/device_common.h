// Device-side helpers shared by the gfx950 kernels of libbfp8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace bfp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// One 16x16x128 FP8 (e4m3 x e4m3) matrix-core product with a zero accumulator input.
// Operand layout (gfx950 v_mfma_f32_16x16x128_f8f6f4, both operands e4m3): lane l
// supplies 32 consecutive K bytes [32*(l/16), 32*(l/16)+32) of row l%16 of its
// operand; result register i of lane l is D[4*(l/16) + i][l%16], where the row index
// runs over src0's rows and the column index over src1's rows. Zero scale operands
// select the unscaled instruction.
__device__ __forceinline__ v4f mfma_block(const v8i& src0, const v8i& src1) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(src0, src1, zero, 0, 0, 0, 0, 0, 0);
}

// float32 -> bf16 bit pattern, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Store 4 consecutive bf16 outputs c[0..3] of one row, with column tail masking.
__device__ __forceinline__ void store_bf16x4(uint16_t* c, int n, int N, bool vec_ok, float v0, float v1,
                                             float v2, float v3) {
  const uint32_t b0 = f32_to_bf16_rne(v0), b1 = f32_to_bf16_rne(v1);
  const uint32_t b2 = f32_to_bf16_rne(v2), b3 = f32_to_bf16_rne(v3);
  if (vec_ok && n + 3 < N) {
    uint2 pk;
    pk.x = b0 | (b1 << 16);
    pk.y = b2 | (b3 << 16);
    *reinterpret_cast<uint2*>(c) = pk;
  } else {
    if (n + 0 < N) c[0] = (uint16_t)b0;
    if (n + 1 < N) c[1] = (uint16_t)b1;
    if (n + 2 < N) c[2] = (uint16_t)b2;
    if (n + 3 < N) c[3] = (uint16_t)b3;
  }
}

// 32 bytes from global memory (16-byte aligned) as an MFMA operand.
__device__ __forceinline__ v8i load_frag_global(const uint8_t* p) {
  const v4i lo = *reinterpret_cast<const v4i*>(p);
  const v4i hi = *reinterpret_cast<const v4i*>(p + 16);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace bfp8
