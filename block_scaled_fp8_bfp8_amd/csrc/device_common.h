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

// Zeroes the bytes of an MFMA operand fragment that lie at or past K in a partial last K block
// (K % 128 != 0, K a multiple of 16): lane (r, kc) holds bytes [32 kc, 32 kc + 32) of the block,
// of which the first `valid` exist. Both operands are masked, so stale bytes (even e4m3 NaN
// codes) past K contribute exact zeros.
__device__ __forceinline__ v8i mask_k_tail(v8i f, int valid, int kc) {
  const int v = valid - 32 * kc;  // a multiple of 16: whole dwords are kept or cleared
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = v >= 4 * (i + 1) ? f[i] : 0;
  return f;
}

// The same product with UE8M0 block scales applied by the hardware and the result added to
// `acc`: D = acc + sum_k (src0[i][k] 2^(e0 - 127)) (src1[j][k] 2^(e1 - 127)). Lane l gives
// the scale code of row l % 16 of each operand in the low byte of e0 / e1 (the instruction
// scales each 32-wide K slice by the code of the lane that holds it, and the four lanes of a
// row carry the same code for a 128-wide block). The sum is formed in the matrix core's own
// wide accumulation, not as IEEE float32 steps; its error against the exact result was
// measured below 2^-19 of |acc| plus the block's absolute mass.
__device__ __forceinline__ v4f mfma_block_e8(const v8i& src0, const v8i& src1, const v4f& acc, int e0, int e1) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(src0, src1, acc, 0, 0, 0, e0, 0, e1);
}

// UE8M0 code of block kb from a row of codes whose start is 4-byte aligned, read through the
// scalar cache as the aligned dword that holds it (inside the row: its length is padded to a
// multiple of 4).
__device__ __forceinline__ int e8_code_scalar(const __attribute__((address_space(4))) uint32_t* row, int kb) {
  return (int)((row[kb >> 2] >> ((kb & 3) * 8)) & 0xffu);
}

// float32 -> bf16 bit pattern, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  // Both results are formed and one selected, so the conversion compiles without branches.
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet_nan = (u >> 16) | 0x40u;
  return (u & 0x7fffffffu) > 0x7f800000u ? quiet_nan : rounded;
}

// Output element n as bf16 bits: the FP32 result rounded to bf16, then, with a bias, the
// bf16 sum bf16(float(c) + float(bias[n])) (the result is formed in the output's dtype and
// the bias added to it, as the linear layer of page "transformers/integrations/deepgemm.py",
// deepgemm_fp8_fp4_linear, does with output.add_(bias)).
__device__ __forceinline__ uint32_t bf16_out(float acc, const uint16_t* bias, int n) {
  uint32_t b = f32_to_bf16_rne(acc);
  if (bias != nullptr) b = f32_to_bf16_rne(__uint_as_float(b << 16) + __uint_as_float((uint32_t)bias[n] << 16));
  return b;
}

// Store 4 consecutive bf16 outputs c[0..3] of one row (columns n .. n+3), with column tail
// masking and an optional bias.
// float32 -> fp16 bit pattern: the hardware conversion rounds to nearest even (default mode),
// overflows to infinity and keeps fp16 subnormals.
__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float f16_value(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Output element n as 16-bit bits: bf16 (bf16_out), or with f16 the same steps in fp16 (the
// linear layer's output dtype follows its input: fp16(float(fp16(C)) + float(bias[n]))).
// The same conversion with the output dtype and the bias presence fixed at compile time; the
// bias arrives as its 16-bit pattern (loaded once per column by the caller).
template <bool kF16, bool kBias>
__device__ __forceinline__ uint32_t conv16(float acc, uint32_t bias_bits) {
  if constexpr (kF16) {
    uint32_t h = f32_to_f16_rne(acc);
    if constexpr (kBias) h = f32_to_f16_rne(f16_value(h) + f16_value(bias_bits));
    return h;
  } else {
    uint32_t b = f32_to_bf16_rne(acc);
    if constexpr (kBias) b = f32_to_bf16_rne(__uint_as_float(b << 16) + __uint_as_float(bias_bits << 16));
    return b;
  }
}

__device__ __forceinline__ uint32_t out16(float acc, const uint16_t* bias, int n, bool f16) {
  if (f16) {
    uint32_t h = f32_to_f16_rne(acc);
    if (bias != nullptr) h = f32_to_f16_rne(f16_value(h) + f16_value(bias[n]));
    return h;
  }
  return bf16_out(acc, bias, n);
}

__device__ __forceinline__ void store_out16x4(uint16_t* c, int n, int N, bool vec_ok, float v0, float v1,
                                              float v2, float v3, const uint16_t* bias, bool f16) {
  const uint32_t b0 = out16(v0, bias, min(n, N - 1), f16), b1 = out16(v1, bias, min(n + 1, N - 1), f16);
  const uint32_t b2 = out16(v2, bias, min(n + 2, N - 1), f16), b3 = out16(v3, bias, min(n + 3, N - 1), f16);
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

// LDS-only workgroup barrier: orders LDS accesses across the barrier without
// waiting for outstanding global loads (unlike a full __syncthreads()).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Direct global -> LDS copies: lane l's 16 (or 4) bytes from sbase + voff land at LDS
// byte address lds + 16 * l (or 4 * l); completion is awaited with wait_copies(). They are
// issued from inline assembly because the compiler, which cannot tell the copies into one
// LDS stage from reads of the other, would otherwise drain every copy in flight before
// each LDS read. The LDS address travels in M0, which the compiler reserves: it is saved
// and restored inside the same statement.
__device__ __forceinline__ void copy16_to_lds(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %2, %1\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(sbase), "v"(voff), "s"(lds)
      : "memory");
}
__device__ __forceinline__ void copy4_to_lds(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dword %2, %1\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(sbase), "v"(voff), "s"(lds)
      : "memory");
}
// The same copies for kernels whose register pressure lets the compiler spill the (wave-uniform)
// base or LDS address: a value reloaded from a spill lands in a vector register, which the
// scalar moves above cannot read, so these pass both through readfirstlane (free for values
// already in scalar registers).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void copy16_to_lds_u(const void* sbase, uint32_t voff, uint32_t lds) {
  copy16_to_lds(uniform_ptr(sbase), voff, __builtin_amdgcn_readfirstlane(lds));
}
__device__ __forceinline__ void copy4_to_lds_u(const void* sbase, uint32_t voff, uint32_t lds) {
  copy4_to_lds(uniform_ptr(sbase), voff, __builtin_amdgcn_readfirstlane(lds));
}
__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// s_waitcnt vmcnt(N): all but this wave's N most recent copies have landed.
template <int N>
__device__ __forceinline__ void wait_copies_upto() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Tile of workgroup `bid`: each XCD (bid % 8) owns a contiguous run of the tiles,
// ordered in groups of `group_m` M-tiles with the M-tile index fastest.
__device__ __forceinline__ void map_tile(int bid, int n_tiles, int m_tiles, int group_m, int& tn, int& tm) {
  const int total = n_tiles * m_tiles;
  int t = bid;
  if (total % 8 == 0) t = (bid % 8) * (total / 8) + bid / 8;
  const int band = group_m * n_tiles;
  const int first_m = (t / band) * group_m;
  const int gm = min(m_tiles - first_m, group_m);
  const int r = t - (t / band) * band;
  tm = first_m + r % gm;
  tn = r / gm;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// XOR swizzle of the 16-byte columns of a 128-byte LDS row. A fragment read has 16 lanes
// reading the same logical column of the 16 rows of a 16-row block, two 16-byte reads per
// lane. Measured on gfx950 with the LDS bank-conflict counter: XOR by (r ^ r / 8) % 8, r the
// row within its block, makes these reads conflict-free, whereas r % 8, (r / 2) % 8 and
// similar XORs still conflict two ways and halve the LDS read rate. It depends on r alone, so
// all fragments of a wave share their swizzled offsets.
__device__ __forceinline__ int lds_swizzle(int row) { return (row ^ ((row >> 3) & 1)) & 7; }

}  // namespace bfp8
