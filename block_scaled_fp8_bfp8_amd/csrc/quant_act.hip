// Per-token-group FP8 activation quantizer for gfx950.
//
// Computes, for every row m and 128-column group g (page "prhub.com.cn ...
// vllm/pull/49932", test source: per_token_group_quant_fp8(A, 128,
// column_major_scales=True); page "transformers/integrations/deepgemm.py",
// per_token_cast_to_fp8 with gran_k=128 and float32 scale factors):
//   s = fl32(max(amax, 1e-10) / 448),  q = e4m3fn_RNE(clamp(fl32(x / s), -448, 448)),
// and writes the scale group-major: as[g * ld_as + m].
//
// UE8M0 variant (page "transformers/integrations/deepgemm.py": _ceil_to_ue8m0 and the
// use_ue8m0 recipe of _select_fp8_cast_kwargs): the same s is rounded up to a power of two
// by adding 2^23 - 1 to its bit pattern and clearing the mantissa; the group is divided by
// that power of two (exactly) and the scale is written as its UE8M0 code, the biased
// exponent byte.
//
// HBM-bound: per element it reads 4 (fp32) or 2 (bf16, fp16) bytes and writes 1, plus
// 4 bytes of scale per 128 elements. Mapping: 16 lanes per group, 8 consecutive
// elements per lane (one or two 16-byte loads), 4 groups per wave, so one wave
// streams 512 consecutive elements of a row. The group's amax is reduced with
// lane shuffles inside each 16-lane quarter; the division is the correctly
// rounded IEEE divide (HIP's default, no fast-math), and the e4m3 encoding uses
// the hardware's round-to-nearest-even OCP e4m3fn conversion on values already
// clamped to +-448 (the conversion itself does not saturate).
#include "device_common.h"
#include "launch.h"

namespace bfp8 {

namespace {

constexpr int kQuantThreads = 256;
constexpr int kGroupsPerBlock = kQuantThreads / 16;

// Gather variant (kGather): output row m quantizes input row src_rows[m] / src_div, and rows
// whose entry is negative are left unwritten (the MoE dispatch's padded buffer: entry = pair
// index, src_div = top_k, so the input row is the pair's token).
template <int kIn, bool kE8, bool kGather>
__global__ __launch_bounds__(kQuantThreads) void quant_act_kernel(const void* __restrict__ x, int64_t ldx,
                                                                  uint8_t* __restrict__ q, int64_t ldq,
                                                                  void* __restrict__ as, int64_t ld_as,
                                                                  int groups_per_row, int64_t total_groups,
                                                                  const int32_t* __restrict__ src_rows, int src_div,
                                                                  int64_t K) {
  const int sub = threadIdx.x & 15;  // which 8-element slice of the group
  const int64_t gid = (int64_t)blockIdx.x * kGroupsPerBlock + (threadIdx.x >> 4);
  const bool valid = gid < total_groups;
  // Out-of-range quarters redo the last group (all 16 lanes of a group agree on
  // `valid`, so shuffles only ever pair lanes of the same state) and store nothing.
  const int64_t g_lin = valid ? gid : total_groups - 1;
  const int64_t m = g_lin / groups_per_row;
  const int g = (int)(g_lin - m * groups_per_row);
  const int64_t col = (int64_t)g * kBlock + sub * 8;
  // A partial last group (K % 128 != 0; K is a multiple of 16) has lanes past K: they load
  // nothing, count as zeros in the amax and store nothing.
  const bool in_k = col < K;
  int64_t src = m;
  bool store = valid && in_k;
  if constexpr (kGather) {
    const int32_t p = src_rows[m];  // the same for the group's 16 lanes
    // An unwritten row is not computed: the group's lanes exchange values only among
    // themselves, so leaving it early does not affect the other groups of the wave.
    if (p < 0) return;
    src = p / src_div;
  }

  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (!in_k) {
  } else if constexpr (kIn == kInBf16) {
    const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + src * ldx + col);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else if constexpr (kIn == kInF16) {
    const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + src * ldx + col);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = f16_value(w[i] & 0xffffu);  // exact widening
      v[2 * i + 1] = f16_value(w[i] >> 16);
    }
  } else {
    const float* p = static_cast<const float*>(x) + src * ldx + col;
    const float4 lo = *reinterpret_cast<const float4*>(p);
    const float4 hi = *reinterpret_cast<const float4*>(p + 4);
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  }

  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int mask = 1; mask < 16; mask <<= 1) amax = fmaxf(amax, __shfl_xor(amax, mask));

  float s = fmaxf(amax, 1e-10f) / 448.0f;  // correctly rounded divide
  if constexpr (kE8) s = __uint_as_float((__float_as_uint(s) + 0x7fffffu) & ~0x7fffffu);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(v[i] / s, -448.0f), 448.0f);

  uint32_t w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
  uint32_t w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);

  if (store) {
    *reinterpret_cast<uint2*>(q + m * ldq + col) = make_uint2(w0, w1);
    if (sub == 0) {
      if constexpr (kE8) {
        static_cast<uint8_t*>(as)[(int64_t)g * ld_as + m] = (uint8_t)(__float_as_uint(s) >> 23);
      } else {
        static_cast<float*>(as)[(int64_t)g * ld_as + m] = s;
      }
    }
  }
}

}  // namespace

namespace {

template <int kIn, bool kE8>
void launch_quant_cfg(const void* x, int64_t ldx, uint8_t* q, int64_t ldq, void* as, int64_t ld_as, int groups_per_row,
                      int64_t total, const int32_t* src_rows, int src_div, int64_t K, hipStream_t stream) {
  const int64_t blocks = (total + kGroupsPerBlock - 1) / kGroupsPerBlock;
  if (src_rows) {
    hipLaunchKernelGGL((quant_act_kernel<kIn, kE8, true>), dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream,
                       x, ldx, q, ldq, as, ld_as, groups_per_row, total, src_rows, src_div, K);
  } else {
    hipLaunchKernelGGL((quant_act_kernel<kIn, kE8, false>), dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream,
                       x, ldx, q, ldq, as, ld_as, groups_per_row, total, src_rows, src_div, K);
  }
}

}  // namespace

hipError_t launch_quant_act(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                            int64_t ldq, void* as, int64_t ld_as, bool e8, hipStream_t stream, const int32_t* src_rows,
                            int src_div) {
  const int groups_per_row = (int)((K + kBlock - 1) / kBlock);
  const int64_t total = M * groups_per_row;
  if (x_dtype == kInBf16) {
    if (e8) launch_quant_cfg<kInBf16, true>(x, ldx, q, ldq, as, ld_as, groups_per_row, total, src_rows, src_div, K, stream);
    else launch_quant_cfg<kInBf16, false>(x, ldx, q, ldq, as, ld_as, groups_per_row, total, src_rows, src_div, K, stream);
  } else if (x_dtype == kInF16) {
    if (e8) launch_quant_cfg<kInF16, true>(x, ldx, q, ldq, as, ld_as, groups_per_row, total, src_rows, src_div, K, stream);
    else launch_quant_cfg<kInF16, false>(x, ldx, q, ldq, as, ld_as, groups_per_row, total, src_rows, src_div, K, stream);
  } else {
    if (e8) launch_quant_cfg<kInF32, true>(x, ldx, q, ldq, as, ld_as, groups_per_row, total, src_rows, src_div, K, stream);
    else launch_quant_cfg<kInF32, false>(x, ldx, q, ldq, as, ld_as, groups_per_row, total, src_rows, src_div, K, stream);
  }
  return hipGetLastError();
}

}  // namespace bfp8
