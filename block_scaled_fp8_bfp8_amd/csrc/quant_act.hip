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
// 1x64 groups (kGroup = 64; the next block-scale layout named on the vLLM torch-backend page,
// section "风险与影响"): the same arithmetic over groups of 64 columns, 8 lanes of 8 elements each.
//
// HBM-bound: per element it reads 4 (fp32) or 2 (bf16, fp16) bytes and writes 1, plus
// 4 bytes of scale per 128 elements. Mapping: L lanes per group, 128 / L consecutive
// elements per lane, 16-byte loads issued together and one store of the lane's codes.
// Inputs of 32768 groups and more take L = 8 (16 elements, 32 or 64 bytes in flight per
// lane): with 16 lanes the bf16 path reached only 3.4-4.0 TB/s at M = 2048 on the
// hidden-5120 shapes, and 8 lanes took K = 25600 from 40.1 to 31.7 us and the fp32
// M = 8192 sweep input from 30.1 to 27.9 us. Smaller inputs keep L = 16 (twice the lanes,
// half the latency per lane: M = 1 2.2 against 2.5 us). The group's amax is reduced with
// lane shuffles inside its L lanes; the division is the correctly rounded IEEE divide
// (HIP's default, no fast-math), and the e4m3 encoding uses the hardware's
// round-to-nearest-even OCP e4m3fn conversion on values already clamped to +-448 (the
// conversion itself does not saturate).
#include "device_common.h"
#include "launch.h"

namespace bfp8 {

namespace {

constexpr int kQuantThreads = 256;
// Groups below this count take 16 lanes per group, others 8.
constexpr int64_t kWideGroups = 32768;

// Gather variant (kGather): output row m quantizes input row src_rows[m] / src_div, and rows
// whose entry is negative are left unwritten (the MoE dispatch's padded buffer: entry = pair
// index, src_div = top_k, so the input row is the pair's token).
// Scattered scales (scale_dst != nullptr): row m's group scale is written to the columns
// scale_dst[m * scale_fan + j], j < scale_fan, that are not negative, instead of column m (the
// codes stay in row m): each token quantized once, its scales placed at its padded rows.
template <int kIn, bool kE8, bool kGather, int kLanesPerGroup, int kGroup = kBlock>
__global__ __launch_bounds__(kQuantThreads) void quant_act_kernel(const void* __restrict__ x, int64_t ldx,
                                                                  uint8_t* __restrict__ q, int64_t ldq,
                                                                  void* __restrict__ as, int64_t ld_as,
                                                                  int groups_per_row, int64_t total_groups,
                                                                  const int32_t* __restrict__ src_rows, int src_div,
                                                                  int64_t K, const int32_t* __restrict__ scale_dst,
                                                                  int scale_fan) {
  constexpr int kPerLane = kGroup / kLanesPerGroup;  // consecutive elements per lane
  constexpr int kGroupsPerBlock = kQuantThreads / kLanesPerGroup;
  static_assert(kLanesPerGroup == 8 || kLanesPerGroup == 16, "8 or 16 lanes per group");
  static_assert(kPerLane == 8 || kPerLane == 16, "8 or 16 elements per lane");
  const int sub = threadIdx.x & (kLanesPerGroup - 1);  // which slice of the group
  const int64_t gid = (int64_t)blockIdx.x * kGroupsPerBlock + threadIdx.x / kLanesPerGroup;
  const bool valid = gid < total_groups;
  // Out-of-range groups redo the last group (all lanes of a group agree on `valid`, so
  // shuffles only ever pair lanes of the same state) and store nothing.
  const int64_t g_lin = valid ? gid : total_groups - 1;
  const int64_t m = g_lin / groups_per_row;
  const int g = (int)(g_lin - m * groups_per_row);
  const int64_t col = (int64_t)g * kGroup + sub * kPerLane;
  // A partial last group (K % 128 != 0; K is a multiple of 16, so a lane's 8 or 16 elements
  // lie wholly before or wholly past K) has lanes past K: they load nothing, count as zeros
  // in the amax and store nothing.
  const bool in_k = col < K;
  int64_t src = m;
  bool store = valid && in_k;
  if constexpr (kGather) {
    const int32_t p = src_rows[m];  // the same for all lanes of the group
    // An unwritten row is not computed: the group's lanes exchange values only among
    // themselves, so leaving it early does not affect the other groups of the wave.
    if (p < 0) return;
    src = p / src_div;
  }

  float v[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) v[i] = 0.f;
  if (!in_k) {
  } else if constexpr (kIn == kInBf16 || kIn == kInF16) {
    constexpr int kLoads = kPerLane / 8;  // 16-byte loads of 8 elements
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + src * ldx + col);
    uint4 r[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) r[j] = p[j];
    uint32_t w[4 * kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      w[4 * j] = r[j].x; w[4 * j + 1] = r[j].y; w[4 * j + 2] = r[j].z; w[4 * j + 3] = r[j].w;
    }
#pragma unroll
    for (int i = 0; i < 4 * kLoads; ++i) {
      if constexpr (kIn == kInBf16) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      } else {
        v[2 * i] = f16_value(w[i] & 0xffffu);  // exact widening
        v[2 * i + 1] = f16_value(w[i] >> 16);
      }
    }
  } else {
    constexpr int kLoads = kPerLane / 4;  // 16-byte loads of 4 elements
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + src * ldx + col);
    float4 f[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) f[j] = p[j];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      v[4 * i] = f[i].x; v[4 * i + 1] = f[i].y; v[4 * i + 2] = f[i].z; v[4 * i + 3] = f[i].w;
    }
  }

  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int mask = 1; mask < kLanesPerGroup; mask <<= 1) amax = fmaxf(amax, __shfl_xor(amax, mask));

  float s = fmaxf(amax, 1e-10f) / 448.0f;  // correctly rounded divide
  if constexpr (kE8) s = __uint_as_float((__float_as_uint(s) + 0x7fffffu) & ~0x7fffffu);
  float y[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) y[i] = fminf(fmaxf(v[i] / s, -448.0f), 448.0f);

  uint32_t wq[kPerLane / 4];
#pragma unroll
  for (int i = 0; i < kPerLane / 4; ++i) {
    wq[i] = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * i], y[4 * i + 1], 0, false);
    wq[i] = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * i + 2], y[4 * i + 3], wq[i], true);
  }

  if (!kE8 && valid && scale_dst != nullptr) {
    // the group's lanes share the destinations (also those past K in a partial last group)
    for (int j = sub; j < scale_fan; j += kLanesPerGroup) {
      const int32_t r = scale_dst[m * scale_fan + j];
      if (r >= 0) static_cast<float*>(as)[(int64_t)g * ld_as + r] = s;
    }
  }
  if (store) {
    if constexpr (kPerLane == 16) {
      *reinterpret_cast<uint4*>(q + m * ldq + col) = make_uint4(wq[0], wq[1], wq[2], wq[3]);
    } else {
      *reinterpret_cast<uint2*>(q + m * ldq + col) = make_uint2(wq[0], wq[1]);
    }
    if (sub == 0 && (kE8 || scale_dst == nullptr)) {  // scattered scales are written above
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

template <int kIn, bool kE8, int L>
void launch_quant_lanes(const void* x, int64_t ldx, uint8_t* q, int64_t ldq, void* as, int64_t ld_as,
                        int groups_per_row, int64_t total, const int32_t* src_rows, int src_div, int64_t K,
                        const int32_t* scale_dst, int scale_fan, hipStream_t stream) {
  constexpr int kGroupsPerBlock = kQuantThreads / L;
  const int64_t blocks = (total + kGroupsPerBlock - 1) / kGroupsPerBlock;
  if (src_rows) {
    hipLaunchKernelGGL((quant_act_kernel<kIn, kE8, true, L>), dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream,
                       x, ldx, q, ldq, as, ld_as, groups_per_row, total, src_rows, src_div, K, scale_dst, scale_fan);
  } else {
    hipLaunchKernelGGL((quant_act_kernel<kIn, kE8, false, L>), dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream,
                       x, ldx, q, ldq, as, ld_as, groups_per_row, total, src_rows, src_div, K, scale_dst, scale_fan);
  }
}

template <int kIn, bool kE8>
void launch_quant_cfg(const void* x, int64_t ldx, uint8_t* q, int64_t ldq, void* as, int64_t ld_as, int groups_per_row,
                      int64_t total, const int32_t* src_rows, int src_div, int64_t K, const int32_t* scale_dst,
                      int scale_fan, hipStream_t stream) {
  if (total < kWideGroups) {
    launch_quant_lanes<kIn, kE8, 16>(x, ldx, q, ldq, as, ld_as, groups_per_row, total, src_rows, src_div, K, scale_dst,
                                     scale_fan, stream);
  } else {
    launch_quant_lanes<kIn, kE8, 8>(x, ldx, q, ldq, as, ld_as, groups_per_row, total, src_rows, src_div, K, scale_dst,
                                    scale_fan, stream);
  }
}

}  // namespace

hipError_t launch_quant_act_1x64(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                                 int64_t ldq, float* as, int64_t ld_as, hipStream_t stream) {
  const int groups_per_row = (int)((K + 63) / 64);
  const int64_t total = M * groups_per_row;
  constexpr int kGroupsPerBlock = kQuantThreads / 8;
  const dim3 grid((unsigned)((total + kGroupsPerBlock - 1) / kGroupsPerBlock));
  if (x_dtype == kInBf16) {
    hipLaunchKernelGGL((quant_act_kernel<kInBf16, false, false, 8, 64>), grid, dim3(kQuantThreads), 0, stream, x, ldx,
                       q, ldq, as, ld_as, groups_per_row, total, nullptr, 1, K, nullptr, 1);
  } else if (x_dtype == kInF16) {
    hipLaunchKernelGGL((quant_act_kernel<kInF16, false, false, 8, 64>), grid, dim3(kQuantThreads), 0, stream, x, ldx,
                       q, ldq, as, ld_as, groups_per_row, total, nullptr, 1, K, nullptr, 1);
  } else {
    hipLaunchKernelGGL((quant_act_kernel<kInF32, false, false, 8, 64>), grid, dim3(kQuantThreads), 0, stream, x, ldx,
                       q, ldq, as, ld_as, groups_per_row, total, nullptr, 1, K, nullptr, 1);
  }
  return hipGetLastError();
}

hipError_t launch_quant_act(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                            int64_t ldq, void* as, int64_t ld_as, bool e8, hipStream_t stream, const int32_t* src_rows,
                            int src_div, const int32_t* scale_dst, int scale_fan) {
  const int groups_per_row = (int)((K + kBlock - 1) / kBlock);
  const int64_t total = M * groups_per_row;
#define BFP8_QUANT_CFG(IN, E8)                                                                                    \
  launch_quant_cfg<IN, E8>(x, ldx, q, ldq, as, ld_as, groups_per_row, total, src_rows, src_div, K, scale_dst, scale_fan, \
                           stream)
  if (x_dtype == kInBf16) {
    if (e8) BFP8_QUANT_CFG(kInBf16, true);
    else BFP8_QUANT_CFG(kInBf16, false);
  } else if (x_dtype == kInF16) {
    if (e8) BFP8_QUANT_CFG(kInF16, true);
    else BFP8_QUANT_CFG(kInF16, false);
  } else {
    if (e8) BFP8_QUANT_CFG(kInF32, true);
    else BFP8_QUANT_CFG(kInF32, false);
  }
#undef BFP8_QUANT_CFG
  return hipGetLastError();
}

}  // namespace bfp8
