// Mixture-of-experts chain around the M-grouped contiguous GEMM, for gfx950.
//
// Role: the routing, gate activation and combine steps of page
// "transformers/integrations/deepgemm.py" (_dispatch_routed_input,
// _build_deepgemm_contiguous_layout, deepgemm_fp8_fp4_experts_forward,
// _combine_routed_output), done on the device without a host round trip:
//   * dispatch: the S = T * top_k (token, expert) pairs get rows in a padded buffer where
//     expert e owns a block of rows starting on a multiple of the alignment. Three small
//     kernels: per-1024-pair expert histograms; one workgroup turning them into aligned
//     expert starts and per-block bases; a placement pass that ranks each pair among the
//     earlier pairs of its expert (wave ballots inside a wave, per-wave counts in LDS across
//     the workgroup), so the order inside an expert is the pair order and the result is the
//     same on every run. A fourth kernel writes the per-row expert id (-1 on padding) that the
//     grouped GEMM reads. Ids outside [0, E) are sentinels: counted nowhere, placed nowhere;
//   * SwiGLU fused with the second quantization: gate and up halves of the bf16 up-projection
//     row are read once, h = bf16(bf16(silu(gate)) * up) stays in registers, and each 1x128
//     group of h is quantized exactly as the activation quantizer does. silu is evaluated in
//     float64 and rounded once to bf16 (through float with round-to-odd, which cannot double
//     round), so the bf16 value, and every FP8 code derived from it, is the exact one (a float32
//     evaluation decides all but the elements near a bf16 rounding midpoint); padding rows are
//     skipped;
//   * combine: per token and 8 output columns, sum_j bf16(out[row] * bf16(w)) in float32 in the
//     order of the token's pairs, rounded once to bf16; sentinel pairs add nothing and their
//     rows are never read.
// All are HBM-bound and small next to the two grouped GEMMs.
#include "device_common.h"
#include "launch.h"

namespace bfp8 {

namespace {

constexpr int kPairsPerBlock = 1024;  // one (token, expert) pair per thread
constexpr int kWavesPerBlock = kPairsPerBlock / 64;

__global__ __launch_bounds__(kPairsPerBlock) void moe_count_kernel(const int32_t* __restrict__ ids, int64_t S, int E,
                                                                    int32_t* __restrict__ block_counts) {
  extern __shared__ int cnt[];  // E counters
  for (int e = threadIdx.x; e < E; e += kPairsPerBlock) cnt[e] = 0;
  __syncthreads();
  const int64_t p = (int64_t)blockIdx.x * kPairsPerBlock + threadIdx.x;
  if (p < S) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPairsPerBlock) block_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// One workgroup: per expert, exclusive prefix of the block counts and its total; aligned expert
// starts (exclusive scan of the totals rounded up to the alignment); then the per-block bases
// become absolute rows.
__global__ __launch_bounds__(1024) void moe_offsets_kernel(int32_t* __restrict__ block_counts, int nblocks, int E,
                                                           int align, int32_t* __restrict__ expert_start,
                                                           int32_t* __restrict__ expert_count) {
  extern __shared__ int start[];  // E + 1
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int b = 0; b < nblocks; ++b) {
      const int c = block_counts[(int64_t)b * E + e];
      block_counts[(int64_t)b * E + e] = run;
      run += c;
    }
    expert_count[e] = run;
    start[e] = (run + align - 1) / align * align;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
      const int a = start[e];
      start[e] = acc;
      acc += a;
    }
    start[E] = acc;
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x) expert_start[e] = start[e];
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    for (int b = 0; b < nblocks; ++b) block_counts[(int64_t)b * E + e] += start[e];
}

// Small dispatches (kMergedMaxBlocks blocks of pairs or fewer, their counters within
// kMergedMaxCounters) in one workgroup: the per-block histograms in LDS, then the per-block bases,
// the aligned starts and the totals exactly as moe_count_kernel and moe_offsets_kernel give them.
constexpr int kMergedMaxBlocks = 16;
constexpr int kMergedMaxCounters = 8192;
__global__ __launch_bounds__(1024) void moe_count_offsets_kernel(const int32_t* __restrict__ ids, int64_t S, int E,
                                                                 int nblocks, int align,
                                                                 int32_t* __restrict__ block_base,
                                                                 int32_t* __restrict__ expert_start,
                                                                 int32_t* __restrict__ expert_count) {
  extern __shared__ int sh[];  // nblocks x E counters, then E + 1 starts
  int* cnt = sh;
  int* start = sh + nblocks * E;
  for (int i = threadIdx.x; i < nblocks * E; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  for (int64_t p = threadIdx.x; p < S; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[(int)(p / kPairsPerBlock) * E + e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int b = 0; b < nblocks; ++b) {
      const int c = cnt[b * E + e];
      cnt[b * E + e] = run;
      run += c;
    }
    expert_count[e] = run;
    start[e] = (run + align - 1) / align * align;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
      const int a = start[e];
      start[e] = acc;
      acc += a;
    }
    start[E] = acc;
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x) expert_start[e] = start[e];
  for (int i = threadIdx.x; i < nblocks * E; i += blockDim.x) block_base[i] = cnt[i] + start[i % E];
}

// Workgroup b of the placement: rows [1024 b, 1024 b + 1024) of the layout get their expert (-1 on
// padding and past the last expert's rows), and the padding rows' pair_of_row entries -1; then, if
// b < nblocks, the pairs [1024 b, 1024 b + 1024) are placed, each writing its row's pair_of_row
// entry. A real row's entry is written by its pair alone and a padding row's by the row fill
// alone, so the two parts need no ordering between workgroups.
__global__ __launch_bounds__(kPairsPerBlock) void moe_fill_place_kernel(
    const int32_t* __restrict__ ids, int64_t S, int E, int nblocks, const int32_t* __restrict__ block_base,
    const int32_t* __restrict__ expert_start, const int32_t* __restrict__ expert_count, int64_t rows,
    int32_t* __restrict__ layout, int32_t* __restrict__ row_of_pair, int32_t* __restrict__ pair_of_row) {
  const int64_t r = (int64_t)blockIdx.x * kPairsPerBlock + threadIdx.x;
  if (r < rows) {
    int e = -1;
    if (r < expert_start[E]) {
      int lo = 0, hi = E;  // largest lo with expert_start[lo] <= r (expert_start[0] = 0 <= r < expert_start[E])
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (expert_start[mid] <= r) lo = mid;
        else hi = mid;
      }
      if (r - expert_start[lo] < expert_count[lo]) e = lo;
    }
    layout[r] = e;
    if (e < 0) pair_of_row[r] = -1;
  }
  if ((int)blockIdx.x >= nblocks) return;  // uniform: no pairs here
  extern __shared__ int wave_cnt[];  // kWavesPerBlock x E
  for (int i = threadIdx.x; i < kWavesPerBlock * E; i += kPairsPerBlock) wave_cnt[i] = 0;
  __syncthreads();
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t p = (int64_t)blockIdx.x * kPairsPerBlock + threadIdx.x;
  const int e = p < S ? ids[p] : -1;
  const bool valid = e >= 0 && e < E;
  // Rank among this wave's lanes below with the same expert: one ballot per distinct expert.
  int rank = 0;
  uint64_t todo = __ballot(valid);
  while (todo) {
    const int leader = __ffsll((unsigned long long)todo) - 1;
    const int ev = __shfl(e, leader);
    const bool mine = valid && e == ev;
    const uint64_t same = __ballot(mine);
    if (mine) rank = __popcll(same & ((1ull << lane) - 1ull));
    if (lane == leader) wave_cnt[w * E + ev] = __popcll(same);
    todo &= ~same;
  }
  __syncthreads();
  if (p < S) {
    if (valid) {
      int pos = block_base[(int64_t)blockIdx.x * E + e] + rank;
      for (int ww = 0; ww < w; ++ww) pos += wave_cnt[ww * E + e];
      row_of_pair[p] = pos;
      pair_of_row[pos] = (int32_t)p;
    } else {
      row_of_pair[p] = -1;
    }
  }
}

// float64 -> bf16 bits, round to nearest even, with a single rounding: truncate to float and
// mark inexactness in the last bit (round to odd), then round that float to bf16.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double d) {
  const float t = __double2float_rz(d);
  uint32_t u = __float_as_uint(t);
  if ((double)t != d && d == d) u |= 1u;
  return f32_to_bf16_rne(__uint_as_float(u));
}

__device__ __forceinline__ float bf16_value(uint32_t bits) { return __uint_as_float(bits << 16); }

// A finite normal float rounded to bf16 (nearest, ties to even) by the hardware conversion;
// inf stays inf and a NaN stays a NaN.
__device__ __forceinline__ float round_bf16(float f) { return (float)(__bf16)f; }

// Float32 ulps of slack around a bf16 rounding midpoint inside which the float32 silu below does
// not decide the rounding: twice its error bound.
constexpr uint32_t kSiluSlackUlps = 16;

// bf16 bits of silu(x) = x / (1 + exp(-x)) from float32 arithmetic, with `decided` false where
// float32 cannot vouch for the rounding (the caller then takes the float64 path).
//
// The exponential: the argument a log2(e) (a = -x, or a = x for x < -20) is split into a float t
// and the remainder tl that t misses (an fma and a product), t into an integer n and a fraction
// f = t - n, and exp(a) = ldexp(2^f (1 + tl ln 2), n): the hardware exp2 (within 1 ulp) on
// |f| <= 1/2, one rounding for the correction, one for the product, an exact ldexp.
//  * x >= -20: silu = x * rcp(1 + exp(-x)) (the sum, the hardware reciprocal within 1 ulp and the
//    product add one rounding each; errors of exp(-x) enter the sum damped by
//    exp(-x) / (1 + exp(-x)) <= 1): at most 8 * 2^-24 relative error, 8 float32 ulps.
//  * x < -20: silu = x e^x (1 - e^x + ...), and e^x < 2^-28, so x * exp(x) with the exponent
//    raised by 64 (no underflow down to x = -131) is silu(x) 2^64 within 6 * 2^-24 relative.
//    Where silu(x) >= 2^-126 the scaling back is exact; below, bf16 rounds on its subnormal grid
//    2^-133, and k = |silu(x)| 2^133 < 128 is known to within 6 * 2^-24 * 128 < 2^-14.
// The bf16 rounding is decided unless the result lies within the slack of a rounding midpoint
// (k within 2^-13 of one on the subnormal grid), or is not a finite normal float32 value on
// the main branch (zero gates excepted: silu(+-0) = +-0 exactly). All branches are selects.
__device__ __forceinline__ uint32_t silu_bf16_f32(float x, bool& decided) {
#pragma clang fp contract(off)  // every step rounds as written (explicit fmaf calls excepted)
  constexpr float kLog2e = 0x1.715476p+0f;    // fl(log2 e)
  constexpr float kLog2eLo = 0x1.4ae0c0p-26f; // fl(log2 e - kLog2e)
  constexpr float kLn2 = 0x1.62e430p-1f;
  const bool tail = x < -20.0f;
  const float a = tail ? x : -x;
  const float t = a * kLog2e;  // rounded (t - n fused with it would count tl twice); at most 29

  const float tl = fmaf(a, kLog2e, -t) + a * kLog2eLo;
  const float n = fminf(fmaxf(rintf(t), -200.0f), 200.0f);
  const float p = __builtin_amdgcn_exp2f(t - n) * fmaf(tl, kLn2, 1.0f);
  const float ex = __builtin_amdgcn_ldexpf(p, (int)n + (tail ? 64 : 0));
  const float s1 = x * (tail ? ex : __builtin_amdgcn_rcpf(1.0f + ex));
  const float s = tail ? s1 * 0x1p-64f : s1;
  const float as = fabsf(s);
  const uint32_t low = __float_as_uint(s) & 0xffffu;
  const bool normal = (low + kSiluSlackUlps - 0x8000u > 2 * kSiluSlackUlps) & (as >= 0x1p-126f) &
                      (as < __builtin_huge_valf());
  const bool sub = tail & !(fabsf(s1) >= 0x1p-62f);
  const float k = fabsf(s1) * 0x1p69f;  // exact scaling
  const float kr = k <= 128.0f ? rintf(k) : 128.0f;
  decided = sub ? (fabsf(k - truncf(k) - 0.5f) > 0x1p-13f) : (normal | (x == 0.0f));
  return sub ? 0x8000u | (uint32_t)kr : (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)s);
}

// bf16(silu(x)), silu evaluated in float64 (exp within an ulp of float64, one divide) and
// rounded to bf16 through round-to-odd, for the elements float32 does not decide.
__device__ __forceinline__ uint32_t silu_bf16_f64(float x) {
  const double xd = (double)x;
  return f64_to_bf16_rne(xd / (1.0 + exp(-xd)));
}

// bf16(a * b) for bf16 values a, b when the float32 product is not exact: below the normal range
// (the product of two 8-bit significands always fits 24 bits otherwise), formed in float64.
__device__ __forceinline__ uint32_t mul_bf16_f64(float a, float b) { return f64_to_bf16_rne((double)a * (double)b); }

// The float32 product a * b of bf16 values is exact unless it left the normal range for a
// nonzero result (underflow to a subnormal or to zero).
__device__ __forceinline__ bool product_exact(float pr, float a, float b) {
  return (fabsf(pr) >= 0x1p-126f) | ((pr == 0.0f) & ((a == 0.0f) | (b == 0.0f))) | (pr != pr);
}

// bf16(a * b) for bf16 values a, b.
__device__ __forceinline__ uint32_t mul_bf16(float a, float b) {
  const float pr = a * b;
  return product_exact(pr, a, b) ? f32_to_bf16_rne(pr) : mul_bf16_f64(a, b);
}

constexpr int kSwigluThreads = 256;
constexpr int kSwigluGroupsPerBlock = kSwigluThreads / 16;

// h = bf16(bf16(silu(gate)) * up) for one row's 1x128 group, 16 lanes per group and 8
// consecutive elements per lane; then either (kQuant) the activation quantizer's steps on h
// into codes and the group scale, or h itself as bf16.
template <bool kQuant>
__global__ __launch_bounds__(kSwigluThreads) void swiglu_kernel(const uint16_t* __restrict__ proj, int64_t ldp, int I,
                                                                const int32_t* __restrict__ layout,
                                                                uint8_t* __restrict__ q, int64_t ldq,
                                                                float* __restrict__ as, int64_t ld_as,
                                                                uint16_t* __restrict__ h_out, int64_t ldh,
                                                                int groups_per_row, int64_t total_groups) {
  const int sub = threadIdx.x & 15;
  const int64_t gid = (int64_t)blockIdx.x * kSwigluGroupsPerBlock + (threadIdx.x >> 4);
  bool valid = gid < total_groups;
  const int64_t g_lin = valid ? gid : total_groups - 1;
  const int64_t m = g_lin / groups_per_row;
  const int g = (int)(g_lin - m * groups_per_row);
  // A padding row is not computed at all; its 16-lane groups exchange values only among
  // themselves, so the other groups of the wave are unaffected.
  if (layout != nullptr && layout[m] < 0) return;
  const int64_t col = (int64_t)g * kBlock + sub * 8;
  const uint4 graw = *reinterpret_cast<const uint4*>(proj + m * ldp + col);
  const uint4 uraw = *reinterpret_cast<const uint4*>(proj + m * ldp + I + col);
  const uint32_t gw[4] = {graw.x, graw.y, graw.z, graw.w};
  const uint32_t uw[4] = {uraw.x, uraw.y, uraw.z, uraw.w};
  float gate[8], up[8], h[8];
  uint32_t slow_silu = 0, slow_mul = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    gate[i] = bf16_value((gw[i / 2] >> (16 * (i & 1))) & 0xffffu);
    up[i] = bf16_value((uw[i / 2] >> (16 * (i & 1))) & 0xffffu);
    bool decided;
    const float sb = bf16_value(silu_bf16_f32(gate[i], decided));
    slow_silu |= (decided ? 0u : 1u) << i;
    const float pr = sb * up[i];
    slow_mul |= (product_exact(pr, sb, up[i]) ? 0u : 1u) << i;
    h[i] = round_bf16(pr);
  }
  // Rare: elements whose silu is near a bf16 midpoint or tiny, or whose product underflows, are
  // formed again in float64 (a wave enters only if one of its lanes has such an element).
  if (slow_silu | slow_mul) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((slow_silu | slow_mul) >> i & 1u) {
        bool decided;
        const uint32_t fast = silu_bf16_f32(gate[i], decided);
        const float sb = bf16_value((slow_silu >> i & 1u) ? silu_bf16_f64(gate[i]) : fast);
        const float pr = sb * up[i];
        h[i] = product_exact(pr, sb, up[i]) ? round_bf16(pr) : bf16_value(mul_bf16_f64(sb, up[i]));
      }
    }
  }
  if constexpr (kQuant) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(h[i]));
#pragma unroll
    for (int mask = 1; mask < 16; mask <<= 1) amax = fmaxf(amax, __shfl_xor(amax, mask));
    const float s = fmaxf(amax, 1e-10f) / 448.0f;  // correctly rounded divide
    float y[8];
    if (s < __builtin_huge_valf()) {
      // h / s without a divide per element: the correctly rounded reciprocal r, q0 = h r and one
      // Newton correction with the exact residual h - q0 s. For every bf16 h and every finite
      // scale of the quantizer this gives the correctly rounded quotient, or a quotient below
      // 2^-10 in magnitude of the same sign (both encode as that signed zero).
      const float r = 1.0f / s;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q0 = h[i] * r;
        const float e = fmaf(-q0, s, h[i]);
        y[i] = fminf(fmaxf(copysignf(fmaf(e, r, q0), h[i]), -448.0f), 448.0f);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(h[i] / s, -448.0f), 448.0f);
    }
    uint32_t w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
    uint32_t w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
    if (valid) {
      *reinterpret_cast<uint2*>(q + m * ldq + col) = make_uint2(w0, w1);
      if (sub == 0) as[(int64_t)g * ld_as + m] = s;
    }
  } else {
    uint4 o;
    o.x = (__float_as_uint(h[0]) >> 16) | (__float_as_uint(h[1]) & 0xffff0000u);
    o.y = (__float_as_uint(h[2]) >> 16) | (__float_as_uint(h[3]) & 0xffff0000u);
    o.z = (__float_as_uint(h[4]) >> 16) | (__float_as_uint(h[5]) & 0xffff0000u);
    o.w = (__float_as_uint(h[6]) >> 16) | (__float_as_uint(h[7]) & 0xffff0000u);
    if (valid) *reinterpret_cast<uint4*>(h_out + m * ldh + col) = o;
  }
}

// y[t, c .. c+7] = bf16( sum_j bf16(out[row(t, j), c ..] * bf16(w[t, j])) ), float32 sum in
// order j; a pair without a row adds zero.
// kWaveToken: the row's chunk count is a multiple of 64, so all lanes of a wave sum for one token;
// its pair rows and weights are then read once per wave, through the scalar cache.
template <bool kWaveToken>
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t* __restrict__ out, int64_t ldo,
                                                          const int32_t* __restrict__ row_of_pair,
                                                          const float* __restrict__ w, int64_t T, int top_k,
                                                          int chunks_per_row, uint16_t* __restrict__ y, int64_t ldy) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * chunks_per_row) return;
  int64_t t = i / chunks_per_row;
  if constexpr (kWaveToken) t = (int64_t)__builtin_amdgcn_readfirstlane((int)t);
  const int c = (int)(i - t * chunks_per_row) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < top_k; ++j) {
    const int64_t p = t * top_k + j;
    const int r = row_of_pair[p];
    if (r < 0) continue;
    const float wb = bf16_value(f32_to_bf16_rne(w[p]));
    const uint4 raw = *reinterpret_cast<const uint4*>(out + (int64_t)r * ldo + c);
    const uint32_t ow[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float o = bf16_value((ow[e / 2] >> (16 * (e & 1))) & 0xffffu);
      acc[e] += bf16_value(mul_bf16(o, wb));
    }
  }
  uint4 res;
  res.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
  res.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
  res.z = f32_to_bf16_rne(acc[4]) | (f32_to_bf16_rne(acc[5]) << 16);
  res.w = f32_to_bf16_rne(acc[6]) | (f32_to_bf16_rne(acc[7]) << 16);
  *reinterpret_cast<uint4*>(y + t * ldy + c) = res;
}

}  // namespace

int64_t moe_dispatch_blocks(int64_t S) { return (S + kPairsPerBlock - 1) / kPairsPerBlock; }

hipError_t launch_moe_dispatch(const int32_t* ids, int64_t S, int E, int align, int64_t rows, int32_t* row_of_pair,
                               int32_t* pair_of_row, int32_t* layout, int32_t* expert_start, int32_t* expert_count,
                               int32_t* block_counts, hipStream_t stream) {
  const int64_t nblocks = moe_dispatch_blocks(S);
  if (nblocks <= kMergedMaxBlocks && nblocks * E <= kMergedMaxCounters) {
    hipLaunchKernelGGL(moe_count_offsets_kernel, dim3(1), dim3(1024), (size_t)(nblocks * E + E + 1) * 4, stream, ids,
                       S, E, (int)nblocks, align, block_counts, expert_start, expert_count);
  } else {
    hipLaunchKernelGGL(moe_count_kernel, dim3((unsigned)nblocks), dim3(kPairsPerBlock), (size_t)E * 4, stream, ids,
                       S, E, block_counts);
    hipLaunchKernelGGL(moe_offsets_kernel, dim3(1), dim3(1024), (size_t)(E + 1) * 4, stream, block_counts,
                       (int)nblocks, E, align, expert_start, expert_count);
  }
  const int64_t row_blocks = (rows + kPairsPerBlock - 1) / kPairsPerBlock;
  const int64_t grid = nblocks > row_blocks ? nblocks : row_blocks;
  if (grid > 0) {
    hipLaunchKernelGGL(moe_fill_place_kernel, dim3((unsigned)grid), dim3(kPairsPerBlock),
                       (size_t)kWavesPerBlock * E * 4, stream, ids, S, E, (int)nblocks, block_counts, expert_start,
                       expert_count, rows, layout, row_of_pair, pair_of_row);
  }
  return hipGetLastError();
}

hipError_t launch_swiglu_quant(const uint16_t* proj, int64_t M, int64_t I, int64_t ldp, const int32_t* layout,
                               uint8_t* q, int64_t ldq, float* as, int64_t ld_as, hipStream_t stream) {
  const int groups_per_row = (int)(I / kBlock);
  const int64_t total = M * groups_per_row;
  const int64_t blocks = (total + kSwigluGroupsPerBlock - 1) / kSwigluGroupsPerBlock;
  hipLaunchKernelGGL(swiglu_kernel<true>, dim3((unsigned)blocks), dim3(kSwigluThreads), 0, stream, proj, ldp, (int)I,
                     layout, q, ldq, as, ld_as, (uint16_t*)nullptr, (int64_t)0, groups_per_row, total);
  return hipGetLastError();
}

hipError_t launch_swiglu(const uint16_t* proj, int64_t M, int64_t I, int64_t ldp, const int32_t* layout, uint16_t* h,
                         int64_t ldh, hipStream_t stream) {
  const int groups_per_row = (int)(I / kBlock);
  const int64_t total = M * groups_per_row;
  const int64_t blocks = (total + kSwigluGroupsPerBlock - 1) / kSwigluGroupsPerBlock;
  hipLaunchKernelGGL(swiglu_kernel<false>, dim3((unsigned)blocks), dim3(kSwigluThreads), 0, stream, proj, ldp, (int)I,
                     layout, (uint8_t*)nullptr, (int64_t)0, (float*)nullptr, (int64_t)0, h, ldh, groups_per_row, total);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const uint16_t* out, int64_t ldo, const int32_t* row_of_pair, const float* w, int64_t T,
                              int top_k, int64_t H, uint16_t* y, int64_t ldy, hipStream_t stream) {
  const int chunks = (int)(H / 8);
  const int64_t n = T * chunks;
  if (chunks % 64 == 0) {
    hipLaunchKernelGGL(moe_combine_kernel<true>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, out, ldo,
                       row_of_pair, w, T, top_k, chunks, y, ldy);
  } else {
    hipLaunchKernelGGL(moe_combine_kernel<false>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, out, ldo,
                       row_of_pair, w, T, top_k, chunks, y, ldy);
  }
  return hipGetLastError();
}

}  // namespace bfp8
