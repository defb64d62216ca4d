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

// Row r's expert (-1 on padding and past the last block); every pair_of_row entry starts at -1.
__global__ __launch_bounds__(256) void moe_fill_kernel(const int32_t* __restrict__ expert_start,
                                                       const int32_t* __restrict__ expert_count, int E, int64_t rows,
                                                       int32_t* __restrict__ layout,
                                                       int32_t* __restrict__ pair_of_row) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
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
  pair_of_row[r] = -1;
}

__global__ __launch_bounds__(kPairsPerBlock) void moe_place_kernel(const int32_t* __restrict__ ids, int64_t S, int E,
                                                                    const int32_t* __restrict__ block_base,
                                                                    int32_t* __restrict__ row_of_pair,
                                                                    int32_t* __restrict__ pair_of_row) {
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

// bf16(silu(x)) for a bf16 input x, equal to rounding the exact silu once. Fast path in float32:
// s = x / (1 + exp(-x)) is within a few float32 ulps of silu(x) (exp within 2 ulps, one rounding
// for the sum and one for the IEEE divide), so its bf16 rounding is the exact one unless s lies
// within 16 float32 ulps of a bf16 rounding midpoint (low 16 bits near 0x8000), or is tiny, where
// float32 loses relative accuracy; those few elements are evaluated again in float64.
__device__ __forceinline__ uint32_t silu_bf16(float x) {
  const float s = x / (1.0f + expf(-x));
  const uint32_t u = __float_as_uint(s);
  const uint32_t low = u & 0xffffu;
  const bool clear = (low < 0x8000u - 16u || low > 0x8000u + 16u) && fabsf(s) >= 0x1p-100f && fabsf(s) < 0x1p100f;
  if (clear) return f32_to_bf16_rne(s);
  const double xd = (double)x;
  return f64_to_bf16_rne(xd / (1.0 + exp(-xd)));
}

// bf16(a * b) for bf16 values a, b: the product has at most 16 significant bits, so float32 holds
// it exactly unless it falls below the normal range; those are formed in float64.
__device__ __forceinline__ uint32_t mul_bf16(float a, float b) {
  const float pr = a * b;
  if (fabsf(pr) >= 0x1p-126f || pr == 0.0f && (a == 0.0f || b == 0.0f)) return f32_to_bf16_rne(pr);
  return f64_to_bf16_rne((double)a * (double)b);
}

constexpr int kSwigluThreads = 256;
constexpr int kSwigluGroupsPerBlock = kSwigluThreads / 16;

// h = bf16(bf16(silu(gate)) * up) for one row's 1x128 group, then the activation quantizer's
// steps on h: 16 lanes per group, 8 consecutive elements per lane.
__global__ __launch_bounds__(kSwigluThreads) void swiglu_quant_kernel(const uint16_t* __restrict__ proj, int64_t ldp,
                                                                      int I, const int32_t* __restrict__ layout,
                                                                      uint8_t* __restrict__ q, int64_t ldq,
                                                                      float* __restrict__ as, int64_t ld_as,
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
  float h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t gb = (gw[i / 2] >> (16 * (i & 1))) & 0xffffu;
    const uint32_t ub = (uw[i / 2] >> (16 * (i & 1))) & 0xffffu;
    const float sb = bf16_value(silu_bf16(bf16_value(gb)));
    h[i] = bf16_value(mul_bf16(sb, bf16_value(ub)));
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(h[i]));
#pragma unroll
  for (int mask = 1; mask < 16; mask <<= 1) amax = fmaxf(amax, __shfl_xor(amax, mask));
  const float s = fmaxf(amax, 1e-10f) / 448.0f;
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(h[i] / s, -448.0f), 448.0f);
  uint32_t w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
  uint32_t w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
  if (valid) {
    *reinterpret_cast<uint2*>(q + m * ldq + col) = make_uint2(w0, w1);
    if (sub == 0) as[(int64_t)g * ld_as + m] = s;
  }
}

// y[t, c .. c+7] = bf16( sum_j bf16(out[row(t, j), c ..] * bf16(w[t, j])) ), float32 sum in
// order j; a pair without a row adds zero.
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t* __restrict__ out, int64_t ldo,
                                                          const int32_t* __restrict__ row_of_pair,
                                                          const float* __restrict__ w, int64_t T, int top_k,
                                                          int chunks_per_row, uint16_t* __restrict__ y, int64_t ldy) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * chunks_per_row) return;
  const int64_t t = i / chunks_per_row;
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
  if (nblocks > 0) {
    hipLaunchKernelGGL(moe_count_kernel, dim3((unsigned)nblocks), dim3(kPairsPerBlock), (size_t)E * 4, stream, ids, S,
                       E, block_counts);
  }
  hipLaunchKernelGGL(moe_offsets_kernel, dim3(1), dim3(1024), (size_t)(E + 1) * 4, stream, block_counts,
                     (int)nblocks, E, align, expert_start, expert_count);
  if (rows > 0) {
    hipLaunchKernelGGL(moe_fill_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, expert_start,
                       expert_count, E, rows, layout, pair_of_row);
  }
  if (nblocks > 0) {
    hipLaunchKernelGGL(moe_place_kernel, dim3((unsigned)nblocks), dim3(kPairsPerBlock),
                       (size_t)kWavesPerBlock * E * 4, stream, ids, S, E, block_counts, row_of_pair, pair_of_row);
  }
  return hipGetLastError();
}

hipError_t launch_swiglu_quant(const uint16_t* proj, int64_t M, int64_t I, int64_t ldp, const int32_t* layout,
                               uint8_t* q, int64_t ldq, float* as, int64_t ld_as, hipStream_t stream) {
  const int groups_per_row = (int)(I / kBlock);
  const int64_t total = M * groups_per_row;
  const int64_t blocks = (total + kSwigluGroupsPerBlock - 1) / kSwigluGroupsPerBlock;
  hipLaunchKernelGGL(swiglu_quant_kernel, dim3((unsigned)blocks), dim3(kSwigluThreads), 0, stream, proj, ldp, (int)I,
                     layout, q, ldq, as, ld_as, groups_per_row, total);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const uint16_t* out, int64_t ldo, const int32_t* row_of_pair, const float* w, int64_t T,
                              int top_k, int64_t H, uint16_t* y, int64_t ldy, hipStream_t stream) {
  const int chunks = (int)(H / 8);
  const int64_t n = T * chunks;
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, out, ldo,
                     row_of_pair, w, T, top_k, chunks, y, ldy);
  return hipGetLastError();
}

}  // namespace bfp8
