// Layout conversion for NN expert weights, for gfx950.
//
// Role: page "transformers/integrations/deepgemm.py" runs experts whose weights are stored
// transposed ([E, K, N], "is_transposed") through a separate NN grouped kernel. Here the weights
// are static, so they are converted once, at load time, to the NT layout [E, N, K] that the
// grouped kernel streams with 128-byte K rows, and the GEMM itself has a single form. The
// conversion is a plain tiled transpose through LDS: a workgroup reads a 64 x 64 byte tile
// along N (coalesced), and writes it along K (coalesced). The block scales [E, K/128, N/128]
// are transposed the same way, element by element.
//
// Scale granularity: page "vllm/pull/19085" (review thread) runs FP8 models quantized per
// tensor on the block kernel by expanding their scales to the block shape. A per-tensor or
// per-token scale is constant over every activation group and weight block, so the expansion
// (a broadcast into the grids the GEMMs read) is exact.
#include "device_common.h"
#include "launch.h"

namespace bfp8 {

namespace {

constexpr int kTile = 64;

__global__ __launch_bounds__(256) void transpose_u8_kernel(const uint8_t* __restrict__ src, int64_t K, int64_t N,
                                                           int64_t ld_src, uint8_t* __restrict__ dst,
                                                           int64_t ld_dst) {
  __shared__ uint8_t tile[kTile][kTile + 4];
  const int64_t e = blockIdx.z;
  const int64_t n0 = (int64_t)blockIdx.x * kTile, k0 = (int64_t)blockIdx.y * kTile;
  const uint8_t* s = src + e * K * ld_src;
  uint8_t* d = dst + e * N * ld_dst;
  const int row = threadIdx.x >> 2, part = (threadIdx.x & 3) * 16;
  // read: tile row = k (64 of them), 16 consecutive n per thread
  if (k0 + row < K) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t n = n0 + part + j;
      tile[row][part + j] = n < N ? s[(k0 + row) * ld_src + n] : 0;
    }
  }
  __syncthreads();
  // write: output row = n, 16 consecutive k per thread
  if (n0 + row < N) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t k = k0 + part + j;
      if (k < K) d[(n0 + row) * ld_dst + k] = tile[part + j][row];
    }
  }
}

__global__ __launch_bounds__(256) void transpose_f32_kernel(const float* __restrict__ src, int64_t R, int64_t C,
                                                            int64_t total, float* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // output index: [e][c][r]
  if (i >= total) return;
  const int64_t e = i / (R * C), rem = i - e * R * C;
  const int64_t c = rem / R, r = rem - c * R;
  dst[i] = src[e * R * C + r * C + c];
}

// as[g * ld_as + m] = s[m * s_stride] for m < M, g < G (group-major activation scales).
__global__ __launch_bounds__(256) void expand_act_scales_kernel(const float* __restrict__ s, int64_t s_stride,
                                                                int64_t M, int64_t G, float* __restrict__ as,
                                                                int64_t ld_as) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * G) return;
  const int64_t g = i / M, m = i - g * M;
  as[g * ld_as + m] = s[m * s_stride];
}

// bs[j * ld_bs + kb] = s[0] for j < NB, kb < KB (one scale for the whole weight).
__global__ __launch_bounds__(256) void fill_weight_scales_kernel(const float* __restrict__ s, int64_t NB, int64_t KB,
                                                                 float* __restrict__ bs, int64_t ld_bs) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= NB * KB) return;
  const int64_t j = i / KB, kb = i - j * KB;
  bs[j * ld_bs + kb] = s[0];
}

}  // namespace

hipError_t launch_expand_act_scales(const float* s, int64_t s_stride, int64_t M, int64_t G, float* as, int64_t ld_as,
                                    hipStream_t stream) {
  const int64_t total = M * G;
  hipLaunchKernelGGL(expand_act_scales_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, s,
                     s_stride, M, G, as, ld_as);
  return hipGetLastError();
}

hipError_t launch_fill_weight_scales(const float* s, int64_t NB, int64_t KB, float* bs, int64_t ld_bs,
                                     hipStream_t stream) {
  const int64_t total = NB * KB;
  hipLaunchKernelGGL(fill_weight_scales_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, s, NB,
                     KB, bs, ld_bs);
  return hipGetLastError();
}

hipError_t launch_transpose_u8(const uint8_t* src, int64_t E, int64_t K, int64_t N, int64_t ld_src, uint8_t* dst,
                               int64_t ld_dst, hipStream_t stream) {
  const dim3 grid((unsigned)((N + kTile - 1) / kTile), (unsigned)((K + kTile - 1) / kTile), (unsigned)E);
  hipLaunchKernelGGL(transpose_u8_kernel, grid, dim3(256), 0, stream, src, K, N, ld_src, dst, ld_dst);
  return hipGetLastError();
}

hipError_t launch_transpose_f32(const float* src, int64_t E, int64_t R, int64_t C, float* dst, hipStream_t stream) {
  const int64_t total = E * R * C;
  hipLaunchKernelGGL(transpose_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, src, R, C,
                     total, dst);
  return hipGetLastError();
}

}  // namespace bfp8
