// Measurement probes for the benchmark: the ceilings the GEMM kernels are compared against
// besides the vendor peaks. Not part of the GEMM path; built into libbfp8_probes.so.
//
//   * FP8 matrix-core loop: every wave issues a long run of independent 16x16x128 FP8 MFMAs
//     on operands held in registers (no memory traffic), either accumulating in the MFMA or,
//     as the float-scale GEMM does, each from a zero accumulator with its product scaled into
//     a float32 sum by four FMAs (the per-128-block promotion of the blockwise method).
//   * the same with the 32x32x64 FP8 MFMA, whose K of 64 is one 1x64 group: accumulating in the
//     MFMA, or each product from a zero accumulator promoted with sixteen FMAs (one per result).
//   * Streaming read: a grid of 256-thread workgroups reads a buffer once with 16-byte loads,
//     eight in flight per thread (HBM bandwidth for a buffer larger than the last-level cache).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bfp8_probes.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;  // independent MFMAs per wave per step

// kMode 0: each MFMA adds into its chain's accumulator (C = previous result);
// kMode 1: each MFMA starts from zero and its result is promoted with four FMAs;
// kMode 2: each MFMA starts from zero and one element of its result is added to a sum.
template <int kMode>
__global__ __launch_bounds__(512) void mfma_loop_kernel(float* out, int iters) {
  constexpr bool kPromote = kMode != 0;
  const int lane = threadIdx.x & 63;
  // e4m3 codes 0x38 (1.0) and 0x30 (0.5), varied per lane so no operand is a constant
  v8i a, b[kChains];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 ^ ((lane + i) & 1);
#pragma unroll
    for (int j = 0; j < kChains; ++j) b[j][i] = 0x30303030 ^ (j << 8) ^ ((lane + 2 * i) & 1);
  }
  v4f acc[kChains];
  float sum[kChains][4];
#pragma unroll
  for (int j = 0; j < kChains; ++j) {
    acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) sum[j][e] = 0.f;
  }
  float s = 1.0f + lane * 1e-7f;
  for (int it = 0; it < iters; ++it) {
    // the operands count as new in every step (no code is emitted), so no product is hoisted
    asm volatile("" : "+v"(a));
#pragma unroll
    for (int j = 0; j < kChains; ++j) {
      if constexpr (kPromote) {
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
        const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[j], zero, 0, 0, 0, 0, 0, 0);
        if constexpr (kMode == 1) {
#pragma unroll
          for (int e = 0; e < 4; ++e) sum[j][e] = fmaf(p[e], s, sum[j][e]);
        } else {
          sum[j][0] += p[0];
        }
      } else {
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[j], acc[j], 0, 0, 0, 0, 0, 0);
      }
    }
    s = s * 0.999999f;  // a new scale per step, as each K block brings its own
  }
  float r = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) r += kPromote ? sum[j][e] : acc[j][e];
  out[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, uint64_t n_vec,
                                                          uint32_t* out) {
  const uint64_t tid = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  uint32_t x = 0;
  uint64_t i = tid;
  for (; i + 7 * stride < n_vec; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n_vec; i += stride) {
    const uint4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[tid] = x;  // one word per thread, so the loads are not dead
}

// Global -> LDS copy throughput: every wave keeps kInflight copies of 8 rows x 128 bytes in
// flight (the GEMMs' copy shape: rows of a [rows][4096] byte matrix, 8 lanes per row, 16 bytes
// per lane), either with the direct-to-LDS load (kDma) or with a load into registers followed
// by an LDS write. Copy c reads row group c % groups (groups a power of two) at column block
// (c / groups) % 32, so a window of groups * 8 rows is swept block by block.
template <int kInflight, bool kDma, int kLanesPerRow = 8>
__global__ __launch_bounds__(512) void copy_lds_kernel(const uint8_t* __restrict__ src, uint32_t groups, int iters,
                                                       uint32_t* out) {
  static_assert(kLanesPerRow == 8 || kLanesPerRow == 16 || kLanesPerRow == 32 || kLanesPerRow == 64, "row shape");
  __shared__ __attribute__((aligned(16))) uint8_t lds[8][kInflight][1024];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: the LDS address goes to M0
  // a copy covers 64 / kLanesPerRow rows of kLanesPerRow * 16 bytes; row groups stay 8 rows, so a
  // wider copy covers fewer rows and a longer stretch of each (kLanesPerRow / 8 column blocks)
  constexpr uint32_t kRows = 64 / kLanesPerRow, kBlocks = kLanesPerRow / 8;
  const uint32_t lrow = lane / kLanesPerRow, lcol = (lane % kLanesPerRow) * 16;
  const uint32_t first = blockIdx.x * 8 + w, step = gridDim.x * 8;
  auto offset = [&](uint32_t c) -> uint32_t {
    const uint32_t sub = (c / groups) % (8 / kRows);  // which rows of the group
    const uint32_t col = ((c / groups / (8 / kRows)) * kBlocks) & 31;
    return ((c & (groups - 1)) * 8 + sub * kRows + lrow) * 4096u + col * 128u + lcol;
  };
  uint32_t x = 0;
  if constexpr (kDma) {
    for (int it = 0; it < iters; it += kInflight) {
#pragma unroll
      for (int j = 0; j < kInflight; ++j) {
        uint32_t saved;
        const uint32_t dst = (uint32_t)(uintptr_t)&lds[w][j][0];
        const uint32_t voff = offset(first + (uint32_t)(it + j) * step);
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %3\n\t"
            "global_load_lds_dwordx4 %2, %1\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(src), "v"(voff), "s"(dst)
            : "memory");
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kInflight - 1) : "memory");
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    uint4 regs[kInflight];
#pragma unroll
    for (int j = 0; j < kInflight; ++j) regs[j] = *reinterpret_cast<const uint4*>(src + offset(first + (uint32_t)j * step));
    for (int it = kInflight; it < iters; it += kInflight) {
#pragma unroll
      for (int j = 0; j < kInflight; ++j) {
        *reinterpret_cast<uint4*>(&lds[w][j][lane * 16]) = regs[j];
        regs[j] = *reinterpret_cast<const uint4*>(src + offset(first + (uint32_t)(it + j) * step));
      }
    }
#pragma unroll
    for (int j = 0; j < kInflight; ++j) *reinterpret_cast<uint4*>(&lds[w][j][lane * 16]) = regs[j];
  }
  __syncthreads();
  x ^= *reinterpret_cast<const uint32_t*>(&lds[w][lane % kInflight][(lane * 16) & 1023]);
  out[blockIdx.x * 512 + threadIdx.x] = x;
}

// 32x32x64 products, kChains32 independent ones per wave per step. kPromote false: each adds
// into its chain's accumulator; true: each starts from zero and its 16 results are scaled into a
// float32 sum by 16 FMAs (the promotion of the 1x64 method).
constexpr int kChains32 = 4;
typedef float v16f __attribute__((ext_vector_type(16)));
template <bool kPromote>
__global__ __launch_bounds__(512) void mfma32_loop_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  v8i a, b[kChains32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 ^ ((lane + i) & 1);
#pragma unroll
    for (int j = 0; j < kChains32; ++j) b[j][i] = 0x30303030 ^ (j << 8) ^ ((lane + 2 * i) & 1);
  }
  v16f acc[kChains32];
#pragma unroll
  for (int j = 0; j < kChains32; ++j) acc[j] = v16f{};
  float s = 1.0f + lane * 1e-7f;
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(a));
#pragma unroll
    for (int j = 0; j < kChains32; ++j) {
      if constexpr (kPromote) {
        const v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[j], v16f{}, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = fmaf(p[e], s, acc[j][e]);
      } else {
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b[j], acc[j], 0, 0, 0, 0, 0, 0);
      }
    }
    s = s * 0.999999f;
  }
  float r = 0.f;
#pragma unroll
  for (int j = 0; j < kChains32; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) r += acc[j][e];
  out[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

}  // namespace

extern "C" {

int bfp8_probe_mfma_loop(float* out, int workgroups, int iters, int mode, void* stream) {
  if (!out || workgroups < 1 || iters < 1 || mode < 0 || mode > 2) return 1;
  if (mode == 0) {
    hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(workgroups), dim3(512), 0, (hipStream_t)stream, out, iters);
  } else if (mode == 1) {
    hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(workgroups), dim3(512), 0, (hipStream_t)stream, out, iters);
  } else {
    hipLaunchKernelGGL(mfma_loop_kernel<2>, dim3(workgroups), dim3(512), 0, (hipStream_t)stream, out, iters);
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

double bfp8_probe_mfma_loop_flops(int workgroups, int iters) {
  // 8 waves per workgroup, kChains MFMAs per step, 2 * 16 * 16 * 128 flops each
  return (double)workgroups * 8.0 * (double)iters * kChains * 2.0 * 16 * 16 * 128;
}

int bfp8_probe_mfma32_loop(float* out, int workgroups, int iters, int mode, void* stream) {
  if (!out || workgroups < 1 || iters < 1 || mode < 0 || mode > 1) return 1;
  if (mode == 0) {
    hipLaunchKernelGGL(mfma32_loop_kernel<false>, dim3(workgroups), dim3(512), 0, (hipStream_t)stream, out, iters);
  } else {
    hipLaunchKernelGGL(mfma32_loop_kernel<true>, dim3(workgroups), dim3(512), 0, (hipStream_t)stream, out, iters);
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

double bfp8_probe_mfma32_loop_flops(int workgroups, int iters) {
  return (double)workgroups * 8.0 * (double)iters * kChains32 * 2.0 * 32 * 32 * 64;
}

int bfp8_probe_stream_read(const void* src, size_t bytes, uint32_t* out, int workgroups, void* stream) {
  if (!src || !out || workgroups < 1 || bytes % 16 != 0 || ((uintptr_t)src & 15)) return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const uint4*>(src), (uint64_t)(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int bfp8_probe_copy_lds(const void* src, uint32_t groups, int iters, int inflight, int dma, uint32_t* out,
                        int workgroups, void* stream) {
  if (!src || !out || workgroups < 1 || iters < 1 || groups < 1 || (groups & (groups - 1)) || dma < 0 || dma > 4)
    return 1;
  if (inflight != 4 && inflight != 8 && inflight != 16) return 1;
  if (iters % inflight) return 1;
  // dma 2, 3, 4: the direct-to-LDS load with 16, 32 or 64 lanes per row (4, 2 or 1 rows of
  // 256, 512 or 1024 bytes per copy), 8 in flight
  if (dma >= 2) {
    if (inflight != 8) return 1;
    const uint8_t* s8 = static_cast<const uint8_t*>(src);
    if (dma == 2)
      hipLaunchKernelGGL((copy_lds_kernel<8, true, 16>), dim3(workgroups), dim3(512), 0, (hipStream_t)stream, s8, groups, iters, out);
    else if (dma == 3)
      hipLaunchKernelGGL((copy_lds_kernel<8, true, 32>), dim3(workgroups), dim3(512), 0, (hipStream_t)stream, s8, groups, iters, out);
    else
      hipLaunchKernelGGL((copy_lds_kernel<8, true, 64>), dim3(workgroups), dim3(512), 0, (hipStream_t)stream, s8, groups, iters, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
  }
  const uint8_t* s8 = static_cast<const uint8_t*>(src);
  const hipStream_t st = (hipStream_t)stream;
#define BFP8_COPY_PROBE(N, D) \
  hipLaunchKernelGGL((copy_lds_kernel<N, D>), dim3(workgroups), dim3(512), 0, st, s8, groups, iters, out)
  if (dma) {
    if (inflight == 4) BFP8_COPY_PROBE(4, true);
    else if (inflight == 8) BFP8_COPY_PROBE(8, true);
    else BFP8_COPY_PROBE(16, true);
  } else {
    if (inflight == 4) BFP8_COPY_PROBE(4, false);
    else if (inflight == 8) BFP8_COPY_PROBE(8, false);
    else BFP8_COPY_PROBE(16, false);
  }
#undef BFP8_COPY_PROBE
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
