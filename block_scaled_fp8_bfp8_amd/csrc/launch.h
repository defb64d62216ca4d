// Host-side launchers of the gfx950 kernels (internal to libbfp8; arguments are
// validated by the C-ABI layer before any of these is called).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bfp8 {

constexpr int kBlock = 128;  // K block of the scale grid, also the N block of the weight scales

constexpr int kInF32 = 0;
constexpr int kInBf16 = 1;

struct GemmArgs {
  const uint8_t* a;  // [M][lda] e4m3 activations
  int64_t lda;
  const float* as;  // [K/128][ld_as] activation scales (group-major)
  int64_t ld_as;
  const uint8_t* b;  // [G][N][ldb] e4m3 weights (G = 1 for the dense GEMM)
  int64_t ldb;
  const float* bs;  // [G][ceil(N/128)][ld_bs] weight block scales
  int64_t ld_bs;
  uint16_t* c;  // [M][ldc] bf16 output
  int64_t ldc;
  int M, N, K;
  const int32_t* layout;  // grouped GEMM only: [M] group id per row, -1 = padding
  int G;
  const uint16_t* bias;  // optional bf16 [N], added to the bf16 output (nullptr = none)
};

// Tiled-schedule plan for a dense GEMM: tile shape, and the workspace it needs (none so far).
struct TiledPlan {
  int bn, bm;  // tile: weight rows x activation rows
  int tiles;   // number of output tiles
  size_t workspace_bytes;
};
TiledPlan plan_tiled(int64_t M, int64_t N, int64_t K);

hipError_t launch_quant_act(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                            int64_t ldq, float* as, int64_t ld_as, hipStream_t stream);

// Largest M the automatic choice gives to the K-split schedule (BFP8_SCHED_SMALL_M); the
// tiled schedule takes larger M.
constexpr int kSmallMaxM = 256;

hipError_t launch_gemm_ksplit(const GemmArgs& args, hipStream_t stream);
hipError_t launch_gemm_tiled(const GemmArgs& args, void* workspace, hipStream_t stream);
hipError_t launch_grouped_tiled(const GemmArgs& args, hipStream_t stream);

}  // namespace bfp8
