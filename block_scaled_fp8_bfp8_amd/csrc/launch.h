// Host-side launchers of the gfx950 kernels (internal to libbfp8; arguments are
// validated by the C-ABI layer before any of these is called).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bfp8 {

constexpr int kBlock = 128;  // K block of the scale grid, also the N block of the weight scales

constexpr int kInF32 = 0;
constexpr int kInBf16 = 1;
constexpr int kInF16 = 2;

struct GemmArgs {
  const uint8_t* a;  // [M][lda] e4m3 activations
  int64_t lda;
  const void* as;  // [K/128][ld_as] activation scales (group-major): float32, or UE8M0 bytes if e8
  int64_t ld_as;
  const uint8_t* b;  // [G][N][ldb] e4m3 weights (G = 1 for the dense GEMM)
  int64_t ldb;
  const void* bs;  // [G][ceil(N/128)][ld_bs] weight block scales: float32, or UE8M0 bytes if e8
  int64_t ld_bs;
  uint16_t* c;  // [M][ldc] bf16 output
  int64_t ldc;
  int M, N, K;
  const int32_t* layout;  // grouped GEMM only: [M] group id per row, -1 = padding
  int G;
  const uint16_t* bias;  // optional bf16 [N], added to the bf16 output (nullptr = none)
  // UE8M0 scales: byte e stands for 2^(e - 127); both scale arrays start 4-byte aligned and
  // have leading dimensions that are multiples of 4. The kernels then apply the scales
  // inside the scaled MFMA and accumulate in its FP32 accumulator (no separate promotion).
  bool e8;
  bool out_f16;  // C (and bias) are fp16 instead of bf16
  // Grouped launches only (ignored elsewhere): a gathered A. When set, GEMM row r reads its codes
  // from activation row a_row_src[r] / a_row_div of a (row 0 where the entry is negative:
  // padding, whose results are never stored); its scales stay at column r of as.
  const int32_t* a_row_src = nullptr;
  int a_row_div = 1;
};

// Tiled-schedule plan for a dense GEMM: tile shape, and the workspace it needs (none so far).
struct TiledPlan {
  int bn, bm;  // tile: weight rows x activation rows
  int tiles;   // number of output tiles
  size_t workspace_bytes;
};
TiledPlan plan_tiled(int64_t M, int64_t N, int64_t K);

// Writes float32 scales to `as`, or with e8 their UE8M0 codes (one byte each). With src_rows,
// output row m quantizes input row src_rows[m] / src_div and rows with a negative entry are
// not written.
hipError_t launch_quant_act(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                            int64_t ldq, void* as, int64_t ld_as, bool e8, hipStream_t stream,
                            const int32_t* src_rows = nullptr, int src_div = 1, const int32_t* scale_dst = nullptr,
                            int scale_fan = 1);

// 1x64 groups: scales [ceil(K/64)][ld_as], float32.
hipError_t launch_quant_act_1x64(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                                 int64_t ldq, float* as, int64_t ld_as, hipStream_t stream);

// MoE chain (moe.hip). Dispatch: block_counts holds moe_dispatch_blocks(S) * E ints of scratch;
// rows = length of layout and pair_of_row.
int64_t moe_dispatch_blocks(int64_t S);
hipError_t launch_moe_dispatch(const int32_t* ids, int64_t S, int E, int align, int64_t rows, int32_t* row_of_pair,
                               int32_t* pair_of_row, int32_t* layout, int32_t* expert_start, int32_t* expert_count,
                               int32_t* block_counts, hipStream_t stream);
hipError_t launch_swiglu_quant(const uint16_t* proj, int64_t M, int64_t I, int64_t ldp, const int32_t* layout,
                               uint8_t* q, int64_t ldq, float* as, int64_t ld_as, hipStream_t stream);
hipError_t launch_swiglu(const uint16_t* proj, int64_t M, int64_t I, int64_t ldp, const int32_t* layout, uint16_t* h,
                         int64_t ldh, hipStream_t stream);
// NN -> NT conversions (layout.hip): dst[e][n][k] = src[e][k][n] for bytes; dst[e][c][r] =
// src[e][r][c] for float32 (contiguous).
hipError_t launch_transpose_u8(const uint8_t* src, int64_t E, int64_t K, int64_t N, int64_t ld_src, uint8_t* dst,
                               int64_t ld_dst, hipStream_t stream);
hipError_t launch_transpose_f32(const float* src, int64_t E, int64_t R, int64_t C, float* dst, hipStream_t stream);
hipError_t launch_expand_act_scales(const float* s, int64_t s_stride, int64_t M, int64_t G, float* as, int64_t ld_as,
                                    hipStream_t stream);
hipError_t launch_fill_weight_scales(const float* s, int64_t NB, int64_t KB, float* bs, int64_t ld_bs,
                                     hipStream_t stream);
hipError_t launch_moe_combine(const uint16_t* out, int64_t ldo, const int32_t* row_of_pair, const float* w, int64_t T,
                              int top_k, int64_t H, uint16_t* y, int64_t ldy, hipStream_t stream);

// Largest M the K-split schedule (BFP8_SCHED_SMALL_M) takes; the tiled schedule takes larger M
// always, and smaller M where its predicted time is clearly lower.
constexpr int kSmallMaxM = 256;

// Predicted time in microseconds of one dense GEMM under each schedule (host arithmetic only),
// from rates measured on MI355X; the automatic schedule choice compares them.
double ksplit_time_us(int64_t M, int64_t N, int64_t K);
double tiled_time_us(int64_t M, int64_t N, int64_t K);

hipError_t launch_gemm_ksplit(const GemmArgs& args, hipStream_t stream);
// 1x64 activation groups / 128x64 weight blocks (float scales): args.as is [ceil(K/64)][ld_as],
// args.bs [ceil(N/128)][ld_bs >= ceil(K/64)]; the K-split kernel at every M.
hipError_t launch_gemm_ksplit_1x64(const GemmArgs& args, hipStream_t stream);
// The same on 256 x 128 tiles with the 32x32x64 matrix-core product, one product per 64-wide
// group (bf16 output, no bias).
hipError_t launch_gemm_g64(const GemmArgs& args, hipStream_t stream);
// The tile shape of that launch.
enum class G64Tile { k128x128, k256x128, k256x256 };
G64Tile g64_tile(int64_t M, int64_t N);
// 1x64 GEMMs with at least this many 256 x 128 output tiles take the tiled schedule (N = K = 4096:
// M >= 385; measured at M = 384 K-split 26.1 us, tiled 27.2; M = 512 28.9 and 27.7 us).
constexpr int64_t kTiled1x64MinTiles = 64;
// The linear layer at small M: the K-split kernel's 16 x 16 tile quantizing the bf16/fp16
// activations (args.a, args.lda in elements; args.as unused) itself, bit-identical to
// launch_quant_act followed by launch_gemm_ksplit. Taken for the shapes ksplit_fused_shape
// accepts (M <= kFusedMaxM, on the K-split schedule's 16 x 16 tile, where it is faster).
constexpr int kFusedMaxM = 8;
bool ksplit_fused_shape(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_ksplit_fused(const GemmArgs& args, int x_dtype, hipStream_t stream);
// persistent != 0 (the forced persistent schedule): launches whose plan runs 256 x 256 tiles take
// the persistent kernel where it supports the arguments.
hipError_t launch_gemm_tiled(const GemmArgs& args, void* workspace, hipStream_t stream, int persistent = 0);
// Persistent 256 x 256 kernel (gemm_persistent.hip): float scales, K % 128 == 0, bf16 output in
// 16-byte aligned rows.
bool persistent_supported(const GemmArgs& args);
hipError_t launch_gemm_persistent(const GemmArgs& args, hipStream_t stream);
hipError_t launch_grouped_tiled(const GemmArgs& args, hipStream_t stream);

}  // namespace bfp8
