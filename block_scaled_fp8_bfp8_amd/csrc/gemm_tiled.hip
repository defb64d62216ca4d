// LDS-tiled blockwise FP8 GEMM schedule for gfx950 (mid and large M), dense and
// M-grouped contiguous.
//
// Role: the mid/large-M schedules of page "lmdeploy/pull/4830", section "Kernel
// design", and the M-grouped contiguous kernel of page
// "transformers/integrations/deepgemm.py" (m_grouped_fp8_fp4_gemm_nt_contiguous,
// _build_deepgemm_contiguous_layout), re-derived for CDNA4:
//   * one workgroup computes a BN x BM tile of C^T = B . A^T (weights on the
//     MFMA's first operand, activations on its second), split over WGN x WGM
//     waves of WN x WM each; one 16x16x128 FP8 MFMA covers one 128-wide K block of
//     a 16x16 sub-tile, so the "block accumulator" of the method is just the MFMA
//     result of that K block;
//   * per K block the B and A tiles (BN and BM rows of 128 bytes) are copied
//     HBM -> registers -> LDS with 16-byte coalesced loads, double buffered: the
//     loads of block kb+1 are in flight while block kb is multiplied, and one
//     barrier per K block separates the two LDS buffers' uses. 16-byte chunks of
//     each 128-byte LDS row are XOR-swizzled by (row mod 8) so that the 16 lanes
//     reading one fragment column spread over the LDS banks;
//   * promotion: acc += P * (As[kb][m] * Bs[n/128][kb]) with one FMA per element;
//     each lane holds one activation row m per M sub-tile (one scale product per
//     sub-tile) and each wave's N range lies inside one 128-row weight-scale strip
//     (one weight scale per K block, loaded once per wave);
//   * grouped: a workgroup's BM rows lie in one 128-row block; its expert id is the
//     largest id among those rows (padding rows carry -1), a block of padding only
//     exits at once, and rows whose id is -1 are not stored.
#include "device_common.h"
#include "launch.h"

namespace bfp8 {

namespace {

template <int BN, int BM, int WGN, int WGM, bool kGrouped>
__global__ __launch_bounds__(WGN * WGM * 64) void gemm_tiled_kernel(GemmArgs args) {
  constexpr int kThreads = WGN * WGM * 64;
  constexpr int WN = BN / WGN, WM = BM / WGM;
  constexpr int TN = WN / 16, TM = WM / 16;
  constexpr int kRows = BN + BM;  // 128-byte LDS rows per stage
  constexpr int kLoads = kRows * 8 / kThreads;
  static_assert(kRows * 8 % kThreads == 0, "tile copy must split evenly over the threads");
  static_assert(kThreads % 8 == 0 && BN % (kThreads / 8) == 0, "each copy step must stay inside B or A rows");
  static_assert(WN % 16 == 0 && WM % 16 == 0, "wave tiles are made of 16x16 MFMA tiles");
  static_assert(kBlock % WN == 0 && BN % WN == 0, "a wave's N range must lie inside one weight-scale strip");
  static_assert(!kGrouped || kBlock % BM == 0, "grouped: a workgroup's rows must lie in one 128-row block");

  __shared__ __attribute__((aligned(16))) uint8_t smem[2][kRows * kBlock];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = w % WGN, wm = w / WGN;
  const int M = args.M, N = args.N;
  const int KB = args.K / kBlock;

  const int n_tiles = (N + BN - 1) / BN;
  const int tile_n = blockIdx.x % n_tiles;
  const int tile_m = blockIdx.x / n_tiles;
  const int n0 = tile_n * BN, m0 = tile_m * BM;

  const uint8_t* bmat = args.b;
  const float* bsmat = args.bs;
  if constexpr (kGrouped) {
    int gid = -1;
    for (int i = lane; i < BM; i += 64) gid = max(gid, args.layout[m0 + i]);
#pragma unroll
    for (int mask = 1; mask < 64; mask <<= 1) gid = max(gid, __shfl_xor(gid, mask));
    gid = __builtin_amdgcn_readfirstlane(gid);
    // A block of padding only exits at once (uniform over the workgroup). An id >= G
    // breaks the layout contract; such a block is skipped rather than read out of bounds.
    if (gid < 0 || gid >= args.G) return;
    bmat += (int64_t)gid * N * args.ldb;
    bsmat += (int64_t)gid * ((N + kBlock - 1) / kBlock) * args.ld_bs;
  }

  // Copy assignment: chunk c = tid + j * kThreads of the stage, row c / 8, 16-byte column c % 8.
  const uint8_t* gsrc[kLoads];
  int ldst[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int c = tid + j * kThreads;
    const int row = c >> 3, col = c & 7;
    if (row < BN) {
      const int n = min(n0 + row, N - 1);
      gsrc[j] = bmat + (int64_t)n * args.ldb + col * 16;
    } else {
      const int m = min(m0 + row - BN, M - 1);
      gsrc[j] = args.a + (int64_t)m * args.lda + col * 16;
    }
    ldst[j] = row * kBlock + ((col ^ (row & 7)) << 4);
  }

  // Scale pointers: one activation row per lane per M sub-tile, one weight strip per wave.
  const int r = lane & 15, kc = lane >> 4;
  const float* asp[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) asp[tm] = args.as + min(m0 + wm * WM + tm * 16 + r, M - 1);
  const float* bsp = bsmat + (int64_t)(min(n0 + wn * WN, N - 1) / kBlock) * args.ld_bs;

  float acc[TN][TM][4];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[tn][tm][e] = 0.f;

  uint4 stage[kLoads];
  float as_next[TM], as_cur[TM];
  float bs_next, bs_cur;

  auto load_global = [&](int kb) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) stage[j] = *reinterpret_cast<const uint4*>(gsrc[j] + (int64_t)kb * kBlock);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) as_next[tm] = asp[tm][(int64_t)kb * args.ld_as];
    bs_next = bsp[kb];
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) *reinterpret_cast<uint4*>(&smem[buf][ldst[j]]) = stage[j];
  };
  auto lds_frag = [&](int buf, int row) -> v8i {
    const uint8_t* base = &smem[buf][row * kBlock];
    const int sw = row & 7;
    const uint4 lo = *reinterpret_cast<const uint4*>(base + (((2 * kc) ^ sw) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(base + (((2 * kc + 1) ^ sw) << 4));
    v8i f;
    f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
    f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
    return f;
  };

  load_global(0);
  store_lds(0);
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) as_cur[tm] = as_next[tm];
  bs_cur = bs_next;
  __syncthreads();

  for (int kb = 0; kb < KB; ++kb) {
    const int cur = kb & 1;
    const bool more = kb + 1 < KB;
    if (more) load_global(kb + 1);

    v8i af[TM];
    float sc[TM];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      af[tm] = lds_frag(cur, BN + wm * WM + tm * 16 + r);
      sc[tm] = as_cur[tm] * bs_cur;
    }
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const v8i bf = lds_frag(cur, wn * WN + tn * 16 + r);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const v4f p = mfma_block(bf, af[tm]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[tn][tm][e] = fmaf(p[e], sc[tm], acc[tn][tm][e]);
      }
    }

    if (more) {
      store_lds(cur ^ 1);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) as_cur[tm] = as_next[tm];
      bs_cur = bs_next;
    }
    __syncthreads();
  }

  const bool vec_ok = ((args.ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(args.c) & 7) == 0);
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int m = m0 + wm * WM + tm * 16 + r;
    bool row_ok = m < M;
    if constexpr (kGrouped) row_ok = row_ok && args.layout[m] >= 0;
    if (!row_ok) continue;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int n = n0 + wn * WN + tn * 16 + 4 * kc;
      if (n < N)
        store_bf16x4(args.c + (int64_t)m * args.ldc + n, n, N, vec_ok, acc[tn][tm][0], acc[tn][tm][1],
                     acc[tn][tm][2], acc[tn][tm][3]);
    }
  }
}

constexpr int kTileBN = 128, kTileBM = 128, kTileWGN = 2, kTileWGM = 2;

}  // namespace

hipError_t launch_gemm_tiled(const GemmArgs& args, hipStream_t stream) {
  const int n_tiles = (args.N + kTileBN - 1) / kTileBN;
  const int m_tiles = (args.M + kTileBM - 1) / kTileBM;
  hipLaunchKernelGGL((gemm_tiled_kernel<kTileBN, kTileBM, kTileWGN, kTileWGM, false>),
                     dim3((unsigned)(n_tiles * m_tiles)), dim3(kTileWGN * kTileWGM * 64), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_grouped_tiled(const GemmArgs& args, hipStream_t stream) {
  const int n_tiles = (args.N + kTileBN - 1) / kTileBN;
  const int m_tiles = args.M / kTileBM;  // M % 128 == 0 (checked by the caller)
  hipLaunchKernelGGL((gemm_tiled_kernel<kTileBN, kTileBM, kTileWGN, kTileWGM, true>),
                     dim3((unsigned)(n_tiles * m_tiles)), dim3(kTileWGN * kTileWGM * 64), 0, stream, args);
  return hipGetLastError();
}

}  // namespace bfp8
