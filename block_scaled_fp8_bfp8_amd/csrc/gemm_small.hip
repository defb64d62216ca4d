// Small-M blockwise FP8 GEMM schedule for gfx950 (decode-sized M, memory bound).
//
// Role: the "M <= 128 single-partition" schedule of page "lmdeploy/pull/4830",
// section "Kernel design", re-derived for CDNA4. At small M the cost is reading
// the weight matrix B once from HBM (N*K bytes); the math is tiny. So:
//   * the problem is computed transposed, C^T = B . A^T, so that the 16 rows of an
//     MFMA's first operand are 16 weight rows (N fills the matrix core's M side,
//     the "transposed schedule" idea of the same page) and its 16 columns are
//     activation rows; one 16x16x128 MFMA covers exactly one 128-wide K block;
//   * each workgroup owns 16*NT weight rows and all (up to 16*MT) activation
//     rows of its blockIdx.y slice; its WAVES waves split the K blocks round-robin
//     (kb = wave, wave + WAVES, ...), so at any time the waves read neighbouring
//     128-byte pieces of the same weight rows;
//   * weight fragments go straight from HBM to registers (each weight byte is used
//     by exactly one MFMA per M slice, so LDS staging would buy nothing), PF
//     K blocks deep so that enough bytes are in flight to cover HBM latency;
//   * per K block the FP32 MFMA result P is promoted into the FP32 accumulator
//     with one FMA per element: acc += P * (As[kb][m] * Bs[n/128][kb]). In the
//     transposed layout every lane holds one activation row m, so it needs one
//     scale product per M tile;
//   * the waves' partial sums are reduced through LDS in a fixed order (wave 0,
//     1, ...), which keeps results bitwise reproducible without atomics or a
//     global workspace, and the sum is rounded once to bf16.
#include "device_common.h"
#include "launch.h"

namespace bfp8 {

namespace {

template <int MT, int NT, int WAVES, int PF>
__global__ __launch_bounds__(WAVES * 64) void gemm_small_kernel(GemmArgs args) {
  constexpr int kTileN = 16 * NT;
  constexpr int kTileM = 16 * MT;
  __shared__ float red[WAVES * NT * MT * 4 * 64];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;   // operand row inside a 16-row tile
  const int kc = lane >> 4;  // 32-byte K chunk inside the 128-byte K block
  const int n0 = blockIdx.x * kTileN;
  const int m0 = blockIdx.y * kTileM;
  const int M = args.M, N = args.N;
  const int KB = args.K / kBlock;

  // Operand row pointers. Rows past the end are clamped into range: their results
  // land only in accumulator slots that are never stored.
  const uint8_t* bp[NT];
  const float* bsp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = min(n0 + nt * 16 + r, N - 1);
    bp[nt] = args.b + (int64_t)n * args.ldb + kc * 32;
    const int strip = min(n0 + nt * 16, N - 1) / kBlock;  // uniform across the wave
    bsp[nt] = args.bs + (int64_t)strip * args.ld_bs;
  }
  const uint8_t* ap[MT];
  const float* asp[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(m0 + mt * 16 + r, M - 1);
    ap[mt] = args.a + (int64_t)m * args.lda + kc * 32;
    asp[mt] = args.as + m;
  }

  float acc[NT][MT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[nt][mt][i] = 0.f;

  v8i bf[PF][NT];
  v8i af[PF][MT];
  float bsv[PF][NT];
  float asv[PF][MT];

  const int nkb = (KB - w + WAVES - 1) / WAVES;  // this wave's K blocks: kb = w + i * WAVES

#pragma unroll
  for (int s = 0; s < PF; ++s) {
    if (s < nkb) {
      const int kb = w + s * WAVES;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bf[s][nt] = load_frag_global(bp[nt] + (int64_t)kb * kBlock);
        bsv[s][nt] = bsp[nt][kb];
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        af[s][mt] = load_frag_global(ap[mt] + (int64_t)kb * kBlock);
        asv[s][mt] = asp[mt][(int64_t)kb * args.ld_as];
      }
    }
  }

  for (int base = 0; base < nkb; base += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int i = base + s;
      if (i < nkb) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const v4f p = mfma_block(bf[s][nt], af[s][mt]);
            const float sc = asv[s][mt] * bsv[s][nt];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[nt][mt][e] = fmaf(p[e], sc, acc[nt][mt][e]);
          }
        }
        if (i + PF < nkb) {
          const int kb = w + (i + PF) * WAVES;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            bf[s][nt] = load_frag_global(bp[nt] + (int64_t)kb * kBlock);
            bsv[s][nt] = bsp[nt][kb];
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            af[s][mt] = load_frag_global(ap[mt] + (int64_t)kb * kBlock);
            asv[s][mt] = asp[mt][(int64_t)kb * args.ld_as];
          }
        }
      }
    }
  }

  // Fixed-order reduction of the waves' partial sums.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[(((w * NT + nt) * MT + mt) * 4 + e) * 64 + lane] = acc[nt][mt][e];
  __syncthreads();

  const bool vec_ok = ((args.ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(args.c) & 7) == 0);
  for (int qd = threadIdx.x; qd < NT * MT * 64; qd += WAVES * 64) {
    const int ln = qd & 63;
    const int tile = qd >> 6;  // nt * MT + mt
    const int nt = tile / MT, mt = tile % MT;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int ww = 0; ww < WAVES; ++ww)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += red[((ww * NT * MT + tile) * 4 + e) * 64 + ln];
    const int m = m0 + mt * 16 + (ln & 15);
    const int n = n0 + nt * 16 + 4 * (ln >> 4);
    if (m < M && n < N) store_bf16x4(args.c + (int64_t)m * args.ldc + n, n, N, vec_ok, v[0], v[1], v[2], v[3]);
  }
}

template <int MT, int PF>
hipError_t launch_small_mt(const GemmArgs& args, hipStream_t stream) {
  constexpr int NT = 1, WAVES = 8;
  const dim3 grid((unsigned)((args.N + 16 * NT - 1) / (16 * NT)), (unsigned)((args.M + 16 * MT - 1) / (16 * MT)));
  hipLaunchKernelGGL((gemm_small_kernel<MT, NT, WAVES, PF>), grid, dim3(WAVES * 64), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_small(const GemmArgs& args, hipStream_t stream) {
  if (args.M <= 16) return launch_small_mt<1, 8>(args, stream);
  if (args.M <= 32) return launch_small_mt<2, 6>(args, stream);
  return launch_small_mt<4, 3>(args, stream);
}

}  // namespace bfp8
