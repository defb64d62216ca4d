// Blockwise FP8 GEMM with 1x64 activation groups and 128x64 weight blocks on gfx950's
// 32x32x64 matrix-core product (mid and large M).
//
// Role: the 1x64 / 128x64 block-scale layouts that page "prhub.com.cn ... vllm/pull/49932",
// section "风险与影响", names as the next ones: C[m, n] = bf16(sum_g P_g[m, n] As[g][m] Bs[n/128][g]),
// g over the 64-wide K groups and P_g the FP32 dot product of the e4m3 codes over group g.
//   * one v_mfma_scale_f32_32x32x64_f8f6f4 covers exactly one group of a 32x32 sub-tile, so each
//     group's sum is one product's result with nothing masked (the 16x16x128 product spans two
//     groups: it takes one product per group with the other half of the operand zeroed, half of
//     the matrix-core work wasted);
//   * tiles, copies and pipeline follow the 1x128 tiled kernel: a tile of C^T (weight rows on
//     the product's first operand, activation rows on its second) computed by 8 waves, LDS
//     stages of (BN + BM) rows of 128 bytes filled by the direct-to-LDS copies with the
//     conflict-free XOR swizzle, plus the block's two groups of activation scales; 128 x 128 and
//     256 x 128 tiles hold a block's fragments of both groups, 256 x 256 tiles (whose
//     accumulators take half the registers) one group's at a time;
//   * promotion: acc += P_g * (As[g][m] * Bs[n/128][g]); lane l holds activation row l % 32 of a
//     sub-tile and 16 of its weight rows, all inside one 128-row scale strip, so a sub-tile and
//     group take one scale product and 16 FMAs, lagging their product by two steps.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace bfp8 {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

// One 32x32x64 FP8 (e4m3 x e4m3) product with a zero accumulator input. Lane l supplies 32 K
// bytes of row l % 32 of each operand, the lanes l < 32 one half of the 64-wide slice and the
// others the other half; both operands are laid out alike, so which K index sits where does not
// change the sum. Result register v of lane l is D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32], the
// row index running over src0's rows and the column index over src1's. Zero scale operands
// select the unscaled instruction.
__device__ __forceinline__ v16f mfma_group(const v8i& src0, const v8i& src1) {
  const v16f zero = {};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(src0, src1, zero, 0, 0, 0, 0, 0, 0);
}

// Zeroes the bytes of a group fragment that lie at or past K in a partial last K block: lane
// (r, kc) holds bytes [64 h + 32 kc, 64 h + 32 kc + 32) of the block, of which the first `valid`
// exist (K a multiple of 16, so whole dwords are kept or cleared).
__device__ __forceinline__ v8i mask_group_tail(v8i f, int valid, int h, int kc) {
  const int v = valid - 64 * h - 32 * kc;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = v >= 4 * (i + 1) ? f[i] : 0;
  return f;
}

// Output of a wave's WN x WM tile (TN x TM sub-tiles of 32 x 32 in acc). Register v of sub-tile
// (tn, tm) holds activation row tm 32 + r and weight row tn 32 + 8 (v / 4) + 4 kc + v % 4, so each
// quad of registers is 4 consecutive outputs of one row. When C's rows allow 16-byte stores, the
// wave stages 32 activation rows (one sub-tile row) at a time in LDS at `out_lds` as bf16 rows
// padded by 16 bytes and stores whole row segments of WN * 2 bytes; otherwise it stores 4 outputs
// per lane straight from the registers.
template <int WN, int WM>
__device__ __forceinline__ void store_tile(const GemmArgs& args, const float (&acc)[WN / 32][WM / 32][16],
                                           uint8_t* out_lds, int m_base, int n_base, int lane) {
  constexpr int TN = WN / 32, TM = WM / 32;
  constexpr int kRowBytes = WN * 2 + 16;
  const int r = lane & 31, kc = lane >> 5;
  const int M = args.M, N = args.N;
  const bool vec16 = ((args.ldc & 7) == 0) && ((reinterpret_cast<uintptr_t>(args.c) & 15) == 0);
  if (vec16) {
    constexpr int kLanesPerRow = WN / 8;  // 16 bytes (8 outputs) per lane
    constexpr int kRowsPerPass = 64 / kLanesPerRow;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint2 pk;
          pk.x = f32_to_bf16_rne(acc[tn][tm][4 * q]) | (f32_to_bf16_rne(acc[tn][tm][4 * q + 1]) << 16);
          pk.y = f32_to_bf16_rne(acc[tn][tm][4 * q + 2]) | (f32_to_bf16_rne(acc[tn][tm][4 * q + 3]) << 16);
          *reinterpret_cast<uint2*>(out_lds + r * kRowBytes + (tn * 32 + 8 * q + 4 * kc) * 2) = pk;
        }
      // The wave's LDS writes are read back by other lanes of the same wave; LDS executes one
      // wave's accesses in order, and this keeps the compiler from reordering them.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
      for (int pass = 0; pass < 32 / kRowsPerPass; ++pass) {
        const int row = pass * kRowsPerPass + lane / kLanesPerRow;
        const int seg = lane % kLanesPerRow;
        const v4i v = *reinterpret_cast<const v4i*>(out_lds + row * kRowBytes + seg * 16);
        const int m = m_base + tm * 32 + row;
        const int n = n_base + seg * 8;
        if (m < M && n < N) {
          uint16_t* cp = args.c + (int64_t)m * args.ldc + n;
          if (n + 8 <= N) {
            *reinterpret_cast<v4i*>(cp) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (n + e < N) cp[e] = (uint16_t)((uint32_t)v[e / 2] >> (16 * (e & 1)));
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    }
    return;
  }
  const bool vec_ok = ((args.ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(args.c) & 7) == 0);
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int m = m_base + tm * 32 + r;
    if (m >= M) continue;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n_base + tn * 32 + 8 * q + 4 * kc;
        if (n < N)
          store_out16x4(args.c + (int64_t)m * args.ldc + n, n, N, vec_ok, acc[tn][tm][4 * q], acc[tn][tm][4 * q + 1],
                        acc[tn][tm][4 * q + 2], acc[tn][tm][4 * q + 3], nullptr, false);
      }
  }
}

template <int BN, int BM, int WGN, int WGM, int STAGES, bool kTail>
__global__ __launch_bounds__(WGN * WGM * 64) void gemm_g64_kernel(GemmArgs args) {
  constexpr int kWaves = WGN * WGM;
  constexpr int WN = BN / WGN, WM = BM / WGM;  // the wave tile
  constexpr int TN = WN / 32, TM = WM / 32;    // 32 x 32 sub-tiles
  constexpr int kRows = BN + BM;               // 128-byte LDS rows per stage: weights, then activations
  constexpr int kStage = kRows * kBlock;
  constexpr int kCopies = kRows / 8 / kWaves;  // 1 KB (8-row) copies per wave per K block
  constexpr int kSteps = TM * TN * 2;          // (tm, tn, group half) per K block
  static_assert(kRows % (8 * kWaves) == 0 && BN % 8 == 0, "each wave copies whole 8-row groups");
  static_assert(kBlock % WN == 0, "a wave's weight rows lie in one scale strip");
  static_assert(WN % 32 == 0 && WM % 32 == 0 && TM >= 2, "32 x 32 sub-tiles, two rows of them or more");
  static_assert(BM % 64 == 0 && 2 * BM / 64 <= kWaves, "activation scales: one 64-lane copy per 64 rows and group");
  static_assert(STAGES >= 3 && STAGES <= 8, "the refill of a stage follows the barrier of the block before");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES][kStage];
  __shared__ __attribute__((aligned(16))) float as_lds[STAGES][2 * BM];  // [group half][activation row]

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = w % WGN, wm = w / WGN;
  const int M = args.M, N = args.N;
  const int n_tiles = (N + BN - 1) / BN, m_tiles = (M + BM - 1) / BM;
  const int KB = (args.K + kBlock - 1) / kBlock;
  const int G = (args.K + 63) / 64;  // 64-wide groups along K
  const int k_tail = kTail ? args.K - (KB - 1) * kBlock : kBlock;
  int tile_n, tile_m;
  map_tile(blockIdx.x, n_tiles, m_tiles, 8, tile_n, tile_m);
  const int n0 = tile_n * BN, m0 = tile_m * BM;

  // Copy plan: wave w copies stage rows [8 kCopies w, 8 kCopies (w + 1)) in 8-row pieces; lane l of a piece
  // lands at row prow + l / 8, physical 16-byte column l % 8, so it loads the logical column
  // (l % 8) ^ swizzle(row). Rows past M or N are clamped to the last row (never stored).
  const int prow_base = w * 8 * kCopies;
  const int lrow = lane >> 3;
  uint32_t coff[kCopies];
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int prow = prow_base + j * 8;  // uniform
    const int lcol = (lane & 7) ^ lds_swizzle(prow + lrow);
    const int row = prow < BN ? min(n0 + prow + lrow, N - 1) : min(m0 + prow - BN + lrow, M - 1);
    const int64_t ld = prow < BN ? args.ldb : args.lda;
    coff[j] = (uint32_t)((int64_t)row * ld + lcol * 16);
  }
  // Activation scales of K block kb: groups 2 kb and 2 kb + 1 (the latter clamped to the last
  // group: a clamped group only meets K bytes past K, which the tail mask zeroes), BM rows
  // each; waves 0 .. 2 BM / 64 - 1 copy 64 of them each, wave w the group half w / (BM / 64) and
  // the rows (w % (BM / 64)) 64 + lane.
  const bool copies_as = w < 2 * BM / 64;
  const int as_h = w / (BM / 64);
  const uint32_t as_voff = (uint32_t)min(m0 + (w % (BM / 64)) * 64 + lane, M - 1) * 4u;
  const uint32_t as_dst_off = (uint32_t)(w * 64 * 4);
  const uint8_t* asmat = static_cast<const uint8_t*>(args.as);

  uint32_t stage_lds[STAGES], as_lds_addr[STAGES];
#pragma unroll
  for (int i = 0; i < STAGES; ++i) {
    stage_lds[i] = lds_addr(&smem[i][0]);
    as_lds_addr[i] = lds_addr(&as_lds[i][0]);
  }
  auto issue_piece = [&](int buf, int kb, int j) __attribute__((always_inline)) {
    const uint8_t* src = prow_base + j * 8 < BN ? args.b + (int64_t)kb * kBlock : args.a + (int64_t)kb * kBlock;
    copy16_to_lds(src, coff[j], stage_lds[buf] + (uint32_t)((prow_base + j * 8) * kBlock));
  };
  auto issue_scales = [&](int buf, int kb) __attribute__((always_inline)) {
    if (copies_as)
      copy4_to_lds(asmat + (int64_t)min(2 * kb + as_h, G - 1) * args.ld_as * 4, as_voff, as_lds_addr[buf] + as_dst_off);
  };

  // Weight scales of the wave's strip through the scalar cache: groups 2 kb and 2 kb + 1 (a
  // second group past K gets 0, so its zeroed fragment adds nothing).
  const __attribute__((address_space(4))) float* bs_row =
      (const __attribute__((address_space(4))) float*)(static_cast<const uint8_t*>(args.bs) +
                                                       (int64_t)(min(n0 + wn * WN, N - 1) / kBlock) * args.ld_bs * 4);
  auto weight_scales = [&](int kb, float (&out)[2]) __attribute__((always_inline)) {
    out[0] = bs_row[2 * kb];
    out[1] = 2 * kb + 1 < G ? bs_row[2 * kb + 1] : 0.f;
  };

  // Group fragments: lane (r, kc) reads row row0 + r, bytes [64 h + 32 kc, +32), i.e. the logical
  // 16-byte columns 4 h + 2 kc and 4 h + 2 kc + 1. Every fragment starts at a multiple of 32 rows,
  // so row % 16 == r % 16 and the swizzle, hence the per-lane offsets, are shared by all of them.
  const int r = lane & 31, kc = lane >> 5;
  const int fsw = lds_swizzle(r);
  uint32_t foff[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int c = 0; c < 2; ++c) foff[h][c] = (uint32_t)(r * kBlock + (((4 * h + 2 * kc + c) ^ fsw) << 4));
  auto frag_at = [&](const uint8_t* stage, int row0, int h) __attribute__((always_inline)) -> v8i {
    const v4i lo = *reinterpret_cast<const v4i*>(stage + foff[h][0] + row0 * kBlock);
    const v4i hi = *reinterpret_cast<const v4i*>(stage + foff[h][1] + row0 * kBlock);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto frag_b = [&](const uint8_t* stage, int tn, int h) __attribute__((always_inline)) {
    return frag_at(stage, wn * WN + tn * 32, h);
  };
  auto frag_a = [&](const uint8_t* stage, int tm, int h) __attribute__((always_inline)) {
    return frag_at(stage, BN + wm * WM + tm * 32, h);
  };
  auto act_scale = [&](int slot, int tm, int h) __attribute__((always_inline)) -> float {
    return as_lds[slot][h * BM + wm * WM + tm * 32 + r];
  };

  float acc[TN][TM][16];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[tn][tm][e] = 0.f;

  // Software pipeline. Step t = (tm TN + tn) 2 + h multiplies weight fragment (tn, h) by
  // activation fragment (tm, h). Block kb is multiplied out of registers while block kb + 1 is
  // read from LDS into the same registers, each fragment right after its last use (activation
  // fragments at the end of their row tm, weight fragments in the last row). The barrier of
  // iteration kb sits at step kBarStep, just before the first read of block kb + 1: past it,
  // block kb + 1 has landed (every wave waited for its own copies of it) and every wave has
  // finished reading block kb (read during iteration kb - 1), so stage kb % STAGES is refilled
  // with block kb + STAGES from there on. The promotion of a step lags its product by two
  // steps, across blocks too: the first two steps of block kb promote the last two of block
  // kb - 1 with that block's scale products.
  v8i fa[TM][2], fb[TN][2];
  float sa[TM][2], bsv[2], sc[TM][2];
  constexpr int kBarStep = 2 * TN - 1;
  constexpr int kCopySpan = kSteps - kBarStep;
  auto copy_step = [](int j) constexpr { return kBarStep + j * kCopySpan / kCopies; };
  static_assert(copy_step(kCopies - 1) < kSteps, "every copy of a refill is issued inside the block");
  auto wait_next_block = [&](bool steady) __attribute__((always_inline)) {
    if (!steady) {
      wait_copies();
    } else if (copies_as) {
      wait_copies_upto<(STAGES - 2) * (kCopies + 1)>();
    } else {
      wait_copies_upto<(STAGES - 2) * kCopies>();
    }
  };
  auto promote = [&](int u, const v16f& pu, float s) __attribute__((always_inline)) {
    const int um = u / (2 * TN), un = (u / 2) % TN;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[un][um][e] = fmaf(pu[e], s, acc[un][um][e]);
    // Pin the promotion here: otherwise the FMAs are sunk past the loop's branch, since their
    // results are only read in the next K block.
#pragma unroll
    for (int e = 0; e < 16; e += 4)
      asm volatile("" : "+v"(acc[un][um][e]), "+v"(acc[un][um][e + 1]), "+v"(acc[un][um][e + 2]),
                   "+v"(acc[un][um][e + 3]));
  };
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) sc[tm][0] = sc[tm][1] = 0.f;
  // The last two products of the previous block (zero before the first block: promoting them
  // adds 0 * 0 to a zero accumulator).
  v16f p1c = {}, p2c = {};

  auto iter = [&](int kb, auto steady_c) __attribute__((always_inline)) {
    constexpr bool kSteady = decltype(steady_c)::value;  // kb + STAGES < KB: refill a stage
    const int cslot = kb % STAGES;
    // The last iteration also reads a (stale, in-bounds) stage, which keeps the steps free of
    // branches; those registers are never used.
    const int nslot = (kb + 1) % STAGES;
    const uint8_t* nstage = &smem[nslot][0];
    const bool mask_next = kTail && kb + 1 == KB - 1;  // uniform
    float bs_next[2];
    weight_scales(min(kb + 1, KB - 1), bs_next);
    v16f p1 = p1c, p2 = p2c;
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      const int tm = t / (2 * TN), tn = (t / 2) % TN, h = t % 2;
      // The scale products of row tm are formed at the row's first step, while sa[tm] still
      // holds this block's activation scales (the row's last step reloads them). Until then
      // sc[TM - 1] keeps the previous block's, which its two lagging promotions use.
      if (tn == 0 && h == 0) {
        sc[tm][0] = sa[tm][0] * bsv[0];
        sc[tm][1] = sa[tm][1] * bsv[1];
      }
      const v16f p = mfma_group(fb[tn][h], fa[tm][h]);
      if (t >= 2) {
        promote(t - 2, p2, sc[(t - 2) / (2 * TN)][t % 2]);
      } else {
        promote(kSteps - 2 + t, p2, sc[TM - 1][t % 2]);
      }
      if (t == kBarStep) {
        wait_next_block(kSteady);
        lds_barrier();
        if constexpr (kSteady) issue_scales(cslot, kb + STAGES);
      }
      if constexpr (kSteady) {
#pragma unroll
        for (int j = 0; j < kCopies; ++j)
          if (t == copy_step(j)) issue_piece(cslot, kb + STAGES, j);
      }
      if (tn == TN - 1 && h == 1) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          fa[tm][hh] = frag_a(nstage, tm, hh);
          if (mask_next) fa[tm][hh] = mask_group_tail(fa[tm][hh], k_tail, hh, kc);
          sa[tm][hh] = act_scale(nslot, tm, hh);
        }
      }
      if (tm == TM - 1) {
        fb[tn][h] = frag_b(nstage, tn, h);
        if (mask_next) fb[tn][h] = mask_group_tail(fb[tn][h], k_tail, h, kc);
      }
      __builtin_amdgcn_sched_barrier(0);
      p2 = p1;
      p1 = p;
    }
    p1c = p1;
    p2c = p2;
    bsv[0] = bs_next[0];
    bsv[1] = bs_next[1];
  };

#pragma unroll
  for (int i = 0; i < STAGES; ++i) {
    const int kb = min(i, KB - 1);
    issue_scales(i, kb);
#pragma unroll
    for (int j = 0; j < kCopies; ++j) issue_piece(i, kb, j);
  }
  // block 0 has landed once the copies of blocks 1 .. STAGES-1 are the only ones left
  if (copies_as) {
    wait_copies_upto<(STAGES - 1) * (kCopies + 1)>();
  } else {
    wait_copies_upto<(STAGES - 1) * kCopies>();
  }
  lds_barrier();
  const bool mask_first = kTail && KB == 1;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      fa[tm][h] = frag_a(&smem[0][0], tm, h);
      if (mask_first) fa[tm][h] = mask_group_tail(fa[tm][h], k_tail, h, kc);
      sa[tm][h] = act_scale(0, tm, h);
    }
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      fb[tn][h] = frag_b(&smem[0][0], tn, h);
      if (mask_first) fb[tn][h] = mask_group_tail(fb[tn][h], k_tail, h, kc);
    }
  }
  weight_scales(0, bsv);
  int kb = 0;
  for (; kb + STAGES < KB; ++kb) iter(kb, std::true_type{});
  for (; kb < KB; ++kb) iter(kb, std::false_type{});
  promote(kSteps - 2, p2c, sc[TM - 1][0]);
  promote(kSteps - 1, p1c, sc[TM - 1][1]);
  // Every wave's LDS reads (the last iteration's stale ones included) are done before the
  // stages are reused below. No copy is in flight: the last iteration waited for all of them.
  lds_barrier();

  // Output, staged in this wave's part of the stages (every wave has finished with them).
  static_assert(kWaves * 32 * (WN * 2 + 16) <= STAGES * kStage, "output staging fits the stages");
  store_tile<WN, WM>(args, acc, &smem[0][0] + w * 32 * (WN * 2 + 16), m0 + wm * WM, n0 + wn * WN, lane);
}


// The 256 x 256 tile for large M: 8 waves of 128 x 64 (4 x 2 sub-tiles), two LDS stages. Its
// accumulators (128 registers per lane) leave no room for all fragments of a block, so the steps
// run group by group and weight fragment by weight fragment: step t = (h TN + tn) TM + tm
// multiplies group h of weight fragment tn by group h of activation fragment tm. The wave holds
// the TM activation fragments of the current group and two weight fragments (the current one and
// the next, read at the first step of the current one). Each activation fragment is refilled
// after its last use in a group with the next group: group 1 of the same block (same stage) or
// group 0 of the next block. The barrier of iteration kb sits at the first read of block kb + 1;
// past it every wave has read block kb's group 1 as well, so its stage takes block kb + 2. One
// iteration covers the copies' latency, as in the 1x128 kernel's 256 x 256 tile.
template <bool kTail>
__global__ __launch_bounds__(512) void gemm_g64_wide_kernel(GemmArgs args) {
  constexpr int BN = 256, BM = 256, WGN = 2, WGM = 4, STAGES = 2;
  constexpr int kWaves = WGN * WGM;
  constexpr int WN = BN / WGN, WM = BM / WGM;  // 128 x 64 per wave
  constexpr int TN = WN / 32, TM = WM / 32;    // 4 x 2 sub-tiles of 32 x 32
  constexpr int kRows = BN + BM;
  constexpr int kStage = kRows * kBlock;
  constexpr int kCopies = kRows / 8 / kWaves;  // 8
  constexpr int kSteps = 2 * TN * TM;          // (group half, tn, tm) per K block
  constexpr int kBarStep = (2 * TN - 1) * TM;  // group 1, last weight fragment, first row: the first read of the next block
  static_assert(kRows % (8 * kWaves) == 0 && BN % 8 == 0 && kBlock % WN == 0 && TM >= 2 && TN % 2 == 0, "tile");
  static_assert(2 * BM / 64 == kWaves, "activation scales: every wave copies 64 of them");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES][kStage];
  __shared__ __attribute__((aligned(16))) float as_lds[STAGES][2 * BM];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = w % WGN, wm = w / WGN;
  const int M = args.M, N = args.N;
  const int n_tiles = (N + BN - 1) / BN, m_tiles = (M + BM - 1) / BM;
  const int KB = (args.K + kBlock - 1) / kBlock;
  const int G = (args.K + 63) / 64;
  const int k_tail = kTail ? args.K - (KB - 1) * kBlock : kBlock;
  int tile_n, tile_m;
  map_tile(blockIdx.x, n_tiles, m_tiles, 8, tile_n, tile_m);
  const int n0 = tile_n * BN, m0 = tile_m * BM;

  // Copy plan and scale copies as in the 256 x 128 kernel; here all 8 waves copy scales (wave w:
  // group half w / 4, rows (w % 4) 64 + lane).
  const int prow_base = w * 8 * kCopies;
  const int lrow = lane >> 3;
  uint32_t coff[kCopies];
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int prow = prow_base + j * 8;  // uniform
    const int lcol = (lane & 7) ^ lds_swizzle(prow + lrow);
    const int row = prow < BN ? min(n0 + prow + lrow, N - 1) : min(m0 + prow - BN + lrow, M - 1);
    const int64_t ld = prow < BN ? args.ldb : args.lda;
    coff[j] = (uint32_t)((int64_t)row * ld + lcol * 16);
  }
  const int as_h = w / (BM / 64);
  const uint32_t as_voff = (uint32_t)min(m0 + (w % (BM / 64)) * 64 + lane, M - 1) * 4u;
  const uint32_t as_dst_off = (uint32_t)(w * 64 * 4);
  const uint8_t* asmat = static_cast<const uint8_t*>(args.as);
  auto issue_piece = [&](int buf, int kb, int j) __attribute__((always_inline)) {
    const uint8_t* src = prow_base + j * 8 < BN ? args.b + (int64_t)kb * kBlock : args.a + (int64_t)kb * kBlock;
    copy16_to_lds(src, coff[j], lds_addr(&smem[buf][0]) + (uint32_t)((prow_base + j * 8) * kBlock));
  };
  auto issue_scales = [&](int buf, int kb) __attribute__((always_inline)) {
    copy4_to_lds(asmat + (int64_t)min(2 * kb + as_h, G - 1) * args.ld_as * 4, as_voff,
                 lds_addr(&as_lds[buf][0]) + as_dst_off);
  };
  const __attribute__((address_space(4))) float* bs_row =
      (const __attribute__((address_space(4))) float*)(static_cast<const uint8_t*>(args.bs) +
                                                       (int64_t)(min(n0 + wn * WN, N - 1) / kBlock) * args.ld_bs * 4);
  auto weight_scales = [&](int kb, float (&out)[2]) __attribute__((always_inline)) {
    out[0] = bs_row[2 * kb];
    out[1] = 2 * kb + 1 < G ? bs_row[2 * kb + 1] : 0.f;
  };

  // Group fragments (see the 256 x 128 kernel); the four per-lane offsets differ only in the
  // group and chunk bits of the 16-byte column, which the XOR swizzle leaves in place.
  const int r = lane & 31, kc = lane >> 5;
  const uint32_t foff0 = (uint32_t)(r * kBlock + (((2 * kc) ^ lds_swizzle(r)) << 4));
  auto frag_at = [&](int slot, int row0, int h) __attribute__((always_inline)) -> v8i {
    const uint8_t* stage = &smem[slot][0] + row0 * kBlock;
    const v4i lo = *reinterpret_cast<const v4i*>(stage + (foff0 ^ (uint32_t)(h << 6)));
    const v4i hi = *reinterpret_cast<const v4i*>(stage + (foff0 ^ (uint32_t)((h << 6) | 16)));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  float acc[TN][TM][16];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[tn][tm][e] = 0.f;

  v8i fa[TM], fb[2];
  float sa[TM][2], bsv[2], sc[TM][2];
  auto promote = [&](int u, const v16f& pu) __attribute__((always_inline)) {
    const int uh = u / (TN * TM), un = (u / TM) % TN, um = u % TM;
    const float s = sc[um][uh];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[un][um][e] = fmaf(pu[e], s, acc[un][um][e]);
#pragma unroll
    for (int e = 0; e < 16; e += 4)
      asm volatile("" : "+v"(acc[un][um][e]), "+v"(acc[un][um][e + 1]), "+v"(acc[un][um][e + 2]),
                   "+v"(acc[un][um][e + 3]));
  };
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) sc[tm][0] = sc[tm][1] = 0.f;
  v16f p1c = {}, p2c = {};

  auto iter = [&](int kb, auto steady_c) __attribute__((always_inline)) {
    constexpr bool kSteady = decltype(steady_c)::value;  // kb + 2 < KB: refill the stage
    const int cslot = kb % STAGES, nslot = (kb + 1) % STAGES;
    const bool mask_cur = kTail && kb == KB - 1;       // uniform
    const bool mask_next = kTail && kb + 1 == KB - 1;  // uniform
    float bs_next[2];
    weight_scales(min(kb + 1, KB - 1), bs_next);
    v16f p1 = p1c, p2 = p2c;
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      const int h = t / (TN * TM), tn = (t / TM) % TN, tm = t % TM;
      // The scale products of (tm, h) are formed at their first step, while sa[tm] still holds
      // this block's activation scales (the last step of tm in group 1 reloads them); the
      // previous block's sc[.][1] serve its two lagging promotions first.
      if (tn == 0) sc[tm][h] = sa[tm][h] * bsv[h];
      const v16f p = mfma_group(fb[tn % 2], fa[tm]);
      promote(t >= 2 ? t - 2 : kSteps - 2 + t, p2);
      if (t == kBarStep) {
        wait_copies();  // block kb + 1 has landed (the only copies in flight)
        lds_barrier();
        if constexpr (kSteady) {
          issue_scales(cslot, kb + STAGES);
#pragma unroll
          for (int j = 0; j < kCopies; ++j) issue_piece(cslot, kb + STAGES, j);
        }
      }
      // The next weight fragment, at the first step of the current one: (h, tn + 1), or group 1
      // of this block's first one, or group 0 of the next block's.
      if (tm == 0) {
        const int nh = tn + 1 < TN ? h : 1 - h;
        const int slot = tn + 1 < TN || h == 0 ? cslot : nslot;
        const bool msk = slot == cslot ? mask_cur : mask_next;
        fb[(tn + 1) % 2] = frag_at(slot, wn * WN + ((tn + 1) % TN) * 32, nh);
        if (msk) fb[(tn + 1) % 2] = mask_group_tail(fb[(tn + 1) % 2], k_tail, nh, kc);
      }
      // Activation fragment tm after its last use in the group, with the next group; at the end
      // of group 1 also block kb + 1's activation scales.
      if (tn == TN - 1) {
        const int slot = h == 0 ? cslot : nslot;
        fa[tm] = frag_at(slot, BN + wm * WM + tm * 32, 1 - h);
        if (h == 0 ? mask_cur : mask_next) fa[tm] = mask_group_tail(fa[tm], k_tail, 1 - h, kc);
        if (h == 1) {
          sa[tm][0] = as_lds[nslot][wm * WM + tm * 32 + r];
          sa[tm][1] = as_lds[nslot][BM + wm * WM + tm * 32 + r];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      p2 = p1;
      p1 = p;
    }
    p1c = p1;
    p2c = p2;
    bsv[0] = bs_next[0];
    bsv[1] = bs_next[1];
  };

#pragma unroll
  for (int i = 0; i < STAGES; ++i) {
    const int kb = min(i, KB - 1);
    issue_scales(i, kb);
#pragma unroll
    for (int j = 0; j < kCopies; ++j) issue_piece(i, kb, j);
  }
  wait_copies_upto<kCopies + 1>();  // block 0 has landed
  lds_barrier();
  const bool mask_first = kTail && KB == 1;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    fa[tm] = frag_at(0, BN + wm * WM + tm * 32, 0);
    if (mask_first) fa[tm] = mask_group_tail(fa[tm], k_tail, 0, kc);
    sa[tm][0] = as_lds[0][wm * WM + tm * 32 + r];
    sa[tm][1] = as_lds[0][BM + wm * WM + tm * 32 + r];
  }
  fb[0] = frag_at(0, wn * WN, 0);
  if (mask_first) fb[0] = mask_group_tail(fb[0], k_tail, 0, kc);
  weight_scales(0, bsv);
  int kb = 0;
  for (; kb + STAGES < KB; ++kb) iter(kb, std::true_type{});
  for (; kb < KB; ++kb) iter(kb, std::false_type{});
  promote(kSteps - 2, p2c);
  promote(kSteps - 1, p1c);
  lds_barrier();

  // Output, staged in this wave's part of the stages (every wave has finished with them).
  static_assert(kWaves * 32 * (WN * 2 + 16) <= STAGES * kStage, "output staging fits the stages");
  store_tile<WN, WM>(args, acc, &smem[0][0] + w * 32 * (WN * 2 + 16), m0 + wm * WM, n0 + wn * WN, lane);
}

}  // namespace

namespace {

template <int BN, int BM, int WGN, int WGM, int STAGES>
hipError_t launch_g64_cfg(const GemmArgs& args, hipStream_t stream) {
  const dim3 grid((unsigned)(((args.N + BN - 1) / BN) * ((args.M + BM - 1) / BM)));
  if (args.K % kBlock) {
    hipLaunchKernelGGL((gemm_g64_kernel<BN, BM, WGN, WGM, STAGES, true>), grid, dim3(WGN * WGM * 64), 0, stream, args);
  } else {
    hipLaunchKernelGGL((gemm_g64_kernel<BN, BM, WGN, WGM, STAGES, false>), grid, dim3(WGN * WGM * 64), 0, stream,
                       args);
  }
  return hipGetLastError();
}

}  // namespace

// The tile shape whose rounds of 256 workgroups (one per CU) take the least time at the time per
// K block of a full round measured at N = K = 4096 (K scales every shape alike): 2.75 us for
// 256 x 256 tiles, 1.55 us for 256 x 128, 1.0 us for 128 x 128; the larger tile on a tie. E.g.
// M = 1024: one round of 128 x 128 tiles (32.9 us) rather than one of 256 x 128 (44.7 us);
// M = 1536: one round of 256 x 128 (45.1 us) rather than two of 128 x 128 (56.7 us); M = 6144:
// three rounds of 256 x 128 (138.6 us) rather than one and a half of 256 x 256 (153.7 us);
// M = 8192: two rounds of 256 x 256 (171.6 us) rather than four of 256 x 128 (198.9 us).
G64Tile g64_tile(int64_t M, int64_t N) {
  auto rounds = [&](int64_t bn, int64_t bm) { return (((N + bn - 1) / bn) * ((M + bm - 1) / bm) + 255) / 256; };
  const double t256x256 = 2.75 * (double)rounds(256, 256);
  const double t256x128 = 1.55 * (double)rounds(256, 128);
  const double t128x128 = 1.0 * (double)rounds(128, 128);
  if (t256x256 <= t256x128 && t256x256 <= t128x128) return G64Tile::k256x256;
  return t256x128 <= t128x128 ? G64Tile::k256x128 : G64Tile::k128x128;
}

// bf16 output without bias (the 1x64 entry point has neither): 256 x 256 tiles (8 waves of
// 128 x 64, two stages, one group's fragments at a time), 256 x 128 (8 waves of 64 x 64, three
// stages) or 128 x 128 (8 waves of 32 x 64, four stages), as g64_tile picks.
hipError_t launch_gemm_g64(const GemmArgs& args, hipStream_t stream) {
  if (args.bias != nullptr || args.out_f16 || args.e8) return hipErrorInvalidValue;
  switch (g64_tile(args.M, args.N)) {
    case G64Tile::k256x256: {
      const dim3 grid((unsigned)(((args.N + 255) / 256) * ((args.M + 255) / 256)));
      if (args.K % kBlock) {
        hipLaunchKernelGGL(gemm_g64_wide_kernel<true>, grid, dim3(512), 0, stream, args);
      } else {
        hipLaunchKernelGGL(gemm_g64_wide_kernel<false>, grid, dim3(512), 0, stream, args);
      }
      return hipGetLastError();
    }
    case G64Tile::k256x128:
      return launch_g64_cfg<256, 128, 4, 2, 3>(args, stream);
    default:
      return launch_g64_cfg<128, 128, 4, 2, 4>(args, stream);
  }
}

}  // namespace bfp8
