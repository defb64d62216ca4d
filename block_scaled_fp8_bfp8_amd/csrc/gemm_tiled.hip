// LDS-tiled blockwise FP8 GEMM schedule for gfx950 (mid and large M), dense and
// M-grouped contiguous.
//
// Role: the mid/large-M schedules of page "lmdeploy/pull/4830", section "Kernel
// design", and the M-grouped contiguous kernel of page
// "transformers/integrations/deepgemm.py" (m_grouped_fp8_fp4_gemm_nt_contiguous,
// _build_deepgemm_contiguous_layout), re-derived for CDNA4:
//   * a workgroup computes a BN x BM tile of C^T = B . A^T (weight rows on the MFMA's
//     first operand, activation rows on its second) with WGN x WGM waves of WN x WM;
//     one 16x16x128 FP8 MFMA covers one 128-wide K block of a 16x16 sub-tile, so the
//     per-block FP32 accumulator of the method is simply that MFMA's result;
//   * promotion: acc += P * (As[kb][m] * Bs[n/128][kb]), one FMA per element per K
//     block; every lane holds one activation row m per M sub-tile (one scale product
//     per sub-tile) and each wave's weight rows lie in one 128-row scale strip;
//   * both operand tiles of a K block (BN + BM rows of 128 bytes) and the block's BM
//     activation scales are copied HBM -> LDS by the gfx950 direct-to-LDS loads
//     (global_load_lds_dwordx4 / _dword), which need no staging registers and no LDS
//     write instructions. The copy of block kb + 1 runs while block kb is multiplied
//     out of the other LDS stage. The loads are issued from inline assembly and their
//     completion is awaited explicitly (the compiler would otherwise drain them before
//     every LDS read); the weight scales come through scalar loads. The 16-byte chunks
//     of each 128-byte LDS row are XOR-swizzled by a function of the row, which the copy
//     realizes by choosing each lane's source chunk, so that fragment reads are free of
//     bank conflicts;
//   * workgroups are mapped to tiles XCD by XCD: the hardware deals consecutive
//     workgroups round-robin to the 8 XCDs, so each XCD is given a contiguous run of
//     tiles in an M-grouped order, and the workgroups resident on one XCD at a time
//     share activation and weight rows in that XCD's L2;
//   * grouped: a workgroup's BM rows lie in one 128-row block; its expert id is the
//     largest id among those rows (padding rows carry -1); a block of padding only
//     exits at once, and rows whose id is -1 are not stored;
//   * UE8M0 scales (kE8; page "transformers/integrations/deepgemm.py", the power-of-two
//     scale factors of _ceil_to_ue8m0 / float8_e8m0fnu): As and Bs are powers of two given
//     by their exponent bytes, so the scaled MFMA applies them exactly in the matrix core
//     and accumulates into the FP32 tile itself; the VALU promotion disappears.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace bfp8 {

namespace {

// Largest divisor of n that is at most cap (0 if cap < 1).
constexpr int largest_divisor_upto(int n, int cap) {
  for (int d = cap < n ? cap : n; d >= 1; --d)
    if (n % d == 0) return d;
  return 0;
}

// The same order for a grid padded to a multiple of 8 workgroups (the grouped launches): each XCD
// gets a run of ceil(total / 8) tiles whatever the tile count; returns false for the padding.
// Without the padding a tile count that is not a multiple of 8 deals consecutive tiles to
// different XCDs: on the MoE down projection (N = 7168, 41 blocks, 1148 tiles) that took 133 us
// against 120 us with the runs (interleaved timings; 656 tiles, a multiple of 8: unchanged).
__device__ __forceinline__ bool map_tile_padded(int bid, int n_tiles, int m_tiles, int group_m, int& tn, int& tm) {
  const int total = n_tiles * m_tiles, per = (total + 7) / 8;
  const int t = (bid % 8) * per + bid / 8;
  if (t >= total) return false;
  const int band = group_m * n_tiles;
  const int first_m = (t / band) * group_m;
  const int gm = min(m_tiles - first_m, group_m);
  const int r = t - (t / band) * band;
  tm = first_m + r % gm;
  tn = r / gm;
  return true;
}

template <int BN, int BM, int WGN, int WGM, int STAGES, int KG, bool kGrouped, bool kE8, bool kTail>
__global__ __launch_bounds__(KG * WGN * WGM * 64) void gemm_tiled_kernel(GemmArgs args) {
  constexpr int kWaves = WGN * WGM;  // waves per K group
  constexpr int WN = BN / WGN, WM = BM / WGM;
  constexpr int TN = WN / 16, TM = WM / 16;
  constexpr int kRows = BN + BM;             // 128-byte LDS rows per stage: weights, then activations
  constexpr int kStage = kRows * kBlock;     // bytes per stage
  constexpr int kCopies = kRows / 8 / kWaves;  // 1 KB (8-row) copies per wave per K block
  static_assert(kRows % (8 * kWaves) == 0, "each wave copies whole 8-row groups");
  static_assert(BM % 64 == 0 && BM / 64 <= kWaves, "activation scales: one 64-lane copy per 64 rows");
  static_assert(WN % 16 == 0 && WM % 16 == 0, "wave tiles are made of 16x16 MFMA tiles");
  static_assert(kBlock % WN == 0 && BN % WN == 0, "a wave's N range must lie inside one weight-scale strip");
  static_assert(!kGrouped || kBlock % BM == 0, "grouped: a workgroup's rows must lie in one 128-row block");

  static_assert(STAGES >= 2 && STAGES <= 8, "2 to 8 pipeline stages");
  static_assert(KG == 1 || KG == 2, "one or two K groups");
  static_assert(KG == 1 || BN * BM * 4 <= KG * STAGES * kStage, "the K-group sum reuses the stages");
  // K groups: KG sets of WGN x WGM waves; group g multiplies the K blocks kb = g, g + KG, ...
  // through its own LDS ring, and the groups' tiles are summed in group order at the end.
  // Activation scales of a stage: BM floats, or with kE8 BM code bytes (one 64-lane dword copy
  // fills 256 bytes).
  constexpr int kAsWords = kE8 ? 64 : BM;
  constexpr int kScaleBytes = kE8 ? 1 : 4;
  static_assert(!kE8 || BM <= 256, "one copy holds the codes of 256 activation rows");
  using ScaleT = std::conditional_t<kE8, int, float>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[KG][STAGES][kStage];
  __shared__ __attribute__((aligned(16))) float as_lds[KG][STAGES][kAsWords];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wg = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wg / kWaves, w = wg % kWaves;  // K group, wave within the group
  const int wn = w % WGN, wm = w / WGN;
  const int M = args.M, N = args.N;

  const int n_tiles = (N + BN - 1) / BN;
  const int m_tiles = (M + BM - 1) / BM;
  // K blocks per group (the plan makes their count a multiple of KG). kTail kernels take a
  // partial last block (K % 128 != 0): its k_tail existing bytes are kept in the fragments and
  // the rest masked to zero; the others compile no mask at all.
  const int KB_all = (args.K + kBlock - 1) / kBlock;
  const int KB = KB_all / KG;
  const int k_tail = kTail ? args.K - (KB_all - 1) * kBlock : kBlock;
  int tile_n, tile_m;
  if constexpr (kGrouped) {
    if (!map_tile_padded(blockIdx.x, n_tiles, m_tiles, 8, tile_n, tile_m)) return;  // uniform
  } else {
    map_tile(blockIdx.x, n_tiles, m_tiles, 8, tile_n, tile_m);
  }
  const int n0 = tile_n * BN, m0 = tile_m * BM;

  const uint8_t* bmat = args.b;
  const uint8_t* bsmat = static_cast<const uint8_t*>(args.bs);
  const uint8_t* asmat = static_cast<const uint8_t*>(args.as);
  const int prow_base = w * 8 * kCopies;
  const int lrow = lane >> 3;
  // Grouped, with a gathered A: the row-map entries of the activation rows this lane copies,
  // loaded first so that their round trip overlaps the layout read below.
  int a_map[kCopies];
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int prow = prow_base + j * 8;  // uniform
    a_map[j] = kGrouped && args.a_row_src != nullptr && prow >= BN ? args.a_row_src[min(m0 + prow - BN + lrow, M - 1)]
                                                                    : 0;
  }
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
    bsmat += (int64_t)gid * ((N + kBlock - 1) / kBlock) * args.ld_bs * kScaleBytes;
  }

  // Copy plan. Wave w copies stage rows [w * 8 * kCopies, ...) in 8-row pieces; lane l of
  // piece j lands at stage row prow + l/8, physical 16-byte column l%8, so it loads the
  // logical column (l%8) ^ swizzle(row) of that row. A piece is all weight rows or all
  // activation rows (BN is a multiple of 8). Rows past M or N are clamped to the last row
  // (their results are never stored).
  uint32_t coff[kCopies];
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int prow = prow_base + j * 8;  // uniform
    const int lcol = (lane & 7) ^ lds_swizzle(prow + lrow);
    // activation rows: the row itself, or with a gathered A the row its map entry names (the
    // codes only: the scales of row r stay at column r); padding entries (< 0) read row 0
    const int arow = !kGrouped || args.a_row_src == nullptr ? min(m0 + prow - BN + lrow, M - 1)
                                                            : (a_map[j] < 0 ? 0 : a_map[j] / args.a_row_div);
    const int row = prow < BN ? min(n0 + prow + lrow, N - 1) : arow;
    const int64_t ld = prow < BN ? args.ldb : args.lda;
    coff[j] = (uint32_t)((int64_t)row * ld + lcol * 16);
  }
  // Activation scales of a K block: waves 0 .. BM/64-1 copy 64 of them each (clamped rows);
  // UE8M0 codes: wave 0 copies 4 codes per lane (dwords clamped to the one holding row M-1,
  // which lies inside the row of codes: its length is a multiple of 4).
  const bool copies_as = kE8 ? w == 0 : w < BM / 64;
  const uint32_t as_voff = kE8 ? (uint32_t)min(m0 + 4 * lane, (M - 1) & ~3)
                               : (uint32_t)min(m0 + (copies_as ? w : 0) * 64 + lane, M - 1) * 4u;
  const uint32_t as_dst_off = kE8 ? 0u : (uint32_t)(w * 64 * 4);

  uint32_t stage_lds[STAGES], as_lds_addr[STAGES];
#pragma unroll
  for (int i = 0; i < STAGES; ++i) {
    stage_lds[i] = lds_addr(&smem[g][i][0]);
    as_lds_addr[i] = lds_addr(&as_lds[g][i][0]);
  }
  // Block index in K of this group's local block i.
  auto gkb = [&](int i) __attribute__((always_inline)) { return i * KG + g; };
  auto issue_copies = [&](int buf, int kb_local) __attribute__((always_inline)) {
    const int kb = gkb(kb_local);
    const uint8_t* bsrc = bmat + (int64_t)kb * kBlock;
    const uint8_t* asrc = args.a + (int64_t)kb * kBlock;
    const uint32_t dst = stage_lds[buf] + (uint32_t)(prow_base * kBlock);
#pragma unroll
    for (int j = 0; j < kCopies; ++j)
      copy16_to_lds(prow_base + j * 8 < BN ? bsrc : asrc, coff[j], dst + (uint32_t)(j * 8 * kBlock));
    if (copies_as) copy4_to_lds(asmat + (int64_t)kb * args.ld_as * kScaleBytes, as_voff, as_lds_addr[buf] + as_dst_off);
  };
  // One piece of a block's copy (for spreading a block's copies over the multiply steps).
  auto issue_piece = [&](int buf, int kb_local, int j) __attribute__((always_inline)) {
    const int kb = gkb(kb_local);
    const uint8_t* src = prow_base + j * 8 < BN ? bmat + (int64_t)kb * kBlock : args.a + (int64_t)kb * kBlock;
    copy16_to_lds(src, coff[j], stage_lds[buf] + (uint32_t)((prow_base + j * 8) * kBlock));
  };
  auto issue_scales = [&](int buf, int kb_local) __attribute__((always_inline)) {
    if (copies_as)
      copy4_to_lds(asmat + (int64_t)gkb(kb_local) * args.ld_as * kScaleBytes, as_voff, as_lds_addr[buf] + as_dst_off);
  };

  const int r = lane & 15, kc = lane >> 4;
  // Weight scale of this wave's strip, through the scalar cache (constant address space).
  const uint8_t* bs_row = bsmat + (int64_t)(min(n0 + wn * WN, N - 1) / kBlock) * args.ld_bs * kScaleBytes;
  auto weight_scale = [&](int kb_global) __attribute__((always_inline)) -> ScaleT {
    if constexpr (kE8) {
      return e8_code_scalar((const __attribute__((address_space(4))) uint32_t*)bs_row, kb_global);
    } else {
      return ((const __attribute__((address_space(4))) float*)bs_row)[kb_global];
    }
  };

  float acc[TN][TM][4];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[tn][tm][e] = 0.f;

  // Fragment rows come in 16-row blocks, so every row a lane reads has row % 16 == r and the
  // same swizzle: a fragment is two 16-byte reads at per-lane offsets from the block's first
  // row, and the block offset folds into the instruction's immediate.
  const int fsw = lds_swizzle(r);
  const uint32_t off_lo = (uint32_t)(r * kBlock + (((2 * kc) ^ fsw) << 4));
  const uint32_t off_hi = (uint32_t)(r * kBlock + (((2 * kc + 1) ^ fsw) << 4));
  auto frag_at = [&](const uint8_t* stage, int row0) __attribute__((always_inline)) -> v8i {
    const v4i lo = *reinterpret_cast<const v4i*>(stage + off_lo + row0 * kBlock);
    const v4i hi = *reinterpret_cast<const v4i*>(stage + off_hi + row0 * kBlock);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto frag_b = [&](const uint8_t* stage, int tn) __attribute__((always_inline)) {
    return frag_at(stage, wn * WN + tn * 16);
  };
  auto frag_a = [&](const uint8_t* stage, int tm) __attribute__((always_inline)) {
    return frag_at(stage, BN + wm * WM + tm * 16);
  };
  auto act_scale = [&](int slot, int tm) __attribute__((always_inline)) -> ScaleT {
    if constexpr (kE8) {
      return reinterpret_cast<const uint8_t*>(&as_lds[g][slot][0])[wm * WM + tm * 16 + r];
    } else {
      return as_lds[g][slot][wm * WM + tm * 16 + r];
    }
  };

  // Software pipeline. Sub-tiles are visited activation-row by activation-row: step
  // t = tm * TN + tn multiplies weight fragment tn by activation fragment tm. Block kb is
  // multiplied out of registers while block kb + 1 is read from LDS into the same registers,
  // each fragment right after its last use in block kb (activation fragment tm after row tm,
  // weight fragment tn in the last row). The promotion of a sub-tile lags its MFMA by two
  // steps. Where the workgroup barrier goes depends on the tile (kMid):
  //   * mid-block (tiles below 256 x 256): the barrier of iteration kb sits at step TN - 1,
  //     just before the first read of block kb + 1, so its first steps multiply fragments
  //     already in registers while the previous iteration's last LDS reads return and late
  //     waves catch up. Past it, block kb + 1 has landed (every wave waited for its own copies
  //     of it first) and every wave has finished reading block kb (read during iteration
  //     kb - 1), so stage kb % STAGES is refilled with block kb + STAGES, one copy per step
  //     from the barrier on. The promotions lag across blocks too: the first two steps of
  //     block kb promote the last two sub-tiles of block kb - 1 with that block's scale;
  //   * end of block (256 x 256, whose registers cannot keep those promotions live across the
  //     barrier): iteration kb refills stage kb % STAGES from its first step on, one copy
  //     every three steps (the barrier that ended iteration kb - 1 follows every read of
  //     block kb), promotes its last two sub-tiles at its end, waits for block kb + 2, which
  //     iteration kb + 1 reads, and ends with the barrier.
  v8i fa[TM];
  v8i fb[TN];
  ScaleT sa[TM];
  ScaleT bsv;
  constexpr int kSteps = TN * TM;
  constexpr bool kMid = BN * BM < 256 * 256;
  constexpr int kBarStep = kMid ? TN - 1 : -1;
  static_assert(TM >= 2 && TN >= 2, "the barrier step precedes every read of the next block");
  // Copy j of a refill goes out at step kFirstCopy + j * kCopyStride, or spread over the
  // remaining steps when there are fewer of them than copies. The 256 x 256 kernel spaces its
  // eight copies three steps apart: measured at M = 4096 and 8192, stride 1 (the first eight
  // steps) was 2-3 % slower, stride 2 about 10 % slower and stride 4 3 % slower.
  constexpr int kFirstCopy = kMid ? kBarStep : 0;
  constexpr int kCopySpan = kSteps - kFirstCopy;
  constexpr int kCopyStride = !kMid && 3 * (kCopies - 1) < kCopySpan ? 3 : 1;
  auto copy_step = [](int j) constexpr {
    return kFirstCopy + (kCopyStride * (kCopies - 1) < kCopySpan ? j * kCopyStride : j * kCopySpan / kCopies);
  };
  static_assert(copy_step(kCopies - 1) < kSteps, "every copy of a refill is issued inside the block");

  // Copies issued per wave per K block. At the mid-block barrier of iteration kb block kb + 1
  // must have landed, at the end-of-block barrier block kb + 2: either way the copies of the
  // STAGES - 2 most recently issued blocks may stay in flight (waits take immediates).
  auto wait_next_block = [&](bool steady) __attribute__((always_inline)) {
    if (!steady || STAGES == 2) {
      wait_copies();
    } else if (copies_as) {
      wait_copies_upto<(STAGES - 2) * (kCopies + 1)>();
    } else {
      wait_copies_upto<(STAGES - 2) * kCopies>();
    }
  };

  float sc[TM];  // scale products As * Bs of the block's activation rows
  if constexpr (kMid) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) sc[tm] = 0.f;
  }
  // kMid: the last two MFMA results of the previous block (zero before the first block:
  // promoting them then adds 0 * 0 to a zero accumulator).
  v4f p1c = {0.f, 0.f, 0.f, 0.f}, p2c = p1c;
  auto promote = [&](int u, const v4f& pu, float s) __attribute__((always_inline)) {
    const int um = u / TN, un = u % TN;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[un][um][e] = fmaf(pu[e], s, acc[un][um][e]);
    // Pin the promotion here: otherwise the FMAs are sunk past the loop's branch,
    // since their results are only read in the next K block.
    asm volatile("" : "+v"(acc[un][um][0]), "+v"(acc[un][um][1]), "+v"(acc[un][um][2]), "+v"(acc[un][um][3]));
  };

  auto iter = [&](int kb, auto steady_c) __attribute__((always_inline)) {
    constexpr bool kSteady = decltype(steady_c)::value;  // kb + STAGES < KB: refill a stage
    const int cslot = kb % STAGES;
    // The last iteration also reads a (stale, in-bounds) stage, which keeps the steps free of
    // branches; those registers are never used.
    const int nslot = (kb + 1) % STAGES;
    const uint8_t* nstage = &smem[g][nslot][0];
    const bool mask_next = kTail && kb + 1 < KB && gkb(kb + 1) == KB_all - 1;  // uniform
    const ScaleT bs_next = weight_scale(gkb(min(kb + 1, KB - 1)));
    // With kMid the scale products live across blocks; otherwise they are this block's alone.
    float sc_block[TM];
    float* const scp = kMid ? sc : sc_block;
    if constexpr (!kE8 && !kMid) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) scp[tm] = sa[tm] * bsv;
    }
    if constexpr (kSteady && !kMid) issue_scales(cslot, kb + STAGES);
    v4f p1 = {0.f, 0.f, 0.f, 0.f}, p2 = p1;  // MFMA results of the previous two steps
    if constexpr (kMid) {
      p1 = p1c;
      p2 = p2c;
    }
    // Step t issues the MFMA of sub-tile t, the promotion FMAs of the sub-tile two steps back
    // (its result is then at least one MFMA old), its share of the copies and of the next
    // block's LDS reads; a scheduling barrier per step keeps this order.
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      const int tm = t / TN, tn = t % TN;
      v4f p;
      if constexpr (kE8) {
        // The scaled product is added to the tile by the MFMA itself.
        const v4f cur = {acc[tn][tm][0], acc[tn][tm][1], acc[tn][tm][2], acc[tn][tm][3]};
        const v4f nxt = mfma_block_e8(fb[tn], fa[tm], cur, bsv, sa[tm]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[tn][tm][e] = nxt[e];
      } else {
        // The scale product of row tm is formed at the row's first step, while sa[tm] still
        // holds this block's activation scale (the row's last step reloads it). Until then
        // sc[TM - 1] keeps the previous block's, which its two lagging promotions use (the
        // last two steps of a block lie in its last row, since TN >= 2).
        if (kMid && tn == 0) scp[tm] = sa[tm] * bsv;
        p = mfma_block(fb[tn], fa[tm]);
        if (t >= 2) {
          promote(t - 2, p2, scp[(t - 2) / TN]);
        } else if constexpr (kMid) {
          promote(kSteps - 2 + t, p2, scp[TM - 1]);
        }
      }
      if (kMid && t == kBarStep) {
        wait_next_block(kSteady);
        lds_barrier();
        if constexpr (kSteady) issue_scales(cslot, kb + STAGES);
      }
      if constexpr (kSteady) {
#pragma unroll
        for (int j = 0; j < kCopies; ++j)
          if (t == copy_step(j)) issue_piece(cslot, kb + STAGES, j);
      }
      if (tn == TN - 1) {
        fa[tm] = frag_a(nstage, tm);
        if (mask_next) fa[tm] = mask_k_tail(fa[tm], k_tail, kc);
        sa[tm] = act_scale(nslot, tm);
      }
      if (tm == TM - 1) {
        fb[tn] = frag_b(nstage, tn);
        if (mask_next) fb[tn] = mask_k_tail(fb[tn], k_tail, kc);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!kE8) {
        p2 = p1;
        p1 = p;
      }
    }
    if constexpr (!kE8 && !kMid) {
      promote(kSteps - 2, p2, scp[TM - 1]);
      promote(kSteps - 1, p1, scp[TM - 1]);
    }
    if constexpr (kMid) {
      p1c = p1;
      p2c = p2;
    }
    bsv = bs_next;
    if constexpr (!kMid) {
      wait_next_block(kSteady);
      lds_barrier();
    }
  };

#pragma unroll
  for (int i = 0; i < STAGES; ++i) issue_copies(i, min(i, KB - 1));
  if constexpr (kMid) {
    // block 0 has landed once the copies of blocks 1 .. STAGES-1 are the only ones left
    if (copies_as) {
      wait_copies_upto<(STAGES - 1) * (kCopies + 1)>();
    } else {
      wait_copies_upto<(STAGES - 1) * kCopies>();
    }
  } else {
    // blocks 0 and 1 have landed once the copies of blocks 2 .. STAGES-1 are the only ones left
    wait_next_block(STAGES <= KB);
  }
  lds_barrier();
  const bool mask_first = kTail && gkb(0) == KB_all - 1;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    fa[tm] = frag_a(&smem[g][0][0], tm);
    if (mask_first) fa[tm] = mask_k_tail(fa[tm], k_tail, kc);
    sa[tm] = act_scale(0, tm);
  }
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    fb[tn] = frag_b(&smem[g][0][0], tn);
    if (mask_first) fb[tn] = mask_k_tail(fb[tn], k_tail, kc);
  }
  bsv = weight_scale(g);
  // every wave has read stage 0 before iteration 0 refills it (with kMid, the refill follows
  // the barrier of iteration 0 instead)
  if constexpr (!kMid) lds_barrier();
  int kb = 0;
  for (; kb + STAGES < KB; ++kb) iter(kb, std::true_type{});
  for (; kb < KB; ++kb) iter(kb, std::false_type{});
  if constexpr (kMid) {
    if constexpr (!kE8 && kMid) {
      promote(kSteps - 2, p2c, sc[TM - 1]);
      promote(kSteps - 1, p1c, sc[TM - 1]);
    }
    // Every wave's LDS reads (the last iteration's stale ones included) are done before the
    // stages are reused below (the end-of-block barrier already covers them).
    lds_barrier();
  }
  // No copy is in flight: the last iteration waited for all of them.

  if constexpr (KG == 2) {
    // Sum of the two groups' tiles, group 0 + group 1: group 1 parks its tile in the stages
    // (every wave has finished with them at the last barrier), group 0 adds and stores.
    float* red = reinterpret_cast<float*>(&smem[0][0][0]);
    if (g == 1) {
#pragma unroll
      for (int t = 0; t < TN * TM; ++t)
        *reinterpret_cast<v4f*>(red + ((w * TN * TM + t) * 64 + lane) * 4) =
            v4f{acc[t / TM][t % TM][0], acc[t / TM][t % TM][1], acc[t / TM][t % TM][2], acc[t / TM][t % TM][3]};
    }
    lds_barrier();
    if (g == 1) return;
#pragma unroll
    for (int t = 0; t < TN * TM; ++t) {
      const v4f o = *reinterpret_cast<const v4f*>(red + ((w * TN * TM + t) * 64 + lane) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t / TM][t % TM][e] += o[e];
    }
  }

  // Output. When C rows allow 16-byte stores, each wave stages its tile in LDS as bf16 rows
  // (padded by 16 bytes, which keeps the transposing writes free of bank conflicts) and then
  // stores whole row segments, WN * 2 contiguous bytes per row; storing straight from the
  // MFMA layout writes 16 rows x 32 bytes per instruction and reaches memory as partial
  // lines. Each wave uses its own part of the stages (after the K-group sum's area), in
  // chunks of 16-row blocks that fit.
  const bool vec16 = ((args.ldc & 7) == 0) && ((reinterpret_cast<uintptr_t>(args.c) & 15) == 0);
  // The staged output, compiled once per output dtype and bias presence so that the
  // per-element conversion has no branches; the bias of the lane's columns is loaded once.
  auto staged = [&](auto f16_c, auto bias_c) {
    constexpr bool kF16 = decltype(f16_c)::value, kBias = decltype(bias_c)::value;
    constexpr int kRowBytes = WN * 2 + 16;
    constexpr int kBase = KG == 2 ? BN * BM * 4 : 0;
    constexpr int kFitRows = (KG * STAGES * kStage - kBase) / (kWaves * kRowBytes);
    constexpr int kChunkTM = largest_divisor_upto(TM, kFitRows / 16);
    static_assert(kChunkTM >= 1 && TM % kChunkTM == 0, "output staging must fit the LDS stages");
    constexpr int kLanesPerRow = WN / 8;  // 16 bytes (8 outputs) per lane
    constexpr int kRowsPerPass = 64 / kLanesPerRow;
    static_assert(64 % kLanesPerRow == 0 && (kChunkTM * 16) % kRowsPerPass == 0, "whole passes");
    uint8_t* out_lds = &smem[0][0][0] + kBase + w * (kChunkTM * 16 * kRowBytes);
    uint32_t bias_bits[TN][4];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int nb = n0 + wn * WN + tn * 16 + 4 * kc + e;  // clamped on tails (not stored)
        bias_bits[tn][e] = kBias ? (uint32_t)args.bias[min(nb, N - 1)] : 0u;
      }
#pragma unroll
    for (int c0 = 0; c0 < TM; c0 += kChunkTM) {
#pragma unroll
      for (int tm = c0; tm < c0 + kChunkTM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          uint2 pk;
          pk.x = conv16<kF16, kBias>(acc[tn][tm][0], bias_bits[tn][0]) |
                 (conv16<kF16, kBias>(acc[tn][tm][1], bias_bits[tn][1]) << 16);
          pk.y = conv16<kF16, kBias>(acc[tn][tm][2], bias_bits[tn][2]) |
                 (conv16<kF16, kBias>(acc[tn][tm][3], bias_bits[tn][3]) << 16);
          *reinterpret_cast<uint2*>(out_lds + ((tm - c0) * 16 + r) * kRowBytes + (tn * 16 + 4 * kc) * 2) = pk;
        }
      // The wave's LDS writes are read back by other lanes of the same wave; LDS executes one
      // wave's accesses in order, and this keeps the compiler from reordering them.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
      for (int pass = 0; pass < kChunkTM * 16 / kRowsPerPass; ++pass) {
        const int row = pass * kRowsPerPass + lane / kLanesPerRow;
        const int seg = lane % kLanesPerRow;
        const v4i v = *reinterpret_cast<const v4i*>(out_lds + row * kRowBytes + seg * 16);
        const int m = m0 + wm * WM + c0 * 16 + row;
        const int n = n0 + wn * WN + seg * 8;
        bool row_ok = m < M;
        if constexpr (kGrouped) row_ok = row_ok && args.layout[m] >= 0;
        if (row_ok && n < N) {
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
  };
  if (vec16) {
    if (args.out_f16) {
      if (args.bias) staged(std::true_type{}, std::true_type{});
      else staged(std::true_type{}, std::false_type{});
    } else {
      if (args.bias) staged(std::false_type{}, std::true_type{});
      else staged(std::false_type{}, std::false_type{});
    }
    return;
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
        store_out16x4(args.c + (int64_t)m * args.ldc + n, n, N, vec_ok, acc[tn][tm][0], acc[tn][tm][1],
                      acc[tn][tm][2], acc[tn][tm][3], args.bias, args.out_f16);
    }
  }
}

template <int BN, int BM, int WGN, int WGM, int STAGES, int KG, bool G, bool T>
hipError_t launch_tiled_cfg(const GemmArgs& args, hipStream_t stream) {
  unsigned tiles = (unsigned)(((args.N + BN - 1) / BN) * ((args.M + BM - 1) / BM));
  if (G) tiles = (tiles + 7) / 8 * 8;  // grouped: a multiple of 8 workgroups (map_tile_padded)
  if (args.e8) {
    hipLaunchKernelGGL((gemm_tiled_kernel<BN, BM, WGN, WGM, STAGES, KG, G, true, T>), dim3(tiles),
                       dim3(KG * WGN * WGM * 64), 0, stream, args);
  } else {
    hipLaunchKernelGGL((gemm_tiled_kernel<BN, BM, WGN, WGM, STAGES, KG, G, false, T>), dim3(tiles),
                       dim3(KG * WGN * WGM * 64), 0, stream, args);
  }
  return hipGetLastError();
}

constexpr int64_t kCUs = 256;  // workgroups that fill MI355X once

// Time of one round of tiles of a shape, from the FLOP rate per CU that each shape reached on
// the N = K = 4096 sweep (one full round, launch included): 256x256 8.5, 256x128 6.3,
// 128x128 4.9 and 128x64 3.2 TFLOP/s per CU.
double round_us(const TiledPlan& p, int64_t K) {
  const double rate = p.bm == 256 ? 8.5 : p.bn == 256 ? 6.3 : p.bm == 128 ? 4.9 : 3.2;
  return 2.0 * p.bn * p.bm * (double)K / (rate * 1e6);
}

double plan_us(const TiledPlan& p, int64_t K) { return (double)((p.tiles + kCUs - 1) / kCUs) * round_us(p, K); }

}  // namespace

// Base tile shape: the largest that still gives every CU a workgroup, which trades bytes copied
// per MFMA (fewer with big tiles) against parallelism. On the N = K = 4096 sweep: 256x256 from
// M = 4096 (8 waves of 128x64, two LDS stages), 256x128 at M = 2048 (three stages, 16 waves of
// 64x32: 3 % under 8 waves of 64x64 at M = 2048, 1.6 % at M = 3072), 128x128 at M = 1024 and
// 128x64 at M = 512 (8 waves of 64x32 or 32x32, four stages: the fourth stage took M = 512 from
// 20.1 to 18.2 us, and 8 waves instead of 4 a further 3-6 % at M = 512-1536; 16 waves of 32x32 on
// 128x128 lost 1-3 %).
TiledPlan plan_tiled(int64_t M, int64_t N, int64_t K) {
  (void)K;
  auto tiles = [&](int bn, int bm) { return (int)(((N + bn - 1) / bn) * ((M + bm - 1) / bm)); };
  if (tiles(256, 256) >= kCUs) return {256, 256, tiles(256, 256), 0};
  if (tiles(256, 128) >= kCUs) return {256, 128, tiles(256, 128), 0};
  if (tiles(128, 128) >= kCUs) return {128, 128, tiles(128, 128), 0};
  return {128, 64, tiles(128, 64), 0};
}

namespace {

// The tile shape a dense launch runs: the plan's, except that with a partial last K block the
// 256 x 256 plan runs 256 x 128 tiles (its masked kernel would spill).
TiledPlan no_masked_256(TiledPlan p, int64_t M, int64_t N, int64_t K) {
  if (K % kBlock && p.bn == 256 && p.bm == 256) p = {256, 128, (int)(((N + 255) / 256) * ((M + 127) / 128)), 0};
  return p;
}
TiledPlan launched_plan(int64_t M, int64_t N, int64_t K) { return no_masked_256(plan_tiled(M, N, K), M, N, K); }

// The shape whose rounds take the least predicted time (the larger tile on a tie).
TiledPlan min_time_plan(int64_t M, int64_t N, int64_t K) {
  auto plan = [&](int bn, int bm) {
    return no_masked_256(TiledPlan{bn, bm, (int)(((N + bn - 1) / bn) * ((M + bm - 1) / bm)), 0}, M, N, K);
  };
  const TiledPlan shapes[] = {plan(256, 256), plan(256, 128), plan(128, 128), plan(128, 64)};
  TiledPlan best = shapes[0];
  for (const TiledPlan& p : shapes)
    if (plan_us(p, K) < plan_us(best, K)) best = p;
  return best;
}

hipError_t launch_planned(const GemmArgs& args, const TiledPlan& p, hipStream_t stream, int persistent) {
  if (persistent && p.bn == 256 && p.bm == 256 && persistent_supported(args)) return launch_gemm_persistent(args, stream);
  if (args.K % kBlock) {
    if (p.bn == 256) return launch_tiled_cfg<256, 128, 4, 2, 3, 1, false, true>(args, stream);
    if (p.bm == 128) return launch_tiled_cfg<128, 128, 2, 2, 3, 1, false, true>(args, stream);
    return launch_tiled_cfg<128, 64, 2, 2, 3, 1, false, true>(args, stream);
  }
  if (p.bn == 256 && p.bm == 256) return launch_tiled_cfg<256, 256, 2, 4, 2, 1, false, false>(args, stream);
  if (p.bn == 256) return launch_tiled_cfg<256, 128, 4, 4, 3, 1, false, false>(args, stream);
  if (p.bm == 128) return launch_tiled_cfg<128, 128, 2, 4, 4, 1, false, false>(args, stream);
  return launch_tiled_cfg<128, 64, 4, 2, 4, 1, false, false>(args, stream);
}

constexpr double kLaunchGapUs = 3.0;  // a second launch on the stream

// What a dense GEMM launches: one plan over all N columns, or (n1 > 0) `lead` over the columns
// [0, n1) and `tail` over the rest, with the predicted time.
struct TiledLaunch {
  TiledPlan lead;
  int n1;
  TiledPlan tail;
  double us;
};

// Wave quantization: when the base plan's tiles fill the 256 CUs some whole number of times plus
// a fraction, that last round runs a few workgroups on an otherwise idle chip. Two remedies,
// each taken only when the per-shape round times predict a gain:
//   * split: the columns of the whole rounds run with the base plan, the remaining columns as a
//     second launch of the same GEMM restricted to them (B, its scales, C and the bias offset by
//     whole 128-column strips) with the tile shape the base rule picks for that narrower problem;
//     on the hidden-5120 layers at M = 2048 this gave QKV 164-174 -> 145 us, o_proj 151-158 ->
//     140 us and down 423-433 -> 371 us;
//   * otherwise, fewer and bigger tiles: the shape with the least predicted time, e.g. 160 tiles
//     of 128x128 in one round instead of 320 of 128x64 in two at M = 640 (N = K = 4096:
//     32.6 -> 22.7 us; M = 768 32.4 -> 22.9, M = 1536 44.0 -> 35.1, M = 3072 70.2 -> 56.0 us).
// The split is preferred when both apply: for o_proj and down at M = 2048 the model ranks one
// partial round of 256x256 tiles first, but it measured 5-8 % slower than the split.
// Each output element is computed exactly as by a single launch of either shape.
TiledLaunch choose_launch(int64_t M, int64_t N, int64_t K) {
  const TiledPlan p = launched_plan(M, N, K);
  const double p_us = plan_us(p, K);
  const int full = p.tiles / (int)kCUs, rest = p.tiles % (int)kCUs;
  if (full >= 1 && rest > 0) {
    const int m_tiles = (int)((M + p.bm - 1) / p.bm);
    const int n1 = (int)(full * kCUs / m_tiles) * p.bn;  // columns of the whole rounds
    if (n1 >= p.bn && n1 < N) {
      TiledPlan lead = p;
      lead.tiles = (n1 / p.bn) * m_tiles;
      const TiledPlan tail = launched_plan(M, N - n1, K);
      const double split_us = plan_us(lead, K) + plan_us(tail, K) + kLaunchGapUs;
      if (split_us < p_us) return {lead, n1, tail, split_us};
    }
  }
  if (rest > 0) {
    const TiledPlan q = min_time_plan(M, N, K);
    if (plan_us(q, K) < p_us) return {q, 0, q, plan_us(q, K)};
  }
  return {p, 0, p, p_us};
}

}  // namespace

// The chosen launch's rounds at the measured per-CU rates, or, where the operands take longer to
// stream from HBM (about 5.5 TB/s, plus 3.5 us for the launch), that.
double tiled_time_us(int64_t M, int64_t N, int64_t K) {
  const double stream_us = ((double)N * (double)K + (double)M * (double)K) / 5.5e6 + 3.5;
  return std::max(choose_launch(M, N, K).us, stream_us);
}

hipError_t launch_gemm_tiled(const GemmArgs& args, void* workspace, hipStream_t stream, int persistent) {
  (void)workspace;
  const TiledLaunch l = choose_launch(args.M, args.N, args.K);
  if (l.n1 == 0) return launch_planned(args, l.lead, stream, persistent);
  const int n1 = l.n1;
  GemmArgs a1 = args;
  a1.N = n1;
  GemmArgs a2 = args;
  a2.N = args.N - n1;
  a2.b = args.b + (int64_t)n1 * args.ldb;
  a2.bs = static_cast<const uint8_t*>(args.bs) + (int64_t)(n1 / kBlock) * args.ld_bs * (args.e8 ? 1 : 4);
  a2.c = args.c + n1;
  if (args.bias) a2.bias = args.bias + n1;
  const hipError_t e = launch_planned(a1, l.lead, stream, persistent);
  if (e != hipSuccess) return e;
  return launch_planned(a2, l.tail, stream, persistent);
}

// Grouped: a workgroup stays inside one 128-row block, so 256 x 128 with 16 waves of 64 x 32
// (8 waves of 64 x 64 with a partial last K block).
hipError_t launch_grouped_tiled(const GemmArgs& args, hipStream_t stream) {
  if (args.K % kBlock) return launch_tiled_cfg<256, 128, 4, 2, 3, 1, true, true>(args, stream);
  return launch_tiled_cfg<256, 128, 4, 4, 3, 1, true, false>(args, stream);
}

}  // namespace bfp8
