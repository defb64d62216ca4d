// K-split blockwise FP8 GEMM schedule for gfx950 (small and mid M, memory bound).
//
// Role: the small-M "single-partition" and mid-M schedules of page "lmdeploy/pull/4830",
// section "Kernel design", re-derived for CDNA4. At small and mid M the cost is moving the
// weight matrix B (N*K bytes, from HBM) and the activation rows (from L2) into the CUs; the
// math is small. So:
//   * the problem is computed transposed, C^T = B . A^T: the 16 rows of an MFMA's first
//     operand are weight rows and its 16 columns activation rows; one 16x16x128 FP8 MFMA
//     covers one 128-wide K block of a 16x16 sub-tile;
//   * a workgroup owns a BN x BM tile of C^T (BN weight rows, BM activation rows), from
//     16 x 16 to 64 x 64, chosen per shape by a model of the bytes each CU copies (small
//     tiles give every CU a workgroup; larger ones copy fewer bytes where K is long); its
//     WAVES waves split the tile's
//     K blocks round-robin (kb = w, w + WAVES, ...), each wave accumulating the whole tile
//     over its own blocks, so waves never wait for one another inside the K loop;
//   * each wave copies its K blocks (BN + BM rows of 128 bytes, and the block's BM
//     activation scales) with the gfx950 direct-to-LDS loads into SLOTS private LDS slots.
//     These copies read whole 128-byte rows with 8 lanes each, several times the rate of
//     loading MFMA operands straight from memory (4 rows per lane quad). The wave reads a
//     block's fragments into registers, refills the slot with its next block and multiplies
//     while that copy is in flight; the 16-byte columns of each LDS row are XOR-swizzled so
//     that the fragment reads are free of bank conflicts;
//   * promotion per K block: acc += P * (As[kb][m] * Bs[n/128][kb]) with one FMA per
//     element (BN is at most 128 and tiles are BN-aligned, so a wave's weight rows share
//     one scale strip);
//   * the workgroups that share weight rows walk their K blocks from different starting
//     points, so that they do not all wait on the same HBM reads;
//   * the waves' partial tiles are summed through LDS in a fixed wave order, which keeps
//     results bitwise reproducible without atomics or a global workspace, and each sum is
//     rounded once to bf16;
//   * UE8M0 scales (kE8): the scale codes are copied like the float scales, and the scaled
//     MFMA applies 2^(ea - 127) * 2^(eb - 127) and accumulates into the wave's tile itself;
//   * 1x64 activation groups with 128x64 weight blocks (kG64; the next block-scale layouts
//     named on the vLLM torch-backend page, section "风险与影响"): each 128-wide K block holds
//     two scale groups. The lanes of an MFMA operand fragment hold K bytes [32 kc, 32 kc + 32),
//     so the activation fragment is split into its kc < 2 half (K 0-63) and its kc >= 2 half,
//     each multiplied by a full MFMA with the other half zeroed and promoted with its own
//     As * Bs (groups 2 kb and 2 kb + 1, in that order); twice the MFMAs and promotions;
//   * fused activation quantization (kFuse = kInBf16 or kInF16, 16-row tiles, M <= kQRows):
//     the linear layer's bf16/fp16 activations are copied instead of codes, the wave's 64
//     lanes covering only the kQRows (1, 4 or 8) rows quantized: 64 / kQRows lanes per row
//     and 2 * kQRows consecutive elements per lane. Each lane quantizes its elements in
//     registers (1x128 groups, the group's amax reduced over the row's lanes) with the
//     per-token-group quantizer's arithmetic, so codes and scales are bit-identical to
//     quantizing first, and writes the codes into the slot's kQRows rows of codes (the
//     swizzled layout the fragment reads expect) and the scale beside them; fragment rows past
//     kQRows read row r % kQRows (their results are never stored). The division by the group
//     scale s is done as q0 = x * r, r = 1 / s correctly rounded, then q0 + (x - q0 * s) * r
//     with fused multiply-adds and x's sign: that is the correctly rounded x / s for every
//     bf16 and fp16 x and every scale the quantizer can produce, except quotients below 2^-10
//     in magnitude, which all encode as zero of x's sign (checked exhaustively against the
//     division); groups whose scale is infinite divide. Every workgroup of the grid repeats
//     this for its M rows (about (N / 16) x kQRows x K element steps in all), which pays only
//     where a separate quantizer launch costs more: small M, N and K.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace bfp8 {

namespace {

template <int TN, int TM, int WAVES, int SLOTS, bool kE8, int kFuse = 0, int kQRows = 16, bool kG64 = false>
__global__ __launch_bounds__(WAVES * 64) void gemm_ksplit_kernel(GemmArgs args) {
  static_assert(!kG64 || (!kE8 && kFuse == 0), "1x64 groups: float scales, quantized activations");
  constexpr int kScaleGroups = kG64 ? 2 : 1;  // activation scale groups per 128-wide K block
  constexpr bool kFused = kFuse != 0;  // args.a holds bf16/fp16 activations (lda in elements)
  static_assert(!kFused || (!kE8 && TM == 1 && (kFuse == kInBf16 || kFuse == kInF16)),
                "fused quantization: float scales, 16 activation rows, bf16 or fp16 input");
  static_assert(kQRows == 1 || kQRows == 4 || kQRows == 8 || kQRows == 16, "1, 4, 8 or 16 quantized rows");

  constexpr int BN = 16 * TN, BM = 16 * TM;
  constexpr int kRows = kFused ? BN : BN + BM;    // 128-byte rows copied per K block
  constexpr int kQLanes = 64 / kQRows;             // fused: lanes per quantized row
  constexpr int kQElems = kBlock / kQLanes;        // fused: consecutive elements per lane
  // fused: the lane's elements arrive as 16-byte pieces (8 elements), or for one row as one
  // 4-byte piece (2 elements)
  constexpr int kXPiece = kQRows == 1 ? 4 : 16;
  constexpr int kXCopies = kFused ? kQElems * 2 / kXPiece : 0;
  // bytes per slot: copied rows; fused: then the kQRows rows of codes and the staged 16-bit
  // activations (kXCopies pieces of 64 lanes x kXPiece bytes)
  constexpr int kSlot = kRows * kBlock + (kFused ? kQRows * kBlock + kXCopies * 64 * kXPiece : 0);
  constexpr int kPieces = kRows / 8;              // 1 KB (8-row) copies per K block
  // 64-lane scale copies per K block: 64 float scales each, or 256 UE8M0 codes (4 per lane).
  constexpr int kAsCopies = kFused ? 0 : kE8 ? 1 : (BM + 63) / 64;
  constexpr int kScaleBytes = kE8 ? 1 : 4;
  static_assert(!kE8 || BM <= 256, "one copy holds the codes of 256 activation rows");
  using ScaleT = std::conditional_t<kE8, int, float>;
  constexpr int kPerBlock = kPieces + kScaleGroups * kAsCopies + kXCopies;  // copies issued per K block
  constexpr int kTileFloats = BN * BM;
  static_assert(kBlock % BN == 0, "a wave's weight rows must share one scale strip");
  static_assert(kTileFloats * 4 <= SLOTS * kSlot, "the reduction reuses the wave's slots");
  static_assert(SLOTS >= 1 && SLOTS <= 3 && (SLOTS - 1) * kPerBlock < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) uint8_t slots[WAVES][SLOTS][kSlot];
  __shared__ __attribute__((aligned(16))) float as_slots[WAVES][SLOTS][kScaleGroups * (kAsCopies > 0 ? kAsCopies : 1) * 64];


  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, kc = lane >> 4;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int M = args.M, N = args.N;
  const int KB = (args.K + kBlock - 1) / kBlock;  // the last block may be partial (K % 128 != 0)
  const int k_tail = args.K - (KB - 1) * kBlock;   // bytes of the last block that exist
  const int G64 = (args.K + 63) / 64;               // kG64: scale groups along K
  const int nkb = KB > w ? (KB - w + WAVES - 1) / WAVES : 0;  // this wave's blocks: w + i * WAVES

  // Copy plan: piece j is slot rows [8j, 8j + 8); lane l lands at row 8j + l/8, physical
  // 16-byte column l%8, so it loads logical column (l%8) ^ swizzle(row) of that row. Rows
  // past N or M are clamped to the last row (their results are never stored).
  uint32_t coff[kPieces];
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {
    const int row = j * 8 + (lane >> 3);
    const int lcol = (lane & 7) ^ lds_swizzle(row);
    const bool is_b = j * 8 < BN;  // uniform: BN is a multiple of 16
    const int src_row = is_b ? min(n0 + row, N - 1) : min(m0 + row - BN, M - 1);
    coff[j] = (uint32_t)((int64_t)src_row * (is_b ? args.ldb : args.lda) + lcol * 16);
  }
  // Float scales: row m0 + 64 c + lane, clamped. UE8M0 codes: the dword of rows m0 + 4 lane ..,
  // clamped to the one holding row M - 1 (inside the row of codes: its length is a multiple of 4).
  uint32_t as_voff[kAsCopies > 0 ? kAsCopies : 1];
#pragma unroll
  for (int c = 0; c < kAsCopies; ++c)
    as_voff[c] = kE8 ? (uint32_t)min(m0 + 4 * lane, (M - 1) & ~3) : (uint32_t)min(m0 + c * 64 + lane, M - 1) * 4u;
  const uint8_t* asmat = static_cast<const uint8_t*>(args.as);
  // Fused: lane l quantizes row qr = l / kQLanes, elements [qc, qc + kQElems) of each K block,
  // copied in pieces of kXPiece bytes (piece j lands at stage byte 64 kXPiece j + kXPiece l). A
  // piece past M or past K is not needed; it copies the block's first piece of row m0 instead
  // (in bounds) and is zeroed after the read, so that every copy instruction is issued with
  // the same count in flight (the waits below count them).
  const int qr = lane / kQLanes, qc = (lane % kQLanes) * kQElems;
  const bool x_row_ok = kFused && m0 + qr < M;
  const uint32_t x_off = (uint32_t)((int64_t)(x_row_ok ? m0 + qr : m0) * args.lda * 2) + (x_row_ok ? 2u * qc : 0u);
  const uint32_t x_off_spare = (uint32_t)((int64_t)m0 * args.lda * 2);
  const uint32_t x_delta = x_off - x_off_spare;  // offset of the lane's piece 0 past the spare
  auto x_piece_ok = [&](int kb, int j) __attribute__((always_inline)) {
    return x_row_ok && qc + (kXPiece / 2) * j < (kb == KB - 1 ? k_tail : kBlock);
  };

  auto issue = [&](int slot, int kb) __attribute__((always_inline)) {
    const uint8_t* bsrc = args.b + (int64_t)kb * kBlock;
    const uint8_t* asrc = args.a + (int64_t)kb * kBlock;
    const uint32_t dst = lds_addr(&slots[w][slot][0]);
#pragma unroll
    for (int j = 0; j < kPieces; ++j) copy16_to_lds(j * 8 < BN ? bsrc : asrc, coff[j], dst + (uint32_t)(j * 8 * kBlock));
    if constexpr (kG64) {
      // groups 2 kb and 2 kb + 1 (clamped to the last group, which a partial last block may end
      // before: that copy is then a duplicate whose scale is never used)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int grp = min(2 * kb + h, G64 - 1);
#pragma unroll
        for (int c = 0; c < kAsCopies; ++c)
          copy4_to_lds(asmat + (int64_t)grp * args.ld_as * 4, as_voff[c], lds_addr(&as_slots[w][slot][(h * kAsCopies + c) * 64]));
      }
    } else {
#pragma unroll
      for (int c = 0; c < kAsCopies; ++c)
        copy4_to_lds(asmat + (int64_t)kb * args.ld_as * kScaleBytes, as_voff[c], lds_addr(&as_slots[w][slot][c * 64]));
    }
    if constexpr (kFused) {
      const uint8_t* xsrc = args.a + (int64_t)kb * kBlock * 2;
      const uint32_t xdst = dst + (uint32_t)((kRows + kQRows) * kBlock);
#pragma unroll
      for (int j = 0; j < kXCopies; ++j) {
        const uint32_t voff = x_off_spare + (x_piece_ok(kb, j) ? x_delta + (uint32_t)(kXPiece * j) : 0u);
        if constexpr (kXPiece == 16) {
          copy16_to_lds(xsrc, voff, xdst + (uint32_t)(j * 64 * kXPiece));
        } else {
          copy4_to_lds(xsrc, voff, xdst + (uint32_t)(j * 64 * kXPiece));
        }
      }
    }
  };

  // Fused: the lane's kQElems staged activations of a block (`raw`) -> e4m3 codes written to
  // its row of the slot's activation rows (swizzled), and the row's group scale to `as_row`
  // (the per-token-group quantizer's arithmetic).
  auto quantize = [&](const uint32_t (&raw)[kXCopies > 0 ? kXCopies * kXPiece / 4 : 1], int kb, uint8_t* arows,
                      float* as_row) __attribute__((always_inline)) {
    float v[kQElems];
#pragma unroll
    for (int j = 0; j < kXCopies; ++j) {
      const bool ok = x_piece_ok(kb, j);
#pragma unroll
      for (int i = 0; i < kXPiece / 4; ++i) {
        const uint32_t p = ok ? raw[j * (kXPiece / 4) + i] : 0u;
        const int e = (kXPiece / 2) * j + 2 * i;
        if constexpr (kFuse == kInBf16) {
          v[e] = __uint_as_float(p << 16);
          v[e + 1] = __uint_as_float(p & 0xffff0000u);
        } else {
          v[e] = f16_value(p & 0xffffu);
          v[e + 1] = f16_value(p >> 16);
        }
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < kQElems; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int mask = 1; mask < kQLanes; mask <<= 1) amax = fmaxf(amax, __shfl_xor(amax, mask));
    const float s = fmaxf(amax, 1e-10f) / 448.0f;  // correctly rounded divide
    float y[kQElems];
    if (s < __builtin_huge_valf()) {
      const float rcp = 1.0f / s;  // correctly rounded
#pragma unroll
      for (int i = 0; i < kQElems; ++i) {
        const float q0 = v[i] * rcp;
        const float e = fmaf(-q0, s, v[i]);  // exact
        y[i] = fminf(fmaxf(copysignf(fmaf(e, rcp, q0), v[i]), -448.0f), 448.0f);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kQElems; ++i) y[i] = fminf(fmaxf(v[i] / s, -448.0f), 448.0f);
    }
    uint32_t wq[(kQElems + 3) / 4];
    if constexpr (kQElems == 2) {
      wq[0] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    } else {
#pragma unroll
      for (int d = 0; d < kQElems / 4; ++d) {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * d], y[4 * d + 1], 0, false);
        wq[d] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4 * d + 2], y[4 * d + 3], lo, true);
      }
    }
    // codes of elements [qc, qc + kQElems): 2 or 8 bytes inside a 16-byte column, or whole columns
    uint8_t* row = arows + qr * kBlock;
    const int sw = lds_swizzle(BN + qr);
    if constexpr (kQElems == 2) {
      *reinterpret_cast<uint16_t*>(row + (((qc >> 4) ^ sw) << 4) + (qc & 15)) = (uint16_t)wq[0];
    } else if constexpr (kQElems == 8) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      *reinterpret_cast<u32x2*>(row + (((qc >> 4) ^ sw) << 4) + (qc & 15)) = u32x2{wq[0], wq[1]};
    } else {
#pragma unroll
      for (int c = 0; c < kQElems / 16; ++c)
        *reinterpret_cast<u32x4*>(row + ((((qc >> 4) + c) ^ sw) << 4)) =
            u32x4{wq[4 * c], wq[4 * c + 1], wq[4 * c + 2], wq[4 * c + 3]};
    }
    as_row[qr] = s;  // every lane of the row stores the same value
  };

  // Fragment rows come in 16-row blocks, so every row a lane reads has row % 16 == r.
  const int fsw = lds_swizzle(r);
  const uint32_t off_lo = (uint32_t)(r * kBlock + (((2 * kc) ^ fsw) << 4));
  const uint32_t off_hi = (uint32_t)(r * kBlock + (((2 * kc + 1) ^ fsw) << 4));
  auto frag_at = [&](const uint8_t* slot, int row0) __attribute__((always_inline)) -> v8i {
    const v4i lo = *reinterpret_cast<const v4i*>(slot + off_lo + row0 * kBlock);
    const v4i hi = *reinterpret_cast<const v4i*>(slot + off_hi + row0 * kBlock);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // Weight scale strip of the tile (scalar loads through the constant address space).
  const uint8_t* bs_row =
      static_cast<const uint8_t*>(args.bs) + (int64_t)(min(n0, N - 1) / kBlock) * args.ld_bs * kScaleBytes;
  auto weight_scale = [&](int kb) __attribute__((always_inline)) -> ScaleT {
    if constexpr (kE8) {
      return e8_code_scalar((const __attribute__((address_space(4))) uint32_t*)bs_row, kb);
    } else {
      return ((const __attribute__((address_space(4))) float*)bs_row)[kb];
    }
  };

  float acc[TN][TM][4];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[tn][tm][e] = 0.f;

  // The workgroups of one weight strip (blockIdx.y = 0 .. gridDim.y - 1) start at different
  // points of their K loops, so that at any time they request different weight blocks: the
  // first to touch a block fetches it from HBM while the others, later, find it in L2,
  // rather than all waiting on the same HBM reads. A wave still visits each of its blocks
  // once, in a cyclically shifted order.
  const int rot = nkb > 0 ? (int)((int64_t)blockIdx.y * nkb / gridDim.y) : 0;
  auto block_of = [&](int i) __attribute__((always_inline)) {
    const int j = i + rot < nkb ? i + rot : i + rot - nkb;
    return w + j * WAVES;
  };

#pragma unroll
  for (int s = 0; s < SLOTS; ++s)
    if (s < nkb) issue(s, block_of(s));

  for (int i = 0; i < nkb; ++i) {
    const int kb = block_of(i);
    const int slot = i % SLOTS;
    // Block i has landed once only the copies of the SLOTS - 1 blocks issued after it remain.
    if (i + SLOTS - 1 < nkb) {
      wait_copies_upto<(SLOTS - 1) * kPerBlock>();
    } else {
      wait_copies();
    }
    const uint8_t* sl = &slots[w][slot][0];
    v8i fb[TN], fa[TM];
    float sc[TM], sc_hi[TM];
    ScaleT ea[TM];
    const ScaleT bs_kb = weight_scale(kG64 ? 2 * kb : kb);
    // kG64: the second group's weight scale, 0 where a partial last block has no second group
    const bool has_hi = kG64 && 2 * kb + 1 < G64;  // wave-uniform
    const float bs_hi = has_hi ? (float)weight_scale(2 * kb + 1) : 0.f;
    const bool tail = kb == KB - 1 && k_tail < kBlock;  // wave-uniform
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      fb[tn] = frag_at(sl, tn * 16);
      if (tail) fb[tn] = mask_k_tail(fb[tn], k_tail, kc);
    }
    if constexpr (kFused) {
      // The staged activations are read and the slot refilled (its copied rows and stage; the
      // activation rows of codes are not copied) before the quantization, which then runs while
      // the next blocks' copies are in flight. The wave reads back its own LDS writes.
      uint32_t raw[kXCopies * kXPiece / 4];
      const uint8_t* stage = sl + (kRows + kQRows) * kBlock;
#pragma unroll
      for (int j = 0; j < kXCopies; ++j) {
        if constexpr (kXPiece == 16) {
          const u32x4 p = *reinterpret_cast<const u32x4*>(stage + j * 64 * kXPiece + lane * 16);
          raw[4 * j] = p[0]; raw[4 * j + 1] = p[1]; raw[4 * j + 2] = p[2]; raw[4 * j + 3] = p[3];
        } else {
          raw[j] = *reinterpret_cast<const uint32_t*>(stage + j * 64 * kXPiece + lane * 4);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (i + SLOTS < nkb) issue(slot, block_of(i + SLOTS));
      float* as_w = &as_slots[w][slot][0];
      quantize(raw, kb, const_cast<uint8_t*>(sl) + kRows * kBlock, as_w);
      // fragment row r reads code row r % kQRows
      const int ra = r % kQRows, fsa = lds_swizzle(ra);
      const uint8_t* ar = sl + (kRows + ra) * kBlock;
      const v4i lo = *reinterpret_cast<const v4i*>(ar + (((2 * kc) ^ fsa) << 4));
      const v4i hi = *reinterpret_cast<const v4i*>(ar + (((2 * kc + 1) ^ fsa) << 4));
      fa[0] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      sc[0] = as_w[ra] * bs_kb;
    } else {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        fa[tm] = frag_at(sl, BN + tm * 16);
        if (tail) fa[tm] = mask_k_tail(fa[tm], k_tail, kc);
        if constexpr (kE8) {
          ea[tm] = reinterpret_cast<const uint8_t*>(&as_slots[w][slot][0])[tm * 16 + r];
        } else {
          sc[tm] = as_slots[w][slot][tm * 16 + r] * bs_kb;
          if constexpr (kG64) sc_hi[tm] = as_slots[w][slot][kAsCopies * 64 + tm * 16 + r] * bs_hi;
        }
      }
      // The slot is refilled only after this wave's reads of it have returned.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (i + SLOTS < nkb) issue(slot, block_of(i + SLOTS));
    }
    // Multiply, promoting sub-tile t - 2 after issuing the MFMA of sub-tile t (the result
    // is then at least one MFMA old); a scheduling barrier per step keeps this order.
    v4f p1 = {0.f, 0.f, 0.f, 0.f}, p2 = p1;
    auto promote = [&](int u, const v4f& pu) __attribute__((always_inline)) {
      const int un = u / TM, um = u % TM;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[un][um][e] = fmaf(pu[e], sc[um], acc[un][um][e]);
      asm volatile("" : "+v"(acc[un][um][0]), "+v"(acc[un][um][1]), "+v"(acc[un][um][2]), "+v"(acc[un][um][3]));
    };
    if constexpr (kG64) {
      // Halves of each activation fragment: K 0-63 in the lanes with kc < 2, K 64-127 in the
      // others. The two products of a sub-tile are promoted in group order, two steps behind.
      const bool lo_lane = kc < 2;
      v8i fa_lo[TM], fa_hi[TM];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          fa_lo[tm][d] = lo_lane ? fa[tm][d] : 0;
          fa_hi[tm][d] = lo_lane ? 0 : fa[tm][d];
        }
      v4f l1 = {0.f, 0.f, 0.f, 0.f}, l2 = l1, h1 = l1, h2 = l1;
      auto promote2 = [&](int u, const v4f& pl, const v4f& ph) __attribute__((always_inline)) {
        const int un = u / TM, um = u % TM;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[un][um][e] = fmaf(pl[e], sc[um], acc[un][um][e]);
          acc[un][um][e] = fmaf(ph[e], sc_hi[um], acc[un][um][e]);
        }
        asm volatile("" : "+v"(acc[un][um][0]), "+v"(acc[un][um][1]), "+v"(acc[un][um][2]), "+v"(acc[un][um][3]));
      };
#pragma unroll
      for (int t = 0; t < TN * TM; ++t) {
        const v4f pl = mfma_block(fb[t / TM], fa_lo[t % TM]);
        const v4f ph = mfma_block(fb[t / TM], fa_hi[t % TM]);
        if (t >= 2) promote2(t - 2, l2, h2);
        __builtin_amdgcn_sched_barrier(0);
        l2 = l1;
        h2 = h1;
        l1 = pl;
        h1 = ph;
      }
      if constexpr (TN * TM >= 2) promote2(TN * TM - 2, l2, h2);
      promote2(TN * TM - 1, l1, h1);
    } else if constexpr (kE8) {
#pragma unroll
      for (int t = 0; t < TN * TM; ++t) {
        const int tn = t / TM, tm = t % TM;
        const v4f cur = {acc[tn][tm][0], acc[tn][tm][1], acc[tn][tm][2], acc[tn][tm][3]};
        const v4f nxt = mfma_block_e8(fb[tn], fa[tm], cur, bs_kb, ea[tm]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[tn][tm][e] = nxt[e];
      }
    } else {
#pragma unroll
      for (int t = 0; t < TN * TM; ++t) {
        const v4f p = mfma_block(fb[t / TM], fa[t % TM]);
        if (t >= 2) promote(t - 2, p2);
        __builtin_amdgcn_sched_barrier(0);
        p2 = p1;
        p1 = p;
      }
      if constexpr (TN * TM >= 2) promote(TN * TM - 2, p2);
      promote(TN * TM - 1, p1);
    }
  }

  // Fixed-order reduction of the waves' partial tiles through LDS. Wave w's partial goes to
  // its own slots, which no other wave touches and in which none of its copies is pending.
  float* red = reinterpret_cast<float*>(&slots[w][0][0]);
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
      *reinterpret_cast<v4f*>(red + ((tn * TM + tm) * 64 + lane) * 4) =
          v4f{acc[tn][tm][0], acc[tn][tm][1], acc[tn][tm][2], acc[tn][tm][3]};
  __syncthreads();

  const bool vec_ok = ((args.ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(args.c) & 7) == 0);
  for (int q = threadIdx.x; q < TN * TM * 64; q += WAVES * 64) {
    const int ln = q & 63, tile = q >> 6;  // tile = tn * TM + tm
    v4f v = *reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(&slots[0][0][0]) + q * 4);
    for (int ww = 1; ww < WAVES; ++ww)
      v += *reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(&slots[ww][0][0]) + q * 4);
    const int m = m0 + (tile % TM) * 16 + (ln & 15);
    const int n = n0 + (tile / TM) * 16 + 4 * (ln >> 4);
    if (m < M && n < N)
      store_out16x4(args.c + (int64_t)m * args.ldc + n, n, N, vec_ok, v[0], v[1], v[2], v[3], args.bias, args.out_f16);
  }
}

template <int TN, int TM, int WAVES, int SLOTS>
hipError_t launch_ksplit_cfg(const GemmArgs& args, hipStream_t stream) {
  const dim3 grid((unsigned)((args.N + 16 * TN - 1) / (16 * TN)), (unsigned)((args.M + 16 * TM - 1) / (16 * TM)));
  if (args.e8) {
    hipLaunchKernelGGL((gemm_ksplit_kernel<TN, TM, WAVES, SLOTS, true>), grid, dim3(WAVES * 64), 0, stream, args);
  } else {
    hipLaunchKernelGGL((gemm_ksplit_kernel<TN, TM, WAVES, SLOTS, false>), grid, dim3(WAVES * 64), 0, stream, args);
  }
  return hipGetLastError();
}

}  // namespace

// Tiles (BN x BM, 8 waves each) and how many workgroups of each fit on a CU (LDS bound).
struct KsplitCfg {
  int bn, bm, per_cu;
};
constexpr KsplitCfg kKsplitCfgs[] = {
    {16, 16, 2},  // two slots per wave
    {16, 32, 1},
    {32, 32, 1},
    {64, 32, 1},  // one slot per wave from here
    {64, 64, 1},
};
constexpr int kKsplitCfgCount = sizeof(kKsplitCfgs) / sizeof(kKsplitCfgs[0]);

namespace {

// Predicted time of one configuration. Every workgroup copies its BN weight rows and its
// activation rows (at most M distinct ones) of every K block from L2 into LDS, at about 50 GB/s
// per CU when all workgroups run at once, about 33 GB/s when they need several rounds (each
// round then also streams its own part of the weights from HBM); the copies of all workgroups
// together run at up to 9.5 TB/s, the weights stream from HBM at about 5.5 TB/s, and a launch
// adds about 3.5 us. Workgroups beyond what the CUs hold at once (per_cu each) run in further
// rounds. Fitted to the N = K = 4096 and hidden-5120 shapes at M = 16-256, where it ranks the
// measured best tile first or within 5 % of it (the 51200-wide gate+up weight at M = 64, four
// rounds of 64x64 tiles: 79 us predicted, 82 us measured).
double cfg_time_us(const KsplitCfg& c, int64_t M, int64_t N, int64_t K) {
  const double wgs = (double)((N + c.bn - 1) / c.bn) * (double)((M + c.bm - 1) / c.bm);
  const double per_wg = (double)(c.bn + (M < c.bm ? M : c.bm)) * (double)K;
  const double rounds = std::ceil(wgs / (256.0 * c.per_cu));
  const double per_cu_rate = rounds > 1.0 ? 3.3e4 : 5.0e4;  // bytes per us
  return std::max({rounds * per_wg / per_cu_rate, wgs * per_wg / 9.5e6, (double)N * (double)K / 5.5e6}) + 3.5;
}

// The tile measured best on the N = K = 4096 sweep (cold weights) for each M: 16x16 up to
// M = 16, 16x32 and 32x32 up to 32 and 64, then 64x32 and 64x64; every choice gives 256 or
// more workgroups at N = 4096.
int default_cfg(int64_t M) { return M <= 16 ? 0 : M <= 32 ? 1 : M <= 64 ? 2 : M <= 128 ? 3 : 4; }

// The default tile, unless the model predicts another at least 10 % faster. That happens where
// K is long and N not much wider than 4096 (hidden-5120 o_proj and down, QKV), where fewer,
// larger tiles copy fewer bytes: down (N = 5120, K = 25600) at M = 128 takes 67 us with 64x64
// tiles against 94 us with 64x32, o_proj at M = 64 19 us with 64x32 against 21 us with 32x32.
int choose_cfg(int64_t M, int64_t N, int64_t K) {
  const int d = default_cfg(M);
  int best = d;
  double best_us = cfg_time_us(kKsplitCfgs[d], M, N, K);
  const double bar = 0.9 * best_us;
  for (int i = 0; i < kKsplitCfgCount; ++i) {
    const double us = cfg_time_us(kKsplitCfgs[i], M, N, K);
    if (us < bar && us < best_us) {
      best = i;
      best_us = us;
    }
  }
  return best;
}

}  // namespace

double ksplit_time_us(int64_t M, int64_t N, int64_t K) {
  return cfg_time_us(kKsplitCfgs[choose_cfg(M, N, K)], M, N, K);
}

// Where the one-launch linear layer is faster than the quantizer launch followed by the GEMM
// (interleaved graph timings on MI355X, N x K from 2048 x 4096 to 5120 x 25600): every
// workgroup quantizes all M rows, which at M = 1 (64 lanes on one row) costs less than a launch
// on every shape measured (1.2-2.4 us saved), at M <= 4 while N * K <= 2^25 (0.7-1.6 us), at
// M <= 8 while N * K <= 2^24 (0.1-1.5 us); beyond that it loses up to 40 us at M = 16.
bool ksplit_fused_shape(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > kFusedMaxM || choose_cfg(M, N, K) != 0) return false;
  const double nk = (double)N * (double)K;
  return M == 1 || (M <= 4 && nk <= 33554432.0) || nk <= 16777216.0;
}

namespace {
template <int kIn>
hipError_t launch_fused_rows(const GemmArgs& args, hipStream_t stream) {
  const dim3 grid((unsigned)((args.N + 15) / 16), 1u);
  if (args.M == 1) {
    hipLaunchKernelGGL((gemm_ksplit_kernel<1, 1, 8, 2, false, kIn, 1>), grid, dim3(8 * 64), 0, stream, args);
  } else if (args.M <= 4) {
    hipLaunchKernelGGL((gemm_ksplit_kernel<1, 1, 8, 2, false, kIn, 4>), grid, dim3(8 * 64), 0, stream, args);
  } else {
    hipLaunchKernelGGL((gemm_ksplit_kernel<1, 1, 8, 2, false, kIn, 8>), grid, dim3(8 * 64), 0, stream, args);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_ksplit_fused(const GemmArgs& args, int x_dtype, hipStream_t stream) {
  if (args.M < 1 || args.M > kFusedMaxM) return hipErrorInvalidValue;
  return x_dtype == kInF16 ? launch_fused_rows<kInF16>(args, stream) : launch_fused_rows<kInBf16>(args, stream);
}

namespace {
template <int TN, int TM, int WAVES, int SLOTS>
hipError_t launch_ksplit_g64(const GemmArgs& args, hipStream_t stream) {
  const dim3 grid((unsigned)((args.N + 16 * TN - 1) / (16 * TN)), (unsigned)((args.M + 16 * TM - 1) / (16 * TM)));
  hipLaunchKernelGGL((gemm_ksplit_kernel<TN, TM, WAVES, SLOTS, false, 0, 16, true>), grid, dim3(WAVES * 64), 0, stream,
                     args);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_ksplit_1x64(const GemmArgs& args, hipStream_t stream) {
  switch (choose_cfg(args.M, args.N, args.K)) {
    case 0: return launch_ksplit_g64<1, 1, 8, 2>(args, stream);
    case 1: return launch_ksplit_g64<1, 2, 8, 2>(args, stream);
    case 2: return launch_ksplit_g64<2, 2, 8, 2>(args, stream);
    case 3: return launch_ksplit_g64<4, 2, 8, 1>(args, stream);
    default: return launch_ksplit_g64<4, 4, 8, 1>(args, stream);
  }
}

hipError_t launch_gemm_ksplit(const GemmArgs& args, hipStream_t stream) {
  switch (choose_cfg(args.M, args.N, args.K)) {
    case 0: return launch_ksplit_cfg<1, 1, 8, 2>(args, stream);
    case 1: return launch_ksplit_cfg<1, 2, 8, 2>(args, stream);
    case 2: return launch_ksplit_cfg<2, 2, 8, 2>(args, stream);
    case 3: return launch_ksplit_cfg<4, 2, 8, 1>(args, stream);
    default: return launch_ksplit_cfg<4, 4, 8, 1>(args, stream);
  }
}

}  // namespace bfp8
