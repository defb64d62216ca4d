// Persistent blockwise FP8 GEMM schedule for gfx950 (large M, MFMA bound).
//
// Role: the large-M schedule of page "lmdeploy/pull/4830", section "Kernel design" (above
// 256 rows a persistent kernel), re-derived for CDNA4. One workgroup per CU walks the 256 x 256
// output tiles of C^T = B . A^T assigned to it (tile bid, bid + grid, ...). Inside a tile the K
// loop is the tiled schedule's 256 x 256 loop: 8 waves of 128 x 64, both operand tiles of a
// 128-wide K block copied into one of two LDS stages by the direct-to-LDS loads, one
// 16x16x128 FP8 MFMA per sub-tile per K block and the promotion acc += P * (As * Bs) two steps
// behind it, so every output is summed in the same order as by that kernel, bit for bit.
//
// What the persistent form adds is the seam between tiles. A one-tile-per-workgroup launch
// pays, per round of tiles, the wait for the first two K blocks (all CUs request at once) and
// then the output step and its burst of C stores with the matrix cores idle. Here, as soon as
// a tile's last block is multiplied:
//   1. the copies of the next tile's first two K blocks are issued (the stages are free);
//   2. the finished tile is converted to 16-bit outputs in registers;
//   3. the wave waits for the copies, which are then the only memory operations in flight
//      (on gfx950 the counter that copies are awaited with also counts stores);
//   4. the finished tile is stored through a small LDS area beside the stages (which already
//      hold the next tile's blocks) in 8-row chunks, so that every store instruction writes whole
//      256-byte row segments (stored straight from the MFMA layout, 64-byte pieces reached memory
//      as 30 % more bytes than C); then the next tile's K loop starts on blocks that have landed,
//      and its first end-of-block wait finds the stores drained into L2.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace bfp8 {

namespace {

constexpr int kPBN = 256, kPBM = 256;  // tile: weight rows x activation rows
constexpr int kPWGN = 2, kPWGM = 4;    // waves along N and M
constexpr int kPWaves = kPWGN * kPWGM;
constexpr int kPWN = kPBN / kPWGN, kPWM = kPBM / kPWGM;  // 128 x 64 per wave
constexpr int kPTN = kPWN / 16, kPTM = kPWM / 16;        // 8 x 4 sub-tiles
constexpr int kPRows = kPBN + kPBM;                       // LDS rows per stage
constexpr int kPStage = kPRows * kBlock;                  // 64 KB
constexpr int kPCopies = kPRows / 8 / kPWaves;            // 1 KB copies per wave per K block

// Tile of virtual workgroup index v (bid + i * grid): each XCD (v % 8; the grid is a multiple
// of 8) owns a contiguous run of the tiles in an M-grouped order, as in the tiled schedule.
__device__ __forceinline__ void persistent_tile(int v, int n_tiles, int m_tiles, int& tn, int& tm) {
  const int total = n_tiles * m_tiles;
  int t = v;
  if (total % 8 == 0) t = (v % 8) * (total / 8) + v / 8;
  constexpr int group_m = 8;
  const int band = group_m * n_tiles;
  const int first_m = (t / band) * group_m;
  const int gm = min(m_tiles - first_m, group_m);
  const int r = t - (t / band) * band;
  tm = first_m + r % gm;
  tn = r / gm;
}

template <bool kF16, bool kBias>
__global__ __launch_bounds__(kPWaves * 64) void gemm_persistent_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2][kPStage];
  __shared__ __attribute__((aligned(16))) float as_lds[2][kPBM];
  // Output staging beside the stages (which hold the next tile's blocks by then): per wave 8 rows
  // of its 128 columns, rows padded by 16 bytes so the writes from the MFMA layout are free of
  // bank conflicts.
  constexpr int kOutRow = kPWN * 2 + 16;
  __shared__ __attribute__((aligned(16))) uint8_t out_lds[kPWaves][8][kOutRow];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = w % kPWGN, wm = w / kPWGN;
  const int M = args.M, N = args.N;
  const int n_tiles = (N + kPBN - 1) / kPBN, m_tiles = (M + kPBM - 1) / kPBM;
  const int total = n_tiles * m_tiles;
  const int KB = args.K / kBlock;  // K % 128 == 0 for this schedule
  // Lane-dependent values used by the K loop are (re)computed at the top of every tile from the
  // lane index taken through a volatile move (lane_here), so that the compiler cannot hoist them
  // out of the tile loop and keep them live through the output step, where the registers are
  // needed for the finished tile.
  auto lane_here = [&]() __attribute__((always_inline)) -> int {
    int l;
    asm volatile("v_mov_b32 %0, %1" : "=v"(l) : "v"(lane));
    return l;
  };
  int r = 0, kc = 0;
  const bool copies_as = w < kPBM / 64;

  // Per-tile copy plan (see the tiled schedule): wave w copies stage rows
  // [w * 8 * kPCopies, ...) in 8-row pieces, lane l of a piece at row prow + l / 8, physical
  // 16-byte column l % 8, loading logical column (l % 8) ^ swizzle(row).
  // A wave's pieces all come from one operand (waves 0-3 weight rows, 4-7 activation rows), so
  // the offset of piece j is computed when it is issued from the wave's first row and two
  // swizzled column offsets (the swizzle of a row depends on its 8-row group's parity), rather
  // than kept in 8 registers through the K loop.
  const int prow_base = w * 8 * kPCopies;
  const bool b_wave = prow_base < kPBN;  // wave-uniform
  int lrow = 0;
  uint32_t colb[2] = {0u, 0u};
  const uint32_t ld_op = (uint32_t)(b_wave ? args.ldb : args.lda);  // operand row stride (bytes)
  const int row_lim = (b_wave ? N : M) - 1;                          // last row of the operand
  int row0 = 0;  // this lane's row of piece 0 (before clamping)
  const uint8_t* bs_row = nullptr;
  int n0 = 0, m0 = 0;
  auto setup_tile = [&](int v) __attribute__((always_inline)) {
    int tn, tm;
    persistent_tile(v, n_tiles, m_tiles, tn, tm);
    n0 = tn * kPBN;
    m0 = tm * kPBM;
    row0 = (b_wave ? n0 + prow_base : m0 + prow_base - kPBN) + lrow;
    bs_row = static_cast<const uint8_t*>(args.bs) + (int64_t)(min(n0 + wn * kPWN, N - 1) / kBlock) * args.ld_bs * 4;
  };
  // Rows past M or N are clamped to the last row (their results are never stored); the operand
  // spans less than 4 GiB, so the offset fits 32 bits.
  auto coff = [&](int j) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)min(row0 + 8 * j, row_lim) * ld_op + colb[j & 1];
  };
  // activation scale of row m0 + 64 w + lane (clamped), for the waves that copy scales
  auto as_voff = [&]() __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)min(m0 + w * 64 + lane, M - 1) * 4u;
  };
  uint32_t stage_lds[2], as_lds_addr[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    stage_lds[i] = lds_addr(&smem[i][0]);
    as_lds_addr[i] = lds_addr(&as_lds[i][0]);
  }
  const uint8_t* asmat = static_cast<const uint8_t*>(args.as);
  auto issue_copies = [&](int buf, int kb) __attribute__((always_inline)) {
    const uint8_t* bsrc = args.b + (int64_t)kb * kBlock;
    const uint8_t* asrc = args.a + (int64_t)kb * kBlock;
    const uint32_t dst = stage_lds[buf] + (uint32_t)(prow_base * kBlock);
#pragma unroll
    for (int j = 0; j < kPCopies; ++j) copy16_to_lds_u(b_wave ? bsrc : asrc, coff(j), dst + (uint32_t)(j * 8 * kBlock));
    if (copies_as) copy4_to_lds_u(asmat + (int64_t)kb * args.ld_as * 4, as_voff(), as_lds_addr[buf] + (uint32_t)(w * 256));
  };
  auto issue_piece = [&](int buf, int kb, int j) __attribute__((always_inline)) {
    const uint8_t* src = b_wave ? args.b + (int64_t)kb * kBlock : args.a + (int64_t)kb * kBlock;
    copy16_to_lds_u(src, coff(j), stage_lds[buf] + (uint32_t)((prow_base + j * 8) * kBlock));
  };
  auto issue_scales = [&](int buf, int kb) __attribute__((always_inline)) {
    if (copies_as) copy4_to_lds_u(asmat + (int64_t)kb * args.ld_as * 4, as_voff(), as_lds_addr[buf] + (uint32_t)(w * 256));
  };
  auto weight_scale = [&](int kb) __attribute__((always_inline)) -> float {
    return ((const __attribute__((address_space(4))) float*)bs_row)[kb];
  };

  uint32_t off_lo = 0, off_hi = 0;
  auto lane_setup = [&]() __attribute__((always_inline)) {
    const int l = lane_here();
    r = l & 15;
    kc = l >> 4;
    lrow = l >> 3;
    colb[0] = (uint32_t)(((l & 7) ^ lds_swizzle(prow_base + lrow)) * 16);
    colb[1] = (uint32_t)(((l & 7) ^ lds_swizzle(prow_base + 8 + lrow)) * 16);
    const int fsw = lds_swizzle(r);
    off_lo = (uint32_t)(r * kBlock + (((2 * kc) ^ fsw) << 4));
    off_hi = (uint32_t)(r * kBlock + (((2 * kc + 1) ^ fsw) << 4));
  };
  auto frag_at = [&](const uint8_t* stage, int row0) __attribute__((always_inline)) -> v8i {
    const v4i lo = *reinterpret_cast<const v4i*>(stage + off_lo + row0 * kBlock);
    const v4i hi = *reinterpret_cast<const v4i*>(stage + off_hi + row0 * kBlock);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto frag_b = [&](const uint8_t* stage, int tn) __attribute__((always_inline)) {
    return frag_at(stage, wn * kPWN + tn * 16);
  };
  auto frag_a = [&](const uint8_t* stage, int tm) __attribute__((always_inline)) {
    return frag_at(stage, kPBN + wm * kPWM + tm * 16);
  };
  auto act_scale = [&](int slot, int tm) __attribute__((always_inline)) -> float {
    return as_lds[slot][wm * kPWM + tm * 16 + r];
  };

  float acc[kPTN][kPTM][4];
  v8i fa[kPTM];
  v8i fb[kPTN];
  float sa[kPTM];
  float bsv;
  constexpr int kSteps = kPTN * kPTM;
  // Refill copy j goes out at step 3j (measured best spacing for this tile in the tiled schedule).
  constexpr int kCopyStride = 3;
  static_assert(kCopyStride * (kPCopies - 1) < kSteps, "every copy of a refill is issued inside the block");

  auto promote = [&](int u, const v4f& pu, float s) __attribute__((always_inline)) {
    const int um = u / kPTN, un = u % kPTN;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[un][um][e] = fmaf(pu[e], s, acc[un][um][e]);
    asm volatile("" : "+v"(acc[un][um][0]), "+v"(acc[un][um][1]), "+v"(acc[un][um][2]), "+v"(acc[un][um][3]));
  };

  // Iteration kb multiplies block kb out of registers, refills stage kb % 2 with block kb + 2
  // and reads block kb + 1's fragments from the other stage, each right after its last use; it
  // ends waiting for block kb + 2 and with a workgroup barrier.
  auto iter = [&](int kb, auto steady_c) __attribute__((always_inline)) {
    constexpr bool kSteady = decltype(steady_c)::value;  // kb + 2 < KB
    const int cslot = kb & 1;
    const int nslot = cslot ^ 1;
    const uint8_t* nstage = &smem[nslot][0];
    const float bs_next = weight_scale(min(kb + 1, KB - 1));
    float sc[kPTM];
#pragma unroll
    for (int tm = 0; tm < kPTM; ++tm) sc[tm] = sa[tm] * bsv;
    if constexpr (kSteady) issue_scales(cslot, kb + 2);
    v4f p1 = {0.f, 0.f, 0.f, 0.f}, p2 = p1;
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      const int tm = t / kPTN, tn = t % kPTN;
      const v4f p = mfma_block(fb[tn], fa[tm]);
      if (t >= 2) promote(t - 2, p2, sc[(t - 2) / kPTN]);
      if constexpr (kSteady) {
#pragma unroll
        for (int j = 0; j < kPCopies; ++j)
          if (t == j * kCopyStride) issue_piece(cslot, kb + 2, j);
      }
      if (tn == kPTN - 1) {
        fa[tm] = frag_a(nstage, tm);
        sa[tm] = act_scale(nslot, tm);
      }
      if (tm == kPTM - 1) fb[tn] = frag_b(nstage, tn);
      __builtin_amdgcn_sched_barrier(0);
      p2 = p1;
      p1 = p;
    }
    promote(kSteps - 2, p2, sc[kPTM - 1]);
    promote(kSteps - 1, p1, sc[kPTM - 1]);
    bsv = bs_next;
    wait_copies();
    lds_barrier();
  };

  // Output registers of the finished tile: per sub-tile (tm, tn), this lane's 4 outputs (row r,
  // columns 4 kc .. 4 kc + 3) as two dwords of 16-bit values.
  uint32_t outw[kPTM][kPTN][2];
  int out_n0 = 0, out_m0 = 0;  // the finished tile's origin
  // (the output steps also take the lane index through lane_here, for the same reason: their
  // lane-dependent addresses must not be kept through the K loop, which has no register to spare)
  auto convert = [&](int tile_n0, int tile_m0) __attribute__((always_inline)) {
    const int kc_here = lane_here() >> 4;
#pragma unroll
    for (int tn = 0; tn < kPTN; ++tn) {
      uint32_t bias_bits[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int nb = tile_n0 + wn * kPWN + tn * 16 + 4 * kc_here + e;  // clamped on tails (not stored)
        bias_bits[e] = kBias ? (uint32_t)args.bias[min(nb, N - 1)] : 0u;
      }
#pragma unroll
      for (int tm = 0; tm < kPTM; ++tm) {
        outw[tm][tn][0] = conv16<kF16, kBias>(acc[tn][tm][0], bias_bits[0]) |
                          (conv16<kF16, kBias>(acc[tn][tm][1], bias_bits[1]) << 16);
        outw[tm][tn][1] = conv16<kF16, kBias>(acc[tn][tm][2], bias_bits[2]) |
                          (conv16<kF16, kBias>(acc[tn][tm][3], bias_bits[3]) << 16);
      }
    }
    out_n0 = tile_n0;
    out_m0 = tile_m0;
  };
  // Stores of the finished tile in 8-row chunks: the lanes holding the chunk's rows write them to
  // the wave's staging rows, then every lane reads back 16 bytes of a row (16 lanes per row, 4
  // rows per pass) and stores them, so each store instruction writes whole row segments.
  uint8_t* const stage_out = &out_lds[w][0][0];
  auto wave_sync = [&]() __attribute__((always_inline)) {
    // the wave's own LDS accesses execute in order; this keeps the compiler from reordering them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  };
  auto store = [&]() __attribute__((always_inline)) {
    const int l = lane_here();
    const int lr = l & 15, lkc = l >> 4;
#pragma unroll
    for (int tm = 0; tm < kPTM; ++tm)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if ((lr >> 3) == half) {
#pragma unroll
          for (int tn = 0; tn < kPTN; ++tn)
            *reinterpret_cast<uint2*>(stage_out + (lr & 7) * kOutRow + (tn * 16 + 4 * lkc) * 2) =
                make_uint2(outw[tm][tn][0], outw[tm][tn][1]);
        }
        wave_sync();
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
          const int row = pass * 4 + (l >> 4), seg = l & 15;
          const uint4 val = *reinterpret_cast<const uint4*>(stage_out + row * kOutRow + seg * 16);
          const int m = out_m0 + wm * kPWM + tm * 16 + half * 8 + row;
          const int n = out_n0 + wn * kPWN + seg * 8;
          if (m < M && n < N) {
            uint16_t* cp = args.c + (int64_t)m * args.ldc + n;
            if (n + 8 <= N) {
              *reinterpret_cast<uint4*>(cp) = val;
            } else {
              const uint32_t wv[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (n + e < N) cp[e] = (uint16_t)(wv[e / 2] >> (16 * (e & 1)));
            }
          }
        }
        wave_sync();
      }
  };

  // Tile body: the K loop of tile v, whose first two blocks have landed; then the next tile's
  // first two blocks go out (if there is one), the finished tile is converted while they
  // travel, and its stores follow the wait for them (that wait also counts stores). Written
  // out once per tile of the workgroup (at most two) rather than as a loop over tiles, which
  // let the compiler keep registers through the K loop that it then had to spill.
  auto tile = [&](int v, bool more) __attribute__((always_inline)) {
    lane_setup();
    lds_barrier();
#pragma unroll
    for (int tm = 0; tm < kPTM; ++tm) {
      fa[tm] = frag_a(&smem[0][0], tm);
      sa[tm] = act_scale(0, tm);
    }
#pragma unroll
    for (int tn = 0; tn < kPTN; ++tn) fb[tn] = frag_b(&smem[0][0], tn);
    bsv = weight_scale(0);
    // every wave has read stage 0 before iteration 0 refills it
    lds_barrier();
#pragma unroll
    for (int tn = 0; tn < kPTN; ++tn)
#pragma unroll
      for (int tm = 0; tm < kPTM; ++tm)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[tn][tm][e] = 0.f;
    int kb = 0;
    for (; kb + 2 < KB; ++kb) iter(kb, std::true_type{});
    for (; kb < KB; ++kb) iter(kb, std::false_type{});
    // No copy is in flight and every wave is done with both stages (the last barrier).
    const int fin_n0 = n0, fin_m0 = m0;
    if (more) {
      setup_tile(v + (int)gridDim.x);
      issue_copies(0, 0);
      issue_copies(1, min(1, KB - 1));
    }
    convert(fin_n0, fin_m0);
    if (more) wait_copies();
    store();
  };

  // Workgroup b computes tile b and, when the grid covers fewer than all tiles, b + grid.
  const int v0 = blockIdx.x, v1 = v0 + (int)gridDim.x;
  if (v0 >= total) return;
  lane_setup();
  setup_tile(v0);
  issue_copies(0, 0);
  issue_copies(1, min(1, KB - 1));
  wait_copies();
  const bool two = v1 < total;  // workgroup-uniform
  tile(v0, two);
  if (two) tile(v1, false);
}

template <bool kF16, bool kBias>
hipError_t launch_persistent_cfg(const GemmArgs& args, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_persistent_kernel<kF16, kBias>), dim3(grid), dim3(kPWaves * 64), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

bool persistent_supported(const GemmArgs& args) {
  // float scales, whole K blocks, bf16 output in 16-byte aligned rows (the fp16 conversion left
  // the compiler two reloads of spilled registers inside the K loop, so fp16 runs tiled)
  return !args.e8 && !args.out_f16 && args.K % kBlock == 0 && (args.ldc & 7) == 0 &&
         (reinterpret_cast<uintptr_t>(args.c) & 15) == 0;
}

int64_t persistent_tiles(int64_t M, int64_t N) { return ((N + kPBN - 1) / kPBN) * ((M + kPBM - 1) / kPBM); }

hipError_t launch_gemm_persistent(const GemmArgs& args, hipStream_t stream) {
  constexpr int64_t kCUs = 256;
  const int64_t tiles = persistent_tiles(args.M, args.N);
  // two tiles per workgroup beyond one round of tiles (one below); a multiple of 8 workgroups,
  // so that a workgroup's two tiles lie in the same XCD's run of the tile order
  const int64_t per_wg = tiles > kCUs ? 2 : 1;
  const unsigned grid = (unsigned)(((tiles + per_wg - 1) / per_wg + 7) / 8 * 8);
  return args.bias ? launch_persistent_cfg<false, true>(args, grid, stream)
                   : launch_persistent_cfg<false, false>(args, grid, stream);
}

}  // namespace bfp8
