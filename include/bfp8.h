/*
 * bfp8 — blockwise-scaled FP8 GEMM for AMD Instinct MI355X (gfx950 / CDNA4).
 *
 * C ABI of libbfp8.so. Every entry point takes plain device pointers, sizes and
 * a HIP stream (passed as void*, NULL = the null stream); no PyTorch or C++
 * types cross this boundary and no exception leaves it.
 *
 * The method (DeepSeek-style blockwise FP8 "W8A8"):
 *   C[m, n] = sum_kb (A_q[m, kb-block] . B_q[n, kb-block]) * As[m, kb] * Bs[n/128, kb]
 * with e4m3fn operands, 1x128 per-token-group activation scales, 128x128 weight
 * block scales, FP32 accumulation and bf16 output. Sources:
 *   - page "prhub.com.cn ... vllm/pull/49932" (torch._scaled_mm block-scale
 *     backend): section "实现拆解" items 2-3 fix the 1x128 activation group and the
 *     128x128 weight block, the column-major (M-major) activation scales and the
 *     call shape _scaled_mm(A, B.t(), scale_a=As, scale_b=Bs.t()); its test
 *     source (section "关键源码片段") fixes e4m3fn operands, fp32 scales of shapes
 *     [M, ceil(K/128)] and [ceil(N/128), ceil(K/128)], bf16 output and the
 *     acceptance metric mean|C - ref| / mean|ref| < 1e-3.
 *   - page "vllm-project/vllm/pull/19085": the dense kernel gemm_fp8_fp8_bf16_nt
 *     ("NT": both operands K-contiguous).
 *   - page "transformers/integrations/deepgemm.py": per_token_cast_to_fp8 with
 *     gran_k = 128 and float32 scale factors (_select_fp8_cast_kwargs), the
 *     caller-allocated output of deepgemm_fp8_fp4_linear, and the M-grouped
 *     contiguous layout (_build_deepgemm_contiguous_layout: 128-row alignment,
 *     one int32 expert id per row, -1 on padding rows).
 *   - page "lmdeploy/pull/4830" (Gluon blocked FP8 GEMM), section "Kernel
 *     design": the schedule is chosen by M (small / mid / large M).
 *
 * Conventions shared by all entry points
 *   - Ownership: the caller allocates and owns every buffer (inputs, outputs,
 *     workspace). The library never allocates, frees or copies between host
 *     and device; it keeps only per-device cached properties and the fixed
 *     staging array of bfp8_linear_noalloc (BFP8_NOALLOC_SCRATCH_BYTES on each
 *     device the library is loaded on, held until the process ends).
 *   - Asynchrony: work is enqueued on `stream`; BFP8_OK means "enqueued".
 *     Errors in the arguments are found on the host before any HIP call and
 *     leave every buffer untouched.
 *   - M == 0 is a valid no-op (BFP8_OK, nothing launched).
 *   - Alignment: every uint8 operand pointer and every row stride in bytes is
 *     a multiple of 16; float pointers are 4-byte aligned; bf16 output
 *     pointers are 2-byte aligned. Violations return BFP8_ERR_MISALIGNED.
 *   - K must be a positive multiple of 16; other K return BFP8_ERR_UNSUPPORTED. The
 *     scale grid has ceil(K/128) K blocks (the pages size it with ceil); when K % 128 != 0
 *     the last block is partial. The GEMMs read operand rows in whole 128-byte blocks, so
 *     lda and ldb must be at least K rounded up to a multiple of 128 (Kp); the bytes between
 *     K and Kp may hold anything (they are zeroed in the kernels' registers).
 *   - Only gfx950 devices are supported (BFP8_ERR_UNSUPPORTED otherwise).
 *   - Size: M, N, K are at most 2^30, and the activation matrix ((M - 1) * lda + Kp
 *     bytes) and each weight matrix ((N - 1) * ldb + Kp bytes) span less than 4 GiB;
 *     larger requests return BFP8_ERR_UNSUPPORTED.
 *   - Determinism: for fixed inputs and sizes every result is bitwise identical
 *     from run to run (fixed reduction orders, no floating-point atomics).
 *   - Thread safety: calls may be made from several host threads; the message
 *     returned by bfp8_last_error_message() is per host thread.
 */
#ifndef BFP8_H_
#define BFP8_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BFP8_ABI_VERSION 15

typedef enum bfp8_status {
  BFP8_OK = 0,
  BFP8_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative or inconsistent size or stride */
  BFP8_ERR_UNSUPPORTED = 2,      /* valid request this library does not implement (K % 16, arch, dtype) */
  BFP8_ERR_MISALIGNED = 3,       /* pointer or stride alignment (see conventions) */
  BFP8_ERR_WORKSPACE = 4,        /* workspace smaller than bfp8_gemm_workspace_bytes() */
  BFP8_ERR_DEVICE = 5,           /* HIP runtime query failed */
  BFP8_ERR_LAUNCH = 6            /* kernel launch failed (message holds hipGetErrorString) */
} bfp8_status_t;

/* Activation dtypes accepted by bfp8_quant_act. */
typedef enum bfp8_in_dtype {
  BFP8_IN_F32 = 0,
  BFP8_IN_BF16 = 1,
  BFP8_IN_F16 = 2
} bfp8_in_dtype_t;

/* GEMM schedules (page "lmdeploy/pull/4830", section "Kernel design": one schedule
 * per M range). AUTO gives M <= 256 to SMALL_M and larger M to TILED; the others force
 * one schedule at any M (for tests and benchmarks). Each schedule is deterministic on
 * its own; the schedules sum the K blocks in different orders, so they agree to FP32
 * rounding, not bitwise. */
typedef enum bfp8_schedule {
  BFP8_SCHED_AUTO = 0,
  BFP8_SCHED_SMALL_M = 1, /* small/mid M: K blocks split across the waves of a workgroup */
  BFP8_SCHED_TILED = 2,   /* LDS-tiled MFMA kernel, one output tile per workgroup */
  BFP8_SCHED_PERSISTENT = 3, /* the tiled schedule, except that launches planned with 256 x 256
                                tiles run a persistent kernel: each workgroup takes two tiles and
                                issues the second tile's first copies before storing the first
                                (float scales, K % 128 == 0, bf16 output in 16-byte aligned rows;
                                otherwise the tiled kernel). Only by override: timed interleaved
                                with the tiled kernel on MI355X it was slower (e.g. 129 vs 120 us
                                at M = 8192, N = K = 4096), so BFP8_SCHED_AUTO never takes it. */
  BFP8_SCHED_COUNT_ = 4
} bfp8_schedule_t;

/* Returns BFP8_ABI_VERSION of the loaded library. */
int bfp8_abi_version(void);

/* Static string naming a status code (never NULL). */
const char* bfp8_status_string(bfp8_status_t status);

/* Why the calling thread's last failing call failed ("" after success). The
 * pointer stays valid until the thread's next bfp8 call. */
const char* bfp8_last_error_message(void);

/*
 * Per-token-group FP8 quantization of activations.
 * Source: page "prhub.com.cn ... vllm/pull/49932", test source
 * (per_token_group_quant_fp8(A, 128, column_major_scales=True)); page
 * "transformers/integrations/deepgemm.py", per_token_cast_to_fp8 with gran_k=128
 * and float32 scale factors.
 *
 * For every row m and group g (columns 128g .. 128g+127):
 *   s        = fl32(max(max_k |x[m,k]|, 1e-10) / 448)      (correctly rounded divide)
 *   q[m,k]   = e4m3fn_RNE(clamp(fl32(x[m,k] / s), -448, 448))
 *   as[g*ld_as + m] = s
 * x is widened to float32 first (exact for bf16).
 *
 *   x       device, [M][ldx] elements of x_dtype, row-major; read only
 *   x_dtype BFP8_IN_F32, BFP8_IN_BF16 or BFP8_IN_F16 (the 16-bit inputs widen to float32 exactly)
 *   M, K    M >= 0, K > 0 and K % 16 == 0 (a last group of K % 128 columns gets its own scale)
 *   ldx     >= K, elements; ldx * sizeof(element) % 16 == 0; x 16-byte aligned
 *   q       device, [M][ldq] bytes (e4m3fn codes); ldq >= K, ldq % 16 == 0; written
 *   as      device, [ceil(K/128)][ld_as] float32, group-major ("column-major" scales:
 *           scale of row m, group g at as[g*ld_as + m]); ld_as >= M; written
 *   stream  hipStream_t or NULL
 * x may not overlap q or as.
 */
bfp8_status_t bfp8_quant_act(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                             uint8_t* q, int64_t ldq, float* as, int64_t ld_as, void* stream);

/* Bytes of device workspace bfp8_gemm needs for this shape under the current schedule
 * (bfp8_set_schedule). Every schedule of this version needs none and returns 0; the
 * argument pair exists so that a schedule with cross-workgroup partial sums can be added
 * without changing the ABI. Contract for a non-zero size: 256-byte aligned, zero-filled
 * before its first use, reusable by later calls ordered after it (same stream), never
 * shared by calls that may run concurrently. bfp8_grouped_gemm_contiguous needs none. */
size_t bfp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * Dense blockwise-scaled FP8 GEMM, NT layout, bf16 output.
 * Source: page "prhub.com.cn ... vllm/pull/49932", section "实现拆解" items 2-3 and
 * the test source (native_w8a8_block_matmul as reference); page
 * "vllm-project/vllm/pull/19085" (gemm_fp8_fp8_bf16_nt); page
 * "transformers/integrations/deepgemm.py" (fp8_fp4_gemm_nt((a, sfa), (b, sfb), out)).
 *
 *   C[m, n] = bf16_RNE( sum_{kb < ceil(K/128)} P_kb[m,n] * as[kb*ld_as + m] * bs[(n/128)*ld_bs + kb] )
 *   P_kb[m, n] = sum_{k = 128 kb}^{min(128 kb + 127, K - 1)} e4m3(a[m*lda + k]) * e4m3(b[n*ldb + k])
 * Each P_kb is accumulated in FP32 by the matrix cores and promoted into an FP32
 * accumulator with the product of the two scales.
 *
 *   a      device, [M][lda] e4m3fn codes (activations), lda >= Kp, 16-byte aligned rows
 *   as     device, [ceil(K/128)][ld_as] float32 activation scales (group-major), ld_as >= M
 *   b      device, [N][ldb] e4m3fn codes (weights, K-contiguous), ldb >= Kp, 16-byte aligned rows
 *   bs     device, [ceil(N/128)][ld_bs] float32 weight block scales, ld_bs >= ceil(K/128)
 *   c      device, [M][ldc] bf16 bit patterns, ldc >= N; written (only columns < N)
 *   M >= 0, N >= 1, K > 0 with K % 16 == 0 (Kp = K rounded up to a multiple of 128)
 *   workspace / workspace_bytes: device scratch of at least
 *          bfp8_gemm_workspace_bytes(M, N, K) bytes under the contract above (may be
 *          NULL when that is 0); BFP8_ERR_WORKSPACE if smaller
 *   stream hipStream_t or NULL
 * Inputs are read only; c may not overlap any input.
 */
bfp8_status_t bfp8_gemm(const uint8_t* a, int64_t lda, const float* as, int64_t ld_as,
                        const uint8_t* b, int64_t ldb, const float* bs, int64_t ld_bs,
                        uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * M-grouped contiguous blockwise FP8 GEMM (mixture-of-experts layers).
 * Source: page "transformers/integrations/deepgemm.py": _build_deepgemm_contiguous_layout
 * (rows of each expert padded to a multiple of 128; per-row int32 expert id, -1 on
 * padding rows), deepgemm_fp8_fp4_experts_forward (m_grouped_fp8_fp4_gemm_nt_contiguous)
 * and DeepGEMM.m_alignment (128).
 *
 * For every row m with g = grouped_layout[m] >= 0:
 *   C[m, n] = the dense product above with b + g*N*ldb and bs + g*ceil(N/128)*ld_bs
 * Rows with grouped_layout[m] == -1 are padding: their A, As and C contents are
 * never used and C rows are not written.
 *
 *   a, as, c, lda, ld_as, ldc  as in bfp8_gemm, with M rows (M % 128 == 0)
 *   b      device, [G][N][ldb] e4m3fn expert weights
 *   bs     device, [G][ceil(N/128)][ld_bs] float32 block scales
 *   grouped_layout device, int32 [M]; contract (not checked on the host: device
 *          data): values in [-1, G), and all non-negative ids within one 128-row
 *          block are equal. A block whose ids are all -1 is skipped; a block whose
 *          largest id is >= G is skipped too (its rows are not written).
 *   G >= 1
 */
bfp8_status_t bfp8_grouped_gemm_contiguous(const uint8_t* a, int64_t lda, const float* as, int64_t ld_as,
                                           const uint8_t* b, int64_t ldb, const float* bs, int64_t ld_bs,
                                           const int32_t* grouped_layout, int32_t G,
                                           uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * bfp8_grouped_gemm_gathered: bfp8_grouped_gemm_contiguous with the activation codes gathered
 * through an index instead of laid out in the padded order (the experts forward quantizes each
 * token once and reads it for each of its experts). Row m of the M-row product reads its codes
 * from row row_src[m] / src_div of a [a_rows][lda]; rows with row_src[m] < 0 read row 0
 * (padding rows: the layout marks them -1, they are not written). Its scales are column m of
 * as, as in bfp8_grouped_gemm_contiguous (bfp8_quant_act_scatter puts them there). With the
 * dispatch, row_src = pair_of_row and src_div = top_k.
 *   a, lda   as in bfp8_gemm for a GEMM of a_rows rows
 *   as, ld_as  device, [ceil(K/128)][ld_as] float32, ld_as >= M: scales of the product's rows
 *   row_src  device, int32 [M], 4-byte aligned; entries -1 or in [0, a_rows * src_div)
 *            (device data, not checked)
 *   src_div  >= 1
 *   b, ldb, bs, ld_bs, grouped_layout, G, c, ldc, M, N, K  as in bfp8_grouped_gemm_contiguous
 * The product equals bfp8_grouped_gemm_contiguous on the gathered codes, bit for bit. Float
 * scales only; no workspace.
 */
bfp8_status_t bfp8_grouped_gemm_gathered(const uint8_t* a, int64_t lda, const float* as, int64_t ld_as,
                                         int64_t a_rows, const int32_t* row_src, int32_t src_div,
                                         const uint8_t* b, int64_t ldb, const float* bs, int64_t ld_bs,
                                         const int32_t* grouped_layout, int32_t G, uint16_t* c, int64_t ldc,
                                         int64_t M, int64_t N, int64_t K, void* stream);

/* Bytes of device workspace bfp8_linear needs (0 when M == 0): the quantized activations
 * (M * K bytes), their scales (4 * M * K / 128 bytes) and the GEMM's workspace, each part
 * 256-byte aligned. The workspace contract of bfp8_gemm applies. */
size_t bfp8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * End-to-end FP8 linear layer, bf16 in and out (page "transformers/integrations/deepgemm.py",
 * deepgemm_fp8_fp4_linear): the activations are quantized per 1x128 group exactly as
 * bfp8_quant_act does, multiplied with the FP8 weight as bfp8_gemm does into a bf16 result,
 * and, when a bias is given, the bias is added to that bf16 result:
 *   out[m, n] = bf16(float(bf16(C[m, n])) + float(bias[n]))   (bias NULL: out = bf16(C)),
 * which is the page's output.add_(bias) on a bf16 output; with fp16 activations the output,
 * the bias and both roundings are fp16 (the page's output dtype follows the input).
 *   x      [M][ldx] activations, x_dtype BFP8_IN_BF16 or BFP8_IN_F16
 *   b, bs  as for bfp8_gemm (weights [N][ldb] e4m3, scales [ceil(N/128)][ld_bs])
 *   bias   NULL or [N] of x's dtype, 2-byte aligned
 *   c      [M][ldc] output of x's dtype
 *   workspace / workspace_bytes: at least bfp8_linear_workspace_bytes(M, N, K) bytes,
 *          256-byte aligned (BFP8_ERR_WORKSPACE if smaller); it holds the quantized
 *          activations, which the call overwrites.
 * Two kernels are enqueued on stream: the quantizer, then the GEMM with the bias in its
 * output conversion; except where bfp8_linear_fuses(M, N, K, ldx) is 1 (small M), where one
 * GEMM kernel quantizes the activations itself, with the same codes and scales bit for bit,
 * and the workspace is not touched. Validation, ownership and errors as for bfp8_quant_act
 * and bfp8_gemm.
 */
bfp8_status_t bfp8_linear(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                          const uint8_t* b, int64_t ldb, const float* bs, int64_t ld_bs,
                          const uint16_t* bias, uint16_t* c, int64_t ldc, int64_t N,
                          void* workspace, size_t workspace_bytes, void* stream);

/* 1 if bfp8_linear (and bfp8_linear_noalloc) with these sizes enqueues one kernel that
 * quantizes the activations inside the GEMM, else 0. That kernel runs on the K-split
 * schedule's 16 x 16 tile (under the current bfp8_set_schedule override) and every workgroup
 * quantizes all M rows itself, which is faster than a separate quantizer launch only at
 * small sizes: M == 1, or M <= 4 with N * K <= 2^25, or M <= 8 with N * K <= 2^24; and the
 * activation rows must be addressable with 32-bit offsets ((M - 1) * ldx * 2 +
 * 2 * ceil(K/128) * 128 < 2^32). Host arithmetic only. */
int bfp8_linear_fuses(int64_t M, int64_t N, int64_t K, int64_t ldx);

/* Size of the device array that bfp8_linear_noalloc stages the quantized activations in. */
#define BFP8_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * bfp8_linear without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The
 * same computation and kernels as bfp8_linear, bit for bit; the quantized activations are
 * staged in a file-scope device array of BFP8_NOALLOC_SCRATCH_BYTES bytes that every device
 * holds once the library is loaded (its address is looked up once per device, on the first
 * call on that device). Nothing is allocated or freed by the call.
 *   Limit: the staging must fit the array, i.e. bfp8_linear_workspace_bytes(M, N, K) <=
 *          BFP8_NOALLOC_SCRATCH_BYTES (e.g. M = 2048 at K <= 30720); larger layers return
 *          BFP8_ERR_UNSUPPORTED (checked on the host before any HIP call) and should call
 *          bfp8_linear with a workspace.
 *   Sharing: all calls on one device share its array and leave their staging in it (no part
 *          of it needs clearing: each call writes every byte it reads). Calls that overlap in
 *          time on one device (different streams or host threads without ordering) race on it;
 *          calls ordered on one stream do not.
 * Arguments, validation and errors otherwise as bfp8_linear.
 */
bfp8_status_t bfp8_linear_noalloc(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                  const uint8_t* b, int64_t ldb, const float* bs, int64_t ld_bs,
                                  const uint16_t* bias, uint16_t* c, int64_t ldc, int64_t N, void* stream);

/*
 * bfp8_gemm with an fp16 output: C[m, n] = fp16(sum_kb P_kb * As * Bs), rounded to nearest even
 * once (overflow to infinity). Everything else as bfp8_gemm. For the linear layer's fp16 form
 * (page "transformers/integrations/deepgemm.py": the output dtype follows the input).
 */
bfp8_status_t bfp8_gemm_f16(const uint8_t* a, int64_t lda, const float* as, int64_t ld_as,
                            const uint8_t* b, int64_t ldb, const float* bs, int64_t ld_bs,
                            uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * 1x64 activation groups with 128x64 weight blocks (the next block-scale layouts named on page
 * "prhub.com.cn ... vllm/pull/49932", section "风险与影响"; the same definitions over K blocks
 * of 64, weight blocks staying 128 rows tall):
 *
 * bfp8_quant_act_1x64: as bfp8_quant_act with groups of 64 columns: the scale of row m, group
 * g = k / 64 is written to as[g * ld_as + m] (float32, ceil(K/64) groups; the last may be
 * shorter). Same arguments, validation and errors.
 *
 * bfp8_gemm_1x64: C[m, n] = bf16(sum_g P_g * As[g][m] * Bs[n / 128][g]), P_g the e4m3 dot
 * product over the 64 columns of group g. as is [ceil(K/64)][ld_as] (ld_as >= M), bs is
 * [ceil(N/128)][ld_bs] with ld_bs >= ceil(K/64); a, b, c and every other rule as bfp8_gemm
 * (operand rows of whole 128-byte blocks). No workspace. Small M runs the K-split kernel (two
 * 16x16x128 matrix-core products per 128-wide K block, each on one group with the other half
 * zeroed); from 64 output tiles of 256 x 128 on, a tiled kernel with one 32x32x64 product per
 * 64-wide group (bfp8_set_schedule forces either). Both round each group's sum once; the float32
 * accumulation error is bounded as for bfp8_gemm with K/64 promotions instead of K/128.
 */
bfp8_status_t bfp8_quant_act_1x64(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                  uint8_t* q, int64_t ldq, float* as, int64_t ld_as, void* stream);
bfp8_status_t bfp8_gemm_1x64(const uint8_t* a, int64_t lda, const float* as, int64_t ld_as,
                             const uint8_t* b, int64_t ldb, const float* bs, int64_t ld_bs,
                             uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * UE8M0 (power-of-two) scale factors (page "transformers/integrations/deepgemm.py":
 * _ceil_to_ue8m0, the use_ue8m0 recipe of _select_fp8_cast_kwargs, and float8_e8m0fnu scales
 * in _coerce_sf_for_kernel). A scale is given by its UE8M0 code, one byte e standing for
 * 2^(e - 127) (torch.float8_e8m0fnu); code 255 (NaN) is outside the contract.
 *
 * bfp8_quant_act_ue8m0: as bfp8_quant_act, but the group's float32 scale
 * fl32(max(amax, 1e-10) / 448) is rounded up to a power of two by adding 2^23 - 1 to its bit
 * pattern and clearing the mantissa bits; the group is divided by it (exactly) and its code
 * is written to as[(k/128) * ld_as + m] (one byte; no alignment needed).
 */
bfp8_status_t bfp8_quant_act_ue8m0(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                   uint8_t* q, int64_t ldq, uint8_t* as, int64_t ld_as, void* stream);

/*
 * bfp8_gemm and bfp8_grouped_gemm_contiguous with UE8M0 scale codes:
 *   C[m, n] = bf16( sum_kb P_kb[m, n] * 2^(as[kb][m] - 127) * 2^(bs[n/128][kb] - 127) ).
 * Same operands, layouts, workspace and errors as the float-scale calls, plus: as and bs
 * 4-byte aligned and ld_as, ld_bs multiples of 4 (BFP8_ERR_MISALIGNED otherwise), since the
 * kernels read the codes four at a time. The scales are applied by gfx950's scaled MFMA,
 * which also accumulates the K blocks in its FP32 accumulator, so there is no separate
 * promotion step; the sum is the matrix core's (within 2^-17 * (K/128 + 1) of the sum of
 * absolute block terms, on top of the float-scale path's error, see the design notes).
 */
bfp8_status_t bfp8_gemm_ue8m0(const uint8_t* a, int64_t lda, const uint8_t* as, int64_t ld_as,
                              const uint8_t* b, int64_t ldb, const uint8_t* bs, int64_t ld_bs,
                              uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                              void* workspace, size_t workspace_bytes, void* stream);
bfp8_status_t bfp8_grouped_gemm_contiguous_ue8m0(const uint8_t* a, int64_t lda, const uint8_t* as, int64_t ld_as,
                                                 const uint8_t* b, int64_t ldb, const uint8_t* bs, int64_t ld_bs,
                                                 const int32_t* grouped_layout, int32_t G,
                                                 uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Mixture-of-experts chain around the M-grouped GEMM (page "transformers/integrations/deepgemm.py":
 * _dispatch_routed_input, _build_deepgemm_contiguous_layout, deepgemm_fp8_fp4_experts_forward,
 * _combine_routed_output). S = T * top_k (token, expert) pairs; pair p = t * top_k + j.
 *
 * bfp8_moe_padded_rows: rows of the padded buffer, the page's upper bound S + min(S, E) * (align - 1)
 * rounded up to a multiple of align (known on the host, no device-to-host sync).
 *
 * bfp8_moe_dispatch: for topk_ids [S] (int32; ids outside [0, E) are sentinels: placed nowhere)
 * writes, on stream:
 *   row_of_pair [S]     the pair's row in the padded buffer (-1 for a sentinel),
 *   pair_of_row [rows]  the pair in each row (-1 on padding),
 *   layout [rows]       each row's expert id, -1 on padding (the grouped GEMM's layout),
 *   expert_start [E+1]  expert e owns rows [expert_start[e], expert_start[e] + count_e), blocks
 *                       aligned to align and in expert order; expert_start[E] = rows in use.
 * Inside an expert the pairs keep their index order (deterministic). 1 <= E <= 1024,
 * 1 <= align <= 4096. workspace: bfp8_moe_dispatch_workspace_bytes(S, E) bytes, 4-byte aligned
 * (scratch, overwritten).
 */
int64_t bfp8_moe_padded_rows(int64_t S, int32_t E, int32_t align);
size_t bfp8_moe_dispatch_workspace_bytes(int64_t S, int32_t E);
bfp8_status_t bfp8_moe_dispatch(const int32_t* topk_ids, int64_t S, int32_t E, int32_t align,
                                int32_t* row_of_pair, int32_t* pair_of_row, int32_t* layout,
                                int32_t* expert_start, void* workspace, size_t workspace_bytes, void* stream);

/*
 * bfp8_quant_act_gather: bfp8_quant_act of a gathered matrix: output row m (of M) quantizes input
 * row row_src[m] / src_div of x [src_rows][ldx]; rows with row_src[m] < 0 are not written (with
 * the dispatch: row_src = pair_of_row, src_div = top_k, so row m holds its pair's token).
 * Entries must be -1 or below src_rows * src_div (device data, not checked).
 */
bfp8_status_t bfp8_quant_act_gather(const void* x, int x_dtype, int64_t src_rows, int64_t K, int64_t ldx,
                                    const int32_t* row_src, int32_t src_div, int64_t M, uint8_t* q,
                                    int64_t ldq, float* as, int64_t ld_as, void* stream);

/*
 * bfp8_quant_act_scatter: bfp8_quant_act of x [M][ldx] (codes into q row m), with each group's
 * scale written to the columns scale_dst[m * scale_fan + j] (j < scale_fan) that are not
 * negative, instead of column m: as[g * ld_as + scale_dst[m * scale_fan + j]]. With the
 * dispatch (scale_dst = row_of_pair, scale_fan = top_k) each token is quantized once and its
 * scales land at its padded rows, ready for bfp8_grouped_gemm_gathered. Entries of scale_dst
 * must be -1 or below ld_as (device data, not checked); x_dtype BFP8_IN_F32, BFP8_IN_BF16 or
 * BFP8_IN_F16; other arguments and checks as in bfp8_quant_act (ld_as >= M).
 */
bfp8_status_t bfp8_quant_act_scatter(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                                     int64_t ldq, float* as, int64_t ld_as, const int32_t* scale_dst,
                                     int32_t scale_fan, void* stream);

/*
 * bfp8_swiglu_quant: the gate activation fused with the second quantization. Row m of
 * proj [M][ldp] (bf16; gate in columns [0, I), up in [I, 2I)) gives
 *   h = bf16( bf16(silu(gate)) * up ),  silu(x) = x / (1 + exp(-x)) rounded once to bf16,
 * quantized per 1x128 group exactly as bfp8_quant_act does into q [M][ldq] and
 * as[(i/128) * ld_as + m]. Rows whose layout entry is -1 are skipped (layout may be NULL).
 * I a multiple of 128; proj and q rows 16-byte aligned.
 */
bfp8_status_t bfp8_swiglu_quant(const uint16_t* proj, int64_t M, int64_t I, int64_t ldp, const int32_t* layout,
                                uint8_t* q, int64_t ldq, float* as, int64_t ld_as, void* stream);

/*
 * bfp8_swiglu: the gate activation of bfp8_swiglu_quant without the quantization:
 * h[m][i] = bf16( bf16(silu(gate)) * up ) as bf16 into h [M][ldh], the same values the fused
 * call quantizes (silu rounded once to bf16, the product rounded once). Rows whose layout entry
 * is -1 are not written (layout may be NULL). I a multiple of 128; proj and h rows 16-byte
 * aligned. For a consumer that takes h in bf16, and to inspect the activation.
 */
bfp8_status_t bfp8_swiglu(const uint16_t* proj, int64_t M, int64_t I, int64_t ldp, const int32_t* layout, uint16_t* h,
                          int64_t ldh, void* stream);

/*
 * bfp8_moe_combine: y[t, :] = bf16( sum_j bf16(out[row_of_pair[p], :] * bf16(topk_weights[p])) ),
 * p = t * top_k + j, the sum in float32 in order j; pairs with row -1 add nothing (their rows
 * are never read). out [rows][ldo], y [T][ldy] bf16 with 16-byte aligned rows; H % 8 == 0.
 */
bfp8_status_t bfp8_moe_combine(const uint16_t* out, int64_t ldo, const int32_t* row_of_pair,
                               const float* topk_weights, int64_t T, int32_t top_k, int64_t H, uint16_t* y,
                               int64_t ldy, void* stream);

/*
 * bfp8_moe_forward: the FP8 experts forward of the page, end to end on stream: dispatch (align
 * 128), gathered quantization of hidden [T][ldh] (bf16), grouped GEMM with
 *   w_up [E][2I][H] e4m3, s_up [E][2I/128][H/128] float32 (row stride H, H/128),
 * SwiGLU + quantization, grouped GEMM with
 *   w_down [E][H][I] e4m3, s_down [E][H/128][I/128] float32 (row stride I, I/128),
 * and the weighted top-k combine into y [T][ldy] bf16. topk_ids / topk_weights are [T][top_k]
 * (int32 / float32). H and I are multiples of 128, 1 <= E <= 1024. workspace:
 * bfp8_moe_forward_workspace_bytes(T, top_k, E, H, I) bytes, 256-byte aligned; it holds the
 * layout and every intermediate (overwritten). Errors and validation as for the calls above;
 * nothing is launched unless every step's arguments are valid.
 */
size_t bfp8_moe_forward_workspace_bytes(int64_t T, int32_t top_k, int32_t E, int64_t H, int64_t I);
bfp8_status_t bfp8_moe_forward(const uint16_t* hidden, int64_t T, int64_t H, int64_t ldh, const int32_t* topk_ids,
                               const float* topk_weights, int32_t top_k, int32_t E, const uint8_t* w_up,
                               const float* s_up, const uint8_t* w_down, const float* s_down, int64_t I,
                               uint16_t* y, int64_t ldy, void* workspace, size_t workspace_bytes, void* stream);

/*
 * NN expert weights (page "transformers/integrations/deepgemm.py": grouped_fp8_fp4_matmul_nn for
 * experts stored transposed, [E, K, N]). The grouped GEMM reads NT weights; NN weights are
 * converted once (they are static) with:
 *   bfp8_transpose_weights: dst[e][n][k] = src[e][k][n], src [E][K][ld_src] (ld_src >= N),
 *                           dst [E][N][ld_dst] (ld_dst >= K), bytes; no overlap.
 *   bfp8_transpose_scales:  dst[e][c][r] = src[e][r][c] for contiguous float32 [E][R][C]
 *                           (NN scales [E][K/128][ceil(N/128)] -> [E][ceil(N/128)][K/128]).
 */
bfp8_status_t bfp8_transpose_weights(const uint8_t* src, int64_t E, int64_t K, int64_t N, int64_t ld_src,
                                     uint8_t* dst, int64_t ld_dst, void* stream);
bfp8_status_t bfp8_transpose_scales(const float* src, int64_t E, int64_t R, int64_t C, float* dst, void* stream);

/*
 * Coarser scales on the block kernels (page "vllm/pull/19085", the review thread on models
 * quantized per tensor: their scales are expanded to the block shape). A per-tensor or
 * per-token scale is constant over every 1x128 activation group and 128x128 weight block, so
 * the GEMMs on the expanded grids compute the per-tensor / per-token FP8 product exactly as
 * defined: C[m][n] = bf16(s_a[m] * s_b * sum_k A[m][k] B[n][k]). A per-output-channel weight
 * scale changes inside a 128-row block and has no block form (not offered).
 *   bfp8_expand_act_scales:   as[g * ld_as + m] = s[m * s_stride] for m < M, g < ceil(K/128):
 *                             s_stride 1 for per-token scales s[M], 0 for one per-tensor scale.
 *                             as is the group-major grid bfp8_gemm reads (ld_as >= M).
 *   bfp8_expand_weight_scale: bs[j * ld_bs + kb] = s[0] for j < ceil(N/128), kb < ceil(K/128)
 *                             (ld_bs >= ceil(K/128)).
 * s, as and bs are device float32 arrays, 4-byte aligned; M = 0 is a no-op. Errors: as for the
 * calls above; the expansion runs on stream, ordered with the GEMMs that read it.
 */
bfp8_status_t bfp8_expand_act_scales(const float* s, int64_t s_stride, int64_t M, int64_t K, float* as,
                                     int64_t ld_as, void* stream);
bfp8_status_t bfp8_expand_weight_scale(const float* s, int64_t N, int64_t K, float* bs, int64_t ld_bs,
                                       void* stream);

/* Process-wide schedule override for bfp8_gemm (tests and benchmarks):
 * BFP8_SCHED_AUTO restores the automatic choice. Returns BFP8_ERR_INVALID_ARGUMENT
 * for an unknown value. The grouped GEMM always uses the tiled schedule. */
bfp8_status_t bfp8_set_schedule(int schedule);
int bfp8_get_schedule(void);

/* The schedule bfp8_gemm would run for this shape under the current override. */
int bfp8_gemm_schedule_for(int64_t M, int64_t N, int64_t K);

#ifdef __cplusplus
}
#endif

#endif /* BFP8_H_ */
