// C ABI of libbfp8 (declared in include/bfp8.h): argument validation, device
// check, schedule choice and launch. No allocation, no host<->device copies.
//
// Validation happens entirely on the host before any HIP call, so a rejected
// call touches no buffer; each rejection states its reason through
// bfp8_last_error_message() (the "can_implement returns an explicit reason"
// contract of page "prhub.com.cn ... vllm/pull/49932", section "实现拆解" item 2).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "bfp8.h"
#include "launch.h"

namespace {

thread_local std::string g_message;
std::atomic<int> g_schedule{BFP8_SCHED_AUTO};

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

bfp8_status_t fail(bfp8_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_message = buf;
  return st;
}

bfp8_status_t ok() {
  g_message.clear();
  return BFP8_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // keeps every in-kernel row index in int32
constexpr int64_t kMaxOperandSpan = ((int64_t)1 << 32) - 1;  // in-kernel copy offsets are 32-bit

// Device check: the current device must be a gfx950. Cached per device id.
bfp8_status_t check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BFP8_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(BFP8_ERR_DEVICE, "device id %d out of range", dev);
  int st = g_arch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(BFP8_ERR_DEVICE, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_release);
    if (st == 2) return fail(BFP8_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev,
                             prop.gcnArchName);
  }
  if (st == 2) return fail(BFP8_ERR_UNSUPPORTED, "device %d is not a gfx950", dev);
  return BFP8_OK;
}

bfp8_status_t launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BFP8_ERR_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// Shared checks of the dense and grouped GEMM arguments; e8: the scales are UE8M0 codes.
bfp8_status_t check_gemm_args(const uint8_t* a, int64_t lda, const void* as, int64_t ld_as, const uint8_t* b,
                              int64_t ldb, const void* bs, int64_t ld_bs, uint16_t* c, int64_t ldc, int64_t M,
                              int64_t N, int64_t K, void* workspace, size_t workspace_bytes, bool grouped,
                              bool e8 = false) {
  if (M < 0) return fail(BFP8_ERR_INVALID_ARGUMENT, "M = %lld is negative", (long long)M);
  if (N < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "N = %lld must be >= 1", (long long)N);
  if (K < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "K = %lld must be >= 1", (long long)K);
  if (K % 16 != 0)
    return fail(BFP8_ERR_UNSUPPORTED, "K = %lld is not a multiple of 16 (16-byte operand pieces)", (long long)K);
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return fail(BFP8_ERR_UNSUPPORTED, "M, N and K must each be at most 2^30");
  // Rows are read in whole 128-byte K blocks; with K % 128 != 0 the last block's bytes past K
  // are read (and masked), so every row must hold ceil(K/128) * 128 bytes.
  const int64_t Kp = (K + bfp8::kBlock - 1) / bfp8::kBlock * bfp8::kBlock;
  if (!b || !bs) return fail(BFP8_ERR_INVALID_ARGUMENT, "b and bs must not be NULL");
  if (M > 0 && (!a || !as || !c)) return fail(BFP8_ERR_INVALID_ARGUMENT, "a, as and c must not be NULL when M > 0");
  if (lda < Kp)
    return fail(BFP8_ERR_INVALID_ARGUMENT, "lda = %lld < K rounded up to 128 = %lld", (long long)lda, (long long)Kp);
  if (ldb < Kp)
    return fail(BFP8_ERR_INVALID_ARGUMENT, "ldb = %lld < K rounded up to 128 = %lld", (long long)ldb, (long long)Kp);
  if (ld_as < M) return fail(BFP8_ERR_INVALID_ARGUMENT, "ld_as = %lld < M = %lld", (long long)ld_as, (long long)M);
  if (workspace && !aligned(workspace, 256))
    return fail(BFP8_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (ld_bs < Kp / bfp8::kBlock)
    return fail(BFP8_ERR_INVALID_ARGUMENT, "ld_bs = %lld < ceil(K/128) = %lld", (long long)ld_bs,
                (long long)(Kp / bfp8::kBlock));
  if (ldc < N) return fail(BFP8_ERR_INVALID_ARGUMENT, "ldc = %lld < N = %lld", (long long)ldc, (long long)N);
  if (lda % 16 || ldb % 16) return fail(BFP8_ERR_MISALIGNED, "lda and ldb must be multiples of 16 bytes");
  if (!aligned(a, 16) || !aligned(b, 16)) return fail(BFP8_ERR_MISALIGNED, "a and b must be 16-byte aligned");
  if (!aligned(as, 4) || !aligned(bs, 4)) return fail(BFP8_ERR_MISALIGNED, "as and bs must be 4-byte aligned");
  if (e8 && (ld_as % 4 || ld_bs % 4))
    return fail(BFP8_ERR_MISALIGNED, "UE8M0 scale rows: ld_as and ld_bs must be multiples of 4 (codes are read as dwords)");
  if (!aligned(c, 2)) return fail(BFP8_ERR_MISALIGNED, "c must be 2-byte aligned");
  // The kernels address a row inside A, and inside one weight matrix of B, with a 32-bit
  // byte offset from the operand's base.
  if ((N - 1) * ldb + Kp > kMaxOperandSpan || (M > 0 && (M - 1) * lda + Kp > kMaxOperandSpan))
    return fail(BFP8_ERR_UNSUPPORTED, "A (M x lda) and each weight matrix (N x ldb) must span less than 4 GiB");
  // One workgroup per output tile, and the smallest tile (64 activation rows x 128 weight rows)
  // must leave the tile count within a 32-bit grid.
  if (((M + 63) / 64) * ((N + 127) / 128) > (int64_t)INT32_MAX)
    return fail(BFP8_ERR_UNSUPPORTED, "M x N = %lld x %lld has more output tiles than one launch grid holds",
                (long long)M, (long long)N);
  const size_t need = grouped ? 0 : bfp8_gemm_workspace_bytes(M, N, K);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(BFP8_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  return BFP8_OK;
}

// Arguments of the activation quantizer (no device access).
bfp8_status_t check_quant_args(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, const uint8_t* q,
                               int64_t ldq, const void* as, int64_t ld_as, bool e8 = false) {
  if (x_dtype != BFP8_IN_F32 && x_dtype != BFP8_IN_BF16 && x_dtype != BFP8_IN_F16)
    return fail(BFP8_ERR_UNSUPPORTED, "x_dtype %d is not BFP8_IN_F32, BFP8_IN_BF16 or BFP8_IN_F16", x_dtype);
  if (M < 0) return fail(BFP8_ERR_INVALID_ARGUMENT, "M = %lld is negative", (long long)M);
  if (K < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "K = %lld must be >= 1", (long long)K);
  if (K % 16 != 0) return fail(BFP8_ERR_UNSUPPORTED, "K = %lld is not a multiple of 16", (long long)K);
  if (M > kMaxDim || K > kMaxDim) return fail(BFP8_ERR_UNSUPPORTED, "M and K must each be at most 2^30");
  if (M == 0) return ok();
  if (!x || !q || !as) return fail(BFP8_ERR_INVALID_ARGUMENT, "x, q and as must not be NULL");
  if (ldx < K) return fail(BFP8_ERR_INVALID_ARGUMENT, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  if (ldq < K) return fail(BFP8_ERR_INVALID_ARGUMENT, "ldq = %lld < K = %lld", (long long)ldq, (long long)K);
  if (ld_as < M) return fail(BFP8_ERR_INVALID_ARGUMENT, "ld_as = %lld < M = %lld", (long long)ld_as, (long long)M);
  const int64_t esize = x_dtype == BFP8_IN_F32 ? 4 : 2;
  if ((ldx * esize) % 16 || ldq % 16) return fail(BFP8_ERR_MISALIGNED, "row strides must be multiples of 16 bytes");
  if (!aligned(x, 16) || !aligned(q, 16)) return fail(BFP8_ERR_MISALIGNED, "x and q must be 16-byte aligned");
  if (!e8 && !aligned(as, 4)) return fail(BFP8_ERR_MISALIGNED, "as must be 4-byte aligned");
  return ok();
}

// Workspace of the linear layer: the codes q [M][K] at offset 0, the scales As [K/128][M]
// after them, then the GEMM's own workspace; each part 256-byte aligned.
struct LinearLayout {
  size_t as_off, gemm_off, total;
};
LinearLayout linear_layout(int64_t M, int64_t N, int64_t K);

// Schedule by shape (the M ranges of page "lmdeploy/pull/4830", section "Kernel design",
// decided here by predicted time): above kSmallMaxM rows the tiled schedule; below, the
// K-split one unless the tiled one is predicted at least 10 % faster. That happens for wide
// weights at M of 64 and more (the hidden-5120 gate+up projection, N = 51200: 2.2x at M = 128),
// where the K-split copies re-read every weight strip once per 32 or 64 activation rows.
int choose_schedule(int64_t M, int64_t N, int64_t K) {
  const int forced = g_schedule.load(std::memory_order_relaxed);
  if (forced != BFP8_SCHED_AUTO) return forced;
  if (M > bfp8::kSmallMaxM) return BFP8_SCHED_TILED;
  return bfp8::tiled_time_us(M, N, K) < 0.9 * bfp8::ksplit_time_us(M, N, K) ? BFP8_SCHED_TILED : BFP8_SCHED_SMALL_M;
}

}  // namespace

extern "C" {

int bfp8_abi_version(void) { return BFP8_ABI_VERSION; }

const char* bfp8_status_string(bfp8_status_t status) {
  switch (status) {
    case BFP8_OK: return "BFP8_OK";
    case BFP8_ERR_INVALID_ARGUMENT: return "BFP8_ERR_INVALID_ARGUMENT";
    case BFP8_ERR_UNSUPPORTED: return "BFP8_ERR_UNSUPPORTED";
    case BFP8_ERR_MISALIGNED: return "BFP8_ERR_MISALIGNED";
    case BFP8_ERR_WORKSPACE: return "BFP8_ERR_WORKSPACE";
    case BFP8_ERR_DEVICE: return "BFP8_ERR_DEVICE";
    case BFP8_ERR_LAUNCH: return "BFP8_ERR_LAUNCH";
  }
  return "BFP8_UNKNOWN_STATUS";
}

const char* bfp8_last_error_message(void) { return g_message.c_str(); }

bfp8_status_t bfp8_quant_act(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq,
                             float* as, int64_t ld_as, void* stream) {
  bfp8_status_t st = check_quant_args(x, x_dtype, M, K, ldx, q, ldq, as, ld_as);
  if (st != BFP8_OK || M == 0) return st;
  st = check_device();
  if (st != BFP8_OK) return st;
  return launched(bfp8::launch_quant_act(x, x_dtype, M, K, ldx, q, ldq, as, ld_as, false, (hipStream_t)stream),
                  "quant_act");
}

bfp8_status_t bfp8_quant_act_ue8m0(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                                   int64_t ldq, uint8_t* as, int64_t ld_as, void* stream) {
  bfp8_status_t st = check_quant_args(x, x_dtype, M, K, ldx, q, ldq, as, ld_as, true);
  if (st != BFP8_OK || M == 0) return st;
  st = check_device();
  if (st != BFP8_OK) return st;
  return launched(bfp8::launch_quant_act(x, x_dtype, M, K, ldx, q, ldq, as, ld_as, true, (hipStream_t)stream),
                  "quant_act_ue8m0");
}

size_t bfp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 16 != 0) return 0;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
  if (choose_schedule(M, N, K) != BFP8_SCHED_TILED) return 0;
  return bfp8::plan_tiled(M, N, K).workspace_bytes;
}

}  // extern "C"

namespace {

// Launch the dense GEMM (arguments already validated) with the schedule for this shape.
bfp8_status_t launch_dense(const uint8_t* a, int64_t lda, const void* as, int64_t ld_as, const uint8_t* b,
                           int64_t ldb, const void* bs, int64_t ld_bs, const uint16_t* bias, uint16_t* c,
                           int64_t ldc, int64_t M, int64_t N, int64_t K, void* workspace, void* stream,
                           bool e8 = false, bool out_f16 = false) {
  const bfp8::GemmArgs args{a,      lda,    as,     ld_as,   b, ldb, bs, ld_bs, c,
                            ldc,    (int)M, (int)N, (int)K,  nullptr, 1, bias, e8, out_f16};
  const int sched = choose_schedule(M, N, K);
  if (sched == BFP8_SCHED_SMALL_M) return launched(bfp8::launch_gemm_ksplit(args, (hipStream_t)stream), "gemm_ksplit");
  return launched(bfp8::launch_gemm_tiled(args, workspace, (hipStream_t)stream, sched == BFP8_SCHED_PERSISTENT),
                  "gemm_tiled");
}

LinearLayout linear_layout(int64_t M, int64_t N, int64_t K) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  LinearLayout L;
  const size_t kp = (size_t)((K + bfp8::kBlock - 1) / bfp8::kBlock);  // K blocks (the last may be partial)
  L.as_off = up((size_t)M * kp * bfp8::kBlock);  // codes in rows of whole 128-byte blocks
  L.gemm_off = L.as_off + up((size_t)4 * (size_t)M * kp);
  L.total = L.gemm_off + bfp8_gemm_workspace_bytes(M, N, K);
  return L;
}

}  // namespace

namespace {

// Whether the linear layer takes the one-launch path (bfp8_linear_fuses). The kernel's copies
// address the activation rows with a 32-bit byte offset, like A's.
bool linear_fuses(int64_t M, int64_t N, int64_t K, int64_t ldx) {
  if (M < 1 || N < 1 || K < 1 || K % 16 || ldx < K || M > kMaxDim || N > kMaxDim || K > kMaxDim) return false;
  const int64_t Kp = (K + bfp8::kBlock - 1) / bfp8::kBlock * bfp8::kBlock;
  return choose_schedule(M, N, K) == BFP8_SCHED_SMALL_M && bfp8::ksplit_fused_shape(M, N, K) &&
         (M - 1) * ldx * 2 + 2 * Kp <= kMaxOperandSpan;
}

// The linear layer on a given workspace (validation, then the quantizer and the GEMM).
bfp8_status_t linear_impl(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, const uint8_t* b,
                          int64_t ldb, const float* bs, int64_t ld_bs, const uint16_t* bias, uint16_t* c,
                          int64_t ldc, int64_t N, void* workspace, size_t workspace_bytes, void* stream) {
  if (x_dtype != BFP8_IN_BF16 && x_dtype != BFP8_IN_F16)
    return fail(BFP8_ERR_UNSUPPORTED,
                "the linear layer takes bf16 or fp16 activations (its output has their dtype), got x_dtype %d", x_dtype);
  if (!aligned(bias, 2)) return fail(BFP8_ERR_MISALIGNED, "bias must be 2-byte aligned");
  if (workspace && !aligned(workspace, 256)) return fail(BFP8_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  // Shapes first (a negative or oversized size must not reach the workspace arithmetic).
  if (M < 0) return fail(BFP8_ERR_INVALID_ARGUMENT, "M = %lld is negative", (long long)M);
  if (N < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "N = %lld must be >= 1", (long long)N);
  if (K < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "K = %lld must be >= 1", (long long)K);
  if (K % 16 != 0) return fail(BFP8_ERR_UNSUPPORTED, "K = %lld is not a multiple of 16", (long long)K);
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return fail(BFP8_ERR_UNSUPPORTED, "M, N and K must each be at most 2^30");
  const size_t need = bfp8_linear_workspace_bytes(M, N, K);
  const int64_t Kp = (K + bfp8::kBlock - 1) / bfp8::kBlock * bfp8::kBlock;  // row stride of the codes
  if (M > 0 && (!workspace || workspace_bytes < need))
    return fail(BFP8_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  bfp8_status_t st = BFP8_OK;
  const LinearLayout L = linear_layout(M, N, K);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* q = M > 0 ? ws : nullptr;
  float* as = M > 0 ? reinterpret_cast<float*>(ws + L.as_off) : nullptr;
  void* gws = M > 0 ? static_cast<void*>(ws + L.gemm_off) : nullptr;
  const size_t gws_bytes = M > 0 ? workspace_bytes - L.gemm_off : 0;
  st = check_quant_args(x, x_dtype, M, K, ldx, q, Kp, as, M);
  if (st != BFP8_OK) return st;
  st = check_gemm_args(q, Kp, as, M, b, ldb, bs, ld_bs, c, ldc, M, N, K, gws, gws_bytes, false);
  if (st != BFP8_OK) return st;
  if (M == 0) return ok();
  st = check_device();
  if (st != BFP8_OK) return st;
  // Small M on the K-split schedule's 16 x 16 tile: one launch that quantizes the activations
  // itself (bit-identical to the two launches below; the workspace is then not touched).
  if (linear_fuses(M, N, K, ldx)) {
    const bfp8::GemmArgs args{static_cast<const uint8_t*>(x), ldx, nullptr, 0, b, ldb, bs, ld_bs, c, ldc,
                              (int)M, (int)N, (int)K, nullptr, 1, bias, false, x_dtype == BFP8_IN_F16};
    return launched(bfp8::launch_gemm_ksplit_fused(args, x_dtype == BFP8_IN_F16 ? bfp8::kInF16 : bfp8::kInBf16,
                                                   (hipStream_t)stream),
                    "gemm_ksplit (fused quantization)");
  }
  st = launched(bfp8::launch_quant_act(x, x_dtype, M, K, ldx, q, Kp, as, M, false, (hipStream_t)stream), "quant_act");
  if (st != BFP8_OK) return st;
  return launch_dense(q, Kp, as, M, b, ldb, bs, ld_bs, bias, c, ldc, M, N, K, gws, stream, false,
                      x_dtype == BFP8_IN_F16);
}

// Staging of bfp8_linear_noalloc: one array per device, resolved once per device with that
// device current. The array's name is only a host-side handle; kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[BFP8_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

bfp8_status_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BFP8_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(BFP8_ERR_DEVICE, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(BFP8_ERR_DEVICE, "hipGetSymbolAddress of the staging array failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BFP8_OK;
}

}  // namespace

extern "C" {

bfp8_status_t bfp8_gemm(const uint8_t* a, int64_t lda, const float* as, int64_t ld_as, const uint8_t* b, int64_t ldb,
                        const float* bs, int64_t ld_bs, uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                        void* workspace, size_t workspace_bytes, void* stream) {
  bfp8_status_t st = check_gemm_args(a, lda, as, ld_as, b, ldb, bs, ld_bs, c, ldc, M, N, K, workspace,
                                     workspace_bytes, false);
  if (st != BFP8_OK) return st;
  if (M == 0) return ok();
  st = check_device();
  if (st != BFP8_OK) return st;
  return launch_dense(a, lda, as, ld_as, b, ldb, bs, ld_bs, nullptr, c, ldc, M, N, K, workspace, stream);
}

bfp8_status_t bfp8_quant_act_1x64(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                                  int64_t ldq, float* as, int64_t ld_as, void* stream) {
  bfp8_status_t st = check_quant_args(x, x_dtype, M, K, ldx, q, ldq, as, ld_as);
  if (st != BFP8_OK || M == 0) return st;
  st = check_device();
  if (st != BFP8_OK) return st;
  return launched(bfp8::launch_quant_act_1x64(x, x_dtype, M, K, ldx, q, ldq, as, ld_as, (hipStream_t)stream),
                  "quant_act_1x64");
}

bfp8_status_t bfp8_gemm_1x64(const uint8_t* a, int64_t lda, const float* as, int64_t ld_as, const uint8_t* b,
                             int64_t ldb, const float* bs, int64_t ld_bs, uint16_t* c, int64_t ldc, int64_t M,
                             int64_t N, int64_t K, void* stream) {
  bfp8_status_t st = check_gemm_args(a, lda, as, ld_as, b, ldb, bs, ld_bs, c, ldc, M, N, K, nullptr, 0, false);
  if (st != BFP8_OK) return st;
  if (ld_bs < (K + 63) / 64)
    return fail(BFP8_ERR_INVALID_ARGUMENT, "ld_bs = %lld < ceil(K/64) = %lld", (long long)ld_bs,
                (long long)((K + 63) / 64));
  if (M == 0) return ok();
  st = check_device();
  if (st != BFP8_OK) return st;
  const bfp8::GemmArgs args{a, lda, as, ld_as, b, ldb, bs, ld_bs, c, ldc, (int)M, (int)N, (int)K, nullptr, 1, nullptr,
                            false, false};
  // The schedule override picks the kernel family; by default the tiled kernel takes the GEMMs
  // with enough 256 x 128 tiles to fill the chip.
  const int sched = g_schedule.load(std::memory_order_relaxed);
  const int64_t tiles = ((N + 255) / 256) * ((M + 127) / 128);
  const bool tiled = sched == BFP8_SCHED_TILED || sched == BFP8_SCHED_PERSISTENT ||
                     (sched == BFP8_SCHED_AUTO && tiles >= bfp8::kTiled1x64MinTiles);
  if (tiled) return launched(bfp8::launch_gemm_g64(args, (hipStream_t)stream), "gemm_g64");
  return launched(bfp8::launch_gemm_ksplit_1x64(args, (hipStream_t)stream), "gemm_ksplit_1x64");
}

bfp8_status_t bfp8_gemm_f16(const uint8_t* a, int64_t lda, const float* as, int64_t ld_as, const uint8_t* b,
                            int64_t ldb, const float* bs, int64_t ld_bs, uint16_t* c, int64_t ldc, int64_t M,
                            int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  bfp8_status_t st = check_gemm_args(a, lda, as, ld_as, b, ldb, bs, ld_bs, c, ldc, M, N, K, workspace,
                                     workspace_bytes, false);
  if (st != BFP8_OK) return st;
  if (M == 0) return ok();
  st = check_device();
  if (st != BFP8_OK) return st;
  return launch_dense(a, lda, as, ld_as, b, ldb, bs, ld_bs, nullptr, c, ldc, M, N, K, workspace, stream, false, true);
}

bfp8_status_t bfp8_gemm_ue8m0(const uint8_t* a, int64_t lda, const uint8_t* as, int64_t ld_as, const uint8_t* b,
                              int64_t ldb, const uint8_t* bs, int64_t ld_bs, uint16_t* c, int64_t ldc, int64_t M,
                              int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  bfp8_status_t st = check_gemm_args(a, lda, as, ld_as, b, ldb, bs, ld_bs, c, ldc, M, N, K, workspace,
                                     workspace_bytes, false, true);
  if (st != BFP8_OK) return st;
  if (M == 0) return ok();
  st = check_device();
  if (st != BFP8_OK) return st;
  return launch_dense(a, lda, as, ld_as, b, ldb, bs, ld_bs, nullptr, c, ldc, M, N, K, workspace, stream, true);
}

}  // extern "C"

namespace {

// gathered: A has a_rows rows and row r of the GEMM reads its codes from A row
// row_src[r] / src_div; its scales stay at column r of as (float scales only).
bfp8_status_t grouped_gemm(const uint8_t* a, int64_t lda, const void* as, int64_t ld_as, const uint8_t* b,
                           int64_t ldb, const void* bs, int64_t ld_bs, const int32_t* grouped_layout, int32_t G,
                           uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K, void* workspace,
                           size_t workspace_bytes, void* stream, bool e8, bool gathered = false,
                           const int32_t* row_src = nullptr, int32_t src_div = 1, int64_t a_rows = 0) {
  bfp8_status_t st;
  if (!gathered) {
    st = check_gemm_args(a, lda, as, ld_as, b, ldb, bs, ld_bs, c, ldc, M, N, K, workspace, workspace_bytes, true, e8);
  } else {
    if (M < 0) return fail(BFP8_ERR_INVALID_ARGUMENT, "M = %lld is negative", (long long)M);
    if (M > kMaxDim) return fail(BFP8_ERR_UNSUPPORTED, "M must be at most 2^30");
    if (M > 0 && a_rows < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "a_rows = %lld must be >= 1", (long long)a_rows);
    if (src_div < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "src_div = %d must be >= 1", (int)src_div);
    if (M > 0 && !row_src) return fail(BFP8_ERR_INVALID_ARGUMENT, "row_src must not be NULL");
    if (!aligned(row_src, 4)) return fail(BFP8_ERR_MISALIGNED, "row_src must be 4-byte aligned");
    // A and its scales as a GEMM of a_rows rows; C as one of M rows (c, ldc and N checked here too)
    st = check_gemm_args(a, lda, as, ld_as, b, ldb, bs, ld_bs, c, ldc, M > 0 ? a_rows : 0, N, K, workspace,
                         workspace_bytes, true, false);
    if (st == BFP8_OK && ld_as < M)
      st = fail(BFP8_ERR_INVALID_ARGUMENT, "ld_as = %lld < M = %lld (one scale column per row of the product)",
                (long long)ld_as, (long long)M);
    if (st == BFP8_OK && M > 0 && ((M + 63) / 64) * ((N + 127) / 128) > (int64_t)INT32_MAX)
      st = fail(BFP8_ERR_UNSUPPORTED, "M x N has more output tiles than one launch grid holds");
  }
  if (st != BFP8_OK) return st;
  if (G < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "G = %d must be >= 1", (int)G);
  if (M % bfp8::kBlock != 0)
    return fail(BFP8_ERR_INVALID_ARGUMENT, "M = %lld is not a multiple of the 128-row group alignment",
                (long long)M);
  if (M > 0 && !grouped_layout) return fail(BFP8_ERR_INVALID_ARGUMENT, "grouped_layout must not be NULL");
  if (!aligned(grouped_layout, 4)) return fail(BFP8_ERR_MISALIGNED, "grouped_layout must be 4-byte aligned");
  if ((int64_t)G * N * ldb > ((int64_t)1 << 40)) return fail(BFP8_ERR_UNSUPPORTED, "G * N * ldb too large");
  if (M == 0) return ok();
  st = check_device();
  if (st != BFP8_OK) return st;
  bfp8::GemmArgs args{a,   lda,    as,     ld_as,  b,              ldb,    bs,      ld_bs, c,
                      ldc, (int)M, (int)N, (int)K, grouped_layout, (int)G, nullptr, e8};
  args.a_row_src = row_src;
  args.a_row_div = src_div;
  return launched(bfp8::launch_grouped_tiled(args, (hipStream_t)stream), "grouped_gemm_tiled");
}

}  // namespace

extern "C" {

bfp8_status_t bfp8_grouped_gemm_contiguous(const uint8_t* a, int64_t lda, const float* as, int64_t ld_as,
                                           const uint8_t* b, int64_t ldb, const float* bs, int64_t ld_bs,
                                           const int32_t* grouped_layout, int32_t G, uint16_t* c, int64_t ldc,
                                           int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  return grouped_gemm(a, lda, as, ld_as, b, ldb, bs, ld_bs, grouped_layout, G, c, ldc, M, N, K, workspace,
                      workspace_bytes, stream, false);
}

bfp8_status_t bfp8_grouped_gemm_gathered(const uint8_t* a, int64_t lda, const float* as, int64_t ld_as, int64_t a_rows,
                                         const int32_t* row_src, int32_t src_div, const uint8_t* b, int64_t ldb,
                                         const float* bs, int64_t ld_bs, const int32_t* grouped_layout, int32_t G,
                                         uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream) {
  return grouped_gemm(a, lda, as, ld_as, b, ldb, bs, ld_bs, grouped_layout, G, c, ldc, M, N, K, nullptr, 0, stream,
                      false, true, row_src, src_div, a_rows);
}

bfp8_status_t bfp8_grouped_gemm_contiguous_ue8m0(const uint8_t* a, int64_t lda, const uint8_t* as, int64_t ld_as,
                                                 const uint8_t* b, int64_t ldb, const uint8_t* bs, int64_t ld_bs,
                                                 const int32_t* grouped_layout, int32_t G, uint16_t* c, int64_t ldc,
                                                 int64_t M, int64_t N, int64_t K, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
  return grouped_gemm(a, lda, as, ld_as, b, ldb, bs, ld_bs, grouped_layout, G, c, ldc, M, N, K, workspace,
                      workspace_bytes, stream, true);
}

size_t bfp8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 16 != 0) return 0;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
  return linear_layout(M, N, K).total;
}

bfp8_status_t bfp8_linear(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, const uint8_t* b,
                          int64_t ldb, const float* bs, int64_t ld_bs, const uint16_t* bias, uint16_t* c,
                          int64_t ldc, int64_t N, void* workspace, size_t workspace_bytes, void* stream) {
  return linear_impl(x, x_dtype, M, K, ldx, b, ldb, bs, ld_bs, bias, c, ldc, N, workspace, workspace_bytes, stream);
}

int bfp8_linear_fuses(int64_t M, int64_t N, int64_t K, int64_t ldx) { return linear_fuses(M, N, K, ldx) ? 1 : 0; }

bfp8_status_t bfp8_linear_noalloc(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, const uint8_t* b,
                                  int64_t ldb, const float* bs, int64_t ld_bs, const uint16_t* bias, uint16_t* c,
                                  int64_t ldc, int64_t N, void* stream) {
  // Sizes first, on the host: a layer whose staging does not fit the device array is rejected
  // before any HIP call.
  if (M < 0 || N < 1 || K < 1 || K % 16 != 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return linear_impl(x, x_dtype, M, K, ldx, b, ldb, bs, ld_bs, bias, c, ldc, N, nullptr, 0, stream);
  const size_t need = M > 0 ? linear_layout(M, N, K).total : 0;
  if (need > BFP8_NOALLOC_SCRATCH_BYTES)
    return fail(BFP8_ERR_UNSUPPORTED,
                "M x K = %lld x %lld needs %zu bytes of staging; bfp8_linear_noalloc holds at most %zu "
                "(use bfp8_linear with a caller workspace)",
                (long long)M, (long long)K, need, (size_t)BFP8_NOALLOC_SCRATCH_BYTES);
  if (M == 0)
    return linear_impl(x, x_dtype, M, K, ldx, b, ldb, bs, ld_bs, bias, c, ldc, N, nullptr, 0, stream);
  bfp8_status_t st = check_device();
  if (st != BFP8_OK) return st;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != BFP8_OK) return st;
  return linear_impl(x, x_dtype, M, K, ldx, b, ldb, bs, ld_bs, bias, c, ldc, N, ws, BFP8_NOALLOC_SCRATCH_BYTES,
                     stream);
}

// ---- MoE chain ------------------------------------------------------------------------------

int64_t bfp8_moe_padded_rows(int64_t S, int32_t E, int32_t align) {
  if (S < 0 || E < 1 || align < 1) return 0;
  const int64_t bound = S + (S < E ? S : (int64_t)E) * (align - 1);
  return (bound + align - 1) / align * align;
}

size_t bfp8_moe_dispatch_workspace_bytes(int64_t S, int32_t E) {
  if (S < 0 || E < 1) return 0;
  return (size_t)(bfp8::moe_dispatch_blocks(S) * E + E) * 4;
}

}  // extern "C"

namespace {

constexpr int32_t kMaxExperts = 1024;  // the placement kernel keeps 16 x E counters in LDS

bfp8_status_t check_dispatch_args(const int32_t* ids, int64_t S, int32_t E, int32_t align, const int32_t* row_of_pair,
                                  const int32_t* pair_of_row, const int32_t* layout, const int32_t* expert_start) {
  if (S < 0) return fail(BFP8_ERR_INVALID_ARGUMENT, "S = %lld is negative", (long long)S);
  if (E < 1 || E > kMaxExperts) return fail(BFP8_ERR_UNSUPPORTED, "E = %d must be in [1, %d]", (int)E, (int)kMaxExperts);
  if (align < 1 || align > 4096) return fail(BFP8_ERR_INVALID_ARGUMENT, "alignment %d must be in [1, 4096]", (int)align);
  if (bfp8_moe_padded_rows(S, E, align) > (int64_t)INT32_MAX)
    return fail(BFP8_ERR_UNSUPPORTED, "the padded buffer of %lld pairs would exceed 2^31 rows", (long long)S);
  if (S > 0 && (!ids || !row_of_pair || !pair_of_row || !layout))
    return fail(BFP8_ERR_INVALID_ARGUMENT, "ids, row_of_pair, pair_of_row and layout must not be NULL when S > 0");
  if (!expert_start) return fail(BFP8_ERR_INVALID_ARGUMENT, "expert_start must not be NULL");
  if (!aligned(ids, 4) || !aligned(row_of_pair, 4) || !aligned(pair_of_row, 4) || !aligned(layout, 4) ||
      !aligned(expert_start, 4))
    return fail(BFP8_ERR_MISALIGNED, "the int32 arrays must be 4-byte aligned");
  return BFP8_OK;
}

bfp8_status_t dispatch(const int32_t* ids, int64_t S, int32_t E, int32_t align, int32_t* row_of_pair,
                       int32_t* pair_of_row, int32_t* layout, int32_t* expert_start, int32_t* scratch,
                       void* stream) {
  const int64_t rows = bfp8_moe_padded_rows(S, E, align);
  int32_t* block_counts = scratch;
  int32_t* expert_count = scratch + bfp8::moe_dispatch_blocks(S) * E;
  return launched(bfp8::launch_moe_dispatch(ids, S, E, align, rows, row_of_pair, pair_of_row, layout, expert_start,
                                            expert_count, block_counts, (hipStream_t)stream),
                  "moe_dispatch");
}

bfp8_status_t check_swiglu_args(const uint16_t* proj, int64_t M, int64_t I, int64_t ldp, const int32_t* layout,
                                const uint8_t* q, int64_t ldq, const float* as, int64_t ld_as) {
  if (M < 0) return fail(BFP8_ERR_INVALID_ARGUMENT, "M = %lld is negative", (long long)M);
  if (I < bfp8::kBlock || I % bfp8::kBlock != 0 || I > kMaxDim)
    return fail(BFP8_ERR_UNSUPPORTED, "I = %lld must be a positive multiple of 128 (at most 2^30)", (long long)I);
  if (M > kMaxDim) return fail(BFP8_ERR_UNSUPPORTED, "M must be at most 2^30");
  if (M == 0) return BFP8_OK;
  if (!proj || !q || !as) return fail(BFP8_ERR_INVALID_ARGUMENT, "proj, q and as must not be NULL");
  if (ldp < 2 * I) return fail(BFP8_ERR_INVALID_ARGUMENT, "ldp = %lld < 2 I = %lld", (long long)ldp, (long long)(2 * I));
  if (ldq < I) return fail(BFP8_ERR_INVALID_ARGUMENT, "ldq = %lld < I = %lld", (long long)ldq, (long long)I);
  if (ld_as < M) return fail(BFP8_ERR_INVALID_ARGUMENT, "ld_as = %lld < M = %lld", (long long)ld_as, (long long)M);
  if ((ldp * 2) % 16 || ldq % 16) return fail(BFP8_ERR_MISALIGNED, "row strides must be multiples of 16 bytes");
  if (!aligned(proj, 16) || !aligned(q, 16) || !aligned(as, 4) || !aligned(layout, 4))
    return fail(BFP8_ERR_MISALIGNED, "proj and q must be 16-byte aligned, as and layout 4-byte aligned");
  return BFP8_OK;
}

bfp8_status_t check_combine_args(const uint16_t* out, int64_t ldo, const int32_t* row_of_pair, const float* w,
                                 int64_t T, int32_t top_k, int64_t H, const uint16_t* y, int64_t ldy) {
  if (T < 0) return fail(BFP8_ERR_INVALID_ARGUMENT, "T = %lld is negative", (long long)T);
  if (top_k < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "top_k = %d must be >= 1", (int)top_k);
  if (H < 8 || H % 8 != 0 || H > kMaxDim)
    return fail(BFP8_ERR_UNSUPPORTED, "H = %lld must be a positive multiple of 8", (long long)H);
  if (T * top_k > (int64_t)INT32_MAX) return fail(BFP8_ERR_UNSUPPORTED, "T * top_k must be below 2^31");
  if (T == 0) return BFP8_OK;
  if (!out || !row_of_pair || !w || !y)
    return fail(BFP8_ERR_INVALID_ARGUMENT, "out, row_of_pair, weights and y must not be NULL");
  if (ldo < H || ldy < H) return fail(BFP8_ERR_INVALID_ARGUMENT, "ldo and ldy must be >= H");
  if ((ldo * 2) % 16 || (ldy * 2) % 16) return fail(BFP8_ERR_MISALIGNED, "row strides must be multiples of 16 bytes");
  if (!aligned(out, 16) || !aligned(y, 16) || !aligned(row_of_pair, 4) || !aligned(w, 4))
    return fail(BFP8_ERR_MISALIGNED, "out and y must be 16-byte aligned, row_of_pair and weights 4-byte aligned");
  return BFP8_OK;
}

// Workspace of the MoE forward, each part 256-byte aligned.
struct MoeLayout {
  size_t row_of_pair, pair_of_row, layout, expert_start, scratch, q, as, proj, q2, as2, out, total;
  int64_t rows;
};

MoeLayout moe_layout(int64_t T, int32_t top_k, int32_t E, int64_t H, int64_t I) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  MoeLayout L{};
  const int64_t S = T * top_k;
  L.rows = bfp8_moe_padded_rows(S, E, bfp8::kBlock);
  const size_t R = (size_t)L.rows;
  size_t off = 0;
  L.row_of_pair = off; off += up(4 * (size_t)S);
  L.pair_of_row = off; off += up(4 * R);
  L.layout = off; off += up(4 * R);
  L.expert_start = off; off += up(4 * ((size_t)E + 1));
  L.scratch = off; off += up(bfp8_moe_dispatch_workspace_bytes(S, E));
  L.q = off; off += up((size_t)T * (size_t)H);  // the tokens quantized once, [T][H]
  L.as = off; off += up(4 * (size_t)(H / bfp8::kBlock) * R);  // their scales at the padded rows
  L.proj = off; off += up(2 * R * 2 * (size_t)I);
  L.q2 = off; off += up(R * (size_t)I);
  L.as2 = off; off += up(4 * (size_t)(I / bfp8::kBlock) * R);
  L.out = off; off += up(2 * R * (size_t)H);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

bfp8_status_t bfp8_moe_dispatch(const int32_t* topk_ids, int64_t S, int32_t E, int32_t align, int32_t* row_of_pair,
                                int32_t* pair_of_row, int32_t* layout, int32_t* expert_start, void* workspace,
                                size_t workspace_bytes, void* stream) {
  bfp8_status_t st = check_dispatch_args(topk_ids, S, E, align, row_of_pair, pair_of_row, layout, expert_start);
  if (st != BFP8_OK) return st;
  const size_t need = bfp8_moe_dispatch_workspace_bytes(S, E);
  if (!workspace || workspace_bytes < need)
    return fail(BFP8_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (!aligned(workspace, 4)) return fail(BFP8_ERR_MISALIGNED, "workspace must be 4-byte aligned");
  st = check_device();
  if (st != BFP8_OK) return st;
  return dispatch(topk_ids, S, E, align, row_of_pair, pair_of_row, layout, expert_start,
                  static_cast<int32_t*>(workspace), stream);
}

bfp8_status_t bfp8_quant_act_gather(const void* x, int x_dtype, int64_t src_rows, int64_t K, int64_t ldx,
                                    const int32_t* row_src, int32_t src_div, int64_t M, uint8_t* q, int64_t ldq,
                                    float* as, int64_t ld_as, void* stream) {
  bfp8_status_t st = check_quant_args(x, x_dtype, M, K, ldx, q, ldq, as, ld_as);
  if (st != BFP8_OK || M == 0) return st;
  if (src_rows < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "src_rows = %lld must be >= 1", (long long)src_rows);
  if (src_div < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "src_div = %d must be >= 1", (int)src_div);
  if (!row_src) return fail(BFP8_ERR_INVALID_ARGUMENT, "row_src must not be NULL");
  if (!aligned(row_src, 4)) return fail(BFP8_ERR_MISALIGNED, "row_src must be 4-byte aligned");
  st = check_device();
  if (st != BFP8_OK) return st;
  return launched(bfp8::launch_quant_act(x, x_dtype, M, K, ldx, q, ldq, as, ld_as, false, (hipStream_t)stream,
                                         row_src, src_div),
                  "quant_act_gather");
}

bfp8_status_t bfp8_swiglu_quant(const uint16_t* proj, int64_t M, int64_t I, int64_t ldp, const int32_t* layout,
                                uint8_t* q, int64_t ldq, float* as, int64_t ld_as, void* stream) {
  bfp8_status_t st = check_swiglu_args(proj, M, I, ldp, layout, q, ldq, as, ld_as);
  if (st != BFP8_OK || M == 0) return st;
  st = check_device();
  if (st != BFP8_OK) return st;
  return launched(bfp8::launch_swiglu_quant(proj, M, I, ldp, layout, q, ldq, as, ld_as, (hipStream_t)stream),
                  "swiglu_quant");
}

bfp8_status_t bfp8_swiglu(const uint16_t* proj, int64_t M, int64_t I, int64_t ldp, const int32_t* layout, uint16_t* h,
                          int64_t ldh, void* stream) {
  if (M < 0) return fail(BFP8_ERR_INVALID_ARGUMENT, "M = %lld is negative", (long long)M);
  if (I < bfp8::kBlock || I % bfp8::kBlock != 0 || I > kMaxDim)
    return fail(BFP8_ERR_UNSUPPORTED, "I = %lld must be a positive multiple of 128 (at most 2^30)", (long long)I);
  if (M > kMaxDim) return fail(BFP8_ERR_UNSUPPORTED, "M must be at most 2^30");
  if (M == 0) return BFP8_OK;
  if (!proj || !h) return fail(BFP8_ERR_INVALID_ARGUMENT, "proj and h must not be NULL");
  if (ldp < 2 * I) return fail(BFP8_ERR_INVALID_ARGUMENT, "ldp = %lld < 2 I = %lld", (long long)ldp, (long long)(2 * I));
  if (ldh < I) return fail(BFP8_ERR_INVALID_ARGUMENT, "ldh = %lld < I = %lld", (long long)ldh, (long long)I);
  if ((ldp * 2) % 16 || (ldh * 2) % 16) return fail(BFP8_ERR_MISALIGNED, "row strides must be multiples of 16 bytes");
  if (!aligned(proj, 16) || !aligned(h, 16) || !aligned(layout, 4))
    return fail(BFP8_ERR_MISALIGNED, "proj and h must be 16-byte aligned, layout 4-byte aligned");
  bfp8_status_t st = check_device();
  if (st != BFP8_OK) return st;
  return launched(bfp8::launch_swiglu(proj, M, I, ldp, layout, h, ldh, (hipStream_t)stream), "swiglu");
}

bfp8_status_t bfp8_quant_act_scatter(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                                     int64_t ldq, float* as, int64_t ld_as, const int32_t* scale_dst,
                                     int32_t scale_fan, void* stream) {
  bfp8_status_t st = check_quant_args(x, x_dtype, M, K, ldx, q, ldq, as, ld_as);
  if (st != BFP8_OK || M == 0) return st;
  if (scale_fan < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "scale_fan = %d must be >= 1", (int)scale_fan);
  if (M * scale_fan > (int64_t)INT32_MAX) return fail(BFP8_ERR_UNSUPPORTED, "M * scale_fan must be below 2^31");
  if (!scale_dst) return fail(BFP8_ERR_INVALID_ARGUMENT, "scale_dst must not be NULL");
  if (!aligned(scale_dst, 4)) return fail(BFP8_ERR_MISALIGNED, "scale_dst must be 4-byte aligned");
  st = check_device();
  if (st != BFP8_OK) return st;
  return launched(bfp8::launch_quant_act(x, x_dtype, M, K, ldx, q, ldq, as, ld_as, false, (hipStream_t)stream,
                                         nullptr, 1, scale_dst, scale_fan),
                  "quant_act_scatter");
}

bfp8_status_t bfp8_moe_combine(const uint16_t* out, int64_t ldo, const int32_t* row_of_pair,
                               const float* topk_weights, int64_t T, int32_t top_k, int64_t H, uint16_t* y,
                               int64_t ldy, void* stream) {
  bfp8_status_t st = check_combine_args(out, ldo, row_of_pair, topk_weights, T, top_k, H, y, ldy);
  if (st != BFP8_OK || T == 0) return st;
  st = check_device();
  if (st != BFP8_OK) return st;
  return launched(bfp8::launch_moe_combine(out, ldo, row_of_pair, topk_weights, T, top_k, H, y, ldy,
                                           (hipStream_t)stream),
                  "moe_combine");
}

size_t bfp8_moe_forward_workspace_bytes(int64_t T, int32_t top_k, int32_t E, int64_t H, int64_t I) {
  if (T <= 0 || top_k < 1 || E < 1 || H < 1 || I < 1) return 0;
  if (T * top_k > (int64_t)INT32_MAX || H > kMaxDim || I > kMaxDim) return 0;
  return moe_layout(T, top_k, E, H, I).total;
}

bfp8_status_t bfp8_moe_forward(const uint16_t* hidden, int64_t T, int64_t H, int64_t ldh, const int32_t* topk_ids,
                               const float* topk_weights, int32_t top_k, int32_t E, const uint8_t* w_up,
                               const float* s_up, const uint8_t* w_down, const float* s_down, int64_t I, uint16_t* y,
                               int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  if (T < 0) return fail(BFP8_ERR_INVALID_ARGUMENT, "T = %lld is negative", (long long)T);
  if (top_k < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "top_k = %d must be >= 1", (int)top_k);
  if (E < 1 || E > kMaxExperts) return fail(BFP8_ERR_UNSUPPORTED, "E = %d must be in [1, %d]", (int)E, (int)kMaxExperts);
  if (H < bfp8::kBlock || H % bfp8::kBlock != 0 || I < bfp8::kBlock || I % bfp8::kBlock != 0)
    return fail(BFP8_ERR_UNSUPPORTED, "H and I must be positive multiples of 128");
  if (H > kMaxDim || I > kMaxDim || T * top_k > (int64_t)INT32_MAX / 2)
    return fail(BFP8_ERR_UNSUPPORTED, "sizes too large");
  if (!w_up || !s_up || !w_down || !s_down) return fail(BFP8_ERR_INVALID_ARGUMENT, "weights must not be NULL");
  if (T == 0) return ok();
  if (!hidden || !topk_ids || !topk_weights || !y)
    return fail(BFP8_ERR_INVALID_ARGUMENT, "hidden, topk_ids, topk_weights and y must not be NULL");
  if (ldh < H || (ldh * 2) % 16 || !aligned(hidden, 16))
    return fail(BFP8_ERR_MISALIGNED, "hidden: ldh >= H, rows 16-byte aligned");
  const MoeLayout L = moe_layout(T, top_k, E, H, I);
  if (!workspace || workspace_bytes < L.total)
    return fail(BFP8_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, L.total);
  if (!aligned(workspace, 256)) return fail(BFP8_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const int64_t S = T * top_k, R = L.rows;
  int32_t* row_of_pair = reinterpret_cast<int32_t*>(ws + L.row_of_pair);
  int32_t* pair_of_row = reinterpret_cast<int32_t*>(ws + L.pair_of_row);
  int32_t* layout = reinterpret_cast<int32_t*>(ws + L.layout);
  int32_t* expert_start = reinterpret_cast<int32_t*>(ws + L.expert_start);
  uint8_t* q = ws + L.q;
  float* as = reinterpret_cast<float*>(ws + L.as);
  uint16_t* proj = reinterpret_cast<uint16_t*>(ws + L.proj);
  uint8_t* q2 = ws + L.q2;
  float* as2 = reinterpret_cast<float*>(ws + L.as2);
  uint16_t* out = reinterpret_cast<uint16_t*>(ws + L.out);
  // Every argument of every step, validated before the first launch.
  bfp8_status_t st = check_dispatch_args(topk_ids, S, E, bfp8::kBlock, row_of_pair, pair_of_row, layout, expert_start);
  if (st == BFP8_OK) st = check_quant_args(hidden, BFP8_IN_BF16, T, H, ldh, q, H, as, R);
  // The up projection reads its codes (T token rows) through the row map and its scales at the
  // R padded rows; its R output rows are the workspace's proj, checked with the SwiGLU step.
  if (st == BFP8_OK)
    st = check_gemm_args(q, H, as, R, w_up, H, s_up, H / bfp8::kBlock, proj, 2 * I, T, 2 * I, H, nullptr, 0, true);
  if (st == BFP8_OK) st = check_swiglu_args(proj, R, I, 2 * I, layout, q2, I, as2, R);
  if (st == BFP8_OK)
    st = check_gemm_args(q2, I, as2, R, w_down, I, s_down, I / bfp8::kBlock, out, H, R, H, I, nullptr, 0, true);
  if (st == BFP8_OK) st = check_combine_args(out, H, row_of_pair, topk_weights, T, top_k, H, y, ldy);
  if (st != BFP8_OK) return st;
  if ((int64_t)E * 2 * I * H > ((int64_t)1 << 40) || (int64_t)E * H * I > ((int64_t)1 << 40))
    return fail(BFP8_ERR_UNSUPPORTED, "expert weights too large");
  st = check_device();
  if (st != BFP8_OK) return st;
  st = dispatch(topk_ids, S, E, bfp8::kBlock, row_of_pair, pair_of_row, layout, expert_start,
                reinterpret_cast<int32_t*>(ws + L.scratch), stream);
  if (st != BFP8_OK) return st;
  // Each token is quantized once, its scales written at its padded rows (row_of_pair); the up
  // projection reads padded row r's codes from token pair_of_row[r] / top_k. Codes and scales
  // are the gathered quantizer's, so the product is that of the quantized padded rows.
  st = launched(bfp8::launch_quant_act(hidden, BFP8_IN_BF16, T, H, ldh, q, H, as, R, false, (hipStream_t)stream,
                                       nullptr, 1, row_of_pair, top_k),
                "quant_act_scatter");
  if (st != BFP8_OK) return st;
  bfp8::GemmArgs up_args{q, H, as, R, w_up, H, s_up, H / bfp8::kBlock, proj, 2 * I, (int)R, (int)(2 * I),
                         (int)H, layout, E, nullptr, false};
  up_args.a_row_src = pair_of_row;
  up_args.a_row_div = top_k;
  st = launched(bfp8::launch_grouped_tiled(up_args, (hipStream_t)stream), "grouped_gemm_up");
  if (st != BFP8_OK) return st;
  st = launched(bfp8::launch_swiglu_quant(proj, R, I, 2 * I, layout, q2, I, as2, R, (hipStream_t)stream),
                "swiglu_quant");
  if (st != BFP8_OK) return st;
  const bfp8::GemmArgs down_args{q2, I, as2, R, w_down, I, s_down, I / bfp8::kBlock, out, H, (int)R, (int)H,
                                 (int)I, layout, E, nullptr, false};
  st = launched(bfp8::launch_grouped_tiled(down_args, (hipStream_t)stream), "grouped_gemm_down");
  if (st != BFP8_OK) return st;
  return launched(bfp8::launch_moe_combine(out, H, row_of_pair, topk_weights, T, top_k, H, y, ldy,
                                           (hipStream_t)stream),
                  "moe_combine");
}

bfp8_status_t bfp8_transpose_weights(const uint8_t* src, int64_t E, int64_t K, int64_t N, int64_t ld_src,
                                     uint8_t* dst, int64_t ld_dst, void* stream) {
  if (E < 1 || K < 1 || N < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "E, K and N must be >= 1");
  if (E > 1024 || K > kMaxDim || N > kMaxDim) return fail(BFP8_ERR_UNSUPPORTED, "E <= 1024, K, N <= 2^30");
  if (ld_src < N || ld_dst < K) return fail(BFP8_ERR_INVALID_ARGUMENT, "ld_src must be >= N and ld_dst >= K");
  if (!src || !dst) return fail(BFP8_ERR_INVALID_ARGUMENT, "src and dst must not be NULL");
  const uint8_t* src_end = src + E * K * ld_src;
  const uint8_t* dst_end = dst + E * N * ld_dst;
  if (src < dst_end && dst < src_end) return fail(BFP8_ERR_INVALID_ARGUMENT, "src and dst must not overlap");
  bfp8_status_t st = check_device();
  if (st != BFP8_OK) return st;
  return launched(bfp8::launch_transpose_u8(src, E, K, N, ld_src, dst, ld_dst, (hipStream_t)stream),
                  "transpose_weights");
}

bfp8_status_t bfp8_transpose_scales(const float* src, int64_t E, int64_t R, int64_t C, float* dst, void* stream) {
  if (E < 1 || R < 1 || C < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "E, R and C must be >= 1");
  if (E * R * C > ((int64_t)1 << 40)) return fail(BFP8_ERR_UNSUPPORTED, "too many scales");
  if (!src || !dst) return fail(BFP8_ERR_INVALID_ARGUMENT, "src and dst must not be NULL");
  if (!aligned(src, 4) || !aligned(dst, 4)) return fail(BFP8_ERR_MISALIGNED, "src and dst must be 4-byte aligned");
  if (src < dst + E * R * C && dst < src + E * R * C)
    return fail(BFP8_ERR_INVALID_ARGUMENT, "src and dst must not overlap");
  bfp8_status_t st = check_device();
  if (st != BFP8_OK) return st;
  return launched(bfp8::launch_transpose_f32(src, E, R, C, dst, (hipStream_t)stream), "transpose_scales");
}

bfp8_status_t bfp8_expand_act_scales(const float* s, int64_t s_stride, int64_t M, int64_t K, float* as,
                                     int64_t ld_as, void* stream) {
  if (M < 0 || K < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "M must be >= 0 and K >= 1");
  if (s_stride < 0) return fail(BFP8_ERR_INVALID_ARGUMENT, "s_stride = %lld is negative", (long long)s_stride);
  const int64_t G = (K + bfp8::kBlock - 1) / bfp8::kBlock;
  if (M > kMaxDim || K > kMaxDim || M * G > ((int64_t)1 << 38)) return fail(BFP8_ERR_UNSUPPORTED, "sizes too large");
  if (M == 0) return ok();
  if (!s || !as) return fail(BFP8_ERR_INVALID_ARGUMENT, "s and as must not be NULL");
  if (ld_as < M) return fail(BFP8_ERR_INVALID_ARGUMENT, "ld_as = %lld < M = %lld", (long long)ld_as, (long long)M);
  if (!aligned(s, 4) || !aligned(as, 4)) return fail(BFP8_ERR_MISALIGNED, "s and as must be 4-byte aligned");
  bfp8_status_t st = check_device();
  if (st != BFP8_OK) return st;
  return launched(bfp8::launch_expand_act_scales(s, s_stride, M, G, as, ld_as, (hipStream_t)stream),
                  "expand_act_scales");
}

bfp8_status_t bfp8_expand_weight_scale(const float* s, int64_t N, int64_t K, float* bs, int64_t ld_bs,
                                       void* stream) {
  if (N < 1 || K < 1) return fail(BFP8_ERR_INVALID_ARGUMENT, "N and K must be >= 1");
  const int64_t NB = (N + bfp8::kBlock - 1) / bfp8::kBlock, KB = (K + bfp8::kBlock - 1) / bfp8::kBlock;
  if (N > kMaxDim || K > kMaxDim) return fail(BFP8_ERR_UNSUPPORTED, "N and K must each be at most 2^30");
  if (!s || !bs) return fail(BFP8_ERR_INVALID_ARGUMENT, "s and bs must not be NULL");
  if (ld_bs < KB) return fail(BFP8_ERR_INVALID_ARGUMENT, "ld_bs = %lld < ceil(K/128) = %lld", (long long)ld_bs,
                              (long long)KB);
  if (!aligned(s, 4) || !aligned(bs, 4)) return fail(BFP8_ERR_MISALIGNED, "s and bs must be 4-byte aligned");
  bfp8_status_t st = check_device();
  if (st != BFP8_OK) return st;
  return launched(bfp8::launch_fill_weight_scales(s, NB, KB, bs, ld_bs, (hipStream_t)stream), "expand_weight_scale");
}

bfp8_status_t bfp8_set_schedule(int schedule) {
  if (schedule < BFP8_SCHED_AUTO || schedule >= BFP8_SCHED_COUNT_)
    return fail(BFP8_ERR_INVALID_ARGUMENT, "unknown schedule %d", schedule);
  g_schedule.store(schedule, std::memory_order_relaxed);
  return ok();
}

int bfp8_get_schedule(void) { return g_schedule.load(std::memory_order_relaxed); }

int bfp8_gemm_schedule_for(int64_t M, int64_t N, int64_t K) { return choose_schedule(M, N, K); }

}  // extern "C"
