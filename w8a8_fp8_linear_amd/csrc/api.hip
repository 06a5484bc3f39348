// The C ABI of libw8a8.so (include/w8a8.h): argument checks on the host,
// the gfx950 device check, then one launcher per entry point.
#include <string.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "../../include/w8a8.h"
#include "launch.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch[kMaxDevices];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return W8A8_ERR_DEVICE;
  }
  if (dev < kMaxDevices) {
    const int known = g_arch[dev].load(std::memory_order_relaxed);
    if (known == 1) return W8A8_OK;
    if (known == 2) return W8A8_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return W8A8_ERR_DEVICE;
  }
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? W8A8_OK : W8A8_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool mul_ok(int64_t a, int64_t b) {  // a, b >= 0; a * b fits in int64
  return a == 0 || b <= INT64_MAX / a;
}

// Sizes accepted by the dense GEMM entry points.
int check_dense_shape(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0 || !mul_ok(M, K) || !mul_ok(N, K) || !mul_ok(M, N) || !mul_ok(M * N, 2) ||
      !mul_ok(M * K, 2))
    return W8A8_ERR_BAD_SHAPE;
  if (K == 0 || K % 16 != 0 || K > (int64_t(1) << 20)) return W8A8_ERR_UNSUPPORTED;
  if (N % 16 != 0 || N > (int64_t(1) << 20) || M > (int64_t(1) << 24)) return W8A8_ERR_UNSUPPORTED;
  return W8A8_OK;
}

int64_t align256(int64_t b) { return (b + 255) & ~int64_t(255); }

// The model page applies the FP8 multiply only to steps with more than 8
// tokens at once; fewer always use the default maths.
constexpr int64_t kFastMathMinTokens = 8;
// fp8_linear's FP8 path takes the single-launch kernel up to this many rows.
constexpr int64_t kFusedFasterMaxM = 16;

int launch_status(hipError_t e) {
  if (e == hipSuccess) return W8A8_OK;
  return W8A8_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int w8a8_abi_version(void) { return W8A8_ABI_VERSION; }

const char* w8a8_status_string(int status) {
  switch (status) {
    case W8A8_OK: return "ok";
    case W8A8_ERR_NULL_ARG: return "null argument";
    case W8A8_ERR_BAD_SHAPE: return "bad shape (negative size or size overflow)";
    case W8A8_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case W8A8_ERR_UNSUPPORTED: return "unsupported size";
    case W8A8_ERR_WORKSPACE: return "workspace too small";
    case W8A8_ERR_DEVICE: return "current device is not gfx950";
    case W8A8_ERR_LAUNCH: return "kernel launch failed";
    case W8A8_ERR_SCRATCH: return "size exceeds the library's static scratch";
    default: return "unknown status";
  }
}

int quantize_per_token(const uint16_t* x_bf16, int64_t M, int64_t K, uint8_t* q_e4m3, float* scale,
                       hipStream_t stream) {
  if (M < 0 || K < 0 || !mul_ok(M, K) || !mul_ok(M * K, 2)) return W8A8_ERR_BAD_SHAPE;
  if (K == 0 || K % 16 != 0 || K > (int64_t(1) << 24)) return W8A8_ERR_UNSUPPORTED;
  if (M == 0) return W8A8_OK;
  if (!x_bf16 || !q_e4m3 || !scale) return W8A8_ERR_NULL_ARG;
  if (!aligned16(x_bf16) || !aligned16(q_e4m3) || !aligned16(scale)) return W8A8_ERR_MISALIGNED;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_quantize_rows(x_bf16, M, K, q_e4m3, scale, stream));
}

static int gemm_checked(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q, const float* w_scale,
                        uint16_t* y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream, hipEvent_t start,
                        hipEvent_t stop) {
  if (M < 0 || N < 0 || K < 0 || !mul_ok(M, K) || !mul_ok(N, K) || !mul_ok(M, N) || !mul_ok(M * N, 2))
    return W8A8_ERR_BAD_SHAPE;
  if (K == 0 || K % 16 != 0 || K > (int64_t(1) << 20)) return W8A8_ERR_UNSUPPORTED;
  if (N % 16 != 0 || N > (int64_t(1) << 20) || M > (int64_t(1) << 24)) return W8A8_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return W8A8_OK;
  if (!a_q || !a_scale || !w_q || !w_scale || !y_bf16) return W8A8_ERR_NULL_ARG;
  if (!aligned16(a_q) || !aligned16(a_scale) || !aligned16(w_q) || !aligned16(w_scale) || !aligned16(y_bf16))
    return W8A8_ERR_MISALIGNED;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_gemm(a_q, a_scale, w_q, w_scale, y_bf16, M, N, K, stream, start, stop));
}

int w8a8_gemm(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q, const float* w_scale,
              uint16_t* y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  return gemm_checked(a_q, a_scale, w_q, w_scale, y_bf16, M, N, K, stream, nullptr, nullptr);
}

int w8a8_gemm_timed(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q, const float* w_scale,
                    uint16_t* y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream, hipEvent_t start,
                    hipEvent_t stop) {
  if (!start || !stop) return W8A8_ERR_NULL_ARG;
  return gemm_checked(a_q, a_scale, w_q, w_scale, y_bf16, M, N, K, stream, start, stop);
}

int w8a16_gemm(const uint16_t* x_bf16, const uint8_t* w_q, const float* w_scale, uint16_t* y_bf16, int64_t M,
               int64_t N, int64_t K, hipStream_t stream) {
  const int c = check_dense_shape(M, N, K);
  if (c != W8A8_OK) return c;
  if (M == 0 || N == 0) return W8A8_OK;
  if (!x_bf16 || !w_q || !w_scale || !y_bf16) return W8A8_ERR_NULL_ARG;
  if (!aligned16(x_bf16) || !aligned16(w_q) || !aligned16(w_scale) || !aligned16(y_bf16)) return W8A8_ERR_MISALIGNED;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_w8a16_gemm(x_bf16, w_q, w_scale, y_bf16, M, N, K, stream));
}

int e4m3_from_f32(const float* v, int64_t n, uint8_t* q_e4m3, hipStream_t stream) {
  if (n < 0) return W8A8_ERR_BAD_SHAPE;
  if (n > (int64_t(1) << 40)) return W8A8_ERR_UNSUPPORTED;
  if (n == 0) return W8A8_OK;
  if (!v || !q_e4m3) return W8A8_ERR_NULL_ARG;
  if (!aligned16(v) || !aligned16(q_e4m3)) return W8A8_ERR_MISALIGNED;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_convert_e4m3(v, n, q_e4m3, stream));
}

int bf16_from_f32(const float* v, int64_t n, uint16_t* y_bf16, hipStream_t stream) {
  if (n < 0) return W8A8_ERR_BAD_SHAPE;
  if (n > (int64_t(1) << 40)) return W8A8_ERR_UNSUPPORTED;
  if (n == 0) return W8A8_OK;
  if (!v || !y_bf16) return W8A8_ERR_NULL_ARG;
  if (!aligned16(v) || !aligned16(y_bf16)) return W8A8_ERR_MISALIGNED;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_convert_bf16(v, n, y_bf16, stream));
}

int64_t read_probe_sink_words(int64_t bytes) {
  if (bytes < 0) return 0;
  return (bytes + w8a8::kProbeBytesPerBlock - 1) / w8a8::kProbeBytesPerBlock;
}

int read_probe(const uint8_t* p, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes < 0) return W8A8_ERR_BAD_SHAPE;
  if (bytes % 16 != 0 || bytes > (int64_t(1) << 40)) return W8A8_ERR_UNSUPPORTED;
  if (bytes == 0) return W8A8_OK;
  if (!p || !sink) return W8A8_ERR_NULL_ARG;
  if (!aligned16(p) || !aligned16(sink)) return W8A8_ERR_MISALIGNED;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_read_probe(p, bytes, sink, stream));
}

int clock_probe(uint64_t* out, int64_t n, hipStream_t stream) {
  if (n < 0) return W8A8_ERR_BAD_SHAPE;
  if (n > 65536) return W8A8_ERR_UNSUPPORTED;
  if (n == 0) return W8A8_OK;
  if (!out) return W8A8_ERR_NULL_ARG;
  if (!aligned16(out)) return W8A8_ERR_MISALIGNED;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_clock_probe(out, n, stream));
}

size_t fp8_linear_workspace_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0 || !mul_ok(M, K)) return 0;
  return (size_t)(align256(M * K) + align256(M * 4));
}

int fp8_linear(const uint16_t* x_bf16, const uint8_t* w_q, const float* w_scale, uint16_t* y_bf16, int64_t M,
               int64_t N, int64_t K, int fast_math, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int c = check_dense_shape(M, N, K);
  if (c != W8A8_OK) return c;
  if (M == 0 || N == 0) return W8A8_OK;
  if (!x_bf16 || !w_q || !w_scale || !y_bf16) return W8A8_ERR_NULL_ARG;
  if (!aligned16(x_bf16) || !aligned16(w_q) || !aligned16(w_scale) || !aligned16(y_bf16)) return W8A8_ERR_MISALIGNED;
  const bool fp8_path = fast_math != 0 && M > kFastMathMinTokens;
  if (fp8_path) {
    if (!workspace) return W8A8_ERR_NULL_ARG;
    if (!aligned16(workspace)) return W8A8_ERR_MISALIGNED;
    if (workspace_bytes < fp8_linear_workspace_bytes(M, K)) return W8A8_ERR_WORKSPACE;
  }
  const int d = check_device();
  if (d != W8A8_OK) return d;
  if (!fp8_path) return launch_status(w8a8::launch_w8a16_gemm(x_bf16, w_q, w_scale, y_bf16, M, N, K, stream));
  // Up to 16 rows the fused kernel (quantisation inside the weight-streaming
  // GEMM, same bits) is the faster of the two: 7.9 / 8.6 us against 8.9 /
  // 9.6 us for the two launches at 9 / 16 rows of an 8192 x 2048 layer; at
  // 32 rows every workgroup's quantisation costs more than the second launch.
  if (M <= kFusedFasterMaxM && K <= w8a8::kFusedDecodeMaxK)
    return launch_status(w8a8::launch_quant_gemm_decode(x_bf16, w_q, w_scale, y_bf16, M, N, K, stream));
  uint8_t* xq = static_cast<uint8_t*>(workspace);
  float* xs = reinterpret_cast<float*>(xq + align256(M * K));
  const hipError_t e = w8a8::launch_quantize_rows(x_bf16, M, K, xq, xs, stream);
  if (e != hipSuccess) return launch_status(e);
  return launch_status(w8a8::launch_gemm(xq, xs, w_q, w_scale, y_bf16, M, N, K, stream));
}

}  // extern "C"

// ---- fp8_linear without allocation ------------------------------------------
namespace {

// The quantised input of fp8_linear_noalloc: codes [M, K], then the M row
// scales, each block 256-byte aligned. One copy per GPU, held until the
// process ends. The name is a host-side stand-in; kernels get the address
// hipGetSymbolAddress reports for the current device.
constexpr int64_t kNoAllocScratchBytes = int64_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::atomic<uint8_t*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// This device's address of `scratch`, looked up once per device (with that
// device current). NULL if the lookup fails.
uint8_t* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (dev < kMaxDevices) {
    uint8_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (dev < kMaxDevices) {
    uint8_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
  }
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (dev < kMaxDevices) g_scratch_ptr[dev].store(static_cast<uint8_t*>(ptr), std::memory_order_release);
  return static_cast<uint8_t*>(ptr);
}

}  // namespace

extern "C" {

size_t fp8_linear_noalloc_max_bytes(void) { return (size_t)kNoAllocScratchBytes; }

int fp8_linear_noalloc(const uint16_t* x_bf16, const uint8_t* w_q, const float* w_scale, uint16_t* y_bf16, int64_t M,
                       int64_t N, int64_t K, int fast_math, hipStream_t stream) {
  const int c = check_dense_shape(M, N, K);
  if (c != W8A8_OK) return c;
  const bool fp8_path = fast_math != 0 && M > kFastMathMinTokens;
  const bool needs_scratch = fp8_path && !(M <= kFusedFasterMaxM && K <= w8a8::kFusedDecodeMaxK);
  if (needs_scratch && fp8_linear_workspace_bytes(M, K) > (size_t)kNoAllocScratchBytes) return W8A8_ERR_SCRATCH;
  if (M == 0 || N == 0) return W8A8_OK;
  if (!x_bf16 || !w_q || !w_scale || !y_bf16) return W8A8_ERR_NULL_ARG;
  if (!aligned16(x_bf16) || !aligned16(w_q) || !aligned16(w_scale) || !aligned16(y_bf16)) return W8A8_ERR_MISALIGNED;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  if (!fp8_path) return launch_status(w8a8::launch_w8a16_gemm(x_bf16, w_q, w_scale, y_bf16, M, N, K, stream));
  if (!needs_scratch)
    return launch_status(w8a8::launch_quant_gemm_decode(x_bf16, w_q, w_scale, y_bf16, M, N, K, stream));
  uint8_t* xq = device_scratch();
  if (!xq) return W8A8_ERR_LAUNCH;
  float* xs = reinterpret_cast<float*>(xq + align256(M * K));
  const hipError_t e = w8a8::launch_quantize_rows(x_bf16, M, K, xq, xs, stream);
  if (e != hipSuccess) return launch_status(e);
  return launch_status(w8a8::launch_gemm(xq, xs, w_q, w_scale, y_bf16, M, N, K, stream));
}

int fp8_linear_single_launch(const uint16_t* x_bf16, const uint8_t* w_q, const float* w_scale, uint16_t* y_bf16,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int c = check_dense_shape(M, N, K);
  if (c != W8A8_OK) return c;
  if (M > w8a8::kFusedDecodeMaxM || K > w8a8::kFusedDecodeMaxK) return W8A8_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return W8A8_OK;
  if (!x_bf16 || !w_q || !w_scale || !y_bf16) return W8A8_ERR_NULL_ARG;
  if (!aligned16(x_bf16) || !aligned16(w_q) || !aligned16(w_scale) || !aligned16(y_bf16)) return W8A8_ERR_MISALIGNED;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_quant_gemm_decode(x_bf16, w_q, w_scale, y_bf16, M, N, K, stream));
}

}  // extern "C"

// ---- routed experts ---------------------------------------------------------
namespace {

constexpr int64_t kMaxExperts = 1024;
constexpr int64_t kMaxGroups = 1024;  // routing groups: E, or topk * E in slot-position-major order
constexpr int64_t kMaxTopk = 64;
constexpr int64_t kFusedIMultiple = 128;  // a gate/up tile holds 128 h columns (256 weight rows)

// Shared checks of the routed-expert calls. Returns W8A8_OK or a status.
int check_moe_shape(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk) {
  if (T < 0 || H < 0 || I < 0 || E < 0 || topk < 0) return W8A8_ERR_BAD_SHAPE;
  if (!mul_ok(T, topk) || !mul_ok(T, H) || !mul_ok(T * H, 4)) return W8A8_ERR_BAD_SHAPE;
  if (E < 1 || E > kMaxExperts || topk < 1 || topk > kMaxTopk) return W8A8_ERR_UNSUPPORTED;
  if (H == 0 || H % 16 != 0 || I == 0 || I % 16 != 0) return W8A8_ERR_UNSUPPORTED;
  // 32-bit element offsets inside the kernels
  if (T * topk > INT32_MAX || T * H > INT32_MAX || 2 * I * H > INT32_MAX || T * topk * I > INT64_C(1) << 40)
    return W8A8_ERR_UNSUPPORTED;
  if (!mul_ok(E * 2 * I, H)) return W8A8_ERR_BAD_SHAPE;
  return W8A8_OK;
}

bool all_aligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!aligned16(p)) return false;
  return true;
}

bool any_null(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p) return true;
  return false;
}

}  // namespace

extern "C" {

size_t moe_route_workspace_bytes(int64_t T, int64_t topk, int64_t E, int order) {
  if (T < 0 || topk < 1 || E < 1 || !mul_ok(T, topk) || (order != 0 && order != 1)) return 0;
  return w8a8::route_workspace_bytes(T, topk, w8a8::route_groups(topk, E, order));
}

int moe_route(const int32_t* topk_ids, int64_t T, int64_t topk, int64_t E, int order, int32_t* counts,
              int32_t* offsets, int32_t* perm, int32_t* slot_row, void* workspace, size_t workspace_bytes,
              hipStream_t stream) {
  if (T < 0 || topk < 0 || E < 0 || !mul_ok(T, topk)) return W8A8_ERR_BAD_SHAPE;
  if (E < 1 || E > kMaxExperts || topk < 1 || topk > kMaxTopk || T * topk > INT32_MAX) return W8A8_ERR_UNSUPPORTED;
  if (order != 0 && order != 1) return W8A8_ERR_UNSUPPORTED;
  if (w8a8::route_groups(topk, E, order) > kMaxGroups) return W8A8_ERR_UNSUPPORTED;
  if (T == 0) return W8A8_OK;
  if (any_null({topk_ids, counts, offsets, perm, workspace})) return W8A8_ERR_NULL_ARG;
  if (!all_aligned({topk_ids, counts, offsets, perm, slot_row, workspace})) return W8A8_ERR_MISALIGNED;
  if (workspace_bytes < w8a8::route_workspace_bytes(T, topk, w8a8::route_groups(topk, E, order)))
    return W8A8_ERR_WORKSPACE;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(
      w8a8::launch_route(topk_ids, T, topk, E, order, counts, offsets, perm, slot_row, workspace, stream));
}

int moe_gate_up_bf16(const uint8_t* x_q, const float* x_scale, const int32_t* perm, const int32_t* offsets,
                     const uint8_t* w13_q, const float* w13_scale, uint16_t* gu_bf16, int64_t T, int64_t H, int64_t I,
                     int64_t E, int64_t topk, int order, hipStream_t stream) {
  const int c = check_moe_shape(T, H, I, E, topk);
  if (c != W8A8_OK) return c;
  if ((order != 0 && order != 1) || w8a8::route_groups(topk, E, order) > kMaxGroups) return W8A8_ERR_UNSUPPORTED;
  if (T == 0) return W8A8_OK;
  if (any_null({x_q, x_scale, perm, offsets, w13_q, w13_scale, gu_bf16})) return W8A8_ERR_NULL_ARG;
  if (!all_aligned({x_q, x_scale, perm, offsets, w13_q, w13_scale, gu_bf16})) return W8A8_ERR_MISALIGNED;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(
      w8a8::launch_grouped_gate_up_bf16(x_q, x_scale, perm, offsets, w13_q, w13_scale, gu_bf16, T, H, I, E, topk, order,
                                        stream));
}

size_t moe_gate_up_swiglu_quant_workspace_bytes(int64_t T, int64_t I, int64_t topk) {
  if (T < 0 || I < 0 || topk < 1 || !mul_ok(T, topk) || !mul_ok(T * topk, I) || !mul_ok(T * topk * I, 4)) return 0;
  return w8a8::gate_up_swiglu_quant_workspace_bytes(T, I, topk);
}

int moe_gate_up_swiglu_quant(const uint8_t* x_q, const float* x_scale, const int32_t* perm, const int32_t* offsets,
                             const int32_t* dst_row, const uint8_t* w13_q, const float* w13_scale, uint8_t* h_q,
                             float* h_scale, float* h_f32, int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                             int order, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int c = check_moe_shape(T, H, I, E, topk);
  if (c != W8A8_OK) return c;
  if ((order != 0 && order != 1) || w8a8::route_groups(topk, E, order) > kMaxGroups) return W8A8_ERR_UNSUPPORTED;
  if (I % kFusedIMultiple != 0) return W8A8_ERR_UNSUPPORTED;
  if (T == 0) return W8A8_OK;
  if (any_null({x_q, x_scale, perm, offsets, w13_q, w13_scale, h_q, h_scale, workspace})) return W8A8_ERR_NULL_ARG;
  if (!all_aligned({x_q, x_scale, perm, offsets, dst_row, w13_q, w13_scale, h_q, h_scale, h_f32, workspace}))
    return W8A8_ERR_MISALIGNED;
  if (workspace_bytes < w8a8::gate_up_swiglu_quant_workspace_bytes(T, I, topk)) return W8A8_ERR_WORKSPACE;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_gate_up_swiglu_quant(x_q, x_scale, perm, offsets, dst_row, w13_q, w13_scale, h_q,
                                                         h_scale, h_f32, T, H, I, E, topk, order, workspace, stream));
}

int moe_down_combine(const uint8_t* h_q, const float* h_scale, const int32_t* perm, const int32_t* offsets,
                     const int32_t* topk_ids, const float* topk_w, const uint8_t* w2_q, const float* w2_scale,
                     uint16_t* out_bf16, float* y_f32, int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                     int order, hipStream_t stream) {
  const int c = check_moe_shape(T, H, I, E, topk);
  if (c != W8A8_OK) return c;
  if ((order != 0 && order != 1) || w8a8::route_groups(topk, E, order) > kMaxGroups) return W8A8_ERR_UNSUPPORTED;
  if (!mul_ok(T * topk, H) || !mul_ok(T * topk * H, 4)) return W8A8_ERR_BAD_SHAPE;
  if (T == 0) return W8A8_OK;
  if (any_null({h_q, h_scale, perm, offsets, topk_ids, topk_w, w2_q, w2_scale, out_bf16, y_f32}))
    return W8A8_ERR_NULL_ARG;
  if (!all_aligned({h_q, h_scale, perm, offsets, topk_ids, topk_w, w2_q, w2_scale, out_bf16, y_f32}))
    return W8A8_ERR_MISALIGNED;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_down_combine(h_q, h_scale, perm, offsets, topk_ids, topk_w, w2_q, w2_scale,
                                                 out_bf16, y_f32, nullptr, nullptr, T, H, I, E, topk, order, stream,
                                                 nullptr));
}

size_t w8a8_grouped_gemm_workspace_bytes(int64_t T, int64_t topk, int64_t E) {
  if (T < 0 || topk < 1 || E < 1 || !mul_ok(T, topk)) return 0;
  return w8a8::grouped_gate_up_workspace_bytes(T, topk, E);
}

int w8a8_grouped_gemm(const uint8_t* x_q, const float* x_scale, const int32_t* topk_ids, const uint8_t* w13_q,
                      const float* w13_scale, uint16_t* gu_bf16, int32_t* perm, int32_t* offsets, int64_t T,
                      int64_t H, int64_t I, int64_t E, int64_t topk, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  const int c = check_moe_shape(T, H, I, E, topk);
  if (c != W8A8_OK) return c;
  if (T == 0) return W8A8_OK;
  if (any_null({x_q, x_scale, topk_ids, w13_q, w13_scale, gu_bf16, perm, offsets, workspace})) return W8A8_ERR_NULL_ARG;
  if (!all_aligned({x_q, x_scale, topk_ids, w13_q, w13_scale, gu_bf16, perm, offsets, workspace}))
    return W8A8_ERR_MISALIGNED;
  if (workspace_bytes < w8a8::grouped_gate_up_workspace_bytes(T, topk, E)) return W8A8_ERR_WORKSPACE;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_grouped_gate_up(x_q, x_scale, topk_ids, w13_q, w13_scale, gu_bf16, perm, offsets,
                                                    T, H, I, E, topk, workspace, stream));
}

size_t moe_w8a8_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk) {
  if (check_moe_shape(T, H, I, E, topk) != W8A8_OK || !mul_ok(T * topk, H) || !mul_ok(T * topk * H, 4)) return 0;
  return w8a8::moe_workspace_bytes(T, H, I, E, topk);
}

int moe_w8a8_grouped(const uint8_t* x_q, const float* x_scale, const int32_t* topk_ids, const float* topk_w,
                     const uint8_t* w13_q, const float* w13_scale, const uint8_t* w2_q, const float* w2_scale,
                     uint16_t* out_bf16, uint8_t* out_q, float* out_scale, int64_t T, int64_t H, int64_t I, int64_t E,
                     int64_t topk, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int c = check_moe_shape(T, H, I, E, topk);
  if (c != W8A8_OK) return c;
  if (I % kFusedIMultiple != 0) return W8A8_ERR_UNSUPPORTED;
  if (!mul_ok(T * topk, H) || !mul_ok(T * topk * H, 4)) return W8A8_ERR_BAD_SHAPE;
  if (T == 0) return W8A8_OK;
  if (any_null({x_q, x_scale, topk_ids, topk_w, w13_q, w13_scale, w2_q, w2_scale, out_bf16, workspace}))
    return W8A8_ERR_NULL_ARG;
  if ((out_q == nullptr) != (out_scale == nullptr)) return W8A8_ERR_NULL_ARG;
  if (!all_aligned({x_q, x_scale, topk_ids, topk_w, w13_q, w13_scale, w2_q, w2_scale, out_bf16, out_q, out_scale,
                    workspace}))
    return W8A8_ERR_MISALIGNED;
  if (workspace_bytes < w8a8::moe_workspace_bytes(T, H, I, E, topk)) return W8A8_ERR_WORKSPACE;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_moe(x_q, x_scale, topk_ids, topk_w, w13_q, w13_scale, w2_q, w2_scale, out_bf16,
                                        out_q, out_scale, T, H, I, E, topk, workspace, stream));
}

}  // extern "C"

// ---- MXFP4 routed experts -----------------------------------------------------
namespace {

constexpr int64_t kMxMultiple = 128;  // one FP4 matrix-core step along K; a gate/up tile holds 128 h columns

int check_mx_moe(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk, int order) {
  const int c = check_moe_shape(T, H, I, E, topk);
  if (c != W8A8_OK) return c;
  if (H % kMxMultiple != 0 || I % kMxMultiple != 0) return W8A8_ERR_UNSUPPORTED;
  if ((order != 0 && order != 1) || w8a8::route_groups(topk, E, order) > kMaxGroups) return W8A8_ERR_UNSUPPORTED;
  if (!mul_ok(T * topk, H) || !mul_ok(T * topk * H, 4)) return W8A8_ERR_BAD_SHAPE;
  return W8A8_OK;
}

}  // namespace

extern "C" {

int mxfp4_quantize(const uint16_t* x_bf16, int64_t M, int64_t K, uint8_t* q_fp4, uint8_t* scale_e8m0,
                   hipStream_t stream) {
  if (M < 0 || K < 0 || !mul_ok(M, K) || !mul_ok(M * K, 2)) return W8A8_ERR_BAD_SHAPE;
  if (K == 0 || K % 32 != 0 || K > (int64_t(1) << 24)) return W8A8_ERR_UNSUPPORTED;
  if (M * K / 8 >= (int64_t(1) << 40)) return W8A8_ERR_UNSUPPORTED;
  if (M == 0) return W8A8_OK;
  if (any_null({x_bf16, q_fp4, scale_e8m0})) return W8A8_ERR_NULL_ARG;
  if (!all_aligned({x_bf16, q_fp4, scale_e8m0})) return W8A8_ERR_MISALIGNED;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_mx_quantize(x_bf16, M, K, q_fp4, scale_e8m0, stream));
}

int moe_mxfp4_gate_up_bf16(const uint8_t* x_q, const uint8_t* x_scale, const int32_t* perm, const int32_t* offsets,
                           const uint8_t* w13_q, const uint8_t* w13_scale, uint16_t* gu_bf16, int64_t T, int64_t H,
                           int64_t I, int64_t E, int64_t topk, int order, hipStream_t stream) {
  const int c = check_mx_moe(T, H, I, E, topk, order);
  if (c != W8A8_OK) return c;
  if (T == 0) return W8A8_OK;
  if (any_null({x_q, x_scale, perm, offsets, w13_q, w13_scale, gu_bf16})) return W8A8_ERR_NULL_ARG;
  if (!all_aligned({x_q, x_scale, perm, offsets, w13_q, w13_scale, gu_bf16})) return W8A8_ERR_MISALIGNED;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_mx_gate_up_bf16(x_q, x_scale, perm, offsets, w13_q, w13_scale, gu_bf16, T, H, I, E,
                                                    topk, order, stream));
}

int moe_mxfp4_gate_up_swiglu_quant(const uint8_t* x_q, const uint8_t* x_scale, const int32_t* perm,
                                   const int32_t* offsets, const int32_t* dst_row, const uint8_t* w13_q,
                                   const uint8_t* w13_scale, uint8_t* h_q, uint8_t* h_scale, int64_t T, int64_t H,
                                   int64_t I, int64_t E, int64_t topk, int order, hipStream_t stream) {
  const int c = check_mx_moe(T, H, I, E, topk, order);
  if (c != W8A8_OK) return c;
  if (T == 0) return W8A8_OK;
  if (any_null({x_q, x_scale, perm, offsets, w13_q, w13_scale, h_q, h_scale})) return W8A8_ERR_NULL_ARG;
  if (!all_aligned({x_q, x_scale, perm, offsets, dst_row, w13_q, w13_scale, h_q, h_scale}))
    return W8A8_ERR_MISALIGNED;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_mx_gate_up_swiglu_quant(x_q, x_scale, perm, offsets, dst_row, w13_q, w13_scale,
                                                            h_q, h_scale, T, H, I, E, topk, order, stream));
}

int moe_mxfp4_down_combine(const uint8_t* h_q, const uint8_t* h_scale, const int32_t* perm, const int32_t* offsets,
                           const int32_t* topk_ids, const float* topk_w, const uint8_t* w2_q, const uint8_t* w2_scale,
                           uint16_t* out_bf16, float* y_f32, uint8_t* out_q, uint8_t* out_scale, int64_t T, int64_t H,
                           int64_t I, int64_t E, int64_t topk, int order, hipStream_t stream) {
  const int c = check_mx_moe(T, H, I, E, topk, order);
  if (c != W8A8_OK) return c;
  if (T == 0) return W8A8_OK;
  if (any_null({h_q, h_scale, perm, offsets, topk_ids, topk_w, w2_q, w2_scale, out_bf16, y_f32}))
    return W8A8_ERR_NULL_ARG;
  if ((out_q == nullptr) != (out_scale == nullptr)) return W8A8_ERR_NULL_ARG;
  if (!all_aligned({h_q, h_scale, perm, offsets, topk_ids, topk_w, w2_q, w2_scale, out_bf16, y_f32, out_q, out_scale}))
    return W8A8_ERR_MISALIGNED;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_mx_down_combine(h_q, h_scale, perm, offsets, topk_ids, topk_w, w2_q, w2_scale,
                                                    out_bf16, y_f32, out_q, out_scale, T, H, I, E, topk, order,
                                                    stream, nullptr));
}

size_t moe_mxfp4_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk) {
  if (check_mx_moe(T, H, I, E, topk, 0) != W8A8_OK) return 0;
  return w8a8::mx_moe_workspace_bytes(T, H, I, E, topk);
}

int moe_mxfp4_grouped(const uint8_t* x_q, const uint8_t* x_scale, const int32_t* topk_ids, const float* topk_w,
                      const uint8_t* w13_q, const uint8_t* w13_scale, const uint8_t* w2_q, const uint8_t* w2_scale,
                      uint16_t* out_bf16, uint8_t* out_q, uint8_t* out_scale, int64_t T, int64_t H, int64_t I,
                      int64_t E, int64_t topk, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int c = check_mx_moe(T, H, I, E, topk, 0);
  if (c != W8A8_OK) return c;
  if (T == 0) return W8A8_OK;
  if (any_null({x_q, x_scale, topk_ids, topk_w, w13_q, w13_scale, w2_q, w2_scale, out_bf16, workspace}))
    return W8A8_ERR_NULL_ARG;
  if ((out_q == nullptr) != (out_scale == nullptr)) return W8A8_ERR_NULL_ARG;
  if (!all_aligned({x_q, x_scale, topk_ids, topk_w, w13_q, w13_scale, w2_q, w2_scale, out_bf16, out_q, out_scale,
                    workspace}))
    return W8A8_ERR_MISALIGNED;
  if (workspace_bytes < w8a8::mx_moe_workspace_bytes(T, H, I, E, topk)) return W8A8_ERR_WORKSPACE;
  const int d = check_device();
  if (d != W8A8_OK) return d;
  return launch_status(w8a8::launch_mx_moe(x_q, x_scale, topk_ids, topk_w, w13_q, w13_scale, w2_q, w2_scale, out_bf16,
                                           out_q, out_scale, T, H, I, E, topk, workspace, stream));
}

}  // extern "C"
