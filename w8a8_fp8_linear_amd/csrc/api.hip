// The C ABI of libw8a8.so (include/w8a8.h): argument checks on the host,
// the gfx950 device check, then one launcher per entry point.
#include <string.h>

#include <atomic>

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

int w8a8_gemm(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q, const float* w_scale,
              uint16_t* y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
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
  return launch_status(w8a8::launch_gemm(a_q, a_scale, w_q, w_scale, y_bf16, M, N, K, stream));
}

}  // extern "C"
