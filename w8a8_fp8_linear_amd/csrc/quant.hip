// Per-row dynamic FP8 quantisation (activations per token, weights per
// output row).
//
// The pages quantise activations per token at run time and give the
// weights a scale for each output channel (Lernex/Metis-1.6-Logos-FP8, "What is in FP8";
// Lernex/Metis-1.6-Praxis-NVFP4, "What is in NVFP4": one scale per output
// row). For a row x: amax = max|x| (exact, on the BF16 bit patterns),
// s = fl32(amax / 448) (s = 1 for an all-zero row), q = E4M3(fl32(x / s))
// with round to nearest even and saturation at 448.
//
// One wave per row: BF16 is read with 16-byte loads (8 values per lane per
// load) and kept in registers, amax is a wave-wide max, then every element
// is scaled and encoded (rows longer than 64 * 8 * 16 values stream through
// twice instead). fl32(x / s) is obtained without a division per
// element: x * r with r = fl32(1 / s), corrected once with its fused
// residual, is the correctly rounded quotient wherever the code depends on
// it (quant8 states the range; rows with a scale below 2^-99 divide). The
// encoding itself is the hardware conversion (round to nearest even) after
// clamping to +-448. An earlier form redid a lane's values with the
// division whenever x * r fell near a rounding boundary or below 2^-6; 0.12%
// of the prefill activations land there after scaling, enough to send 9
// waves in 10 into it, and the 4096 x 2048 quantisation ran at 7.8 us
// against 4.9 us with the correction.
#include "device.h"
#include "launch.h"

namespace w8a8 {
namespace {

constexpr int kRowsPerBlock = 4;  // one wave per row, 256 threads

template <int NCH>
__global__ __launch_bounds__(256) void quant_rows_regs(const uint16_t* __restrict__ x, int64_t M,
                                                        int64_t K, uint8_t* __restrict__ q,
                                                        float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;
  const int nch = (int)(K >> 3);
  const v4i* xr = reinterpret_cast<const v4i*>(x + row * K);
  uint4 v[NCH];
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    v4i t = v4i{0, 0, 0, 0};
    if (c < nch) t = xr[c];
    v[i] = make_uint4((uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w);
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const uint32_t m = absmax8(v[i]);
    amax = amax > m ? amax : m;
  }
  amax = wave_max_u32(amax);
  const float s = row_scale(amax);
  const float r = 1.0f / s;
  uint2* qr = reinterpret_cast<uint2*>(q + row * K);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) qr[c] = quant8(v[i], s, r);
  }
  if (lane == 0) scale[row] = s;
}

__global__ __launch_bounds__(256) void quant_rows_stream(const uint16_t* __restrict__ x, int64_t M,
                                                          int64_t K, uint8_t* __restrict__ q,
                                                          float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;
  const int64_t nch = K >> 3;
  const uint4* xr = reinterpret_cast<const uint4*>(x + row * K);
  uint32_t amax = 0;
  for (int64_t c = lane; c < nch; c += 64) {
    const uint32_t m = absmax8(xr[c]);
    amax = amax > m ? amax : m;
  }
  amax = wave_max_u32(amax);
  const float s = row_scale(amax);
  const float r = 1.0f / s;
  uint2* qr = reinterpret_cast<uint2*>(q + row * K);
  for (int64_t c = lane; c < nch; c += 64) qr[c] = quant8(xr[c], s, r);
  if (lane == 0) scale[row] = s;
}

// The two conversions every output of this library ends with, applied to
// caller-given float32 values: the E4M3 encoding of the quantisers (clamp
// to +-448, then the hardware round-to-nearest-even conversion, e4m3x4) and
// the BF16 rounding of every BF16 result (bf16x2_rne). Four values per
// thread; the tail is guarded per element.
__global__ __launch_bounds__(256) void convert_e4m3(const float* __restrict__ v, int64_t n, uint8_t* __restrict__ q) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float a[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) a[k] = i + k < n ? clamp448(v[i + k]) : 0.f;
  const uint32_t w = e4m3x4(a[0], a[1], a[2], a[3]);
  if (i + 4 <= n) {
    *reinterpret_cast<uint32_t*>(q + i) = w;
  } else {
    for (int k = 0; i + k < n; ++k) q[i + k] = (uint8_t)(w >> (8 * k));
  }
}

__global__ __launch_bounds__(256) void convert_bf16(const float* __restrict__ v, int64_t n, uint16_t* __restrict__ y) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float a[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) a[k] = i + k < n ? v[i + k] : 0.f;
  const uint32_t lo = bf16x2_rne(a[0], a[1]), hi = bf16x2_rne(a[2], a[3]);
  if (i + 4 <= n) {
    *reinterpret_cast<uint2*>(y + i) = make_uint2(lo, hi);
  } else {
    const uint32_t w[2] = {lo, hi};
    for (int k = 0; i + k < n; ++k) y[i + k] = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
  }
}

}  // namespace

hipError_t launch_convert_e4m3(const float* v, int64_t n, uint8_t* q, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(convert_e4m3, dim3((unsigned)((n + 1023) / 1024)), dim3(256), 0, stream, v, n, q);
  return hipGetLastError();
}

hipError_t launch_convert_bf16(const float* v, int64_t n, uint16_t* y, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(convert_bf16, dim3((unsigned)((n + 1023) / 1024)), dim3(256), 0, stream, v, n, y);
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* scale,
                                hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const dim3 grid((unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock));
  const dim3 block(64 * kRowsPerBlock);
  const int64_t per_lane = (K / 8 + 63) / 64;  // 16-byte chunks per lane
  if (per_lane <= 1)
    hipLaunchKernelGGL(quant_rows_regs<1>, grid, block, 0, stream, x, M, K, q, scale);
  else if (per_lane <= 2)
    hipLaunchKernelGGL(quant_rows_regs<2>, grid, block, 0, stream, x, M, K, q, scale);
  else if (per_lane <= 4)
    hipLaunchKernelGGL(quant_rows_regs<4>, grid, block, 0, stream, x, M, K, q, scale);
  else if (per_lane <= 8)
    hipLaunchKernelGGL(quant_rows_regs<8>, grid, block, 0, stream, x, M, K, q, scale);
  else if (per_lane <= 16)
    hipLaunchKernelGGL(quant_rows_regs<16>, grid, block, 0, stream, x, M, K, q, scale);
  else
    hipLaunchKernelGGL(quant_rows_stream, grid, block, 0, stream, x, M, K, q, scale);
  return hipGetLastError();
}

}  // namespace w8a8
