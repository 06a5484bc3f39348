// The default maths: Y[m, n] = bf16( sw[n] * sum_k x[m, k] * dec(W[n, k]) ).
//
// Without the fast-math flag the model page's runtime widens the FP8 weights
// to 16 bits as it multiplies and runs the product in BF16, so the weights
// are the only rounded operand (Lernex/Metis-1.6-Logos-FP8, "What
// --fast-math does"). Here every E4M3 weight byte is widened to BF16 in
// registers (exact: each E4M3 value is a BF16 value) and the product runs on
// the 16x16x32 BF16 MFMA with float32 accumulators; the activations are used
// as given, with no quantisation and no activation scale.
//
// Two kernels, the same split as the FP8 path:
//  * w8a16_tiled: many tokens. 256 x 192 tiles, 2 x 4 waves of 128 x 48; each
//    64-deep K step stages the BF16 activation rows (128 bytes) and the E4M3
//    weight rows (64 bytes) global -> LDS with direct buffer loads, double
//    buffered. A lane reads 16 weight bytes (K 16g .. 16g + 15 of its row, g =
//    lane / 16) and the matching 16 activation values, widens the weights, and
//    issues two MFMAs, one per half of that K range. Both operands use the
//    same K assignment, so each pair of MFMAs sums the whole 64-deep step.
//  * w8a16_skinny: at most 32 tokens (decode), limited by the weight stream
//    (the model page: generation for a single conversation is set by how fast
//    the weights are read, "What --fast-math does"). 16 weight rows per
//    workgroup, the 4 waves split K, every lane loads its weight bytes and
//    activation values straight from global memory.
#include "device.h"
#include "launch.h"

namespace w8a8 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ inline v4f mfma_16x16x32_bf16(v4i a, v4i b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Two float32 values that are exact in BF16 -> their BF16 halves packed (a in the low half).
__device__ inline uint32_t pack_bf16(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// 8 E4M3 codes (bytes of w0 then w1, value 0 in the low byte) -> 8 BF16 values.
// The hardware conversion decodes E4M3 exactly into float32 (checked on gfx950
// against the format's definition for all 256 codes).
__device__ inline v4i widen8(uint32_t w0, uint32_t w1) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
  return v4i{(int)pack_bf16(a[0], a[1]), (int)pack_bf16(b[0], b[1]), (int)pack_bf16(c[0], c[1]),
             (int)pack_bf16(d[0], d[1])};
}

// 64-byte weight rows: 16-byte chunk c of row r sits at c ^ ((r >> 1) & 3), so
// 8 consecutive rows at one logical chunk cover 8 different 16-byte bank
// groups of a 128-byte bank window.
__device__ inline int wrow_off(int row, int c) { return row * 64 + ((c ^ ((row >> 1) & 3)) << 4); }

template <int BM, int BN, int WGM, int WGN>
struct Tiled16 {
  static constexpr int kThreads = 64 * WGM * WGN;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int SM = WM / 16, SN = WN / 16;
  static constexpr int kWBytes = BN * 64;               // E4M3 weight part of a stage
  static constexpr int kStage = kWBytes + BM * 128;     // + BF16 activation part
  static constexpr int kSlotsW = BN * 4, kSlots = kSlotsW + BM * 8;  // 16-byte LDS slots
  static constexpr int kLoads = (kSlots + kThreads - 1) / kThreads;
  static constexpr int kEpiStride = BN * 2 + 16;
  static constexpr int kEpi = BM * kEpiStride;
  static constexpr int kLds = (2 * kStage > kEpi) ? 2 * kStage : kEpi;
  static_assert(kSlotsW % 64 == 0 && kSlots % 64 == 0, "every load instruction must stay in one part");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
};

template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(1, 2)))
void w8a16_tiled(const uint16_t* __restrict__ X, const uint8_t* __restrict__ W, const float* __restrict__ sw,
                 uint16_t* __restrict__ Y, int M, int N, int K, int tiles_m, int tiles_n) {
  using C = Tiled16<BM, BN, WGM, WGN>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLds];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  map_tile<4>(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const auto rW = make_rsrc(W + (int64_t)n0 * K, (int64_t)(N - n0) * K);
  const auto rX = make_rsrc(X + (int64_t)m0 * K, (int64_t)(M - m0) * K * 2);
  const uint32_t xrow = (uint32_t)K * 2u;  // bytes per activation row

  // Loader: slot s = tid + kThreads * i. Slots [0, kSlotsW) are weight row
  // s / 4, physical chunk s % 4; the rest are activation row s' / 8, physical
  // chunk s' % 8 (s' = s - kSlotsW). Each lane loads the global chunk that
  // belongs in its slot (the inverse of the read swizzle). A wave's 64 slots
  // never straddle the two parts, so the part is wave-uniform.
  uint32_t off[C::kLoads];  // byte offset of the slot's chunk in the first K step
  int kc[C::kLoads];        // first K index of that chunk inside a step
  bool isw[C::kLoads], live[C::kLoads];
#pragma unroll
  for (int i = 0; i < C::kLoads; ++i) {
    const int s = tid + C::kThreads * i;
    live[i] = s < C::kSlots;
    isw[i] = s < C::kSlotsW;
    if (isw[i]) {
      const int row = s >> 2, c = (s & 3) ^ ((row >> 1) & 3);  // 16 E4M3 values per chunk
      kc[i] = c << 4;
      off[i] = (uint32_t)row * (uint32_t)K + (uint32_t)kc[i];
    } else {
      const int s2 = s - C::kSlotsW, row = s2 >> 3, c = (s2 & 7) ^ (row & 7);  // 8 BF16 values per chunk
      kc[i] = c << 3;
      off[i] = (uint32_t)row * xrow + (uint32_t)(c << 4);
    }
  }
  auto issue = [&](int stage, int k0) {  // k0: first K index of the step
    uint8_t* base = smem + stage * C::kStage;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      if (!live[i]) continue;
      const int s0 = wave * 64 + C::kThreads * i;
      const bool kin = k0 + kc[i] < K;  // K is a multiple of 16: a chunk is all in or all out
      if (isw[i]) {
        buffer_load16_lds(rW, base + s0 * 16, kin ? off[i] + (uint32_t)k0 : kOutOfRange);
      } else {
        buffer_load16_lds(rX, base + C::kWBytes + (s0 - C::kSlotsW) * 16, kin ? off[i] + (uint32_t)k0 * 2u : kOutOfRange);
      }
    }
  };

  const int wm = wave % WGM, wn = wave / WGM;
  const int r16 = lane & 15, g = lane >> 4;
  v4f acc[C::SN][C::SM];
#pragma unroll
  for (int i = 0; i < C::SN; ++i)
#pragma unroll
    for (int j = 0; j < C::SM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // The epilogue's weight-row scales are loaded before the K loop, so that
  // their latency passes under it.
  float4 sWv[C::SN];
#pragma unroll
  for (int i = 0; i < C::SN; ++i) {
    const int nl = wn * C::WN + i * 16 + 4 * g;
    sWv[i] = n0 + nl < N ? *reinterpret_cast<const float4*>(sw + n0 + nl) : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  const int nk = (K + 63) >> 6;
  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmem_all();
    __syncthreads();
    if (kt + 1 < nk) issue((kt + 1) & 1, (kt + 1) << 6);
    const uint8_t* st = smem + (kt & 1) * C::kStage;
    const uint8_t* sx = st + C::kWBytes;
    v4i xlo[C::SM], xhi[C::SM];
#pragma unroll
    for (int j = 0; j < C::SM; ++j) {
      const int row = wm * C::WM + j * 16 + r16;
      xlo[j] = *reinterpret_cast<const v4i*>(sx + stage_off(row, 2 * g));
      xhi[j] = *reinterpret_cast<const v4i*>(sx + stage_off(row, 2 * g + 1));
    }
#pragma unroll
    for (int i = 0; i < C::SN; ++i) {
      const int row = wn * C::WN + i * 16 + r16;
      const v4i w = *reinterpret_cast<const v4i*>(st + wrow_off(row, g));
      const v4i wlo = widen8((uint32_t)w.x, (uint32_t)w.y), whi = widen8((uint32_t)w.z, (uint32_t)w.w);
#pragma unroll
      for (int j = 0; j < C::SM; ++j) {
        acc[i][j] = mfma_16x16x32_bf16(wlo, xlo[j], acc[i][j]);
        acc[i][j] = mfma_16x16x32_bf16(whi, xhi[j], acc[i][j]);
      }
    }
  }

  // Epilogue: acc[i][j][r] = Y[m][n], m = m-tile j row lane % 16, n = n-tile i,
  // 4 * (lane / 16) + r. Scale, round to BF16, stage in LDS, store row segments.
  __syncthreads();
#pragma unroll
  for (int i = 0; i < C::SN; ++i) {
    const int nl = wn * C::WN + i * 16 + 4 * g;
    const float4 s = sWv[i];
#pragma unroll
    for (int j = 0; j < C::SM; ++j) {
      const int ml = wm * C::WM + j * 16 + r16;
      const v4f a = acc[i][j];
      const uint32_t p0 = bf16x2_rne(a[0] * s.x, a[1] * s.y);
      const uint32_t p1 = bf16x2_rne(a[2] * s.z, a[3] * s.w);
      *reinterpret_cast<uint2*>(smem + ml * C::kEpiStride + nl * 2) = make_uint2(p0, p1);
    }
  }
  __syncthreads();
  constexpr int kRowChunks = BN / 8;
  for (int c = tid; c < BM * kRowChunks; c += C::kThreads) {
    const int row = c / kRowChunks, col = (c % kRowChunks) * 8;
    const int m = m0 + row, n = n0 + col;
    if (m < M && n < N)
      *reinterpret_cast<uint4*>(Y + (int64_t)m * N + n) =
          *reinterpret_cast<const uint4*>(smem + row * C::kEpiStride + col * 2);
  }
}

// Small M: 16 weight rows per workgroup, K split over the 4 waves in 64-deep
// blocks, U blocks of loads in flight per wave. MT = number of 16-token tiles.
template <int MT, int U>
__global__ __launch_bounds__(256) void w8a16_skinny(const uint16_t* __restrict__ X, const uint8_t* __restrict__ W,
                                                    const float* __restrict__ sw, uint16_t* __restrict__ Y, int M,
                                                    int N, int K) {
  __shared__ v4f red[3][MT][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16;
  const auto rW = make_rsrc(W + (int64_t)n0 * K, (int64_t)(N - n0) * K);
  const auto rX = make_rsrc(X, (int64_t)M * K * 2);
  const int r16 = lane & 15, g = lane >> 4;
  const uint32_t wrow = (uint32_t)r16 * (uint32_t)K;
  // the epilogue's weight scales first, so that their latency overlaps the stream
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (wave == 0 && n0 + 4 * g < N) s = *reinterpret_cast<const float4*>(sw + n0 + 4 * g);
  v4f acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  const int nk = (K + 63) >> 6;
  for (int kt = wave; kt < nk; kt += 4 * U) {
    v4i wv[U], xl[U][MT], xh[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = ((kt + 4 * u) << 6) + 16 * g;  // this lane's 16 K values
      const bool live = kt + 4 * u < nk && k < K;
      wv[u] = buffer_load16(rW, live ? wrow + (uint32_t)k : kOutOfRange);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const uint32_t xo = (uint32_t)(t * 16 + r16) * (uint32_t)K * 2u + (uint32_t)k * 2u;
        xl[u][t] = buffer_load16(rX, live ? xo : kOutOfRange);
        xh[u][t] = buffer_load16(rX, live ? xo + 16u : kOutOfRange);
      }
    }
    // every load of this round ahead of the first MFMA: bytes in flight are the limit
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const v4i wlo = widen8((uint32_t)wv[u].x, (uint32_t)wv[u].y);
      const v4i whi = widen8((uint32_t)wv[u].z, (uint32_t)wv[u].w);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        acc[t] = mfma_16x16x32_bf16(wlo, xl[u][t], acc[t]);
        acc[t] = mfma_16x16x32_bf16(whi, xh[u][t], acc[t]);
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t) red[wave - 1][t][lane] = acc[t];
  }
  __syncthreads();
  if (wave != 0) return;
  const int n = n0 + 4 * g;
  if (n >= N) return;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const v4f a = acc[t] + red[0][t][lane] + red[1][t][lane] + red[2][t][lane];
    const int m = t * 16 + r16;
    if (m < M) {
      const uint32_t p0 = bf16x2_rne(a[0] * s.x, a[1] * s.y);
      const uint32_t p1 = bf16x2_rne(a[2] * s.z, a[3] * s.w);
      *reinterpret_cast<uint2*>(Y + (int64_t)m * N + n) = make_uint2(p0, p1);
    }
  }
}

}  // namespace

hipError_t launch_w8a16_gemm(const uint16_t* x, const uint8_t* w, const float* sw, uint16_t* y, int64_t M, int64_t N,
                             int64_t K, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const dim3 skinny_grid((unsigned)((N + 15) / 16));
  if (M <= 16) {
    hipLaunchKernelGGL((w8a16_skinny<1, 4>), skinny_grid, dim3(256), 0, stream, x, w, sw, y, (int)M, (int)N, (int)K);
    return hipGetLastError();
  }
  if (M <= 32) {
    hipLaunchKernelGGL((w8a16_skinny<2, 4>), skinny_grid, dim3(256), 0, stream, x, w, sw, y, (int)M, (int)N, (int)K);
    return hipGetLastError();
  }
  constexpr int BM = 256, BN = 192;
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  hipLaunchKernelGGL((w8a16_tiled<BM, BN, 2, 4>), dim3(tiles_m * tiles_n), dim3(512), 0, stream, x, w, sw, y, (int)M,
                     (int)N, (int)K, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace w8a8
