// Scaled FP8 GEMM: Y[m, n] = bf16( sa[m] * sw[n] * sum_k dec(A[m, k]) * dec(W[n, k]) ).
//
// This is the multiply of the pages' fast-math path: the per-token FP8
// version of a layer's input times the FP8 weights, computed on the FP8
// matrix units (Lernex/Metis-1.6-Logos-FP8, "What --fast-math does"),
// weights stored [out, in], each output row with its own scale (Lernex/Metis-1.6-
// Praxis-NVFP4, "What is in NVFP4"). Both operands are K-contiguous.
//
// Two kernels:
//  * gemm_tiled: many tokens (prompt reading). A workgroup of WGM x WGN
//    waves owns a BM x BN output tile (256 x 192 with 2 x 4 waves, two waves
//    per SIMD). Each 128-deep K step of both operand tiles is copied
//    global -> LDS by buffer loads that write LDS directly (no VGPR
//    staging), double-buffered; each wave runs 16x16x128 E4M3 MFMAs on its
//    (BM/WGM) x (BN/WGN) sub-tile with fp32 accumulators. The two wave
//    groups run a ping-pong schedule: one reads its fragments from LDS while
//    the other issues MFMAs, then they swap. The epilogue applies
//    both scales in fp32, rounds to BF16 and goes through LDS so that every
//    global store is a full 16-byte row segment. Workgroup ids are renumbered
//    so that each of the 8 XCDs walks a compact block of tiles (its own L2).
//  * gemm_skinny: at most 32 tokens (decode). The time is the weight stream:
//    the pages note that single-stream generation is limited by weight
//    bandwidth rather than arithmetic ("What --fast-math does"). A workgroup
//    owns 16 or 32 weight rows, its 4 waves split K, each lane loads its
//    weight operands straight from global memory with 16-byte loads (every
//    weight byte is read once), and the partial sums meet in LDS. The input
//    rows are loaded the same way, or at 17 to 32 rows staged through LDS.
//  * gemm_skinny_q: gemm_skinny with the per-token quantisation of its BF16
//    input fused in (one launch instead of two). For K <= 2048 one round of
//    the skinny loop covers all of K, so the 4 waves of a workgroup load
//    every input element exactly once, as BF16; each lane folds the
//    magnitudes of its chunks into per-row maxima, the maxima meet over the
//    lane groups (shuffles) and the waves (LDS), and each lane then
//    quantises its own chunks with the per-token rule, the same code as
//    quantize_per_token, so the codes and the result are identical to the
//    two-launch chain. Every workgroup quantises the whole input (no
//    workgroup can see another's codes without a grid-wide barrier), which
//    costs more vector-ALU time than the separate quantisation launch saves.
//
// Within one 128-byte K slice, lane group g (lane / 16) of an MFMA operand
// holds the 16-byte chunks g and g + 4 of its row. A and W use the same
// assignment, so the product is the full dot product over the slice.
#include <hip/hip_ext.h>

#include "device.h"
#include "launch.h"

namespace w8a8 {
namespace {

template <int BM, int BN, int WGM, int WGN>
struct Tiled {
  static constexpr int kThreads = 64 * WGM * WGN;
  static constexpr int WM = BM / WGM, WN = BN / WGN;   // per-wave tile
  static constexpr int SM = WM / 16, SN = WN / 16;     // 16x16 MFMA tiles per wave
  static constexpr int kRows = BM + BN;                // rows of one K-slice stage
  static constexpr int kStage = kRows * 128;           // bytes per stage
  static constexpr int kLoaders = kThreads / 2;        // wave group 0 issues the loads
  static constexpr int kRowsPerPass = kLoaders / 8;    // rows one load instruction covers
  static constexpr int kLoadsW = BN / kRowsPerPass;    // W loads per loading thread per stage
  static constexpr int kLoads = kRows / kRowsPerPass;  // all loads per loading thread per stage
  static constexpr int kEpiStride = BN * 2 + 16;       // bytes per staged output row
  static constexpr int kEpi = BM * kEpiStride;
  static constexpr int kLds = (2 * kStage > kEpi) ? 2 * kStage : kEpi;
  static_assert(WGM == 2, "the ping-pong schedule needs two wave groups");
  static_assert(BN % kRowsPerPass == 0 && BM % kRowsPerPass == 0, "stage must split evenly over the loaders");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
};

template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(1, 2)))
void gemm_tiled(const uint8_t* __restrict__ A, const float* __restrict__ sa,
                const uint8_t* __restrict__ W, const float* __restrict__ sw,
                uint16_t* __restrict__ Y, int M, int N, int K, int tiles_m, int tiles_n) {
  using C = Tiled<BM, BN, WGM, WGN>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLds];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps rsrc / LDS bases scalar
  int tm, tn;
  map_tile<4>(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const auto rW = make_rsrc(W + (int64_t)n0 * K, (int64_t)(N - n0) * K);
  const auto rA = make_rsrc(A + (int64_t)m0 * K, (int64_t)(M - m0) * K);

  // Ping-pong schedule. Wave group 0 (waves 0..WGN-1, the tile's top BM/2
  // rows) and group 1 (the rest) hold one wave per SIMD each and alternate:
  // while one group reads its fragments of a K step from LDS, the other runs
  // the MFMAs of the step it read before, so each SIMD's matrix unit is fed
  // while its other wave reads. Group 0 also issues every global -> LDS load,
  // one K step ahead. Step kt's stage is read by group 0 in phase 2 kt and by
  // group 1 in phase 2 kt + 1; the loads of step kt + 1 go to the other
  // stage at the start of phase 2 kt (both groups finished reading it by the
  // end of phase 2 kt - 1) and are waited for at the end of phase 2 kt + 1.
  // Every wave passes 2 nk + 2 barriers.
  //
  // Loader (group 0's threads, tid < kLoaders): slot s = tid + kLoaders * i
  // is a 16-byte LDS slot; rows 0..BN-1 of a stage hold W, rows BN.. hold A.
  // Lanes of a wave fill consecutive slots (8 rows of 128 bytes) and pick
  // the global chunk that belongs in their slot. Slot s holds row
  // (tid >> 3) + kRowsPerPass * i, and its logical chunk
  // (tid & 7) ^ (row & 7) does not depend on i.
  const int lchunk = ((tid & 7) ^ ((tid >> 3) & 7)) << 4;
  const uint32_t lbase = (uint32_t)(tid >> 3) * (uint32_t)K + (uint32_t)lchunk;
  auto issue = [&](int stage, int k0) {
    uint8_t* base = smem + stage * C::kStage;
    const bool kin = k0 + lchunk < K;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int s0 = wave * 64 + C::kLoaders * i;  // first slot of this wave's 64
      const int ii = i < C::kLoadsW ? i : i - C::kLoadsW;
      const uint32_t off =
          kin ? lbase + (uint32_t)(C::kRowsPerPass * ii) * (uint32_t)K + (uint32_t)k0 : kOutOfRange;
      if (i < C::kLoadsW) buffer_load16_lds(rW, base + s0 * 16, off);
      else                buffer_load16_lds(rA, base + s0 * 16, off);
    }
  };

  const int wm = wave / WGN, wn = wave % WGN;
  const bool loader = wm == 0;
  const int r16 = lane & 15, g = lane >> 4;
  v4f acc[C::SN][C::SM];
#pragma unroll
  for (int i = 0; i < C::SN; ++i)
#pragma unroll
    for (int j = 0; j < C::SM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // The epilogue's scales are loaded before the K loop, so that their
  // latency passes under it instead of following the last MFMAs.
  float sA[C::SM];
  float4 sWv[C::SN];
#pragma unroll
  for (int j = 0; j < C::SM; ++j) {
    const int m = m0 + wm * C::WM + j * 16 + r16;
    sA[j] = m < M ? sa[m] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < C::SN; ++i) {
    const int nl = wn * C::WN + i * 16 + 4 * g;
    sWv[i] = n0 + nl < N ? *reinterpret_cast<const float4*>(sw + n0 + nl) : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  const int nk = (K + 127) >> 7;
  v8i xf[C::SM], wf[C::SN];
  // The first two K steps are requested together, and only the first is
  // waited for: the second one's latency then runs under the first step
  // instead of after it.
  if (loader) {
    issue(0, 0);
    if (nk > 1) {
      issue(1, 128);
      wait_vmcnt<C::kLoads>();
    } else {
      wait_vmem_all();
    }
  }
  lds_barrier();
  if (!loader) lds_barrier();
  for (int kt = 0; kt < nk; ++kt) {
    if (loader && kt >= 1 && kt + 1 < nk) issue((kt + 1) & 1, (kt + 1) << 7);
    const uint8_t* st = smem + (kt & 1) * C::kStage;
#pragma unroll
    for (int j = 0; j < C::SM; ++j) xf[j] = lds_frag(st, BN + wm * C::WM + j * 16 + r16, g);
#pragma unroll
    for (int i = 0; i < C::SN; ++i) wf[i] = lds_frag(st, wn * C::WN + i * 16 + r16, g);
    lds_barrier();
#pragma unroll
    for (int i = 0; i < C::SN; ++i)
#pragma unroll
      for (int j = 0; j < C::SM; ++j) acc[i][j] = mfma_16x16x128_e4m3(wf[i], xf[j], acc[i][j]);
    // The wait must stay behind the MFMAs: an s_waitcnt is no scheduling
    // barrier, and hoisted above them it would make every step wait for the
    // loads it has just issued.
    __builtin_amdgcn_sched_barrier(0);
    if (loader) wait_vmem_all();
    lds_barrier();
  }
  if (loader) lds_barrier();

  // Epilogue. acc[i][j][r] is Y[m][n] with m = m-tile j, lane % 16 and
  // n = n-tile i, 4 * (lane / 16) + r: four consecutive outputs of one row.
  __syncthreads();
#pragma unroll
  for (int i = 0; i < C::SN; ++i) {
    const int nl = wn * C::WN + i * 16 + 4 * g;
    const float4 sW = sWv[i];
#pragma unroll
    for (int j = 0; j < C::SM; ++j) {
      const int ml = wm * C::WM + j * 16 + r16;
      const v4f a = acc[i][j];
      const uint32_t p0 = bf16x2_rne(a[0] * sA[j] * sW.x, a[1] * sA[j] * sW.y);
      const uint32_t p1 = bf16x2_rne(a[2] * sA[j] * sW.z, a[3] * sA[j] * sW.w);
      *reinterpret_cast<uint2*>(smem + ml * C::kEpiStride + nl * 2) = make_uint2(p0, p1);
    }
  }
  __syncthreads();
  constexpr int kRowChunks = BN / 8;
  for (int c = tid; c < BM * kRowChunks; c += C::kThreads) {
    const int row = c / kRowChunks, col = (c % kRowChunks) * 8;
    const int m = m0 + row, n = n0 + col;
    if (m < M && n < N)
      store16_nt(Y + (int64_t)m * N + n, *reinterpret_cast<const uint4*>(smem + row * C::kEpiStride + col * 2));
  }
}

// Small-M kernel: NT tiles of 16 weight rows per workgroup, K split over
// the 4 waves, U K-steps of loads in flight per wave. MT = number of 16-token
// tiles. Every workgroup reads all M input rows (from L2), so for M > 16 two
// weight tiles per workgroup halve that traffic; a wave's input fragments
// serve both tiles. Each output's sum runs in the same order for any NT.
// XL = the input rows go global -> LDS as whole 128-byte row pieces (one
// load instruction per 8 rows and K step) instead of straight into the MFMA
// layout (16 rows x 64 bytes per instruction); the sums are the same.
template <int MT, int U, int NT = 1, bool XL = false>
__global__ __launch_bounds__(256) void gemm_skinny(const uint8_t* __restrict__ A, const float* __restrict__ sa,
                                                   const uint8_t* __restrict__ W, const float* __restrict__ sw,
                                                   uint16_t* __restrict__ Y, int M, int N, int K) {
  __shared__ v4f red[3][NT][MT][64];
  // XL: each wave's input rows for its U steps, [U][16 MT rows][128 bytes],
  // the 16-byte pieces of a row swizzled by (row & 7)
  constexpr int kXRows = 16 * MT;
  __shared__ __attribute__((aligned(1024))) uint8_t xs[XL ? 4 : 1][XL ? U : 1][XL ? kXRows * 128 : 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16 * NT;
  const auto rW = make_rsrc(W + (int64_t)n0 * K, (int64_t)(N - n0) * K);
  const auto rA = make_rsrc(A, (int64_t)M * K);
  const int r16 = lane & 15, g = lane >> 4;
  // The epilogue's scales are loaded first, so that their latency overlaps
  // the weight stream instead of following it.
  float4 sW[NT];
  float sA[MT];
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int n = n0 + i * 16 + 4 * g;
      sW[i] = n < N ? *reinterpret_cast<const float4*>(sw + n) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = t * 16 + r16;
      sA[t] = m < M ? sa[m] : 0.f;
    }
  }
  v4f acc[NT][MT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};
  const int nk = (K + 127) >> 7;
  const int xr8 = lane >> 3, xslot = lane & 7;
  for (int kt = wave; kt < nk; kt += 4 * U) {
    v8i wf[U][NT], xf[U][MT];
    if constexpr (XL) {
      // The input rows first, as whole 128-byte row pieces into this wave's
      // LDS slice: instruction (u, q) takes rows 8q .. 8q + 7 of step u, lane
      // l row 8q + l / 8 and the piece (l % 8) ^ (row % 8), which lands in
      // slot l % 8 of the row. Rows at or past M are not loaded: their MFMA
      // columns are never stored.
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k0 = (kt + 4 * u) << 7;
        const bool live = kt + 4 * u < nk;
#pragma unroll
        for (int q = 0; q < 2 * MT; ++q) {
          if (8 * q < M) {
            const int row = 8 * q + xr8;
            const int piece = xslot ^ (row & 7);
            const int c = k0 + 16 * piece;
            const uint32_t off =
                (live && row < M && c < K) ? (uint32_t)row * (uint32_t)K + (uint32_t)c : kOutOfRange;
            buffer_load16_lds(rA, &xs[wave][u][8 * q * 128], off);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k0 = (kt + 4 * u) << 7;
      const int c0 = k0 + 16 * g, c1 = c0 + 64;
      const bool live = kt + 4 * u < nk;
      const uint32_t o0 = (live && c0 < K) ? (uint32_t)c0 : kOutOfRange;
      const uint32_t o1 = (live && c1 < K) ? (uint32_t)c1 : kOutOfRange;
      // The input fragments (L2-resident, short latency) are issued before
      // the weight fragments, so they are in hand by the time the weights
      // arrive from memory: measured 1.5-2% faster for 8 to 16 rows.
      if constexpr (!XL) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const uint32_t xrow = (uint32_t)(t * 16 + r16) * (uint32_t)K;
          const v4i xl = buffer_load16(rA, o0 == kOutOfRange ? o0 : xrow + o0);
          const v4i xh = buffer_load16(rA, o1 == kOutOfRange ? o1 : xrow + o1);
          xf[u][t] = v8i{xl.x, xl.y, xl.z, xl.w, xh.x, xh.y, xh.z, xh.w};
        }
      }
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const uint32_t wrow = (uint32_t)(i * 16 + r16) * (uint32_t)K;
        const v4i lo = buffer_load16(rW, o0 == kOutOfRange ? o0 : wrow + o0);
        const v4i hi = buffer_load16(rW, o1 == kOutOfRange ? o1 : wrow + o1);
        wf[u][i] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
    }
    if constexpr (XL) {
      // the input pieces have landed once only the weight loads are outstanding
      wait_vmcnt<2 * U * NT>();
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const int row = t * 16 + r16;
          const uint8_t* xrow = &xs[wave][u][row * 128];
          const v4i xl = *reinterpret_cast<const v4i*>(xrow + ((g ^ (row & 7)) << 4));
          const v4i xh = *reinterpret_cast<const v4i*>(xrow + (((g + 4) ^ (row & 7)) << 4));
          xf[u][t] = v8i{xl.x, xl.y, xl.z, xl.w, xh.x, xh.y, xh.z, xh.w};
        }
    }
    // keep every load of this round ahead of the first MFMA: bytes in flight
    // are what this kernel is limited by
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[i][t] = mfma_16x16x128_e4m3(wf[u][i], xf[u][t], acc[i][t]);
  }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int t = 0; t < MT; ++t) red[wave - 1][i][t][lane] = acc[i][t];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int n = n0 + i * 16 + 4 * g;
    if (n >= N) continue;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const v4f a = acc[i][t] + red[0][i][t][lane] + red[1][i][t][lane] + red[2][i][t][lane];
      const int m = t * 16 + r16;
      if (m < M) {
        const float s = sA[t];
        const uint32_t p0 = bf16x2_rne(a[0] * s * sW[i].x, a[1] * s * sW[i].y);
        const uint32_t p1 = bf16x2_rne(a[2] * s * sW[i].z, a[3] * s * sW[i].w);
        *reinterpret_cast<uint2*>(Y + (int64_t)m * N + n) = make_uint2(p0, p1);
      }
    }
  }
}

// Fused decode: X BF16 [M, K] with M <= 16 * MT and K <= 512 * U (one round).
// NT tiles of 16 weight rows per workgroup share its quantised input, so
// two tiles halve both the input re-reads and the quantisation work per
// weight row.
template <int MT, int U, int NT = 1>
__global__ __launch_bounds__(256) void gemm_skinny_q(const uint16_t* __restrict__ X, const uint8_t* __restrict__ W,
                                                     const float* __restrict__ sw, uint16_t* __restrict__ Y, int M,
                                                     int N, int K) {
  __shared__ v4f red[3][NT][MT][64];
  __shared__ uint32_t wmax[4][MT * 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16 * NT;
  const auto rW = make_rsrc(W + (int64_t)n0 * K, (int64_t)(N - n0) * K);
  const auto rX = make_rsrc(X, (int64_t)M * K * 2);
  const int r16 = lane & 15, g = lane >> 4;
  const int nk = (K + 127) >> 7;
  // The epilogue's weight scales first (so their latency overlaps the
  // stream), then the weights (their latency is the longest), then this
  // wave's BF16 chunks: for K slice kt = wave + 4u, elements
  // [128 kt + 16 g, +16) and [128 kt + 64 + 16 g, +16) of each row, 32 bytes each.
  float4 sW[NT];
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int n = n0 + i * 16 + 4 * g;
      sW[i] = n < N ? *reinterpret_cast<const float4*>(sw + n) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  v8i wf[U][NT];
  uint4 xb[U][MT][4];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k0 = (wave + 4 * u) << 7;
    const int c0 = k0 + 16 * g, c1 = c0 + 64;
    const bool live = wave + 4 * u < nk;
    const uint32_t o0 = (live && c0 < K) ? (uint32_t)c0 : kOutOfRange;
    const uint32_t o1 = (live && c1 < K) ? (uint32_t)c1 : kOutOfRange;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const uint32_t wrow = (uint32_t)(i * 16 + r16) * (uint32_t)K;
      const v4i lo = buffer_load16(rW, o0 == kOutOfRange ? o0 : wrow + o0);
      const v4i hi = buffer_load16(rW, o1 == kOutOfRange ? o1 : wrow + o1);
      wf[u][i] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint32_t xrow = (uint32_t)(t * 16 + r16) * (uint32_t)K * 2u;
      const uint32_t b0 = o0 == kOutOfRange ? o0 : xrow + 2u * o0;
      const uint32_t b1 = o1 == kOutOfRange ? o1 : xrow + 2u * o1;
      const v4i a0 = buffer_load16(rX, b0), a1 = buffer_load16(rX, b0 == kOutOfRange ? b0 : b0 + 16u);
      const v4i a2 = buffer_load16(rX, b1), a3 = buffer_load16(rX, b1 == kOutOfRange ? b1 : b1 + 16u);
      xb[u][t][0] = make_uint4(a0.x, a0.y, a0.z, a0.w);
      xb[u][t][1] = make_uint4(a1.x, a1.y, a1.z, a1.w);
      xb[u][t][2] = make_uint4(a2.x, a2.y, a2.z, a2.w);
      xb[u][t][3] = make_uint4(a3.x, a3.y, a3.z, a3.w);
    }
  }
  // Row maxima of |x| (integer max on the BF16 bits, as quantize_per_token).
  uint32_t am[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    am[t] = 0;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) am[t] = max(am[t], absmax8(xb[u][t][c]));
    am[t] = max(am[t], (uint32_t)__shfl_xor((int)am[t], 16, 64));
    am[t] = max(am[t], (uint32_t)__shfl_xor((int)am[t], 32, 64));
    if (g == 0) wmax[wave][t * 16 + r16] = am[t];
  }
  __syncthreads();
  float s[MT], r[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int row = t * 16 + r16;
    const uint32_t a = max(max(wmax[0][row], wmax[1][row]), max(wmax[2][row], wmax[3][row]));
    s[t] = row_scale(a);
    r[t] = 1.0f / s[t];
  }
  v4f acc[NT][MT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint2 q0 = quant8(xb[u][t][0], s[t], r[t]), q1 = quant8(xb[u][t][1], s[t], r[t]);
      const uint2 q2 = quant8(xb[u][t][2], s[t], r[t]), q3 = quant8(xb[u][t][3], s[t], r[t]);
      const v8i xf = v8i{(int)q0.x, (int)q0.y, (int)q1.x, (int)q1.y, (int)q2.x, (int)q2.y, (int)q3.x, (int)q3.y};
#pragma unroll
      for (int i = 0; i < NT; ++i) acc[i][t] = mfma_16x16x128_e4m3(wf[u][i], xf, acc[i][t]);
    }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int t = 0; t < MT; ++t) red[wave - 1][i][t][lane] = acc[i][t];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int n = n0 + i * 16 + 4 * g;
    if (n >= N) continue;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const v4f a = acc[i][t] + red[0][i][t][lane] + red[1][i][t][lane] + red[2][i][t][lane];
      const int m = t * 16 + r16;
      if (m < M) {
        const uint32_t p0 = bf16x2_rne(a[0] * s[t] * sW[i].x, a[1] * s[t] * sW[i].y);
        const uint32_t p1 = bf16x2_rne(a[2] * s[t] * sW[i].z, a[3] * s[t] * sW[i].w);
        *reinterpret_cast<uint2*>(Y + (int64_t)m * N + n) = make_uint2(p0, p1);
      }
    }
  }
}

// The read floor of the decode weight stream: the launch shape of
// gemm_skinny (256 threads per 32 KB, each lane's eight 16-byte loads in
// flight together) with no arithmetic but an XOR of what was read, one
// word per workgroup so the loads are kept.
__global__ __launch_bounds__(256) void read_probe(const uint8_t* __restrict__ p, int64_t bytes,
                                                  uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * kProbeBytesPerBlock;
  const auto r = make_rsrc(p + base, bytes - base);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v4i v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
    v[u] = buffer_load16(r, (uint32_t)((wave * 8 + u) * 1024 + lane * 16));
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) x ^= (uint32_t)(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
  __shared__ uint32_t part[4];
  for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, 64);
  if (lane == 0) part[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// The shader clock: lane 0 of each one-wave workgroup spins until the
// constant 100 MHz clock has advanced by kClockProbeTicks and counts the
// shader cycles (s_memtime) over the same span.
constexpr unsigned long long kClockProbeTicks = 400;  // 4 us

__global__ __launch_bounds__(64) void clock_probe(uint64_t* __restrict__ out) {
  if (threadIdx.x != 0) return;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  unsigned long long r1;
  do {
    r1 = __builtin_amdgcn_s_memrealtime();
  } while (r1 - r0 < kClockProbeTicks);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  out[2 * blockIdx.x] = (uint64_t)(t1 - t0);
  out[2 * blockIdx.x + 1] = (uint64_t)(r1 - r0);
}

// A launch, optionally with two events that the runtime stamps with the
// kernel's own start and end (hipExtLaunchKernel), so that an elapsed time
// between them is the kernel alone, without the dispatch in front of it.
template <typename F, typename... Args>
hipError_t launch_k(F kernel, dim3 grid, dim3 block, hipStream_t stream, hipEvent_t start, hipEvent_t stop,
                    Args... args) {
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN>
hipError_t run_tiled(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* y,
                     int64_t M, int64_t N, int64_t K, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  return launch_k(gemm_tiled<BM, BN, WGM, WGN>, dim3(tiles_m * tiles_n), dim3(64 * WGM * WGN), stream, start, stop,
                  a, sa, w, sw, y, (int)M, (int)N, (int)K, tiles_m, tiles_n);
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw, uint16_t* y,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (M == 0 || N == 0) return hipSuccess;
  // Up to 4 rows one 16-row weight tile per workgroup keeps the most bytes
  // in flight; from 5 rows two tiles per workgroup share each input
  // fragment, halving the input rows read per weight byte (8 rows of an
  // 8192 x 2048 layer: 5.62 against 5.75 us; 1 row: 5.26 against 5.47 us).
  if (M <= 4) {
    return launch_k(gemm_skinny<1, 4>, dim3((unsigned)((N + 15) / 16)), dim3(256), stream, start, stop, a, sa, w, sw, y,
                    (int)M, (int)N, (int)K);
  }
  if (M <= 16) {
    return launch_k(gemm_skinny<1, 4, 2>, dim3((unsigned)((N + 31) / 32)), dim3(256), stream, start, stop, a, sa, w, sw, y,
                    (int)M, (int)N, (int)K);
  }
  // 17 to 32 rows: the input rows go through LDS as whole 128-byte row
  // pieces (7.2 -> 6.6 us for 32 rows of the 8192 x 2048 layer; at 8 to 16
  // rows the extra LDS hop costs as much as it saves)
  if (M <= 32) {
    return launch_k(gemm_skinny<2, 4, 2, true>, dim3((unsigned)((N + 31) / 32)), dim3(256), stream, start, stop, a, sa, w, sw, y,
                    (int)M, (int)N, (int)K);
  }
  return run_tiled<256, 192, 2, 4>(a, sa, w, sw, y, M, N, K, stream, start, stop);
}

hipError_t launch_read_probe(const uint8_t* p, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  hipLaunchKernelGGL(read_probe, dim3((unsigned)((bytes + kProbeBytesPerBlock - 1) / kProbeBytesPerBlock)), dim3(256),
                     0, stream, p, bytes, sink);
  return hipGetLastError();
}

hipError_t launch_clock_probe(uint64_t* out, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(clock_probe, dim3((unsigned)n), dim3(64), 0, stream, out);
  return hipGetLastError();
}

hipError_t launch_quant_gemm_decode(const uint16_t* x, const uint8_t* w, const float* sw, uint16_t* y, int64_t M,
                                    int64_t N, int64_t K, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const dim3 grid((unsigned)((N + 31) / 32));
  if (M <= 16)
    hipLaunchKernelGGL((gemm_skinny_q<1, 4, 2>), grid, dim3(256), 0, stream, x, w, sw, y, (int)M, (int)N, (int)K);
  else
    hipLaunchKernelGGL((gemm_skinny_q<2, 4, 2>), grid, dim3(256), 0, stream, x, w, sw, y, (int)M, (int)N, (int)K);
  return hipGetLastError();
}

}  // namespace w8a8
