// Routed experts: expert-sorted permutation, grouped FP8 GEMMs, fused
// SwiGLU + per-slot requantisation, and the router-weighted top-k combine.
//
// The pages put the routed experts in FP8 with the same per-row scheme as
// the other large matrices (Lernex/Metis-1.6-Logos-FP8, "What is in FP8"),
// route every token to its top-k experts (Lernex/Metis-1.6-Praxis,
// "Architecture"), store experts in global expert order (the "Files"
// section of the model pages), and run the expert stage for every token on
// both passes with the same weights (sglang-metis 0.1.0, "How the model maps
// onto SGLang"). The expert activation, the gate/up layout, the requantised
// expert input and the combine are not printed; the readings taken are:
// W13[e] = [gate; up] rows, h = silu(g) * u in float32, one E4M3 scale per
// routed copy (slot) of h, out[t] = bf16(sum_j w[t,j] * y[t,j]) with float32
// sums.
//
// Kernels
//  * route_count / route_scatter: slots t*k+j are grouped by expert, in
//    increasing slot order inside an expert (a stable sort), ids outside
//    [0, E) dropped. Chunk histograms, then one wave per sub-chunk walks its
//    slots in order; lanes holding the same expert are matched with
//    log2(E) ballots, so each slot's rank among earlier equal ids is a
//    popcount. No host synchronisation: every later kernel reads the
//    offsets from device memory and derives its own tile from them.
//  * grouped_tiled<.., GATE_UP>: like the dense tiled GEMM, with A rows
//    gathered through the permutation (slot -> token) and the weight of the
//    tile's expert; BF16 output in sorted order.
//  * gate_up_swiglu_quant: one workgroup owns 64 sorted slots and all 2I
//    gate/up columns, so each slot's h row is complete in one place. A
//    (64 gathered token rows) is staged in LDS by direct buffer loads;
//    each wave streams its own 64 gate + 64 matching up weight rows straight
//    into registers and runs 32x32x64 E4M3 MFMAs. The epilogue forms
//    h = silu(g) * u in float32, stages h in LDS, and requantises every row
//    (amax, scale = amax / 448, correctly rounded division, E4M3 RNE).
//  * grouped_tiled<.., DOWN>: A = the requantised rows (already sorted and
//    contiguous), B = W2 of the tile's expert; the epilogue multiplies by
//    the slot scale, the channel scale and the router weight, stages the
//    tile in LDS and adds it into a float32 [T, H] accumulator with atomics
//    whose 64 lanes cover 64 consecutive outputs of one row.
//  * finalize: float32 accumulator -> BF16 (round to nearest even).
#include "device.h"
#include "launch.h"

namespace w8a8 {
namespace {

constexpr int kRouteChunk = 4096;       // slots per routing block (4 waves x 1024)
constexpr int kRouteSub = kRouteChunk / 4;

__device__ inline int bits_for(int v) {  // bits needed to tell 0..v apart
  int b = 1;
  while ((1 << b) <= v) ++b;
  return b;
}

// Lanes whose key equals this lane's key (all 64 lanes must be active).
__device__ inline uint64_t match_peers(int key, int nbits) {
  uint64_t peers = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

__global__ __launch_bounds__(256) void route_count(const int32_t* __restrict__ ids, int64_t n, int E,
                                                   int32_t* __restrict__ chunk_counts) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kRouteChunk;
  for (int i = threadIdx.x; i < kRouteChunk; i += 256) {
    const int64_t s = base + i;
    if (s < n) {
      const int e = ids[s];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// LDS: before[E] | base[4][E] | whist[4][E]
__global__ __launch_bounds__(256) void route_scatter(const int32_t* __restrict__ ids, int64_t n, int E, int nchunks,
                                                     const int32_t* __restrict__ chunk_counts,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm) {
  extern __shared__ int sm[];
  int* before = sm;              // slots of expert e in earlier chunks, plus the expert's offset
  int* base = sm + E;            // per wave running position
  int* whist = sm + 5 * E;       // per wave histogram of its sub-chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  for (int e = tid; e < 4 * E; e += 256) whist[e] = 0;
  // totals and the exclusive scan over experts: wave 0 walks experts 64 at a time
  if (wave == 0) {
    int carry = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      int tot = 0, bef = 0;
      if (e < E) {
        for (int cc = 0; cc < nchunks; ++cc) {
          const int v = chunk_counts[(int64_t)cc * E + e];
          tot += v;
          if (cc < c) bef += v;
        }
      }
      int incl = tot;
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
      }
      const int off = carry + incl - tot;
      if (e < E) {
        before[e] = off + bef;
        if (c == 0) {
          counts[e] = tot;
          offsets[e] = off;
        }
      }
      carry += __shfl(incl, 63, 64);
    }
    if (c == 0 && lane == 0) offsets[E] = carry;
    // the unused tail of perm (dropped ids) is set to -1
    const int64_t lo = (int64_t)c * kRouteChunk, hi = min(n, lo + kRouteChunk);
    for (int64_t s = lo + lane; s < hi; s += 64)
      if (s >= carry) perm[s] = -1;
  }
  __syncthreads();
  const int nbits = bits_for(E + 1);
  const int64_t sub0 = (int64_t)c * kRouteChunk + (int64_t)wave * kRouteSub;
  // pass 1: histogram of this wave's sub-chunk
  for (int i = 0; i < kRouteSub; i += 64) {
    const int64_t s = sub0 + i + lane;
    int key = E + 1;
    if (s < n) {
      const int e = ids[s];
      key = (e >= 0 && e < E) ? e : E;
    }
    const uint64_t peers = match_peers(key, nbits);
    const bool leader = lane == 63 - __clzll(peers);
    if (leader && key < E) whist[wave * E + key] += __popcll(peers);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    int b = before[e];
    for (int w = 0; w < 4; ++w) {
      base[w * E + e] = b;
      b += whist[w * E + e];
    }
  }
  __syncthreads();
  // pass 2: stable scatter
  const uint64_t lt = (1ull << lane) - 1;
  for (int i = 0; i < kRouteSub; i += 64) {
    const int64_t s = sub0 + i + lane;
    int key = E + 1;
    if (s < n) {
      const int e = ids[s];
      key = (e >= 0 && e < E) ? e : E;
    }
    const uint64_t peers = match_peers(key, nbits);
    if (key < E) {
      const int pos = base[wave * E + key] + __popcll(peers & lt);
      perm[pos] = (int32_t)s;
    }
    __builtin_amdgcn_wave_barrier();
    const bool leader = lane == 63 - __clzll(peers);
    if (leader && key < E) base[wave * E + key] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

// Which expert and which rows the m-tile `mt` covers, from the device-side
// offsets (each wave computes it; the answer is uniform).
__device__ inline bool find_tile(const int32_t* __restrict__ offsets, int E, int BM, int mt, int& e_out,
                                 int& row0, int& rows) {
  const int lane = threadIdx.x & 63;
  int acc = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    int cnt = 0, start = 0;
    if (e < E) {
      start = offsets[e];
      cnt = offsets[e + 1] - start;
    }
    const int tiles = (cnt + BM - 1) / BM;
    int incl = tiles;
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    const int excl = incl - tiles;
    const bool hit = e < E && mt >= acc + excl && mt < acc + incl;
    const uint64_t b = __ballot(hit);
    if (b) {
      const int src = __ffsll((unsigned long long)b) - 1;
      const int ex = __shfl(excl, src, 64), st = __shfl(start, src, 64), ct = __shfl(cnt, src, 64);
      const int local = mt - acc - ex;
      e_out = __builtin_amdgcn_readfirstlane(e0 + src);
      row0 = __builtin_amdgcn_readfirstlane(st + local * BM);
      rows = __builtin_amdgcn_readfirstlane(min(BM, ct - local * BM));
      return true;
    }
    acc += __shfl(incl, 63, 64);
  }
  return false;
}

enum { kGateUp = 0, kDown = 1 };

template <int BM, int BN, int MODE>
struct Grouped {
  static constexpr int kThreads = 256;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int SM = WM / 16, SN = WN / 16;
  static constexpr int kRows = BM + BN;
  static constexpr int kStage = kRows * 128;
  static constexpr int kLoads = kRows * 8 / kThreads;
  static constexpr int kOutElt = MODE == kGateUp ? 2 : 4;       // bf16 or fp32 staging
  static constexpr int kEpiStride = BN * kOutElt + 16;
  static constexpr int kEpi = BM * kEpiStride;
  static constexpr int kLds = (2 * kStage > kEpi) ? 2 * kStage : kEpi;
  static_assert((kRows * 8) % kThreads == 0, "stage must split evenly");
};

// Grouped GEMM over expert-sorted slots. M = sorted slots, N = output
// columns of one expert's weight [N, K], K = reduction.
//  GATE_UP: A row r = xq[perm[r] / topk] (gathered), out = gu bf16 [nslots, N]
//           with scales xs[token] * sB[e, n].
//  DOWN:    A row r = qh[r] (sorted, contiguous), out adds
//           w[slot] * sh[r] * sB[e, n] * acc into acc32[token, n].
template <int BM, int BN, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_tiled(const uint8_t* __restrict__ A, const float* __restrict__ sA, int64_t a_rows,
                   const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets, int E, int topk,
                   const uint8_t* __restrict__ B, const float* __restrict__ sB, const float* __restrict__ tw,
                   uint16_t* __restrict__ out_bf16, float* __restrict__ out_acc, int N, int K, int tiles_n,
                   int tiles_m_max) {
  using C = Grouped<BM, BN, MODE>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLds];
  __shared__ int row_tok[BM];     // token of each tile row (-1 = empty row)
  __shared__ float row_scale[BM]; // activation scale (times router weight for DOWN)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // tile id -> (m-tile, n-tile); consecutive ids share the m-tile (A rows)
  const int total = tiles_m_max * tiles_n;
  const int per = total >> 3;
  int t = blockIdx.x;
  if ((int)blockIdx.x < (per << 3)) t = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  const int mt = t / tiles_n, nt = t - mt * tiles_n;
  int e, row0, rows;
  if (!find_tile(offsets, E, BM, mt, e, row0, rows)) return;
  const int n0 = nt * BN;

  for (int i = tid; i < BM; i += C::kThreads) {
    int tok = -1;
    float sc = 0.f;
    if (i < rows) {
      const int slot = perm[row0 + i];
      tok = slot / topk;
      sc = MODE == kGateUp ? sA[tok] : sA[row0 + i] * tw[slot];
    }
    row_tok[i] = tok;
    row_scale[i] = sc;
  }
  __syncthreads();

  const auto rB = make_rsrc(B + ((int64_t)e * N + n0) * K, (int64_t)(N - n0) * K);
  const auto rA = MODE == kGateUp ? make_rsrc(A, a_rows * K) : make_rsrc(A + (int64_t)row0 * K, (int64_t)rows * K);
  // Loader (as in the dense kernel): thread tid fills rows (tid >> 3) + 32 i,
  // always with logical chunk (tid & 7) ^ ((tid >> 4) & 7). B rows first.
  const int lchunk = ((tid & 7) ^ ((tid >> 4) & 7)) << 4;
  constexpr int kLoadsB = BN / 32, kLoadsA = BM / 32;
  const uint32_t bbase = (uint32_t)(tid >> 3) * (uint32_t)K + (uint32_t)lchunk;
  uint32_t aoff[kLoadsA];
#pragma unroll
  for (int j = 0; j < kLoadsA; ++j) {
    const int lr = (tid >> 3) + 32 * j;
    if (MODE == kGateUp) {
      const int tok = row_tok[lr];
      aoff[j] = tok < 0 ? kOutOfRange : (uint32_t)tok * (uint32_t)K + (uint32_t)lchunk;
    } else {
      aoff[j] = (uint32_t)lr * (uint32_t)K + (uint32_t)lchunk;
    }
  }
  auto issue = [&](int stage, int k0) {
    uint8_t* base = smem + stage * C::kStage;
    const bool kin = k0 + lchunk < K;
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
      const int s0 = wave * 64 + C::kThreads * i;
      if (i < kLoadsB) {
        const uint32_t off = kin ? bbase + (uint32_t)(32 * i) * (uint32_t)K + (uint32_t)k0 : kOutOfRange;
        buffer_load16_lds(rB, base + s0 * 16, off);
      } else {
        const uint32_t a = aoff[i - kLoadsB];
        const uint32_t off = (kin && a != kOutOfRange) ? a + (uint32_t)k0 : kOutOfRange;
        buffer_load16_lds(rA, base + s0 * 16, off);
      }
    }
  };

  const int wm = wave & 1, wn = wave >> 1;
  const int r16 = lane & 15, g = lane >> 4;
  v4f acc[C::SN][C::SM];
#pragma unroll
  for (int i = 0; i < C::SN; ++i)
#pragma unroll
    for (int j = 0; j < C::SM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const int nk = (K + 127) >> 7;
  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmem_all();
    __syncthreads();
    if (kt + 1 < nk) issue((kt + 1) & 1, (kt + 1) << 7);
    const uint8_t* st = smem + (kt & 1) * C::kStage;
    v8i xf[C::SM];
#pragma unroll
    for (int j = 0; j < C::SM; ++j) {
      const int row = BN + wm * C::WM + j * 16 + r16;
      const v4i lo = *reinterpret_cast<const v4i*>(st + stage_off(row, g));
      const v4i hi = *reinterpret_cast<const v4i*>(st + stage_off(row, g + 4));
      xf[j] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
#pragma unroll
    for (int i = 0; i < C::SN; ++i) {
      const int row = wn * C::WN + i * 16 + r16;
      const v4i lo = *reinterpret_cast<const v4i*>(st + stage_off(row, g));
      const v4i hi = *reinterpret_cast<const v4i*>(st + stage_off(row, g + 4));
      const v8i wf = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int j = 0; j < C::SM; ++j) acc[i][j] = mfma_16x16x128_e4m3(wf, xf[j], acc[i][j]);
    }
  }
  __syncthreads();
  // stage the scaled tile in LDS: acc[i][j][r] is row (m-tile j, lane % 16), columns
  // (n-tile i, 4 * (lane / 16) + r)
#pragma unroll
  for (int i = 0; i < C::SN; ++i) {
    const int nl = wn * C::WN + i * 16 + 4 * g;
    float4 sW = make_float4(0.f, 0.f, 0.f, 0.f);
    if (n0 + nl < N) sW = *reinterpret_cast<const float4*>(sB + (int64_t)e * N + n0 + nl);
#pragma unroll
    for (int j = 0; j < C::SM; ++j) {
      const int ml = wm * C::WM + j * 16 + r16;
      const float s = row_scale[ml];
      const v4f a = acc[i][j];
      if (MODE == kGateUp) {
        const uint32_t b0 = f32_to_bf16_rne(a[0] * s * sW.x), b1 = f32_to_bf16_rne(a[1] * s * sW.y);
        const uint32_t b2 = f32_to_bf16_rne(a[2] * s * sW.z), b3 = f32_to_bf16_rne(a[3] * s * sW.w);
        *reinterpret_cast<uint2*>(smem + ml * C::kEpiStride + nl * 2) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
      } else {
        *reinterpret_cast<float4*>(smem + ml * C::kEpiStride + nl * 4) =
            make_float4(a[0] * s * sW.x, a[1] * s * sW.y, a[2] * s * sW.z, a[3] * s * sW.w);
      }
    }
  }
  __syncthreads();
  if (MODE == kGateUp) {
    constexpr int kRowChunks = BN / 8;
    for (int c = tid; c < BM * kRowChunks; c += C::kThreads) {
      const int row = c / kRowChunks, col = (c % kRowChunks) * 8;
      if (row < rows && n0 + col < N)
        *reinterpret_cast<uint4*>(out_bf16 + (int64_t)(row0 + row) * N + n0 + col) =
            *reinterpret_cast<const uint4*>(smem + row * C::kEpiStride + col * 2);
    }
  } else {
    // one wave per row at a time, 64 consecutive columns per atomic instruction
    for (int row = wave; row < rows; row += 4) {
      const int tok = row_tok[row];
      float* dst = out_acc + (int64_t)tok * N + n0;
      const float* src = reinterpret_cast<const float*>(smem + row * C::kEpiStride);
      for (int col = lane; col < BN && n0 + col < N; col += 64) atomicAdd(dst + col, src[col]);
    }
  }
}

// ---- fused gate/up + SwiGLU + per-slot requantisation ----------------------
// Workgroup: 64 sorted slots x all 2I columns; wave w owns gate columns
// [64w, 64w + 64) and up columns [I + 64w, I + 64w + 64). K steps of 64.
constexpr int kFBM = 64;
constexpr int kFStageA = kFBM * 64;      // 64 rows x 64 bytes

template <int WAVES>
struct Fused {
  static_assert(WAVES == 4 || WAVES == 8, "the A loader uses 256 threads; rows split over 4 or 8 waves");
  static constexpr int I = 64 * WAVES;
  static constexpr int kThreads = 64 * WAVES;
  static constexpr int kHStride = I * 4 + 16;               // fp32 h row in LDS
  static constexpr int kH = kFBM * kHStride;
  static constexpr int kLds = (2 * kFStageA > kH) ? 2 * kFStageA : kH;
};

// byte offset of 16-byte chunk c (0..3) of row `row` in a 64-byte-row stage
__device__ inline int stage64_off(int row, int c) { return row * 64 + ((c ^ ((row >> 2) & 3)) << 4); }

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(1, 2)))
void gate_up_swiglu_quant(const uint8_t* __restrict__ xq, const float* __restrict__ xs, int64_t T,
                          const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets, int E, int topk,
                          const uint8_t* __restrict__ w13, const float* __restrict__ s13,
                          uint8_t* __restrict__ qh, float* __restrict__ sh, int H) {
  using F = Fused<WAVES>;
  constexpr int I = F::I;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[F::kLds];
  __shared__ int row_tok[kFBM];
  __shared__ float row_xs[kFBM];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int e, row0, rows;
  if (!find_tile(offsets, E, kFBM, blockIdx.x, e, row0, rows)) return;
  for (int i = tid; i < kFBM; i += F::kThreads) {
    int tok = -1;
    float s = 0.f;
    if (i < rows) {
      tok = perm[row0 + i] / topk;
      s = xs[tok];
    }
    row_tok[i] = tok;
    row_xs[i] = s;
  }
  __syncthreads();
  const auto rA = make_rsrc(xq, T * H);
  const auto rB = make_rsrc(w13 + (int64_t)e * 2 * I * H, (int64_t)2 * I * H);
  // A loader: threads 0..255 each move one 16-byte chunk per K step
  uint32_t aoff = kOutOfRange;
  int achunk = 0;
  if (tid < 256) {
    const int row = tid >> 2, c = (tid & 3) ^ ((row >> 2) & 3);
    achunk = c << 4;
    const int tok = row_tok[row];
    if (tok >= 0) aoff = (uint32_t)tok * (uint32_t)H + (uint32_t)achunk;
  }
  auto issueA = [&](int stage, int k0) {
    if (wave < 4) {
      const uint32_t off = (aoff != kOutOfRange && k0 + achunk < H) ? aoff + (uint32_t)k0 : kOutOfRange;
      buffer_load16_lds(rA, smem + stage * kFStageA + wave * 1024, off);
    }
  };
  // B: lane holds row (lane % 32) of each of its 4 column tiles, 16-byte
  // chunks hb and hb + 2 of the 64-byte K slice (hb = lane / 32)
  const int r32 = lane & 31, hb = lane >> 5;
  uint32_t brow[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int col = (ct < 2 ? 0 : I) + 64 * wave + 32 * (ct & 1) + r32;
    brow[ct] = (uint32_t)col * (uint32_t)H;
  }
  auto loadB = [&](v8i (&bf)[4], int k0) {
    const int c0 = k0 + 16 * hb, c1 = c0 + 32;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const v4i lo = buffer_load16(rB, c0 < H ? brow[ct] + c0 : kOutOfRange);
      const v4i hi = buffer_load16(rB, c1 < H ? brow[ct] + c1 : kOutOfRange);
      bf[ct] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
  };
  v16f acc[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[rt][ct][q] = 0.f;
  const int nk = (H + 63) >> 6;
  v8i bcur[4], bnext[4];
  issueA(0, 0);
  loadB(bcur, 0);
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmem_all();
    __syncthreads();
    if (kt + 1 < nk) {
      issueA((kt + 1) & 1, (kt + 1) << 6);
      loadB(bnext, (kt + 1) << 6);
    }
    const uint8_t* st = smem + (kt & 1) * kFStageA;
    v8i af[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int row = rt * 32 + r32;
      const v4i lo = *reinterpret_cast<const v4i*>(st + stage64_off(row, hb));
      const v4i hi = *reinterpret_cast<const v4i*>(st + stage64_off(row, hb + 2));
      af[rt] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) acc[rt][ct] = mfma_32x32x64_e4m3(bcur[ct], af[rt], acc[rt][ct]);
    if (kt + 1 < nk) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) bcur[ct] = bnext[ct];
    }
  }
  __syncthreads();
  // Epilogue 1: acc[rt][ct][q] = column (ct tile, 8 * (q / 4) + 4 * (lane / 32) + q % 4),
  // slot row (rt * 32 + lane % 32). Gate tiles ct = 0, 1 pair with up tiles ct = 2, 3.
  float* hbuf = reinterpret_cast<float*>(smem);
  {
    const int ml0 = r32;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int ml = rt * 32 + ml0;
      const float s = row_xs[ml];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int cl = 8 * (q >> 2) + 4 * hb + (q & 3);       // 0..31 inside the tile
          const int j = 64 * wave + 32 * half + cl;           // h column
          const float gs = s13[(int64_t)e * 2 * I + j], us = s13[(int64_t)e * 2 * I + I + j];
          const float gv = acc[rt][half][q] * s * gs;
          const float uv = acc[rt][2 + half][q] * s * us;
          const float h = gv / (1.0f + __expf(-gv)) * uv;
          hbuf[ml * (F::kHStride / 4) + j] = h;
        }
      }
    }
  }
  __syncthreads();
  // Epilogue 2: one wave per row: amax, scale, E4M3 codes (I / 64 values per lane)
  constexpr int PER = I / 64;
  for (int row = wave; row < rows; row += WAVES) {
    const float* hr = hbuf + row * (F::kHStride / 4);
    float v[PER];
    float amax = 0.f;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      v[p] = hr[lane * PER + p];
      amax = fmaxf(amax, fabsf(v[p]));
    }
    amax = wave_max_f32(amax);
    const float s = amax == 0.f ? 1.0f : amax / 448.0f;
    uint8_t* dst = qh + (int64_t)(row0 + row) * I + lane * PER;
    uint32_t words[PER / 4];
#pragma unroll
    for (int p = 0; p < PER / 4; ++p) {
      words[p] = e4m3_rne_sat(v[4 * p] / s) | (e4m3_rne_sat(v[4 * p + 1] / s) << 8) |
                 (e4m3_rne_sat(v[4 * p + 2] / s) << 16) | (e4m3_rne_sat(v[4 * p + 3] / s) << 24);
    }
#pragma unroll
    for (int p = 0; p < PER / 4; ++p) reinterpret_cast<uint32_t*>(dst)[p] = words[p];
    if (lane == 0) sh[row0 + row] = s;
  }
}

__global__ __launch_bounds__(256) void fill_zero_f32(float* __restrict__ p, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) reinterpret_cast<float4*>(p)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__global__ __launch_bounds__(256) void finalize_bf16(const float* __restrict__ acc, uint16_t* __restrict__ out,
                                                     int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float4 a = reinterpret_cast<const float4*>(acc)[2 * i];
  const float4 b = reinterpret_cast<const float4*>(acc)[2 * i + 1];
  uint4 o;
  o.x = f32_to_bf16_rne(a.x) | (f32_to_bf16_rne(a.y) << 16);
  o.y = f32_to_bf16_rne(a.z) | (f32_to_bf16_rne(a.w) << 16);
  o.z = f32_to_bf16_rne(b.x) | (f32_to_bf16_rne(b.y) << 16);
  o.w = f32_to_bf16_rne(b.z) | (f32_to_bf16_rne(b.w) << 16);
  reinterpret_cast<uint4*>(out)[i] = o;
}

int64_t align256(int64_t b) { return (b + 255) & ~int64_t(255); }

int route_chunks(int64_t n) { return (int)((n + kRouteChunk - 1) / kRouteChunk); }

constexpr int kGUBM = 128, kGUBN = 256;   // bf16 gate/up tiles
constexpr int kDNBM = 128, kDNBN = 256;   // down + combine tiles

}  // namespace

size_t route_workspace_bytes(int64_t T, int64_t topk, int64_t E) {
  return (size_t)align256((int64_t)route_chunks(T * topk) * E * 4);
}

hipError_t launch_route(const int32_t* ids, int64_t T, int64_t topk, int64_t E, int32_t* counts, int32_t* offsets,
                        int32_t* perm, void* scratch, hipStream_t stream) {
  const int64_t n = T * topk;
  const int nch = route_chunks(n);
  if (nch == 0) return hipSuccess;
  int32_t* chunk_counts = static_cast<int32_t*>(scratch);
  hipLaunchKernelGGL(route_count, dim3(nch), dim3(256), (size_t)E * 4, stream, ids, n, (int)E, chunk_counts);
  hipLaunchKernelGGL(route_scatter, dim3(nch), dim3(256), (size_t)E * 9 * 4, stream, ids, n, (int)E, nch,
                     chunk_counts, counts, offsets, perm);
  return hipGetLastError();
}

static int64_t m_tiles_max(int64_t nslots, int64_t E, int BM) { return (nslots + BM - 1) / BM + E; }

hipError_t launch_grouped_gate_up_bf16(const uint8_t* xq, const float* xs, const int32_t* perm,
                                       const int32_t* offsets, const uint8_t* w13, const float* s13, uint16_t* gu,
                                       int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                                       hipStream_t stream) {
  const int N = (int)(2 * I);
  const int tiles_n = (N + kGUBN - 1) / kGUBN;
  const int tiles_m = (int)m_tiles_max(T * topk, E, kGUBM);
  hipLaunchKernelGGL((grouped_tiled<kGUBM, kGUBN, kGateUp>), dim3(tiles_m * tiles_n), dim3(256), 0, stream, xq, xs,
                     T, perm, offsets, (int)E, (int)topk, w13, s13, (const float*)nullptr, gu, (float*)nullptr, N,
                     (int)H, tiles_n, tiles_m);
  return hipGetLastError();
}

hipError_t launch_gate_up_swiglu_quant(const uint8_t* xq, const float* xs, const int32_t* perm,
                                       const int32_t* offsets, const uint8_t* w13, const float* s13, uint8_t* qh,
                                       float* sh, int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                                       hipStream_t stream) {
  const dim3 grid((unsigned)m_tiles_max(T * topk, E, kFBM));
  switch (I) {
#define W8A8_FUSED(WV)                                                                                   \
  case 64 * WV:                                                                                          \
    hipLaunchKernelGGL((gate_up_swiglu_quant<WV>), grid, dim3(64 * WV), 0, stream, xq, xs, T, perm,       \
                       offsets, (int)E, (int)topk, w13, s13, qh, sh, (int)H);                             \
    break;
    W8A8_FUSED(4) W8A8_FUSED(8)
#undef W8A8_FUSED
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_down_combine(const uint8_t* qh, const float* sh, const int32_t* perm, const int32_t* offsets,
                               const float* tw, const uint8_t* w2, const float* s2, uint16_t* out, float* acc,
                               int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk, hipStream_t stream) {
  const int64_t n4 = T * H / 4;
  hipLaunchKernelGGL(fill_zero_f32, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, acc, n4);
  const int N = (int)H;
  const int tiles_n = (N + kDNBN - 1) / kDNBN;
  const int tiles_m = (int)m_tiles_max(T * topk, E, kDNBM);
  hipLaunchKernelGGL((grouped_tiled<kDNBM, kDNBN, kDown>), dim3(tiles_m * tiles_n), dim3(256), 0, stream, qh, sh,
                     T * topk, perm, offsets, (int)E, (int)topk, w2, s2, tw, (uint16_t*)nullptr, acc, N, (int)I,
                     tiles_n, tiles_m);
  const int64_t n8 = T * H / 8;
  hipLaunchKernelGGL(finalize_bf16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, acc, out, n8);
  return hipGetLastError();
}

// Workspace of the full pass: counts | offsets | perm | route scratch | qh | sh | acc
struct MoeLayout {
  int64_t counts, offsets, perm, route, qh, sh, acc, total;
};

static MoeLayout moe_layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk) {
  MoeLayout L;
  int64_t o = 0;
  const int64_t n = T * topk;
  L.counts = o; o += align256(E * 4);
  L.offsets = o; o += align256((E + 1) * 4);
  L.perm = o; o += align256(n * 4);
  L.route = o; o += (int64_t)route_workspace_bytes(T, topk, E);
  L.qh = o; o += align256(n * I);
  L.sh = o; o += align256(n * 4);
  L.acc = o; o += align256(T * H * 4);
  L.total = o;
  return L;
}

size_t moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk) {
  return (size_t)moe_layout(T, H, I, E, topk).total;
}

hipError_t launch_moe(const uint8_t* xq, const float* xs, const int32_t* ids, const float* tw, const uint8_t* w13,
                      const float* s13, const uint8_t* w2, const float* s2, uint16_t* out, int64_t T, int64_t H,
                      int64_t I, int64_t E, int64_t topk, void* ws, hipStream_t stream) {
  const MoeLayout L = moe_layout(T, H, I, E, topk);
  uint8_t* b = static_cast<uint8_t*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(b + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(b + L.perm);
  uint8_t* qh = b + L.qh;
  float* sh = reinterpret_cast<float*>(b + L.sh);
  float* acc = reinterpret_cast<float*>(b + L.acc);
  hipError_t err = launch_route(ids, T, topk, E, counts, offsets, perm, b + L.route, stream);
  if (err != hipSuccess) return err;
  err = launch_gate_up_swiglu_quant(xq, xs, perm, offsets, w13, s13, qh, sh, T, H, I, E, topk, stream);
  if (err != hipSuccess) return err;
  return launch_down_combine(qh, sh, perm, offsets, tw, w2, s2, out, acc, T, H, I, E, topk, stream);
}

hipError_t launch_grouped_gate_up(const uint8_t* xq, const float* xs, const int32_t* ids, const uint8_t* w13,
                                  const float* s13, uint16_t* gu, int32_t* perm, int32_t* offsets, int64_t T,
                                  int64_t H, int64_t I, int64_t E, int64_t topk, void* ws, hipStream_t stream) {
  uint8_t* b = static_cast<uint8_t*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(b);
  hipError_t err = launch_route(ids, T, topk, E, counts, offsets, perm, b + align256(E * 4), stream);
  if (err != hipSuccess) return err;
  return launch_grouped_gate_up_bf16(xq, xs, perm, offsets, w13, s13, gu, T, H, I, E, topk, stream);
}

size_t grouped_gate_up_workspace_bytes(int64_t T, int64_t topk, int64_t E) {
  return (size_t)(align256(E * 4) + (int64_t)route_workspace_bytes(T, topk, E));
}

}  // namespace w8a8
