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
// routed copy (slot) of h, and out[t] = bf16(sum_j w[t,j] * y[t,j]) with the
// weighted copies kept in float32 and summed in float32, rounded once.
//
// Kernels
//  * route_count / route_scatter: slots t*k+j are grouped by expert (or by
//    (top-k position, expert)), in increasing slot order inside a group (a
//    stable sort), ids outside [0, E) dropped. Chunk histograms, then one
//    wave per sub-chunk walks its slots in order; lanes holding the same key
//    are matched with log2(G) ballots, so each slot's rank among earlier
//    equal keys is a popcount. Optionally also the inverse map slot -> row.
//    No host synchronisation: every later kernel reads the offsets from
//    device memory and derives its own tile from them.
//  * grouped_tiled: the dense tiled pipeline (WGM x WGN waves, 128-deep K
//    steps staged global -> LDS by direct buffer loads, double-buffered for
//    the large tiles and in one stage for the small ones, 16x16x128 E4M3
//    MFMAs) over sorted slots, one expert per m-tile:
//      GATE_UP    A rows gathered through the permutation (slot -> token),
//                 BF16 gate/up output in sorted order;
//      GATE_UP_H  the same product with gate and up weight blocks
//                 interleaved in the tile, so the epilogue forms
//                 h = silu(g) * u in float32 in registers, stores h and
//                 folds each row's max |h| into an integer atomicMax;
//      DOWN_Y     A = the requantised rows (sorted, contiguous), B = W2 of
//                 the tile's expert; the epilogue applies the row scale, the
//                 channel scale and the router weight and stores the slot's
//                 float32 product y to its own row (or, in the full pass, to
//                 its sorted row), staged through LDS into whole row pieces.
//  * requant_rows: elementwise E4M3 requantisation of h once the row maxima
//    are known (scale = amax / 448, correctly rounded division, RNE).
//  * combine_slots: out[t] = bf16(sum_j y[t*k + j]) over valid slots
//    (float32 rows and sums, one rounding), added in the fixed order
//    j = 0, 1, ... (deterministic, no atomics; float32 atomics measured ~3x
//    slower than this whole stage). The k rows of a token are contiguous in
//    the per-stage layout and gathered through the slot -> row map in the
//    full pass; either way one streaming pass. combine_quant also quantises
//    each output row per token (the next pass's input) in the same pass.
#include <algorithm>

#include "device.h"
#include "grouped.h"
#include "launch.h"

namespace w8a8 {
namespace {

constexpr int kRouteChunk = 1024;       // slots per routing block (4 waves x 256)
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

// Group key of slot s with expert id e: e itself (expert-major order), or
// (s % kdiv) * Eids + e (slot-position-major order, kdiv = top-k); -1 if the
// id is outside [0, Eids).
__device__ inline int group_key(int64_t s, int e, int Eids, int kdiv) {
  if (e < 0 || e >= Eids) return -1;
  return kdiv ? (int)(s % kdiv) * Eids + e : e;
}

__global__ __launch_bounds__(256) void route_count(const int32_t* __restrict__ ids, int64_t n, int Eids, int kdiv,
                                                   int G, int32_t* __restrict__ chunk_counts) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < G; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kRouteChunk;
  for (int i = threadIdx.x; i < kRouteChunk; i += 256) {
    const int64_t s = base + i;
    if (s < n) {
      const int key = group_key(s, ids[s], Eids, kdiv);
      if (key >= 0) atomicAdd(&hist[key], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G; e += 256) chunk_counts[(int64_t)blockIdx.x * G + e] = hist[e];
}

// LDS: before[E] | base[4][E] | whist[4][E]
__global__ __launch_bounds__(256) void route_scatter(const int32_t* __restrict__ ids, int64_t n, int Eids, int kdiv,
                                                     int E, int nchunks, const int32_t* __restrict__ chunk_counts,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm, int32_t* __restrict__ slot_row,
                                                     uint32_t* __restrict__ zero, int64_t zero_n) {
  extern __shared__ int sm[];
  // side job for the full pass: clear the gate/up stage's row maxima
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < zero_n; i += (int64_t)gridDim.x * 256) zero[i] = 0;
  int* before = sm;              // slots of expert e in earlier chunks, plus the expert's offset
  int* base = sm + E;            // per wave running position
  int* whist = sm + 5 * E;       // per wave histogram of its sub-chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  // this wave's keys, loaded once up front so that their latency overlaps
  // the chunk-count reads (E + 1: dropped id, E + 2: past the end)
  const int64_t sub0 = (int64_t)c * kRouteChunk + (int64_t)wave * kRouteSub;
  int keys[kRouteSub / 64];
#pragma unroll
  for (int i = 0; i < kRouteSub / 64; ++i) {
    const int64_t s = sub0 + 64 * i + lane;
    int key = E + 1;
    if (s < n) {
      const int k2 = group_key(s, ids[s], Eids, kdiv);
      key = k2 >= 0 ? k2 : E;
    }
    keys[i] = key;
  }
  for (int e = tid; e < 4 * E; e += 256) whist[e] = 0;
  // group totals and the counts of earlier chunks: every thread takes groups
  // tid, tid + 256, ...; the exclusive scan over groups is then done by wave 0
  for (int e = tid; e < E; e += 256) {
    int tot = 0, bef = 0;
#pragma unroll 8
    for (int cc = 0; cc < nchunks; ++cc) {
      const int v = chunk_counts[(int64_t)cc * E + e];
      tot += v;
      bef += cc < c ? v : 0;
    }
    base[e] = tot;      // base[] is free until the scatter; use it for totals
    before[e] = bef;
  }
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int tot = e < E ? base[e] : 0;
      int incl = tot;
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
      }
      const int off = carry + incl - tot;
      if (e < E) {
        before[e] += off;
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
  // pass 1: histogram of this wave's sub-chunk
#pragma unroll
  for (int i = 0; i < kRouteSub / 64; ++i) {
    const int key = keys[i];
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
#pragma unroll
  for (int i = 0; i < kRouteSub / 64; ++i) {
    const int64_t s = sub0 + 64 * i + lane;
    const int key = keys[i];
    const uint64_t peers = match_peers(key, nbits);
    if (key < E) {
      const int pos = base[wave * E + key] + __popcll(peers & lt);
      perm[pos] = (int32_t)s;
      if (slot_row) slot_row[s] = pos;
    } else if (slot_row && key == E) {
      slot_row[s] = -1;  // dropped id
    }
    __builtin_amdgcn_wave_barrier();
    const bool leader = lane == 63 - __clzll(peers);
    if (leader && key < E) base[wave * E + key] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

enum { kGateUp = 0, kGateUpH = 1, kDownY = 2 };

template <int BM, int BN, int WGM, int WGN, int MODE, int NS>
struct Grouped {
  static constexpr int kThreads = 64 * WGM * WGN;
  static constexpr int WM = BM / WGM, WN = BN / WGN;   // per-wave tile
  static constexpr int SM = WM / 16, SN = WN / 16;     // 16x16 MFMA tiles per wave
  static constexpr int kRows = BM + BN;
  static constexpr int kStage = kRows * 128;
  static constexpr int kRowsPerPass = kThreads / 8;    // rows one load instruction covers
  static constexpr int kLoadsB = BN / kRowsPerPass, kLoadsA = BM / kRowsPerPass;
  static constexpr int kEpiStride = BN * 2 + 16;       // BF16 staging row (GATE_UP)
  static constexpr int kEpi = MODE == kGateUp ? BM * kEpiStride : 0;
  static constexpr int kLds = (NS * kStage > kEpi) ? NS * kStage : kEpi;
  // The down epilogue stages a wave row block's float32 rows in kJH parts,
  // each no larger than the K loop's stages.
  static constexpr int kJH = (MODE == kDownY && WM * BN * 4 > kLds) ? 2 : 1;
  static_assert(NS == 1 || NS == 2, "one or two stages");
  static_assert(BN % kRowsPerPass == 0 && BM % kRowsPerPass == 0, "stage must split evenly over the threads");
  static_assert(kRowsPerPass % 8 == 0, "the loader's chunk swizzle needs 8-row passes");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(MODE != kGateUpH || (SN % 2 == 0 && BN % 32 == 0), "gate/up block pairs must stay in one wave");
};

struct GroupedArgs {
  const uint8_t* A;         // GATE_UP*: x codes [a_rows, K]; DOWN_Y: sorted h codes [a_rows, K]
  const float* sA;          // GATE_UP*: token scales; DOWN_Y: sorted row scales
  int64_t a_rows;           // rows of A (tokens, or sorted rows)
  const int32_t* perm;      // sorted row -> slot
  const int32_t* offsets;   // [G + 1] group starts (device)
  int G, Eids, topk;        // groups, experts (group g uses expert g % Eids), top-k
  const uint8_t* B;         // [E, N, K] weight codes
  const float* sB;          // [E, N] weight row scales
  const float* tw;          // DOWN_Y: router weights [slots]
  uint16_t* out_bf16;       // GATE_UP: [rows, N]
  float* out_f32;           // GATE_UP_H: h [rows, N / 2]; DOWN_Y: y [slots, N]
  uint32_t* row_amax;       // GATE_UP_H: max |h| bits per output row (cleared by the caller)
  const int32_t* dst_row;   // GATE_UP_H: slot -> output row (NULL: the sorted row itself)
  int32_t* slot_row;        // DOWN_Y: NULL, y row = slot; else y row = sorted row, and slot_row[slot] = it
  int N, K, tiles_n, tiles_m_max;
};

// Grouped GEMM over sorted slots: M = sorted rows, N = output columns of the
// group's expert weight [N, K], K = reduction. Same pipeline as the dense
// tiled kernel (WGM x WGN waves, 128-deep K steps staged global -> LDS by
// direct buffer loads, 16x16x128 E4M3 MFMAs). NS = 2: two stages, the next
// step loads into one while the MFMAs read the other. NS = 1: one stage,
// half the LDS so that more workgroups fit on a CU; each wave takes the
// step's fragments into registers, the workgroup meets, and the next step's
// loads then overlap the MFMAs.
//  GATE_UP:   A row = x[perm[r] / topk] (gathered); out = BF16 [r, N] with the
//             scales x_scale[token] * sB[e, n].
//  GATE_UP_H: as GATE_UP, but the stage's weight rows alternate a block of 16
//             gate rows and the block of the 16 matching up rows (n-tile nt
//             covers h columns [nt * BN/2, (nt + 1) * BN/2)), so the g and u
//             of one h element land in the same lane and register. The
//             epilogue forms h = silu(g) * u in float32, stores it to row
//             dst_row[slot] (or r) of out_f32 [*, N/2], and posts the row's
//             partial max |h| with an integer atomicMax on the float bits
//             (order-independent, so the row maximum is exact).
//  DOWN_Y:    A row = h codes of sorted row r (contiguous); the epilogue
//             stores w[slot] * sA[r] * sB[e, n] * acc in float32 to row
//             `slot` of out_f32 [T * topk, N] (every slot is written once),
//             or with slot_row to row r (a tile's rows are then one
//             contiguous block; the n-tile 0 workgroups record
//             slot_row[slot] = r for the combine), staged through LDS so
//             that every store instruction writes whole row pieces.
template <int BM, int BN, int WGM, int WGN, int MODE, int OCC, int NS>
__global__ __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(1, OCC)))
void grouped_tiled(const GroupedArgs p) {
  using C = Grouped<BM, BN, WGM, WGN, MODE, NS>;
  // One LDS object: the stages (or the epilogue's staging), then the row
  // tables. With a single object the compiler does not make the LDS reads
  // of a K step wait for the next step's direct-to-LDS loads.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLds + BM * 12];
  int* const row_tok = reinterpret_cast<int*>(smem + C::kLds);                // token of each tile row (-1 = empty)
  float* const row_scale = reinterpret_cast<float*>(smem + C::kLds + BM * 4); // A scale (times the router weight for DOWN)
  int* const row_dst = reinterpret_cast<int*>(smem + C::kLds + BM * 8);       // GATE_UP_H: output row (-1 = none)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = p.N, K = p.K;
  // tile id -> (m-tile, n-tile): each XCD walks a contiguous range, so the
  // n-tiles of one m-tile (same A rows) and neighbouring m-tiles of one
  // expert (same weights) share an L2
  const int total = p.tiles_m_max * p.tiles_n;
  const int per = total >> 3;
  int t = blockIdx.x;
  if ((int)blockIdx.x < (per << 3)) t = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  const int mt = t / p.tiles_n, nt = t - mt * p.tiles_n;
  constexpr bool kIsDown = MODE == kDownY;
  const int cap = (int)(kIsDown ? p.a_rows : p.a_rows * p.topk);  // sorted-row capacity
  int grp, row0, rows;
  if (!find_tile(p.offsets, p.G, BM, mt, cap, grp, row0, rows)) return;
  const int e = grp % p.Eids;
  const int n0 = nt * BN;

  // The row tables. A down-projection tile reads contiguous rows, so its
  // first stage of loads is issued before these (their loads overlap); the
  // first barrier of the K loop orders the tables before their use.
  auto setup_rows = [&]() {
    for (int i = tid; i < BM; i += C::kThreads) {
      int tok = -1, dst = -1;
      float sc = 0.f;
      if (i < rows) {
        const int slot = p.perm[row0 + i];
        if (slot >= 0 && slot < cap) {
          tok = MODE == kDownY ? slot : slot / p.topk;  // DOWN_Y keeps the slot: its output row
          sc = kIsDown ? p.sA[row0 + i] * p.tw[slot] : p.sA[tok];
          if (MODE == kGateUpH) {
            dst = p.dst_row ? p.dst_row[slot] : row0 + i;
            if (dst >= cap) dst = -1;
          }
        }
      }
      row_tok[i] = tok;
      row_scale[i] = sc;
      row_dst[i] = dst;
    }
  };
  if (!kIsDown) {
    setup_rows();
    __syncthreads();
  }

  const auto rB = MODE == kGateUpH ? make_rsrc(p.B + (int64_t)e * N * K, (int64_t)N * K)
                                    : make_rsrc(p.B + ((int64_t)e * N + n0) * K, (int64_t)(N - n0) * K);
  const auto rA = kIsDown ? make_rsrc(p.A + (int64_t)row0 * K, (int64_t)rows * K) : make_rsrc(p.A, p.a_rows * K);
  // Loader (as in the dense kernel): LDS slot tid + kThreads * i holds stage
  // row (tid >> 3) + kRowsPerPass * i, logical chunk (tid & 7) ^ (row & 7).
  // Stage rows 0..BN-1 hold B, rows BN.. hold A.
  const int lchunk = ((tid & 7) ^ ((tid >> 3) & 7)) << 4;
  const int lrow = tid >> 3;
  uint32_t boff[C::kLoadsB], aoff[C::kLoadsA];
#pragma unroll
  for (int i = 0; i < C::kLoadsB; ++i) {
    const int r = lrow + C::kRowsPerPass * i;
    int wr = r;
    if (MODE == kGateUpH) {  // 16-row block b: even = gate rows, odd = the matching up rows
      const int b = r >> 4;
      wr = (b & 1 ? N / 2 : 0) + (n0 >> 1) + (b >> 1) * 16 + (r & 15);
    }
    boff[i] = (uint32_t)wr * (uint32_t)K + (uint32_t)lchunk;
  }
#pragma unroll
  for (int j = 0; j < C::kLoadsA; ++j) {
    const int lr = lrow + C::kRowsPerPass * j;
    if (!kIsDown) {
      const int tok = row_tok[lr];
      aoff[j] = tok < 0 ? kOutOfRange : (uint32_t)tok * (uint32_t)K + (uint32_t)lchunk;
    } else {
      aoff[j] = lr < rows ? (uint32_t)lr * (uint32_t)K + (uint32_t)lchunk : kOutOfRange;
    }
  }
  auto issue = [&](int stage, int k0) {
    uint8_t* base = smem + stage * C::kStage;
    const bool kin = k0 + lchunk < K;
#pragma unroll
    for (int i = 0; i < C::kLoadsB + C::kLoadsA; ++i) {
      const int s0 = wave * 64 + C::kThreads * i;  // first LDS slot of this wave's 64
      if (i < C::kLoadsB) {
        buffer_load16_lds(rB, base + s0 * 16, kin ? boff[i] + (uint32_t)k0 : kOutOfRange);
      } else {
        const uint32_t a = aoff[i - C::kLoadsB];
        buffer_load16_lds(rA, base + s0 * 16, (kin && a != kOutOfRange) ? a + (uint32_t)k0 : kOutOfRange);
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
  const int nk = (K + 127) >> 7;
  // The epilogue's weight-row scales (per lane: four consecutive columns of
  // each of its SN column blocks; for GATE_UP_H block i holds gate columns
  // when i is even and the matching up columns when i is odd). The large
  // tiles (two waves per SIMD, registers to spare) load them before the K
  // loop, so that their latency passes under it; the small tiles, at three
  // waves per SIMD, load them after it.
  float4 esc[C::SN];
  auto load_scales = [&]() {
#pragma unroll
    for (int i = 0; i < C::SN; ++i) {
      if (MODE == kGateUpH) {
        const int hc = (n0 >> 1) + (((wn * C::WN + (i & ~1) * 16) >> 5) << 4) + 4 * g;
        esc[i] = *reinterpret_cast<const float4*>(p.sB + (int64_t)e * N + (i & 1 ? N / 2 : 0) + hc);
      } else {
        const int n = n0 + wn * C::WN + i * 16 + 4 * g;
        esc[i] = n < N ? *reinterpret_cast<const float4*>(p.sB + (int64_t)e * N + n) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  constexpr bool kScalesFirst = OCC <= 2;
  if (kScalesFirst) load_scales();
  issue(0, 0);
  if (kIsDown) {
    setup_rows();
    if (p.slot_row != nullptr && nt == 0)
      for (int i = tid; i < rows; i += C::kThreads) {
        const int slot = p.perm[row0 + i];
        if (slot >= 0 && slot < cap) p.slot_row[slot] = row0 + i;
      }
  }
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmem_all();
    __syncthreads();
    if (NS == 2 && kt + 1 < nk) issue((kt + 1) & 1, (kt + 1) << 7);
    const uint8_t* st = smem + (NS == 2 ? (kt & 1) * C::kStage : 0);
    v8i xf[C::SM];
#pragma unroll
    for (int j = 0; j < C::SM; ++j) xf[j] = lds_frag(st, BN + wm * C::WM + j * 16 + r16, g);
    if (NS == 1) {
      // one stage: every fragment of this step in registers, then the next
      // step's loads, which overlap this step's MFMAs
      v8i wfa[C::SN];
#pragma unroll
      for (int i = 0; i < C::SN; ++i) wfa[i] = lds_frag(st, wn * C::WN + i * 16 + r16, g);
      lds_barrier();
      if (kt + 1 < nk) issue(0, (kt + 1) << 7);
#pragma unroll
      for (int i = 0; i < C::SN; ++i)
#pragma unroll
        for (int j = 0; j < C::SM; ++j) acc[i][j] = mfma_16x16x128_e4m3(wfa[i], xf[j], acc[i][j]);
    } else {
#pragma unroll
      for (int i = 0; i < C::SN; ++i) {
        const v8i wf = lds_frag(st, wn * C::WN + i * 16 + r16, g);
#pragma unroll
        for (int j = 0; j < C::SM; ++j) acc[i][j] = mfma_16x16x128_e4m3(wf, xf[j], acc[i][j]);
      }
    }
  }

  // acc[i][j][r]: tile row wm * WM + 16 j + lane % 16, stage (weight) row
  // wn * WN + 16 i + 4 (lane / 16) + r.
  if constexpr (MODE == kDownY) {
    // The weighted copy in float32, staged through LDS (the K loop's stages
    // are free now) one wm's rows (or half of them) at a time, then written as whole row
    // pieces: one store instruction covers BN * 4 contiguous bytes of each
    // of 256 / BN rows. Straight from the MFMA registers an instruction would
    // cover 16 rows x 64 bytes, which the memory system drains markedly
    // slower (a plain write stream of each shape: 3.9 against 5.9 TB/s).
    // Staged rows are XOR-swizzled by 16-byte chunk so that both the
    // register writes (16 rows per lane group) and the row reads are free of
    // bank conflicts.
    constexpr int kChunks = BN / 4;                 // 16-byte chunks of a staged row
    constexpr int kRowsPerInst = 64 / kChunks;
    constexpr int kJH = C::kJH, kPartRows = C::WM / kJH, kPartJ = C::SM / kJH;
    static_assert(kPartRows * BN * 4 <= C::kLds && C::SM % kJH == 0, "a part of a wm's rows must fit in the LDS");
    static_assert(kChunks >= 16 && 64 % kChunks == 0, "row pieces must tile a wave");
    if (!kScalesFirst) load_scales();
    const float4* const sW = esc;
#pragma unroll
    for (int pass = 0; pass < WGM * kJH; ++pass) {
      const int pw = pass / kJH, ph = pass % kJH;
      __syncthreads();  // the K-loop stages (pass 0) or the previous pass's rows are read
      if (wm == pw) {
#pragma unroll
        for (int jl = 0; jl < kPartJ; ++jl) {
          const int j = ph * kPartJ + jl;
          const int rl = jl * 16 + r16;
          const float s = row_scale[wm * C::WM + j * 16 + r16];
#pragma unroll
          for (int i = 0; i < C::SN; ++i) {
            const int chunk = wn * (C::WN / 4) + i * 4 + g;
            const v4f a = acc[i][j];
            *reinterpret_cast<float4*>(smem + rl * (BN * 4) + ((chunk ^ (rl & 15)) << 4)) =
                make_float4(a[0] * s * sW[i].x, a[1] * s * sW[i].y, a[2] * s * sW[i].z, a[3] * s * sW[i].w);
          }
        }
      }
      __syncthreads();
      // The large tiles: all of a thread's LDS reads first, then its stores
      // (one LDS latency). The small tiles, at three waves per SIMD, one
      // piece at a time, to stay in their register budget.
      const int c = lane % kChunks;
      const int n = n0 + c * 4;
      constexpr int kStep = (C::kThreads / 64) * kRowsPerInst;
      constexpr int kPieces = kPartRows / kStep;
      constexpr int kBatch = OCC <= 2 ? kPieces : 1;
      static_assert(kPartRows % kStep == 0 && kPieces % kBatch == 0, "the staged rows must split evenly");
      const int rl0 = wave * kRowsPerInst + lane / kChunks;
#pragma unroll 1
      for (int b = 0; b < kPieces; b += kBatch) {
        float4 piece[kBatch];
        int slot[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          const int rl = rl0 + (b + q) * kStep;
          piece[q] = *reinterpret_cast<const float4*>(smem + rl * (BN * 4) + ((c ^ (rl & 15)) << 4));
          slot[q] = row_tok[pw * C::WM + ph * kPartRows + rl];
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          const int ml = pw * C::WM + ph * kPartRows + rl0 + (b + q) * kStep;
          const int64_t yrow = p.slot_row != nullptr ? (int64_t)(row0 + ml) : (int64_t)slot[q];
          if (slot[q] >= 0 && n < N) store16_nt(p.out_f32 + yrow * N + n, piece[q]);
        }
      }
    }
    return;
  }
  if (MODE == kGateUpH) {
    const int Ih = N / 2;
    int dsts[C::SM];
    float rs[C::SM], amax[C::SM];
#pragma unroll
    for (int j = 0; j < C::SM; ++j) {
      const int ml = wm * C::WM + j * 16 + r16;
      dsts[j] = row_dst[ml];
      rs[j] = row_scale[ml];
      amax[j] = 0.f;
    }
    if (!kScalesFirst) load_scales();  // gate and up scales, loaded together
#pragma unroll
    for (int i = 0; i < C::SN; i += 2) {  // i: gate block, i + 1: its up block
      const int sr = wn * C::WN + i * 16;
      const int hc = (n0 >> 1) + ((sr >> 5) << 4) + 4 * g;  // h column of this lane's first value
      const float4 gs4 = esc[i], us4 = esc[i + 1];
      const float gs[4] = {gs4.x, gs4.y, gs4.z, gs4.w}, us[4] = {us4.x, us4.y, us4.z, us4.w};
#pragma unroll
      for (int j = 0; j < C::SM; ++j) {
        const v4f ga = acc[i][j], ua = acc[i + 1][j];
        float h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gv = ga[r] * rs[j] * gs[r];
          const float uv = ua[r] * rs[j] * us[r];
          h[r] = silu_f32(gv) * uv;
          amax[j] = fmaxf(amax[j], fabsf(h[r]));
        }
        if (dsts[j] >= 0)
          store16_nt(p.out_f32 + (int64_t)dsts[j] * Ih + hc, make_float4(h[0], h[1], h[2], h[3]));
      }
    }
    // lane groups g = 0..3 hold the same rows: reduce over them, one atomic per row
#pragma unroll
    for (int j = 0; j < C::SM; ++j) {
      float m = amax[j];
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (g == 0 && dsts[j] >= 0) atomicMax(p.row_amax + dsts[j], __float_as_uint(m));
    }
    return;
  }
  // GATE_UP: scale, round to BF16, stage in LDS, store full row segments
  if (!kScalesFirst) load_scales();  // the weight scales, loaded together before the barrier
  __syncthreads();
#pragma unroll
  for (int i = 0; i < C::SN; ++i) {
    const int nl = wn * C::WN + i * 16 + 4 * g;
    const float4 sW = esc[i];
#pragma unroll
    for (int j = 0; j < C::SM; ++j) {
      const int ml = wm * C::WM + j * 16 + r16;
      const float s = row_scale[ml];
      const v4f a = acc[i][j];
      const uint32_t p0 = bf16x2_rne(a[0] * s * sW.x, a[1] * s * sW.y);
      const uint32_t p1 = bf16x2_rne(a[2] * s * sW.z, a[3] * s * sW.w);
      *reinterpret_cast<uint2*>(smem + ml * C::kEpiStride + nl * 2) = make_uint2(p0, p1);
    }
  }
  __syncthreads();
  constexpr int kRowChunks = BN / 8;
  for (int c = tid; c < BM * kRowChunks; c += C::kThreads) {
    const int row = c / kRowChunks, col = (c % kRowChunks) * 8;
    if (row < rows && n0 + col < N)
      store16_nt(p.out_bf16 + (int64_t)(row0 + row) * N + n0 + col,
                 *reinterpret_cast<const uint4*>(smem + row * C::kEpiStride + col * 2));
  }
}

// Requantisation of float32 h rows, elementwise once the row maxima are
// known: s_r = fl32(amax_r / 448) (1 for an all-zero row), q = E4M3(fl32(h / s_r))
// (round to nearest even, saturating). As in the activation quantiser, h * r
// with r = fl32(1 / s_r) stands in for the correctly rounded quotient unless
// it lies within a few ulp of an E4M3 rounding boundary (or below 2^-6),
// where the thread redoes its values with the division. One thread per 16
// values of a row; rows from the valid count on are left alone.
__global__ __launch_bounds__(256) void requant_rows(const float* __restrict__ h, const uint32_t* __restrict__ amax_bits,
                                                    const int32_t* __restrict__ nvalid, int64_t cap, int I,
                                                    uint8_t* __restrict__ qh, float* __restrict__ sh) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = I >> 4;
  const int64_t row = i / per_row;
  const int64_t nrows = min((int64_t)*nvalid, cap);
  if (row >= nrows) return;
  const int c0 = (int)(i - row * per_row) << 4;
  const float amax = __uint_as_float(amax_bits[row]);
  const float s = amax == 0.f ? 1.0f : amax / 448.0f;
  const float r = 1.0f / s;
  const float4* src = reinterpret_cast<const float4*>(h + row * I + c0);
  float x[16], q[16];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 v = src[k];
    x[4 * k] = v.x; x[4 * k + 1] = v.y; x[4 * k + 2] = v.z; x[4 * k + 3] = v.w;
  }
  bool near = !(r < 3.0e38f);  // a subnormal scale: 1 / s overflows, divide everything
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    q[k] = x[k] * r;
    near |= e4m3_boundary_near(q[k]);
  }
  if (__builtin_expect(near, 0)) {
#pragma unroll
    for (int k = 0; k < 16; ++k) q[k] = x[k] / s;
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) q[k] = clamp448(q[k]);
  *reinterpret_cast<uint4*>(qh + row * I + c0) =
      make_uint4(e4m3x4(q[0], q[1], q[2], q[3]), e4m3x4(q[4], q[5], q[6], q[7]), e4m3x4(q[8], q[9], q[10], q[11]),
                 e4m3x4(q[12], q[13], q[14], q[15]));
  if (c0 == 0) sh[row] = s;
}

__global__ __launch_bounds__(256) void fill_zero_u32(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// out[t, c] = bf16( sum_j y[t * topk + j, c] ) over the token's valid slots.
// One thread per 8 columns.
__global__ __launch_bounds__(256) void combine_slots(const float* __restrict__ y, const int32_t* __restrict__ ids,
                                                     const int32_t* __restrict__ slot_row, int64_t T, int topk,
                                                     int Eids, int H,
                                                     uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = H >> 3;
  const int64_t t = i / per_row;
  if (t >= T) return;
  int ca, cb;
  split_cols8((int)(i - t * per_row), H, ca, cb);
  float4 a, b;
  sum_slots_split(y, ids, slot_row, t, topk, Eids, H, ca, cb, a, b);
  const uint4 o = to_bf16x8(a, b);
  *reinterpret_cast<uint2*>(out + t * H + ca) = make_uint2(o.x, o.y);
  *reinterpret_cast<uint2*>(out + t * H + cb) = make_uint2(o.z, o.w);
}

// The combine with the next pass's per-token quantisation fused in: one
// workgroup per token, PER chunks of 8 columns per thread (H <= 2048 * PER).
// Writes out[t] (BF16) and q[t] / qs[t], exactly what quantize_per_token
// makes of out[t]: amax on the BF16 bits, s = fl32(amax / 448), codes of
// fl32(x / s) (the same shared quantiser code).
template <int PER>
__global__ __launch_bounds__(256) void combine_quant(const float* __restrict__ y, const int32_t* __restrict__ ids,
                                                     const int32_t* __restrict__ slot_row, int topk, int Eids, int H, uint16_t* __restrict__ out,
                                                     uint8_t* __restrict__ q, float* __restrict__ qs) {
  __shared__ uint32_t wmax[4];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint4 vb[PER];
  uint32_t amax = 0;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int r8 = tid + 256 * p;
    vb[p] = make_uint4(0u, 0u, 0u, 0u);
    if ((r8 << 3) < H) {
      int ca, cb;
      split_cols8(r8, H, ca, cb);
      float4 a, b;
      sum_slots_split(y, ids, slot_row, t, topk, Eids, H, ca, cb, a, b);
      vb[p] = to_bf16x8(a, b);
      *reinterpret_cast<uint2*>(out + t * H + ca) = make_uint2(vb[p].x, vb[p].y);
      *reinterpret_cast<uint2*>(out + t * H + cb) = make_uint2(vb[p].z, vb[p].w);
      const uint32_t m = absmax8(vb[p]);
      amax = amax > m ? amax : m;
    }
  }
  amax = wave_max_u32(amax);
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  amax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float s = row_scale(amax);
  const float r = 1.0f / s;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int r8 = tid + 256 * p;
    if ((r8 << 3) < H) {
      int ca, cb;
      split_cols8(r8, H, ca, cb);
      const uint2 c = quant8(vb[p], s, r);
      *reinterpret_cast<uint32_t*>(q + t * H + ca) = c.x;
      *reinterpret_cast<uint32_t*>(q + t * H + cb) = c.y;
    }
  }
  if (tid == 0) qs[t] = s;
}

int64_t align256(int64_t b) { return (b + 255) & ~int64_t(255); }

int route_chunks(int64_t n) { return (int)((n + kRouteChunk - 1) / kRouteChunk); }

// Tile shapes (both on expert-major groups of about T*k/E rows): 256 x 256
// tiles, 8 waves of 128 x 64, two waves per SIMD. Measured on the 16384-token
// two-pass workload against 128 x 256, 256 x 128 and 128 x 128 tiles for the
// gate/up, and 128 x 256, 128 x 128 and a persistent variant with split
// load / store roles for the down projection: this shape was the fastest.
constexpr int kGuBM = 256, kGuBN = 256, kGuWGM = 2, kGuWGN = 4, kGuOcc = 2;
constexpr int kDnBM = 256, kDnBN = 256, kDnWGM = 2, kDnWGN = 4, kDnOcc = 2;
// Smaller groups (few tokens per expert, e.g. 128 or 192 experts at top-4)
// take smaller tiles: with 256-row tiles much of each group's last tile
// would be padding, and a pass has too few tiles to fill the chip. Below
// kSmallGroupRows rows on average: 128 x 128 tiles of 2 x 2 waves; below
// kTinyGroupRows: 64 x 128 tiles of 1 x 2 waves. Both with one LDS stage
// (NS = 1) and up to three waves per SIMD: six 64 x 128 workgroups fit on a
// CU instead of three, and three 128 x 128 ones instead of two. Against the
// double-buffered form with its lower occupancy, the same results bit for
// bit: 7-10% less time for a whole two-pass FFN at 128 and 192 experts, and
// 3.5% at 4096 tokens, top-8 of 64.
// Timed at 4096 tokens with 128 and 192 experts (128 and 85 rows per group),
// at 8192 and 12288 tokens with 128 experts (256 and 384 rows) against
// 128 x 256, 64 x 256, 64 x 64 and 4-wave 64 x 128 tiles, and at 4096
// tokens, top-8 of 64 experts (512 rows): 128 x 128 tiles 5% faster than
// 256 x 256 there, with 31% of the issued rows padding in the latter.
constexpr int64_t kSmallGroupRows = 1024, kTinyGroupRows = 192;


template <int BM, int BN, int WGM, int WGN, int MODE, int OCC, int NS = 2>
hipError_t run_grouped(GroupedArgs a, int64_t max_rows, hipStream_t stream) {
  a.tiles_n = (a.N + BN - 1) / BN;
  a.tiles_m_max = (int)((max_rows + BM - 1) / BM + a.G);  // every group adds at most one partial tile
  const int64_t blocks = (int64_t)a.tiles_m_max * a.tiles_n;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_tiled<BM, BN, WGM, WGN, MODE, OCC, NS>), dim3((unsigned)blocks), dim3(64 * WGM * WGN), 0,
                     stream, a);
  return hipGetLastError();
}

// One grouped launch in the tile shape that suits the average group size.
template <int MODE>
hipError_t run_grouped_auto(const GroupedArgs& a, int64_t max_rows, int64_t avg_rows, hipStream_t stream) {
  if (avg_rows < kTinyGroupRows) return run_grouped<64, 128, 1, 2, MODE, 3, 1>(a, max_rows, stream);
  if (avg_rows < kSmallGroupRows) return run_grouped<128, 128, 2, 2, MODE, 3, 1>(a, max_rows, stream);
  if (MODE == kDownY) return run_grouped<kDnBM, kDnBN, kDnWGM, kDnWGN, MODE, kDnOcc>(a, max_rows, stream);
  return run_grouped<kGuBM, kGuBN, kGuWGM, kGuWGN, MODE, kGuOcc>(a, max_rows, stream);
}

GroupedArgs gate_up_args(const uint8_t* xq, const float* xs, const int32_t* perm, const int32_t* offsets, int G,
                         const uint8_t* w13, const float* s13, int64_t T, int64_t H, int64_t I, int64_t E,
                         int64_t topk) {
  GroupedArgs a{};
  a.A = xq;
  a.sA = xs;
  a.a_rows = T;
  a.perm = perm;
  a.offsets = offsets;
  a.G = G;
  a.Eids = (int)E;
  a.topk = (int)topk;
  a.B = w13;
  a.sB = s13;
  a.N = (int)(2 * I);
  a.K = (int)H;
  return a;
}

}  // namespace

size_t route_workspace_bytes(int64_t T, int64_t topk, int64_t G) {
  return (size_t)align256((int64_t)route_chunks(T * topk) * G * 4);
}

int64_t route_groups(int64_t topk, int64_t E, int order) { return order ? topk * E : E; }

hipError_t launch_route(const int32_t* ids, int64_t T, int64_t topk, int64_t E, int order, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* slot_row, void* scratch, hipStream_t stream,
                        uint32_t* zero, int64_t zero_n) {
  const int64_t n = T * topk;
  const int nch = route_chunks(n);
  if (nch == 0) return hipSuccess;
  const int G = (int)route_groups(topk, E, order);
  const int kdiv = order ? (int)topk : 0;
  int32_t* chunk_counts = static_cast<int32_t*>(scratch);
  hipLaunchKernelGGL(route_count, dim3(nch), dim3(256), (size_t)G * 4, stream, ids, n, (int)E, kdiv, G,
                     chunk_counts);
  hipLaunchKernelGGL(route_scatter, dim3(nch), dim3(256), (size_t)G * 9 * 4, stream, ids, n, (int)E, kdiv, G, nch,
                     chunk_counts, counts, offsets, perm, slot_row, zero, zero_n);
  return hipGetLastError();
}

hipError_t launch_grouped_gate_up_bf16(const uint8_t* xq, const float* xs, const int32_t* perm,
                                       const int32_t* offsets, const uint8_t* w13, const float* s13, uint16_t* gu,
                                       int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk, int order,
                                       hipStream_t stream) {
  GroupedArgs a = gate_up_args(xq, xs, perm, offsets, (int)route_groups(topk, E, order), w13, s13, T, H, I, E, topk);
  a.out_bf16 = gu;
  return run_grouped_auto<kGateUp>(a, T * topk, T * topk / a.G, stream);
}

size_t gate_up_swiglu_quant_workspace_bytes(int64_t T, int64_t I, int64_t topk) {
  const int64_t n = T * topk;
  return (size_t)(align256(n * 4) + align256(n * I * 4));
}

// Workspace: row maxima [T*k] (uint32 float bits) | h [T*k, I] float32.
hipError_t launch_gate_up_swiglu_quant(const uint8_t* xq, const float* xs, const int32_t* perm,
                                       const int32_t* offsets, const int32_t* dst_row, const uint8_t* w13,
                                       const float* s13, uint8_t* qh, float* sh, float* h_out, int64_t T,
                                       int64_t H, int64_t I, int64_t E, int64_t topk, int order, void* ws,
                                       hipStream_t stream, bool amax_zeroed) {
  const int64_t n = T * topk;
  if (n == 0) return hipSuccess;
  const int G = (int)route_groups(topk, E, order);
  uint32_t* amax = static_cast<uint32_t*>(ws);
  float* h = h_out ? h_out : reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + align256(n * 4));
  if (!amax_zeroed) hipLaunchKernelGGL(fill_zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, amax, n);
  GroupedArgs a = gate_up_args(xq, xs, perm, offsets, G, w13, s13, T, H, I, E, topk);
  a.out_f32 = h;
  a.row_amax = amax;
  a.dst_row = dst_row;
  hipError_t err = run_grouped_auto<kGateUpH>(a, n, n / G, stream);
  if (err != hipSuccess) return err;
  const int64_t threads = n * (I / 16);
  hipLaunchKernelGGL(requant_rows, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, h, amax,
                     offsets + G, n, (int)I, qh, sh);
  return hipGetLastError();
}

// Down projection of the sorted rows (any order: every slot's product goes
// to its own row of y, or with slot_row to its sorted row), then the
// per-token combine.
hipError_t launch_down_combine(const uint8_t* qh, const float* sh, const int32_t* perm, const int32_t* offsets,
                               const int32_t* ids, const float* tw, const uint8_t* w2, const float* s2, uint16_t* out,
                               float* y, uint8_t* out_q, float* out_s, int64_t T, int64_t H, int64_t I, int64_t E,
                               int64_t topk, int order, hipStream_t stream, int32_t* slot_row) {
  GroupedArgs a{};
  a.slot_row = slot_row;
  a.A = qh;
  a.sA = sh;
  a.a_rows = T * topk;
  a.perm = perm;
  a.offsets = offsets;
  a.G = (int)route_groups(topk, E, order);
  a.Eids = (int)E;
  a.topk = (int)topk;
  a.B = w2;
  a.sB = s2;
  a.tw = tw;
  a.out_f32 = y;
  a.N = (int)H;
  a.K = (int)I;
  const hipError_t err = run_grouped_auto<kDownY>(a, T * topk, T * topk / a.G, stream);
  if (err != hipSuccess) return err;
  if (out_q != nullptr && H <= 2048 * 4) {
    const dim3 grid((unsigned)T);
    if (H <= 2048)
      hipLaunchKernelGGL(combine_quant<1>, grid, dim3(256), 0, stream, y, ids, slot_row, (int)topk, (int)E, (int)H, out, out_q, out_s);
    else if (H <= 4096)
      hipLaunchKernelGGL(combine_quant<2>, grid, dim3(256), 0, stream, y, ids, slot_row, (int)topk, (int)E, (int)H, out, out_q, out_s);
    else
      hipLaunchKernelGGL(combine_quant<4>, grid, dim3(256), 0, stream, y, ids, slot_row, (int)topk, (int)E, (int)H, out, out_q, out_s);
    return hipGetLastError();
  }
  const int64_t threads = T * (H / 8);
  hipLaunchKernelGGL(combine_slots, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, y, ids, slot_row, T,
                     (int)topk, (int)E, (int)H, out);
  if (out_q == nullptr) return hipGetLastError();
  const hipError_t cerr = hipGetLastError();  // rows longer than the fused kernel holds: quantise separately
  if (cerr != hipSuccess) return cerr;
  return launch_quantize_rows(out, T, H, out_q, out_s, stream);
}

size_t down_combine_scratch_bytes(int64_t T, int64_t H, int64_t topk) { return (size_t)(T * topk * H * 4); }

// Workspace of the full pass:
//   counts | offsets | perm | route scratch | qh | sh | amax | big
// where big holds h [T*k, I] float32 during the gate/up and then the
// weighted slot products y [T*k, H] float32 of the down projection.
struct MoeLayout {
  int64_t counts, offsets, perm, route, qh, sh, amax, big, total;
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
  L.amax = o; o += align256(n * 4);  // amax | big is the gate/up stage's workspace
  L.big = o; o += std::max(align256(n * I * 4), align256(n * H * 4));
  L.total = o;
  return L;
}

size_t moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk) {
  return (size_t)moe_layout(T, H, I, E, topk).total;
}

// One pass, all on the expert-major order: route, gate/up + SwiGLU +
// requantisation, down projection into per-slot rows, combine.
hipError_t launch_moe(const uint8_t* xq, const float* xs, const int32_t* ids, const float* tw, const uint8_t* w13,
                      const float* s13, const uint8_t* w2, const float* s2, uint16_t* out, uint8_t* out_q,
                      float* out_s, int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk, void* ws,
                      hipStream_t stream) {
  const MoeLayout L = moe_layout(T, H, I, E, topk);
  uint8_t* b = static_cast<uint8_t*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(b + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(b + L.perm);
  uint8_t* qh = b + L.qh;
  float* sh = reinterpret_cast<float*>(b + L.sh);
  // the routing launch also clears the gate/up stage's row maxima
  hipError_t err = launch_route(ids, T, topk, E, 0, counts, offsets, perm, nullptr, b + L.route, stream,
                                reinterpret_cast<uint32_t*>(b + L.amax), T * topk);
  if (err != hipSuccess) return err;
  err = launch_gate_up_swiglu_quant(xq, xs, perm, offsets, nullptr, w13, s13, qh, sh, nullptr, T, H, I, E, topk, 0,
                                    b + L.amax, stream, true);
  if (err != hipSuccess) return err;
  // the down projection writes y in sorted order (each tile's rows one
  // block) and the slot -> row map into the row maxima's words, free by then
  return launch_down_combine(qh, sh, perm, offsets, ids, tw, w2, s2, out, reinterpret_cast<float*>(b + L.big), out_q,
                             out_s, T, H, I, E, topk, 0, stream, reinterpret_cast<int32_t*>(b + L.amax));
}

hipError_t launch_grouped_gate_up(const uint8_t* xq, const float* xs, const int32_t* ids, const uint8_t* w13,
                                  const float* s13, uint16_t* gu, int32_t* perm, int32_t* offsets, int64_t T,
                                  int64_t H, int64_t I, int64_t E, int64_t topk, void* ws, hipStream_t stream) {
  uint8_t* b = static_cast<uint8_t*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(b);
  hipError_t err = launch_route(ids, T, topk, E, 0, counts, offsets, perm, nullptr, b + align256(E * 4), stream);
  if (err != hipSuccess) return err;
  return launch_grouped_gate_up_bf16(xq, xs, perm, offsets, w13, s13, gu, T, H, I, E, topk, 0, stream);
}

size_t grouped_gate_up_workspace_bytes(int64_t T, int64_t topk, int64_t E) {
  return (size_t)(align256(E * 4) + (int64_t)route_workspace_bytes(T, topk, E));
}

}  // namespace w8a8
