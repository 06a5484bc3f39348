// MXFP4 routed experts: E2M1 expert weights and expert inputs with one
// power-of-two (E8M0) scale per 32 consecutive inputs, on the gfx950
// block-scaled FP4 matrix cores.
//
// The 4-bit model page stores the routed experts as 4-bit E2M1 values with a
// scale per small block of inputs, and under fast-math rounds every expert
// input to FP4 as well (Lernex/Metis-1.6-Praxis-NVFP4, "What is in NVFP4" and
// "What --fast-math does"). Its blocks are 16 wide with E4M3 scales; the
// block-scaled format these matrix cores take natively is the OCP
// microscaling MXFP4, used here:
//   value = dec(E2M1 code) * 2^(e - 127), e the block's E8M0 byte;
//   block exponent = floor(log2(amax)) - 2, clamped to [-127, 127] (an
//   all-zero block gets e = 127); elements divided by the scale (exact) and
//   rounded to nearest, ties to even, saturating at 6.
// Layout: codes [rows, K/2] with element 2i in the low nibble of byte i;
// scales [rows, K/32], so block b of a row is code bytes 16b..16b+15 and
// scale byte b.
//
// Kernels
//  * mx_quant_bf16: BF16 rows -> MXFP4, four lanes per block. The block
//    exponent comes from the bit pattern of the block maximum and the
//    division by a power of two is exact, so the codes are bit-exact.
//  * mx_grouped: the grouped expert pipeline with 256-deep K steps: per row
//    and stage, 128 bytes of codes (staged and swizzled as in the FP8
//    kernel) and the row's 8 scale bytes, both by direct buffer -> LDS
//    loads, double-buffered (NS = 2) or, for the small tiles, in one
//    stage (NS = 1) that the next step's loads refill while the stage's
//    second half of MFMAs runs. A stage is two 16x16x128 FP4 MFMAs per tile
//    pair; the lane that holds a row's 32-element block also hands the MFMA
//    that block's E8M0 byte, so the scales are applied inside the matrix
//    core and the epilogue has no per-row scale.
//      GATE_UP    BF16 gate/up output in sorted order;
//      GATE_UP_Q  gate and up weight blocks interleaved as in the FP8
//                 kernel; the epilogue forms h = silu(g) * u in float32, and
//                 each wave's 32 h columns of a row are one MX block, so
//                 the block maximum (a shuffle over the 4 lanes holding the
//                 block), the exponent and the E2M1 codes are made in
//                 registers and stored: no float32 h round trip, no row
//                 maximum, no atomics, no second kernel;
//      DOWN_Y     per-slot float32 y = w[slot] * acc, staged through LDS
//                 and stored as whole row pieces to the slot's own row (or,
//                 in the full pass, to its sorted row, recording the
//                 slot -> row map).
//  * combine_mx: the ordered per-token slot sum of the FP8 combine (float32
//    rows and sums, one BF16 rounding), with the BF16 result optionally
//    quantised to MXFP4 in the same pass (the next pass's expert input).
#include "device.h"
#include "grouped.h"
#include "launch.h"

namespace w8a8 {
namespace {

// ---- the MX block quantiser ------------------------------------------------

// E8M0 byte of a block from the float32 bit pattern of its largest
// magnitude: floor(log2(amax)) - 2 + 127 = biased exponent - 2, clamped at 0
// (float32 subnormals and the two smallest binades); 127 for an all-zero
// block.
__device__ inline uint32_t mx_scale_code(uint32_t amax_bits) {
  if (amax_bits == 0) return 127u;
  const uint32_t e = amax_bits >> 23;
  return e > 2u ? e - 2u : 0u;
}

// 2^(127 - code), the exact reciprocal of the block scale (codes 0..252 are
// the ones finite inputs produce; all give a normal float32).
__device__ inline float mx_inv_scale(uint32_t code) { return __uint_as_float((254u - code) << 23); }

// float32 -> E2M1 code, round to nearest, ties to the even code, |v| > 6
// saturating to 6, the sign kept on zero. The magnitude code counts the
// midpoints between neighbouring magnitudes (0, 0.5, 1, 1.5, 2, 3, 4, 6)
// that |v| passes: a midpoint itself goes down when the lower neighbour's
// mantissa bit is 0 (strict >) and up otherwise (>=).
__device__ inline uint32_t e2m1(float v) {
  const float a = fabsf(v);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

// N values times m -> N nibbles, value 0 in the low nibble.
template <int N>
__device__ inline uint32_t e2m1_pack(const float* v, float m) {
  uint32_t w = 0;
#pragma unroll
  for (int k = 0; k < N; ++k) w |= e2m1(v[k] * m) << (4 * k);
  return w;
}

__device__ inline void bf16x8_to_f32(uint4 v, float* x) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
}

// Quantise 8 BF16 values held by each lane of an aligned quad of lanes (the
// quad holds one 32-element block, lane q of it elements 8q .. 8q+7).
// Returns the lane's 4 code bytes; *code gets the block's E8M0 byte.
__device__ inline uint32_t mx_quad_quant(uint4 v, uint32_t* code) {
  uint32_t m = absmax8(v);
  m = max(m, (uint32_t)__shfl_xor((int)m, 1, 64));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2, 64));
  const uint32_t c = mx_scale_code(m << 16);
  float x[8];
  bf16x8_to_f32(v, x);
  *code = c;
  return e2m1_pack<8>(x, mx_inv_scale(c));
}

// The same for 4 BF16 values per lane (w0, w1) held by an aligned group of 8
// lanes (lane p of it elements 4p .. 4p+3 of the block). Returns the lane's 2
// code bytes; *code gets the block's E8M0 byte.
__device__ inline uint32_t mx_oct_quant(uint32_t w0, uint32_t w1, uint32_t* code) {
  uint32_t m = max(max(w0 & 0x7FFFu, (w0 >> 16) & 0x7FFFu), max(w1 & 0x7FFFu, (w1 >> 16) & 0x7FFFu));
  m = max(m, (uint32_t)__shfl_xor((int)m, 1, 64));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2, 64));
  m = max(m, (uint32_t)__shfl_xor((int)m, 4, 64));
  const uint32_t c = mx_scale_code(m << 16);
  const float x[4] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1)};
  *code = c;
  return e2m1_pack<4>(x, mx_inv_scale(c));
}

// One thread per 8 values; chunks = M * K / 8 with K % 32 == 0, so the four
// threads of a block are an aligned quad of one row and leave together.
__global__ __launch_bounds__(256) void mx_quant_bf16(const uint16_t* __restrict__ x, int64_t chunks,
                                                     uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= chunks) return;
  const uint4 v = reinterpret_cast<const uint4*>(x)[i];
  uint32_t code;
  reinterpret_cast<uint32_t*>(q)[i] = mx_quad_quant(v, &code);
  if ((i & 3) == 0) s[i >> 2] = (uint8_t)code;
}

// ---- the grouped FP4 GEMM --------------------------------------------------

enum { kMxGateUp = 0, kMxGateUpQ = 1, kMxDownY = 2 };

__device__ inline v4f mfma_16x16x128_mxfp4(v8i a, v8i b, v4f c, int scale_a, int scale_b) {
  // cbsz = blgp = 4: both operands E2M1 (only the first 4 dwords of each are
  // read); op_sel 0: byte 0 of each lane's scale register is its block's E8M0.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, 0, scale_a, 0, scale_b);
}

__device__ inline void buffer_load4_lds(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 4, voff, 0, 0, 0);
}

template <int BM, int BN, int WGM, int WGN, int MODE, int NS>
struct MxTile {
  static constexpr int kThreads = 64 * WGM * WGN;
  static constexpr int WM = BM / WGM, WN = BN / WGN;   // per-wave tile
  static constexpr int SM = WM / 16, SN = WN / 16;     // 16x16 MFMA tiles per wave
  static constexpr int kRows = BM + BN;
  static constexpr int kCodes = kRows * 128;           // 256 K elements per row and stage
  static constexpr int kStage = kCodes + kRows * 8;    // + the rows' 8 E8M0 bytes
  static constexpr int kRowsPerPass = kThreads / 8;
  static constexpr int kLoadsB = BN / kRowsPerPass, kLoadsA = BM / kRowsPerPass;
  static constexpr int kScaleDw = kRows * 2;           // scale dwords per stage
  static constexpr int kScaleLoads = (kScaleDw + kThreads - 1) / kThreads;
  static constexpr int kEpiStride = BN * 2 + 16;       // BF16 staging row (GATE_UP)
  static constexpr int kEpi = MODE == kMxGateUp ? BM * kEpiStride : 0;
  static constexpr int kLds = (NS * kStage > kEpi) ? NS * kStage : kEpi;
  // The down epilogue stages a wave row block's rows in JH parts, each no
  // larger than the K loop's stages.
  static constexpr int kJH = (MODE == kMxDownY && WM * BN * 4 > kLds) ? 2 : 1;
  static_assert(NS == 1 || NS == 2, "one or two stages");
  static_assert(BN % kRowsPerPass == 0 && BM % kRowsPerPass == 0, "stage must split evenly over the threads");
  static_assert(kRowsPerPass % 8 == 0, "the loader's chunk swizzle needs 8-row passes");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(BN % 32 == 0 && kScaleDw % 64 == 0, "a wave's scale rows must be all weight or all input rows");
  static_assert(MODE != kMxGateUpQ || (WN % 64 == 0 && BN % 64 == 0),
                "a wave's gate/up blocks must make whole 32-column h blocks");
};

struct MxArgs {
  const uint8_t* A;         // GATE_UP*: token codes [a_rows, K/2]; DOWN_Y: sorted h codes
  const uint8_t* sA;        // their E8M0 scales [a_rows, K/32]
  int64_t a_rows;
  const int32_t* perm;      // sorted row -> slot
  const int32_t* offsets;   // [G + 1] group starts (device)
  int G, Eids, topk;
  const uint8_t* B;         // [E, N, K/2] weight codes
  const uint8_t* sB;        // [E, N, K/32] weight scales
  const float* tw;          // DOWN_Y: router weights [slots]
  uint16_t* out_bf16;       // GATE_UP: [rows, N]
  float* out_f32;           // DOWN_Y: y [slots, N]
  int32_t* slot_row;        // DOWN_Y: NULL, y row = slot; else y row = sorted row, and slot_row[slot] = it
  uint8_t* out_q;           // GATE_UP_Q: h codes [rows, N/4]
  uint8_t* out_s;           // GATE_UP_Q: h scales [rows, N/64]
  const int32_t* dst_row;   // GATE_UP_Q: slot -> output row (NULL: the sorted row)
  int N, K, tiles_n, tiles_m_max;
};

template <int BM, int BN, int WGM, int WGN, int MODE, int OCC, int NS>
__global__ __launch_bounds__(64 * WGM * WGN) __attribute__((amdgpu_waves_per_eu(1, OCC)))
void mx_grouped(const MxArgs p) {
  using C = MxTile<BM, BN, WGM, WGN, MODE, NS>;
  // One LDS object: the stages (or the epilogue's staging), then the row
  // tables. With a single object the compiler does not make the LDS reads
  // of a K step wait for the next step's direct-to-LDS loads.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kLds + BM * 12];
  int* const row_tok = reinterpret_cast<int*>(smem + C::kLds);             // token (gate/up) or slot (down), -1 = empty
  float* const row_w = reinterpret_cast<float*>(smem + C::kLds + BM * 4);  // DOWN_Y: router weight of the row's slot
  int* const row_dst = reinterpret_cast<int*>(smem + C::kLds + BM * 8);    // GATE_UP_Q: output row (-1 = none)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = p.N, Kb = p.K >> 1, Ks = p.K >> 5;
  const int total = p.tiles_m_max * p.tiles_n;
  const int per = total >> 3;
  int t = blockIdx.x;
  if ((int)blockIdx.x < (per << 3)) t = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  const int mt = t / p.tiles_n, nt = t - mt * p.tiles_n;
  constexpr bool kIsDown = MODE == kMxDownY;
  const int cap = (int)(kIsDown ? p.a_rows : p.a_rows * p.topk);
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
      float w = 0.f;
      if (i < rows) {
        const int slot = p.perm[row0 + i];
        if (slot >= 0 && slot < cap) {
          tok = kIsDown ? slot : slot / p.topk;
          if (kIsDown) w = p.tw[slot];
          if (MODE == kMxGateUpQ) {
            dst = p.dst_row ? p.dst_row[slot] : row0 + i;
            if (dst >= cap) dst = -1;
          }
        }
      }
      row_tok[i] = tok;
      row_w[i] = w;
      row_dst[i] = dst;
    }
  };
  if (!kIsDown) {
    setup_rows();
    __syncthreads();
  }

  const int64_t eN = (int64_t)e * N;
  const bool whole_b = MODE == kMxGateUpQ;  // interleaved gate/up rows address the expert's whole W13
  const auto rB = whole_b ? make_rsrc(p.B + eN * Kb, (int64_t)N * Kb)
                          : make_rsrc(p.B + (eN + n0) * Kb, (int64_t)(N - n0) * Kb);
  const auto rsB = whole_b ? make_rsrc(p.sB + eN * Ks, (int64_t)N * Ks)
                           : make_rsrc(p.sB + (eN + n0) * Ks, (int64_t)(N - n0) * Ks);
  const auto rA = kIsDown ? make_rsrc(p.A + (int64_t)row0 * Kb, (int64_t)rows * Kb) : make_rsrc(p.A, p.a_rows * Kb);
  const auto rsA = kIsDown ? make_rsrc(p.sA + (int64_t)row0 * Ks, (int64_t)rows * Ks)
                           : make_rsrc(p.sA, p.a_rows * Ks);
  // Weight row of stage row r (r < BN), relative to the resource base.
  auto weight_row = [&](int r) {
    if (MODE == kMxGateUpQ) {  // 16-row block b: even = gate rows, odd = the matching up rows
      const int b = r >> 4;
      return (b & 1 ? N / 2 : 0) + (n0 >> 1) + (b >> 1) * 16 + (r & 15);
    }
    return r;
  };
  // Input row of stage row BN + lr, or -1 (zero fill).
  auto input_row = [&](int lr) { return kIsDown ? (lr < rows ? lr : -1) : row_tok[lr]; };

  // Codes: LDS slot tid + kThreads * i holds stage row (tid >> 3) +
  // kRowsPerPass * i, logical chunk (tid & 7) ^ (row & 7), as in the FP8
  // kernel. Stage rows 0..BN-1 hold B, rows BN.. hold A.
  const int lchunk = ((tid & 7) ^ ((tid >> 3) & 7)) << 4;
  const int lrow = tid >> 3;
  uint32_t boff[C::kLoadsB], aoff[C::kLoadsA], soff[C::kScaleLoads];
#pragma unroll
  for (int i = 0; i < C::kLoadsB; ++i)
    boff[i] = (uint32_t)weight_row(lrow + C::kRowsPerPass * i) * (uint32_t)Kb + (uint32_t)lchunk;
#pragma unroll
  for (int j = 0; j < C::kLoadsA; ++j) {
    const int r = input_row(lrow + C::kRowsPerPass * j);
    aoff[j] = r < 0 ? kOutOfRange : (uint32_t)r * (uint32_t)Kb + (uint32_t)lchunk;
  }
  // Scales: dword d = i * kThreads + tid of the stage's scale area is half
  // (d & 1) of stage row d >> 1's 8 bytes.
#pragma unroll
  for (int i = 0; i < C::kScaleLoads; ++i) {
    const int d = i * C::kThreads + tid, row = d >> 1, half = d & 1;
    soff[i] = kOutOfRange;
    if (row < BN) {
      soff[i] = (uint32_t)weight_row(row) * (uint32_t)Ks + 4u * half;
    } else if (row < C::kRows) {
      const int r = input_row(row - BN);
      if (r >= 0) soff[i] = (uint32_t)r * (uint32_t)Ks + 4u * half;
    }
  }
  auto issue = [&](int stage, int kt) {
    uint8_t* base = smem + stage * C::kStage;
    const uint32_t kb0 = (uint32_t)kt << 7;
    const bool kin = kb0 + lchunk < (uint32_t)Kb;
#pragma unroll
    for (int i = 0; i < C::kLoadsB + C::kLoadsA; ++i) {
      const int s0 = wave * 64 + C::kThreads * i;
      if (i < C::kLoadsB) {
        buffer_load16_lds(rB, base + s0 * 16, kin ? boff[i] + kb0 : kOutOfRange);
      } else {
        const uint32_t a = aoff[i - C::kLoadsB];
        buffer_load16_lds(rA, base + s0 * 16, (kin && a != kOutOfRange) ? a + kb0 : kOutOfRange);
      }
    }
    const uint32_t ks0 = (uint32_t)kt << 3;
#pragma unroll
    for (int i = 0; i < C::kScaleLoads; ++i) {
      const int d0 = i * C::kThreads + wave * 64;  // wave-uniform
      if (d0 < C::kScaleDw) {
        const bool sin = ks0 + 4u * (tid & 1) < (uint32_t)Ks && soff[i] != kOutOfRange;
        buffer_load4_lds((d0 >> 1) < BN ? rsB : rsA, base + C::kCodes + d0 * 4, sin ? soff[i] + ks0 : kOutOfRange);
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
  const int nk = (Kb + 127) >> 7;
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
    if (NS == 2 && kt + 1 < nk) issue((kt + 1) & 1, kt + 1);
    const uint8_t* st = smem + (NS == 2 ? (kt & 1) * C::kStage : 0);
    const uint8_t* ss = st + C::kCodes;
    // Pass s of the stage takes chunk g + 4s of each row (elements
    // 128s + 32g .. +31, the row's block 8kt + 4s + g) and the row's scale
    // byte of that block: byte g of scale dword s. The operands of one pass
    // at a time keep the register count down; consecutive MFMAs on one
    // accumulator are SN * SM instructions apart.
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v8i xa[C::SM];
      int sx[C::SM];
#pragma unroll
      for (int j = 0; j < C::SM; ++j) {
        // rows 16 apart share (row & 7), so one swizzled base serves them all
        const int row0x = BN + wm * C::WM + r16;
        const v4i c = *reinterpret_cast<const v4i*>(st + stage_off(row0x, g + 4 * s) + j * 16 * 128);
        xa[j] = v8i{c.x, c.y, c.z, c.w, c.x, c.y, c.z, c.w};
        sx[j] = (int)(*reinterpret_cast<const uint32_t*>(ss + row0x * 8 + 4 * s + j * 16 * 8) >> (8 * g));
      }
      if (NS == 1 && s == 1) {
        // one stage: the last pass's operands in registers, then the next
        // step's loads, which overlap this pass's MFMAs
        v4i wc[C::SN];
        int sw[C::SN];
#pragma unroll
        for (int i = 0; i < C::SN; ++i) {
          const int row0w = wn * C::WN + r16;
          wc[i] = *reinterpret_cast<const v4i*>(st + stage_off(row0w, g + 4 * s) + i * 16 * 128);
          sw[i] = (int)(*reinterpret_cast<const uint32_t*>(ss + row0w * 8 + 4 * s + i * 16 * 8) >> (8 * g));
        }
        lds_barrier();
        // unconditional, so that the loop body stays one block and the first
        // pass's MFMAs stay ahead of this pass's reads; past the last step
        // every load is out of range and only zero-fills the stage
        issue(0, kt + 1);
#pragma unroll
        for (int i = 0; i < C::SN; ++i) {
          const v8i wb = v8i{wc[i].x, wc[i].y, wc[i].z, wc[i].w, wc[i].x, wc[i].y, wc[i].z, wc[i].w};
#pragma unroll
          for (int j = 0; j < C::SM; ++j) acc[i][j] = mfma_16x16x128_mxfp4(wb, xa[j], acc[i][j], sw[i], sx[j]);
        }
        continue;
      }
#pragma unroll
      for (int i = 0; i < C::SN; ++i) {
        const int row0w = wn * C::WN + r16;
        const v4i c = *reinterpret_cast<const v4i*>(st + stage_off(row0w, g + 4 * s) + i * 16 * 128);
        const v8i wb = v8i{c.x, c.y, c.z, c.w, c.x, c.y, c.z, c.w};
        const int sw = (int)(*reinterpret_cast<const uint32_t*>(ss + row0w * 8 + 4 * s + i * 16 * 8) >> (8 * g));
#pragma unroll
        for (int j = 0; j < C::SM; ++j) acc[i][j] = mfma_16x16x128_mxfp4(wb, xa[j], acc[i][j], sw, sx[j]);
      }
      if (NS == 1) {
        // pin the first pass's MFMAs here: otherwise they are sunk below the
        // next step's loads, and both passes' operands are live together
#pragma unroll
        for (int i = 0; i < C::SN; ++i)
#pragma unroll
          for (int j = 0; j < C::SM; ++j) asm volatile("" ::"a"(acc[i][j]));
      }
    }
  }

  if (NS == 1) {
    // the last step's zero-fill loads land before the epilogue reuses the LDS
    wait_vmem_all();
    __syncthreads();
  }
  // acc[i][j][r]: tile row wm * WM + 16 j + lane % 16, stage (weight) row
  // wn * WN + 16 i + 4 (lane / 16) + r.
  if constexpr (MODE == kMxDownY) {
    // y = w * acc in float32, staged through LDS one wm's rows (or half of
    // them) at a time and
    // written as whole row pieces (BN * 4 contiguous bytes of each of
    // 256 / BN rows per store instruction), as in the FP8 down projection:
    // straight from the MFMA registers an instruction covers 16 rows x 64
    // bytes, which drains markedly slower. 16-byte chunks XOR-swizzled by row.
    constexpr int kChunks = BN / 4;
    constexpr int kRowsPerInst = 64 / kChunks;
    constexpr int kJH = C::kJH, kPartRows = C::WM / kJH, kPartJ = C::SM / kJH;
    static_assert(kPartRows * BN * 4 <= C::kLds && C::SM % kJH == 0, "a part of a wm's rows must fit in the LDS");
    static_assert(kChunks >= 16 && 64 % kChunks == 0, "row pieces must tile a wave");
#pragma unroll
    for (int pass = 0; pass < WGM * kJH; ++pass) {
      const int pw = pass / kJH, ph = pass % kJH;
      __syncthreads();  // the K-loop stages (pass 0) or the previous pass's rows are read
      if (wm == pw) {
#pragma unroll
        for (int jl = 0; jl < kPartJ; ++jl) {
          const int j = ph * kPartJ + jl;
          const int rl = jl * 16 + r16;
          const float w = row_w[wm * C::WM + j * 16 + r16];
#pragma unroll
          for (int i = 0; i < C::SN; ++i) {
            const int chunk = wn * (C::WN / 4) + i * 4 + g;
            const v4f a = acc[i][j];
            *reinterpret_cast<float4*>(smem + rl * (BN * 4) + ((chunk ^ (rl & 15)) << 4)) =
                make_float4(a[0] * w, a[1] * w, a[2] * w, a[3] * w);
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
  if (MODE == kMxGateUpQ) {
    // Tiles 4q .. 4q+3 of the wave are (gate, up) of h columns hc .. hc+15
    // and (gate, up) of hc+16 .. hc+31 with hc = n0/2 + wn*WN/2 + 32q: one
    // MX block per row. Lane group g holds columns 4g..4g+3 of each half.
    const int hrow_bytes = N >> 2, hrow_scales = N >> 6;
#pragma unroll
    for (int j = 0; j < C::SM; ++j) {
      const int dst = row_dst[wm * C::WM + j * 16 + r16];
#pragma unroll
      for (int q = 0; q < C::SN / 4; ++q) {
        float h[8];
        float amax = 0.f;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const v4f ga = acc[4 * q + 2 * half][j], ua = acc[4 * q + 2 * half + 1][j];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gv = ga[r], uv = ua[r];
            const float hv = silu_f32(gv) * uv;
            h[4 * half + r] = hv;
            amax = fmaxf(amax, fabsf(hv));
          }
        }
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const uint32_t code = mx_scale_code(__float_as_uint(amax));
        const float m = mx_inv_scale(code);
        // this lane's 4 columns of each half: 16 code bits per half
        const uint32_t mine = e2m1_pack<4>(h, m) | (e2m1_pack<4>(h + 4, m) << 16);
        // lane group g stores block columns 8g .. 8g+7: half g >> 1, from
        // lane groups 2 (g & 1) and 2 (g & 1) + 1
        const int src = r16 + 32 * (g & 1);
        const uint32_t a = (uint32_t)__shfl((int)mine, src, 64), b = (uint32_t)__shfl((int)mine, src + 16, 64);
        const uint32_t word = g < 2 ? ((a & 0xFFFFu) | (b << 16)) : ((a >> 16) | (b & 0xFFFF0000u));
        if (dst >= 0) {
          const int hc = (n0 >> 1) + wn * (C::WN / 2) + 32 * q;
          *reinterpret_cast<uint32_t*>(p.out_q + (int64_t)dst * hrow_bytes + (hc >> 1) + 4 * g) = word;
          if (g == 0) p.out_s[(int64_t)dst * hrow_scales + (hc >> 5)] = (uint8_t)code;
        }
      }
    }
    return;
  }
  // GATE_UP: round to BF16, stage in LDS, store full row segments
  __syncthreads();
#pragma unroll
  for (int i = 0; i < C::SN; ++i) {
    const int nl = wn * C::WN + i * 16 + 4 * g;
#pragma unroll
    for (int j = 0; j < C::SM; ++j) {
      const int ml = wm * C::WM + j * 16 + r16;
      const v4f a = acc[i][j];
      const uint32_t p0 = bf16x2_rne(a[0], a[1]);
      const uint32_t p1 = bf16x2_rne(a[2], a[3]);
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

// out[t, c] = bf16( sum_j y[t * topk + j, c] ) over the token's valid slots,
// in the order j = 0, 1, ...; with QUANT also the MXFP4 codes and scales of
// the BF16 row (exactly what mx_quant_bf16 makes of it). One thread per 8
// columns: two runs of 4 (split_cols8) if SPLIT, so that every load
// instruction reads 1 KB contiguous. Otherwise 8 consecutive columns, and
// with H % 32 == 0 a block's four threads form an aligned quad. With SPLIT
// and QUANT H % 64 == 0: both halves of every 512-column block (or of the
// row's shorter last block) are whole 32-column blocks, each held by an
// aligned group of 8 threads, 4 columns each.
template <bool QUANT, bool SPLIT>
__global__ __launch_bounds__(256) void combine_mx(const float* __restrict__ y, const int32_t* __restrict__ ids,
                                                  const int32_t* __restrict__ slot_row, int64_t T, int topk, int Eids,
                                                  int H, uint16_t* __restrict__ out,
                                                  uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = H >> 3;
  const int64_t t = i / per_row;
  if (t >= T) return;
  float4 a, b;
  if constexpr (SPLIT) {
    int ca, cb;
    split_cols8((int)(i - t * per_row), H, ca, cb);
    sum_slots_split(y, ids, slot_row, t, topk, Eids, H, ca, cb, a, b);
    const uint4 v = to_bf16x8(a, b);
    *reinterpret_cast<uint2*>(out + t * H + ca) = make_uint2(v.x, v.y);
    *reinterpret_cast<uint2*>(out + t * H + cb) = make_uint2(v.z, v.w);
    if constexpr (QUANT) {
      uint32_t code_a, code_b;
      const uint32_t qa = mx_oct_quant(v.x, v.y, &code_a);
      const uint32_t qb = mx_oct_quant(v.z, v.w, &code_b);
      uint8_t* qrow = q + t * (H / 2);
      *reinterpret_cast<uint16_t*>(qrow + ca / 2) = (uint16_t)qa;
      *reinterpret_cast<uint16_t*>(qrow + cb / 2) = (uint16_t)qb;
      if ((i & 7) == 0) {
        s[t * (H / 32) + ca / 32] = (uint8_t)code_a;
        s[t * (H / 32) + cb / 32] = (uint8_t)code_b;
      }
    }
  } else {
    // 8 consecutive columns per thread: a quad of threads holds one block
    const int c0 = (int)(i - t * per_row) << 3;
    sum_slots8(y, ids, slot_row, t, topk, Eids, H, c0, a, b);
    const uint4 v = to_bf16x8(a, b);
    *reinterpret_cast<uint4*>(out + t * H + c0) = v;
    if constexpr (QUANT) {
      uint32_t code;
      reinterpret_cast<uint32_t*>(q)[i] = mx_quad_quant(v, &code);
      if ((i & 3) == 0) s[i >> 2] = (uint8_t)code;
    }
  }
}

// Tile shapes: 256 x 256 tiles of 8 waves from 1024 rows per group on
// average; 128 x 128 tiles of 2 x 2 waves from 448 to 1023 rows; 64 x 128
// tiles of 1 x 2 waves below 448. Both small shapes take one LDS stage at three
// waves per SIMD: the 64 x 128 tiles need 26 KB instead of 52 KB and 78-82
// VGPRs, so six workgroups fit on a CU instead of three (16-19% less time
// for a whole two-pass FFN at 128 and 192 experts); the 128 x 128 tiles 36 KB
// instead of 70 KB and 75-80 VGPRs, three workgroups instead of two. With
// both in one stage the 64 x 128 tiles were 2-5% faster than the 128 x 128
// ones up to 384 rows per group (the FP8 tiles cross over near 256 rows and
// keep their threshold), and the 128 x 128 tiles beat the 256 x 256 ones at
// 512 and 768 rows (5% and 1.4%). The same results bit for bit.
constexpr int64_t kMxSmallGroupRows = 1024, kMxTinyGroupRows = 448;

template <int BM, int BN, int WGM, int WGN, int MODE, int OCC, int NS = 2>
hipError_t run_mx(MxArgs a, int64_t max_rows, hipStream_t stream) {
  a.tiles_n = (a.N + BN - 1) / BN;
  a.tiles_m_max = (int)((max_rows + BM - 1) / BM + a.G);  // every group adds at most one partial tile
  const int64_t blocks = (int64_t)a.tiles_m_max * a.tiles_n;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((mx_grouped<BM, BN, WGM, WGN, MODE, OCC, NS>), dim3((unsigned)blocks), dim3(64 * WGM * WGN), 0,
                     stream, a);
  return hipGetLastError();
}

template <int MODE>
hipError_t run_mx_auto(const MxArgs& a, int64_t max_rows, int64_t avg_rows, hipStream_t stream) {
  if (avg_rows < kMxTinyGroupRows) return run_mx<64, 128, 1, 2, MODE, 3, 1>(a, max_rows, stream);
  if (avg_rows < kMxSmallGroupRows) return run_mx<128, 128, 2, 2, MODE, 3, 1>(a, max_rows, stream);
  return run_mx<256, 256, 2, 4, MODE, 2>(a, max_rows, stream);
}

MxArgs mx_gate_up_args(const uint8_t* xq, const uint8_t* xs, const int32_t* perm, const int32_t* offsets, int G,
                       const uint8_t* w13, const uint8_t* s13, int64_t T, int64_t H, int64_t I, int64_t E,
                       int64_t topk) {
  MxArgs a{};
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

hipError_t launch_mx_quantize(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, uint8_t* s, hipStream_t stream) {
  const int64_t chunks = M * K / 8;
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_quant_bf16, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream, x, chunks, q, s);
  return hipGetLastError();
}

hipError_t launch_mx_gate_up_bf16(const uint8_t* xq, const uint8_t* xs, const int32_t* perm, const int32_t* offsets,
                                  const uint8_t* w13, const uint8_t* s13, uint16_t* gu, int64_t T, int64_t H,
                                  int64_t I, int64_t E, int64_t topk, int order, hipStream_t stream) {
  MxArgs a = mx_gate_up_args(xq, xs, perm, offsets, (int)route_groups(topk, E, order), w13, s13, T, H, I, E, topk);
  a.out_bf16 = gu;
  return run_mx_auto<kMxGateUp>(a, T * topk, T * topk / a.G, stream);
}

hipError_t launch_mx_gate_up_swiglu_quant(const uint8_t* xq, const uint8_t* xs, const int32_t* perm,
                                          const int32_t* offsets, const int32_t* dst_row, const uint8_t* w13,
                                          const uint8_t* s13, uint8_t* qh, uint8_t* sh, int64_t T, int64_t H,
                                          int64_t I, int64_t E, int64_t topk, int order, hipStream_t stream) {
  MxArgs a = mx_gate_up_args(xq, xs, perm, offsets, (int)route_groups(topk, E, order), w13, s13, T, H, I, E, topk);
  a.out_q = qh;
  a.out_s = sh;
  a.dst_row = dst_row;
  return run_mx_auto<kMxGateUpQ>(a, T * topk, T * topk / a.G, stream);
}

hipError_t launch_mx_down_combine(const uint8_t* qh, const uint8_t* sh, const int32_t* perm, const int32_t* offsets,
                                  const int32_t* ids, const float* tw, const uint8_t* w2, const uint8_t* s2,
                                  uint16_t* out, float* y, uint8_t* out_q, uint8_t* out_s, int64_t T, int64_t H,
                                  int64_t I, int64_t E, int64_t topk, int order, hipStream_t stream,
                                  int32_t* slot_row) {
  MxArgs a{};
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
  const hipError_t err = run_mx_auto<kMxDownY>(a, T * topk, T * topk / a.G, stream);
  if (err != hipSuccess) return err;
  const int64_t threads = T * (H / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (out_q != nullptr && H % 64 == 0)
    hipLaunchKernelGGL((combine_mx<true, true>), grid, dim3(256), 0, stream, y, ids, slot_row, T, (int)topk, (int)E,
                       (int)H, out, out_q, out_s);
  else if (out_q != nullptr)
    hipLaunchKernelGGL((combine_mx<true, false>), grid, dim3(256), 0, stream, y, ids, slot_row, T, (int)topk, (int)E,
                       (int)H, out, out_q, out_s);
  else
    hipLaunchKernelGGL((combine_mx<false, true>), grid, dim3(256), 0, stream, y, ids, slot_row, T, (int)topk, (int)E,
                       (int)H, out, nullptr, nullptr);
  return hipGetLastError();
}

// Workspace of the full pass: counts | offsets | perm | route scratch |
// h codes [T*k, I/2] | h scales [T*k, I/32] | slot -> row [T*k] |
// y [T*k, H] float32 (in sorted order).
struct MxLayout {
  int64_t counts, offsets, perm, route, qh, sh, slot_row, y, total;
};

static MxLayout mx_layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk) {
  MxLayout L;
  int64_t o = 0;
  const int64_t n = T * topk;
  auto al = [](int64_t b) { return (b + 255) & ~int64_t(255); };
  L.counts = o; o += al(E * 4);
  L.offsets = o; o += al((E + 1) * 4);
  L.perm = o; o += al(n * 4);
  L.route = o; o += (int64_t)route_workspace_bytes(T, topk, E);
  L.qh = o; o += al(n * I / 2);
  L.sh = o; o += al(n * I / 32);
  L.slot_row = o; o += al(n * 4);
  L.y = o; o += al(n * H * 4);
  L.total = o;
  return L;
}

size_t mx_moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk) {
  return (size_t)mx_layout(T, H, I, E, topk).total;
}

hipError_t launch_mx_moe(const uint8_t* xq, const uint8_t* xs, const int32_t* ids, const float* tw,
                         const uint8_t* w13, const uint8_t* s13, const uint8_t* w2, const uint8_t* s2, uint16_t* out,
                         uint8_t* out_q, uint8_t* out_s, int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                         void* ws, hipStream_t stream) {
  const MxLayout L = mx_layout(T, H, I, E, topk);
  uint8_t* b = static_cast<uint8_t*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(b + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  int32_t* perm = reinterpret_cast<int32_t*>(b + L.perm);
  hipError_t err = launch_route(ids, T, topk, E, 0, counts, offsets, perm, nullptr, b + L.route, stream);
  if (err != hipSuccess) return err;
  err = launch_mx_gate_up_swiglu_quant(xq, xs, perm, offsets, nullptr, w13, s13, b + L.qh, b + L.sh, T, H, I, E, topk,
                                       0, stream);
  if (err != hipSuccess) return err;
  return launch_mx_down_combine(b + L.qh, b + L.sh, perm, offsets, ids, tw, w2, s2, out,
                                reinterpret_cast<float*>(b + L.y), out_q, out_s, T, H, I, E, topk, 0, stream,
                                reinterpret_cast<int32_t*>(b + L.slot_row));
}

}  // namespace w8a8
