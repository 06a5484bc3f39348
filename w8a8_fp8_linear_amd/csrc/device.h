// Device-side helpers shared by the gfx950 kernels of this library.
//
// Formats: activations and outputs are BF16 (the model's dtype; Lernex/
// Metis-1.6-Logos-FP8, "What --fast-math does"), FP8 is OCP E4M3FN (the
// F8_E4M3 tensor type of the checkpoints; Lernex/Metis-1.6-Praxis-NVFP4, hub
// sidebar), scales are float32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource word 3 for raw (untyped) buffers on gfx9-class parts.
constexpr int kBufferFlags = 0x00020000;
// Any voffset at or above this is outside every resource built by make_rsrc,
// so the hardware returns zeros for the load.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Raw buffer resource over [base, base + bytes); bytes is clamped so that
// kOutOfRange always lies outside it.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  if (bytes > 0x7FFFFFF0ll) bytes = 0x7FFFFFF0ll;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}

__device__ inline v4i buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}

// 16 bytes per lane from a buffer straight into LDS: lane i of the wave
// writes lds_base + 16 * i (lds_base must be wave-uniform).
__device__ inline void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, 0, 0, 0);
}

// FP8 x FP8 -> FP32 matrix-core step, 16x16 outputs, 128-deep. cbsz/blgp 0
// select E4M3 for both operands; zero scale operands select the unscaled
// instruction.
__device__ inline v4f mfma_16x16x128_e4m3(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Two float32 -> two BF16 bit patterns (a in the low half), round to nearest
// even, with the gfx950 packed conversion (v_cvt_pk_bf16_f32): one
// instruction per pair. On the GPU it was compared with the integer rule
// (u + 0x7FFF + ((u >> 16) & 1)) >> 16 on every non-NaN float32 bit pattern:
// 0 mismatches; NaN stays NaN.
__device__ inline uint32_t bf16x2_rne(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// silu(g) = g / (1 + e^-g) in float32 with the hardware exponential and
// reciprocal (each within about 1 ulp): a few instructions instead of a
// correctly rounded division. The result stays within a few float32 ulps of
// the exact value (e^-g overflowing to infinity gives -0).
__device__ inline float silu_f32(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Four float32 values in [-448, 448] -> four E4M3FN codes (value 0 in byte 0)
// with the hardware conversion: round to nearest, ties to even, the sign kept
// on a zero result. On gfx950 this was compared with an integer encoder
// written from the format's bit fields for every float32 bit pattern of
// magnitude <= 448, both signs (0 mismatches); the quantiser's bit-exact
// parity tests against the oracle cover it on every BF16 (amax, x) pair over
// 21 binades.
__device__ inline uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ inline float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// True when the E4M3 code of a float32 within 2 ulp of v may differ from
// that of v: v lies within 3 ulp of a round-to-nearest boundary of the
// normal E4M3 range (the 20 bits below the kept mantissa are near one half),
// or 0 < |v| < 2^-6 (the subnormal range, whose boundaries sit elsewhere).
__device__ inline bool e4m3_boundary_near(float v) {
  const uint32_t a = __float_as_uint(v) & 0x7FFFFFFFu;
  return (a - 1u < 0x3C7FFFFFu) | (((a & 0xFFFFFu) - 0x7FFFDu) < 7u);
}

// ---- the per-row quantiser: shared by quantize_per_token and the fused
// quantisation of the routed-expert output

__device__ inline uint32_t absmax8(uint4 v) {
  uint32_t m = 0;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
    m = m > lo ? m : lo;
    m = m > hi ? m : hi;
  }
  return m;
}

// Smallest row scale for which quant8 takes the quotient without dividing.
constexpr float kQuotientMinScale = 0x1p-99f;

// 8 BF16 values -> 8 E4M3 codes of fl32(x / s) (little-endian, element 0 in
// byte 0), for a row scale s = fl32(amax / 448) of a BF16 row maximum (or 1)
// and r = fl32(1 / s), both correctly rounded divisions.
//
// The quotient comes from one residual correction of x * r (Markstein's
// method, with fused multiply-adds): q0 = fl32(x * r), q = fl32(q0 +
// fl32(x - q0 * s) * r), with the sign of x put back on a zero result. For
// s >= 2^-99, every BF16 x with |x| <= amax and both signs, this q equals
// fl32(x / s) bit for bit wherever |x / s| >= 2^-12, and elsewhere has
// magnitude below 2^-11 and the sign of x, so the E4M3 code is the same
// (an exhaustive check over all 1.07e9 (amax, x) pairs runs with the CPU
// tests). Below 2^-99 the residual can underflow and the row divides; s is
// one value per row, so the branch does not split a wave working on one row.
__device__ inline uint2 quant8(uint4 v, float s, float r) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float x[8], q[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
  if (__builtin_expect(s >= kQuotientMinScale, 1)) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float q0 = x[k] * r;
      q[k] = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, s, x[k]), r, q0), x[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k] = x[k] / s;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) q[k] = clamp448(q[k]);
  return make_uint2(e4m3x4(q[0], q[1], q[2], q[3]), e4m3x4(q[4], q[5], q[6], q[7]));
}

__device__ inline float row_scale(uint32_t amax_bits) {
  if (amax_bits == 0) return 1.0f;
  return __uint_as_float(amax_bits << 16) / 448.0f;
}

__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

// 16-byte stores of large write-once outputs (the GEMM's Y, the routed
// copies' y rows, the float32 h rows) with the non-temporal hint: they are
// streamed out rather than kept in the L2 of the writing XCD. Measured 6-11%
// faster for the down projection, about 1% for the prefill GEMM.
__device__ inline void store16_nt(void* p, uint4 v) {
  __builtin_nontemporal_store(v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, reinterpret_cast<v4i*>(p));
}
__device__ inline void store16_nt(void* p, float4 v) {
  __builtin_nontemporal_store(v4f{v.x, v.y, v.z, v.w}, reinterpret_cast<v4f*>(p));
}

__device__ inline void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// At most N vector memory operations of this wave outstanding (vmcnt(N));
// the other counters are not waited for.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  constexpr int kImm = (N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14);
  __builtin_amdgcn_s_waitcnt(kImm);
}

// A workgroup barrier that orders LDS only: this wave's LDS accesses are
// complete, then all waves meet. Unlike __syncthreads() it does not wait for
// the wave's outstanding global loads and stores (on this GPU one counter
// covers both), so stores can drain while the workgroup moves on. The empty
// asm keeps the compiler from moving memory accesses across, the scheduling
// barriers keep other instructions on their side.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Round-robin dispatch puts workgroup b on XCD b % 8. Renumber so that
// each XCD gets a contiguous run of tile ids, then walk tile ids in groups
// of G tile rows so that concurrently running tiles share A and W panels.
template <int G>
__device__ inline void map_tile(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int per = total >> 3;
  int t = bid;
  if (bid < (per << 3)) t = (bid & 7) * per + (bid >> 3);
  const int span = G * tiles_n;
  const int group = t / span;
  const int first_m = group * G;
  const int gsize = min(tiles_m - first_m, G);
  const int within = t - group * span;
  tm = first_m + within % gsize;
  tn = within / gsize;
}

// Byte offset of logical 16-byte chunk c of a staged 128-byte row. A
// ds_read_b128 is served 8 lanes at a time over 128 bytes of banks; the 8
// lanes of a group read 8 consecutive rows at the same logical chunk, and
// the XOR with (row & 7) puts them on 8 different 16-byte bank groups.
__device__ inline int stage_off(int row, int c) { return row * 128 + ((c ^ (row & 7)) << 4); }

// One MFMA operand fragment from a staged K slice: chunks c and c + 4 of
// row `row`.
__device__ inline v8i lds_frag(const uint8_t* st, int row, int c) {
  const v4i lo = *reinterpret_cast<const v4i*>(st + stage_off(row, c));
  const v4i hi = *reinterpret_cast<const v4i*>(st + stage_off(row, c + 4));
  return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

}  // namespace w8a8
