// Internal launchers behind the C ABI (include/w8a8.h). Arguments are
// validated by the ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w8a8 {

// Per-row quantiser: x bf16 [M,K] -> q e4m3 [M,K], scale f32 [M].
hipError_t launch_quantize_rows(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* scale,
                                hipStream_t stream);

// The final conversions of the quantisers and of every BF16 result, on
// caller-given float32 values: E4M3 of clamp(v, -448, 448), and BF16 RNE.
hipError_t launch_convert_e4m3(const float* v, int64_t n, uint8_t* q, hipStream_t stream);
hipError_t launch_convert_bf16(const float* v, int64_t n, uint16_t* y, hipStream_t stream);

// Dense scaled FP8 GEMM: y[m,n] = bf16(sa[m] * sw[n] * sum_k a[m,k] w[n,k]).
// start / stop: optional events stamped with the kernel's own start and end
hipError_t launch_gemm(const uint8_t* a, const float* sa, const uint8_t* w, const float* sw,
                       uint16_t* y, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                       hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

// Per-token quantisation fused into the decode GEMM (one launch), for
// M <= kFusedDecodeMaxM and K <= kFusedDecodeMaxK; bit-identical to
// launch_quantize_rows followed by launch_gemm.
constexpr int64_t kFusedDecodeMaxM = 32, kFusedDecodeMaxK = 2048;
hipError_t launch_quant_gemm_decode(const uint16_t* x, const uint8_t* w, const float* sw, uint16_t* y, int64_t M,
                                    int64_t N, int64_t K, hipStream_t stream);

// The read floor of the decode weight stream (gemm.hip): every byte of p read
// in gemm_skinny's launch shape, kProbeBytesPerBlock bytes per 256-thread
// workgroup; sink gets one XOR word per workgroup.
constexpr int64_t kProbeBytesPerBlock = 32768;
hipError_t launch_read_probe(const uint8_t* p, int64_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_clock_probe(uint64_t* out, int64_t n, hipStream_t stream);

// Default maths (w8a16.hip): y[m,n] = bf16(sw[n] * sum_k x[m,k] w[n,k]), x BF16,
// w E4M3 widened to BF16, BF16 MFMA.
hipError_t launch_w8a16_gemm(const uint16_t* x, const uint8_t* w, const float* sw, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream);

// Routed-expert pipeline (moe.hip). offsets/perm are device arrays made by
// launch_route; the grouped kernels derive their tiles from them on device.
// order 0: groups are experts (E groups); order 1: groups are (top-k
// position j, expert) pairs, key j * E + e (topk * E groups).
int64_t route_groups(int64_t topk, int64_t E, int order);
size_t route_workspace_bytes(int64_t T, int64_t topk, int64_t G);
size_t grouped_gate_up_workspace_bytes(int64_t T, int64_t topk, int64_t E);
size_t moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk);

size_t gate_up_swiglu_quant_workspace_bytes(int64_t T, int64_t I, int64_t topk);

// slot_row (may be NULL): slot -> its sorted row, -1 for a dropped id.
// zero (may be NULL): zero_n words the same launch clears.
hipError_t launch_route(const int32_t* ids, int64_t T, int64_t topk, int64_t E, int order, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* slot_row, void* scratch, hipStream_t stream,
                        uint32_t* zero = nullptr, int64_t zero_n = 0);

hipError_t launch_grouped_gate_up_bf16(const uint8_t* xq, const float* xs, const int32_t* perm,
                                       const int32_t* offsets, const uint8_t* w13, const float* s13,
                                       uint16_t* gu, int64_t T, int64_t H, int64_t I, int64_t E,
                                       int64_t topk, int order, hipStream_t stream);

// dst_row (may be NULL): slot -> output row of h_q / h_scale; NULL keeps
// the sorted order of perm. h_out (may be NULL): where the float32 h rows go
// (in the same rows as h_q) instead of the workspace.
// ws: gate_up_swiglu_quant_workspace_bytes bytes,
// whose first T * topk words (the row maxima) it clears first unless
// amax_zeroed says an earlier launch on the stream already did.
hipError_t launch_gate_up_swiglu_quant(const uint8_t* xq, const float* xs, const int32_t* perm,
                                       const int32_t* offsets, const int32_t* dst_row, const uint8_t* w13,
                                       const float* s13, uint8_t* qh, float* sh, float* h_out, int64_t T,
                                       int64_t H, int64_t I, int64_t E, int64_t topk, int order, void* ws,
                                       hipStream_t stream, bool amax_zeroed = false);

// y: [T*topk, H] float32 scratch (down_combine_scratch_bytes).
size_t down_combine_scratch_bytes(int64_t T, int64_t H, int64_t topk);
// out_q / out_s (both NULL or both set): also quantize_per_token(out).
// slot_row (may be NULL): [T*topk] int32 scratch; when given, y holds the
// products in sorted order and slot_row the slot -> row map.
hipError_t launch_down_combine(const uint8_t* qh, const float* sh, const int32_t* perm,
                               const int32_t* offsets, const int32_t* ids, const float* tw,
                               const uint8_t* w2, const float* s2, uint16_t* out, float* y,
                               uint8_t* out_q, float* out_s, int64_t T, int64_t H, int64_t I,
                               int64_t E, int64_t topk, int order, hipStream_t stream, int32_t* slot_row);

hipError_t launch_grouped_gate_up(const uint8_t* xq, const float* xs, const int32_t* ids,
                                  const uint8_t* w13, const float* s13, uint16_t* gu, int32_t* perm,
                                  int32_t* offsets, int64_t T, int64_t H, int64_t I, int64_t E,
                                  int64_t topk, void* ws, hipStream_t stream);

hipError_t launch_moe(const uint8_t* xq, const float* xs, const int32_t* ids, const float* tw,
                      const uint8_t* w13, const float* s13, const uint8_t* w2, const float* s2,
                      uint16_t* out, uint8_t* out_q, float* out_s, int64_t T, int64_t H, int64_t I,
                      int64_t E, int64_t topk, void* ws, hipStream_t stream);

// MXFP4 routed experts (mx.hip): codes [rows, K/2] (two E2M1 per byte, the
// even element in the low nibble) and E8M0 scales [rows, K/32]. The grouped
// calls need H % 128 == 0 and I % 128 == 0.
hipError_t launch_mx_quantize(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, uint8_t* s, hipStream_t stream);

hipError_t launch_mx_gate_up_bf16(const uint8_t* xq, const uint8_t* xs, const int32_t* perm, const int32_t* offsets,
                                  const uint8_t* w13, const uint8_t* s13, uint16_t* gu, int64_t T, int64_t H,
                                  int64_t I, int64_t E, int64_t topk, int order, hipStream_t stream);

hipError_t launch_mx_gate_up_swiglu_quant(const uint8_t* xq, const uint8_t* xs, const int32_t* perm,
                                          const int32_t* offsets, const int32_t* dst_row, const uint8_t* w13,
                                          const uint8_t* s13, uint8_t* qh, uint8_t* sh, int64_t T, int64_t H,
                                          int64_t I, int64_t E, int64_t topk, int order, hipStream_t stream);

// y: [T*topk, H] float32 scratch; out_q / out_s (both NULL or both set): also
// the MXFP4 quantisation of out; slot_row as for launch_down_combine.
hipError_t launch_mx_down_combine(const uint8_t* qh, const uint8_t* sh, const int32_t* perm, const int32_t* offsets,
                                  const int32_t* ids, const float* tw, const uint8_t* w2, const uint8_t* s2,
                                  uint16_t* out, float* y, uint8_t* out_q, uint8_t* out_s, int64_t T, int64_t H,
                                  int64_t I, int64_t E, int64_t topk, int order, hipStream_t stream,
                                  int32_t* slot_row);

size_t mx_moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk);

hipError_t launch_mx_moe(const uint8_t* xq, const uint8_t* xs, const int32_t* ids, const float* tw,
                         const uint8_t* w13, const uint8_t* s13, const uint8_t* w2, const uint8_t* s2, uint16_t* out,
                         uint8_t* out_q, uint8_t* out_s, int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                         void* ws, hipStream_t stream);

}  // namespace w8a8
