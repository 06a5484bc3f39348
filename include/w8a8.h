/*
 * w8a8.h — C ABI of libw8a8.so, the W8A8 FP8 linear layer for AMD MI355X
 * (gfx950).
 *
 * What the library computes is the FP8 "fast-math" linear layer of the
 * Metis-1.6 model pages: each token's BF16 input row is rounded to FP8 with
 * one scale per token and multiplied with FP8 weights that carry one scale
 * per output channel, on the GPU's FP8 matrix units (Lernex/Metis-1.6-Logos-
 * FP8, "What --fast-math does" and "What is in FP8"; sglang-metis 0.1.0,
 * "Serve", memory paragraph). The routed experts use the same scheme
 * ("What is in FP8") and are run by the grouped entry points.
 *
 * Formats
 *   BF16   uint16_t bit patterns.
 *   E4M3   uint8_t codes of the OCP FP8 E4M3FN format (tensor type F8_E4M3;
 *          Lernex/Metis-1.6-Praxis-NVFP4, hub sidebar): bias 7, largest
 *          magnitude 448, no infinities, NaN = 0x7F / 0xFF.
 *   scale  float32.
 *   All matrices are dense and row-major. Weights are [out, in], each output
 *   row with its own scale (Lernex/Metis-1.6-Praxis-NVFP4, "What is in NVFP4").
 *
 * Conventions shared by every call
 *   Pointers     Device pointers owned by the caller. The library allocates
 *                and frees nothing and keeps no pointer after a call returns.
 *   Alignment    Every pointer must be 16-byte aligned.
 *   Streams      Work is enqueued on `stream` (0 = the null stream) and runs
 *                asynchronously; the caller keeps the buffers alive until
 *                the stream has passed the call.
 *   Errors       Every call returns a status code (W8A8_*). Arguments are
 *                checked on the host before anything is enqueued, so a
 *                non-zero status means nothing was written. A fault inside
 *                a kernel surfaces at the caller's next synchronisation,
 *                like any HIP error.
 *   Empty input  M == 0 (or N == 0) is a valid no-op.
 *   NaN / Inf    Inputs holding NaN or infinity are outside the contract; the
 *                outputs for them are unspecified.
 *   Threads      Calls are reentrant; the only shared state is a per-device
 *                cache of the architecture check.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W8A8_ABI_VERSION 2

enum {
  W8A8_OK = 0,
  W8A8_ERR_NULL_ARG = 1,      /* a required pointer is NULL                        */
  W8A8_ERR_BAD_SHAPE = 2,     /* a negative size, or a size product that overflows */
  W8A8_ERR_MISALIGNED = 3,    /* a pointer is not 16-byte aligned                  */
  W8A8_ERR_UNSUPPORTED = 4,   /* a size the kernels do not handle (see each call)  */
  W8A8_ERR_WORKSPACE = 5,     /* workspace smaller than the *_workspace_bytes size */
  W8A8_ERR_DEVICE = 6,        /* the current device is not gfx950, or no device    */
  W8A8_ERR_LAUNCH = 7,        /* the HIP runtime refused a launch                  */
  W8A8_ERR_SCRATCH = 8        /* the sizes need more than the static scratch holds */
};

/* W8A8_ABI_VERSION of the built library. */
int w8a8_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* w8a8_status_string(int status);

/*
 * quantize_per_token — dynamic per-row FP8 quantisation.
 *
 * Activations are quantised per token at run time, weights once per output
 * row; both are this call (Lernex/Metis-1.6-Logos-FP8, "What is in FP8"). For
 * each row m of x:
 *   amax      = max_k |x[m,k]|                       (exact)
 *   scale[m]  = fl32(amax / 448), or 1 if amax == 0
 *   q[m,k]    = E4M3(fl32(x[m,k] / scale[m]))        round to nearest even,
 *               |v| >= 448 saturates to 448, a negative value rounding to
 *               zero gives 0x80. Division is IEEE float32, subnormals kept.
 * The row's largest-magnitude element therefore always becomes +-448.
 *
 *   x_bf16  [M, K] BF16 input (read only)
 *   M, K    rows and row length; K must be a positive multiple of 16
 *   q_e4m3  [M, K] output codes
 *   scale   [M] output scales
 * Errors: NULL_ARG, BAD_SHAPE (M < 0, K < 0, M*K overflows),
 *         UNSUPPORTED (K == 0 or K % 16 != 0, K > 2^24), MISALIGNED, DEVICE,
 *         LAUNCH.
 */
int quantize_per_token(const uint16_t* x_bf16, int64_t M, int64_t K, uint8_t* q_e4m3, float* scale,
                       hipStream_t stream);

/*
 * w8a8_gemm — scaled FP8 x FP8 matrix product with a BF16 result.
 *
 * The fast-math multiply: the FP8-rounded input times the FP8 weights on the
 * matrix units, rescaled by the per-token and per-output-channel scales
 * (Lernex/Metis-1.6-Logos-FP8, "What --fast-math does"):
 *   y[m,n] = bf16( a_scale[m] * w_scale[n] * sum_k dec(a[m,k]) * dec(w[n,k]) )
 * Products are exact, sums are float32, the scale product is applied in
 * float32 in the epilogue and the result is rounded to nearest even. No bias.
 * M <= 32 runs a weight-streaming kernel (decode); larger M a tiled one.
 *
 *   a_q      [M, K] E4M3 input      a_scale [M] per-row scales
 *   w_q      [N, K] E4M3 weights    w_scale [N] per-output-row scales
 *   y_bf16   [M, N] output (must not overlap the inputs)
 *   M, N, K  K and N must be positive multiples of 16, K <= 2^20, N <= 2^20,
 *            M <= 2^24
 * Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED, MISALIGNED, DEVICE, LAUNCH.
 */
int w8a8_gemm(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q, const float* w_scale,
              uint16_t* y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * w8a8_gemm_timed — w8a8_gemm whose kernel the runtime times, for measurement.
 *
 * The same checks, kernels and result bits as w8a8_gemm. The kernel is
 * launched with hipExtLaunchKernel, which records `start` when the kernel
 * begins and `stop` when it ends, so hipEventElapsedTime(start, stop) is the
 * kernel's own duration, without the dispatch that precedes it on the
 * stream. This is how the throughput comparison of the fast-math layer is
 * measured here (Lernex/Metis-1.6-Logos-FP8, "What --fast-math does").
 *
 *   start, stop  caller-created events (hipEventCreate, timing enabled);
 *                neither may be NULL. When M == 0 or N == 0 no kernel runs
 *                and the events are not recorded.
 * Errors: those of w8a8_gemm; NULL_ARG also for a NULL event.
 */
int w8a8_gemm_timed(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q, const float* w_scale,
                    uint16_t* y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream, hipEvent_t start,
                    hipEvent_t stop);


/*
 * e4m3_from_f32, bf16_from_f32 — the final conversions of this library on
 * caller-given float32 values, for checking them on the device.
 *
 * Every FP8 byte the quantisers write is the E4M3 code of a float32 scaled
 * value (the OCP E4M3FN format the checkpoints store, Lernex/Metis-1.6-
 * Logos-FP8, "What is in FP8"), and every BF16 result is a float32 value
 * rounded to the model's dtype (same page, "What --fast-math does"). These
 * two calls run exactly those device steps:
 *   q_e4m3[i] = E4M3(clamp(v[i], -448, 448))   round to nearest even, the
 *               sign kept on a zero result
 *   y_bf16[i] = BF16(v[i])                     round to nearest even
 *   v          [n] float32 input (read only); NaN gives an unspecified code
 *   q_e4m3 / y_bf16  [n] output
 * Errors: NULL_ARG, BAD_SHAPE (n < 0), UNSUPPORTED (n > 2^40), MISALIGNED,
 *         DEVICE, LAUNCH.
 */
int e4m3_from_f32(const float* v, int64_t n, uint8_t* q_e4m3, hipStream_t stream);
int bf16_from_f32(const float* v, int64_t n, uint16_t* y_bf16, hipStream_t stream);

/*
 * read_probe — the read floor of the decode weight stream, for measurement.
 *
 * A decode step is bound by how fast the GPU reads the weights (Lernex/
 * Metis-1.6-Logos-FP8, "What --fast-math does"). This call reads every byte
 * of p in the decode GEMM's launch shape (one 256-thread workgroup per
 * 32 KB, each lane's 16-byte loads issued together) and does nothing else:
 * sink[b] = XOR of the 32-bit words of block b. Timed like the decode GEMM,
 * it is the floor that GEMM's weight stream is compared with.
 *   p      [bytes] device data; bytes a multiple of 16, at most 2^40
 *   sink   [read_probe_sink_words(bytes)] uint32 output
 * Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED, MISALIGNED, DEVICE, LAUNCH.
 */
int64_t read_probe_sink_words(int64_t bytes);
int read_probe(const uint8_t* p, int64_t bytes, uint32_t* sink, hipStream_t stream);

/*
 * clock_probe — the shader clock, for measurement.
 *
 * The pages compare the fast-math path's throughput with the default maths
 * (Lernex/Metis-1.6-Logos-FP8, "What --fast-math does"); on this GPU the
 * throughput of a steady load depends on the clock the power controller
 * sets, which this call reads. It launches n workgroups of one wave; lane 0
 * of workgroup b spins until the constant 100 MHz clock has advanced by 400
 * ticks (4 us) and writes the shader cycles counted over the same span to
 * out[2 b] and the constant-clock ticks to out[2 b + 1], so
 * 0.1 * out[2 b] / out[2 b + 1] is the shader clock in GHz. Enqueued right
 * after a kernel on the same stream, it shows the clock that kernel ran at
 * as far as the power controller's setting goes.
 *   out  [2 n] uint64 output, 16-byte aligned
 *   n    number of workgroups, 0 .. 65536
 * Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED, MISALIGNED, DEVICE, LAUNCH.
 */
int clock_probe(uint64_t* out, int64_t n, hipStream_t stream);

/*
 * w8a16_gemm — the default maths: BF16 activations times the E4M3 weights
 * widened to BF16, on the BF16 matrix units.
 *
 * Without the fast-math flag the model page's runtime widens the FP8 weights
 * to 16 bits as it multiplies and does the product in BF16, so the weights
 * are the only rounded operand (Lernex/Metis-1.6-Logos-FP8, "What --fast-math
 * does"):
 *   y[m,n] = bf16( w_scale[n] * sum_k x[m,k] * dec(w[n,k]) )
 * Every E4M3 value is exact in BF16; products are exact, sums are float32,
 * the scale is applied in float32 and the result is rounded to nearest even.
 * No activation quantisation, no activation scale, no bias. M <= 32 runs a
 * weight-streaming kernel; larger M a tiled one.
 *
 *   x_bf16   [M, K] BF16 activations
 *   w_q      [N, K] E4M3 weights    w_scale [N] per-output-row scales
 *   y_bf16   [M, N] output (must not overlap the inputs)
 *   M, N, K  as for w8a8_gemm
 * Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED, MISALIGNED, DEVICE, LAUNCH.
 */
int w8a16_gemm(const uint16_t* x_bf16, const uint8_t* w_q, const float* w_scale, uint16_t* y_bf16, int64_t M,
               int64_t N, int64_t K, hipStream_t stream);

/* Bytes of scratch fp8_linear needs on its FP8 path: M*K codes + M scales,
 * each rounded up to 256 bytes (0 for invalid sizes). */
size_t fp8_linear_workspace_bytes(int64_t M, int64_t K);

/*
 * fp8_linear — the layer as the model page's runtime chooses it: with
 * fast_math != 0 and more than 8 tokens (M > 8), quantize_per_token into the
 * workspace followed by w8a8_gemm (for M <= 16 and K <= 2048 as the single
 * launch of fp8_linear_single_launch, which gives the same bits); otherwise
 * w8a16_gemm. The page states that
 * the flag changes only steps that handle many tokens at once (prompt reading,
 * more than 8 conversations) and that a single conversation's generation uses
 * the default maths either way (Lernex/Metis-1.6-Logos-FP8, "What --fast-math
 * does").
 *   workspace  fp8_linear_workspace_bytes(M, K) bytes of device scratch; only
 *              read on the FP8 path (may be NULL otherwise)
 * Other arguments and errors as w8a16_gemm, plus WORKSPACE.
 */
int fp8_linear(const uint16_t* x_bf16, const uint8_t* w_q, const float* w_scale, uint16_t* y_bf16, int64_t M,
               int64_t N, int64_t K, int fast_math, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fp8_linear_noalloc — fp8_linear for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, dispatch and results as fp8_linear (bit
 * for bit), without the workspace: the quantised input (M*K codes + M scales,
 * each rounded up to 256 bytes) goes to a static device array of the library,
 * fp8_linear_noalloc_max_bytes() bytes (64 MiB) per GPU, held until the
 * process ends. The call allocates nothing (no hipMalloc, no allocating
 * library routine); on its first call on a device it looks up that device's
 * address of the array.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other threads) race and must be ordered by the caller.
 * The array needs no clearing: each call writes every byte it reads.
 * Errors: as fp8_linear (no WORKSPACE), plus SCRATCH when the FP8 path would
 * need more than fp8_linear_noalloc_max_bytes() (checked before any launch).
 */
size_t fp8_linear_noalloc_max_bytes(void);
int fp8_linear_noalloc(const uint16_t* x_bf16, const uint8_t* w_q, const float* w_scale, uint16_t* y_bf16, int64_t M,
                       int64_t N, int64_t K, int fast_math, hipStream_t stream);

/*
 * fp8_linear_single_launch — the FP8 multiply of fp8_linear (per-token
 * quantisation, then the scaled FP8 GEMM; Lernex/Metis-1.6-Logos-FP8, "What
 * --fast-math does") in one kernel launch with no workspace, for the few-token
 * steps: 1 <= M <= 32, K <= 2048. Every workgroup derives the row scales from
 * the BF16 input it loads and quantises it in registers with the
 * quantize_per_token rule, so the result is bit-identical to
 * quantize_per_token followed by w8a8_gemm. Each workgroup quantises the whole
 * input, which makes this slower than the two launches on MI355X; it is for
 * callers that need a single launch.
 *   x_bf16 [M, K], w_q [N, K] E4M3, w_scale [N], y_bf16 [M, N]
 * Errors: as w8a16_gemm; UNSUPPORTED also for M > 32 or K > 2048.
 */
int fp8_linear_single_launch(const uint16_t* x_bf16, const uint8_t* w_q, const float* w_scale, uint16_t* y_bf16,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Routed experts
 *
 * The routed experts are FP8 with the same scheme (Lernex/Metis-1.6-Logos-FP8,
 * "What is in FP8"); each token goes to its top-k experts (Lernex/Metis-1.6-
 * Praxis, "Architecture"); experts are stacked in global expert order (the
 * "Files" section of the model pages); the stack, and so this expert stage,
 * runs twice per token with one set of weights (sglang-metis 0.1.0, "How the
 * model maps onto SGLang"). Readings taken where the pages are silent:
 * W13[e] holds [gate; up] rows; h = silu(g) * u in float32; h is requantised
 * with one E4M3 scale per routed copy; each routed copy's output, weighted
 * by its router weight, stays in float32 (no page puts a rounding between
 * the experts and the top-k sum: Lernex/Metis-1.6-Logos-FP8, "What is in
 * FP8"); the k weighted copies of a token are summed in float32 in the
 * order j = 0, 1, ... and rounded once to BF16.
 *
 * Shapes (all row-major)
 *   x_q      [T, H]       E4M3 tokens, quantised once per token (quantize_per_token)
 *   x_scale  [T]          float32
 *   topk_ids [T, topk]    int32 expert ids; ids outside [0, E) are dropped
 *   topk_w   [T, topk]    float32 router weights (used as given)
 *   w13_q    [E, 2I, H]   E4M3; rows 0..I-1 gate, rows I..2I-1 up
 *   w13_scale[E, 2I]      float32 per output row
 *   w2_q     [E, H, I]    E4M3
 *   w2_scale [E, H]       float32 per output row
 * A slot is the flat index t * topk + j. Two sorted orders of the valid
 * slots exist, both stable (increasing slot index inside a group):
 *   order 0, expert-major:        E groups, group of slot = its expert id e;
 *   order 1, slot-position-major: topk * E groups, group = j * E + e.
 * The fused pass uses order 0, whose groups are k times larger than those
 * of order 1 (less padding in partial tiles); every stage accepts either.
 * Limits: 1 <= E <= 1024, 1 <= topk <= 64, at most 1024 routing groups
 * (E, or topk * E in order 1), H and I positive multiples of 16,
 * T * topk, T * H and 2 * I * H below 2^31. The fused calls need I to be a
 * multiple of 128. T == 0 is a no-op. offsets/perm passed to the stage calls must come
 * from moe_route (they are read on the device, never on the host).
 * ------------------------------------------------------------------------- */

/* Bytes of scratch moe_route needs (0 for invalid sizes). */
size_t moe_route_workspace_bytes(int64_t T, int64_t topk, int64_t E, int order);

/*
 * moe_route — sorted permutation of the routed slots (order 0 or 1, above).
 * With G groups (G = E for order 0, topk * E for order 1):
 *   counts  [G]       number of valid slots per group
 *   offsets [G + 1]   exclusive prefix of counts; offsets[G] = valid slots
 *   perm    [T*topk]  perm[offsets[g] + i] = i-th slot (increasing) of group
 *                     g; entries from offsets[G] on are set to -1
 *   slot_row [T*topk] optional (NULL = not written): the inverse map,
 *                     slot_row[perm[r]] = r, and -1 for a slot whose id is
 *                     dropped
 *   workspace         device scratch of moe_route_workspace_bytes bytes
 * Bit-exact, deterministic. Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED,
 * MISALIGNED, WORKSPACE, DEVICE, LAUNCH.
 */
int moe_route(const int32_t* topk_ids, int64_t T, int64_t topk, int64_t E, int order, int32_t* counts,
              int32_t* offsets, int32_t* perm, int32_t* slot_row, void* workspace, size_t workspace_bytes,
              hipStream_t stream);

/*
 * moe_gate_up_bf16 — grouped gate/up projection, BF16 result.
 *   gu_bf16[r, :] = bf16( x_scale[t] * w13_scale[e, :] * (x_q[t, :] . w13_q[e]^T) )
 * for the r-th sorted slot (t = perm[r] / topk, e its expert); gu_bf16 is
 * [T*topk, 2I], rows from offsets[G] on are left untouched. `order` is the
 * order perm/offsets were made with.
 */
int moe_gate_up_bf16(const uint8_t* x_q, const float* x_scale, const int32_t* perm, const int32_t* offsets,
                     const uint8_t* w13_q, const float* w13_scale, uint16_t* gu_bf16, int64_t T, int64_t H,
                     int64_t I, int64_t E, int64_t topk, int order, hipStream_t stream);

/* Bytes of scratch moe_gate_up_swiglu_quant needs: T*topk*(4 I + 4) rounded
 * up (0 for invalid sizes). */
size_t moe_gate_up_swiglu_quant_workspace_bytes(int64_t T, int64_t I, int64_t topk);

/*
 * moe_gate_up_swiglu_quant — grouped gate/up projection with the expert
 * activation and the requantisation fused in:
 *   g, u = the gate and up halves of the slot's float32 gate/up row
 *   h    = silu(g) * u                       (float32)
 *   h_scale[r] = fl32(max|h| / 448) (1 if h == 0),
 *   h_q[r, i]  = E4M3(fl32(h[i] / h_scale[r]))  (round to nearest even, saturating)
 * h_q [T*topk, I] and h_scale [T*topk]. The row r a slot's h goes to is its
 * sorted row under perm, or dst_row[slot] when dst_row is given (a
 * slot_row array of moe_route in the other order: the tiles then follow
 * `perm`, the output rows the other order). Rows from offsets[G] on are left
 * untouched. I must be a multiple of 128. `order` is the order perm/offsets
 * were made with. The workspace holds the row maxima and, unless h_f32 is
 * given, the float32 h rows.
 *   h_f32 [T*topk, I]  optional (NULL: not written): the float32 h rows the
 *                      codes were made from, in the same rows as h_q, so that
 *                      a caller can check the requantisation bit for bit.
 */
int moe_gate_up_swiglu_quant(const uint8_t* x_q, const float* x_scale, const int32_t* perm, const int32_t* offsets,
                             const int32_t* dst_row, const uint8_t* w13_q, const float* w13_scale, uint8_t* h_q,
                             float* h_scale, float* h_f32, int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                             int order, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_down_combine — grouped down projection and router-weighted combine:
 *   y[slot, :]   = topk_w[slot] * h_scale[r] * w2_scale[e, :] * (h_q[r, :] . w2_q[e]^T)
 *                  for the slot of sorted row r (product and scaling in float32)
 *   out_bf16[t]  = bf16( sum over j = 0..topk-1 with a valid id of y[t*topk + j] )
 * Each routed copy is kept in float32; the sum is float32, always taken in
 * the order j = 0, 1, ... (so the result does not depend on the sorted
 * order and is deterministic), and rounded to BF16 once. No page puts a
 * rounding between the experts and the top-k sum (Lernex/Metis-1.6-Logos-
 * FP8, "What is in FP8"; sglang-metis 0.1.0, "How the model maps onto
 * SGLang"). perm/offsets may be in either order (`order`); topk_ids tells
 * the valid slots. y_f32 [T*topk, H] is caller-provided float32 scratch. A
 * token with no valid slot gets zeros.
 */
int moe_down_combine(const uint8_t* h_q, const float* h_scale, const int32_t* perm, const int32_t* offsets,
                     const int32_t* topk_ids, const float* topk_w, const uint8_t* w2_q, const float* w2_scale,
                     uint16_t* out_bf16, float* y_f32, int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                     int order, hipStream_t stream);

/* Bytes of scratch w8a8_grouped_gemm needs (0 for invalid sizes). */
size_t w8a8_grouped_gemm_workspace_bytes(int64_t T, int64_t topk, int64_t E);

/*
 * w8a8_grouped_gemm — moe_route followed by moe_gate_up_bf16: the routed
 * gate/up grouped GEMM on per-token FP8 activations with a BF16 result.
 * Outputs gu_bf16 [T*topk, 2I] in sorted order, perm [T*topk] and
 * offsets [E + 1] (as moe_route) so the caller can map rows back to slots.
 */
int w8a8_grouped_gemm(const uint8_t* x_q, const float* x_scale, const int32_t* topk_ids, const uint8_t* w13_q,
                      const float* w13_scale, uint16_t* gu_bf16, int32_t* perm, int32_t* offsets, int64_t T,
                      int64_t H, int64_t I, int64_t E, int64_t topk, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Bytes of scratch moe_w8a8_grouped needs (0 for invalid sizes). */
size_t moe_w8a8_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk);

/*
 * moe_w8a8_grouped — one routed-expert pass on buffers carved from
 * `workspace`, all in order 0: moe_route, moe_gate_up_swiglu_quant, then
 * moe_down_combine. out_bf16 [T, H]. I must be a multiple of 128.
 *   out_q [T, H], out_scale [T]  optional (both NULL, or both set): also
 *                 writes quantize_per_token(out_bf16), bit for bit, fused into
 *                 the combine — the input of the next pass of the stack
 *                 (sglang-metis 0.1.0, "How the model maps onto SGLang": every
 *                 token passes through the stack twice on one set of weights).
 * Running the two passes is two calls; the second takes the first call's
 * out_q / out_scale as x_q / x_scale.
 */
int moe_w8a8_grouped(const uint8_t* x_q, const float* x_scale, const int32_t* topk_ids, const float* topk_w,
                     const uint8_t* w13_q, const float* w13_scale, const uint8_t* w2_q, const float* w2_scale,
                     uint16_t* out_bf16, uint8_t* out_q, float* out_scale, int64_t T, int64_t H, int64_t I, int64_t E,
                     int64_t topk, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * MXFP4 routed experts
 *
 * The 4-bit model page keeps the routed experts in a 4-bit format (E2M1
 * values with a scale per small block of inputs) and under fast-math rounds
 * each expert input to FP4 as well (Lernex/Metis-1.6-Praxis-NVFP4, "What is
 * in NVFP4" and "What --fast-math does"). Its blocks are 16 inputs with an
 * E4M3 scale; these calls use the block format that gfx950's scaled matrix
 * cores take natively, OCP MXFP4: blocks of 32 consecutive inputs along K,
 * one E8M0 (power-of-two) scale each.
 *
 * Formats
 *   E2M1   4-bit codes, two per byte: element 2i of a row in the low nibble of
 *          byte i. Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign.
 *   E8M0   one byte per block, value 2^(e - 127) (0xFF is NaN, never written).
 *   A row of K values is K/2 code bytes and K/32 scale bytes; matrices are
 *   row-major: codes [rows, K/2], scales [rows, K/32].
 * Quantisation of a block (OCP MX v1.0): X = floor(log2(max |x|)) - 2,
 * clamped to [-127, 127] (an all-zero block gets X = 0); each element is
 * x / 2^X (exact) rounded to nearest, ties to even, magnitudes above 6
 * saturating to 6, a negative value that rounds to zero giving 0x8.
 *
 * The expert chain is that of the FP8 calls above with every expert input
 * and weight in MXFP4: tokens are quantised once over H, h = silu(g) * u
 * (float32) is quantised per routed copy over I, y = topk_w * product in
 * float32, and the k weighted copies of a token are summed in float32 in the
 * order j = 0, 1, ... and rounded once to BF16.
 * Shapes: x_q [T, H/2] / x_scale [T, H/32]; w13_q [E, 2I, H/2] /
 * w13_scale [E, 2I, H/32] (rows 0..I-1 gate, I..2I-1 up); w2_q [E, H, I/2] /
 * w2_scale [E, H, I/32]; h_q [T*topk, I/2] / h_scale [T*topk, I/32].
 * Limits: as the FP8 expert calls, and H and I positive multiples of 128.
 * Scales are applied inside the matrix-core product; products of two E2M1
 * values are exact, sums are float32.
 * ------------------------------------------------------------------------- */

/*
 * mxfp4_quantize — BF16 rows -> MXFP4 codes and E8M0 block scales, by the
 * rule above. Bit-exact and deterministic.
 *   x_bf16 [M, K]; q_fp4 [M, K/2]; scale_e8m0 [M, K/32]
 *   K a positive multiple of 32, K <= 2^24.
 * Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED, MISALIGNED, DEVICE, LAUNCH.
 */
int mxfp4_quantize(const uint16_t* x_bf16, int64_t M, int64_t K, uint8_t* q_fp4, uint8_t* scale_e8m0,
                   hipStream_t stream);

/*
 * moe_mxfp4_gate_up_bf16 — grouped gate/up projection on MXFP4 operands,
 * BF16 result: gu_bf16[r, :] = bf16( x[t] . W13[e]^T ) for the r-th sorted
 * slot (t = perm[r] / topk, e its expert), gu_bf16 [T*topk, 2I]; rows from
 * offsets[G] on are left untouched. perm/offsets from moe_route in `order`.
 */
int moe_mxfp4_gate_up_bf16(const uint8_t* x_q, const uint8_t* x_scale, const int32_t* perm, const int32_t* offsets,
                           const uint8_t* w13_q, const uint8_t* w13_scale, uint16_t* gu_bf16, int64_t T, int64_t H,
                           int64_t I, int64_t E, int64_t topk, int order, hipStream_t stream);

/*
 * moe_mxfp4_gate_up_swiglu_quant — the gate/up projection with the expert
 * activation and the MXFP4 quantisation of h fused in: h = silu(g) * u in
 * float32 from the slot's gate/up row, then h_q / h_scale of h by the block
 * rule. The row a slot's h goes to is its sorted row under perm, or
 * dst_row[slot] when dst_row is given (as for moe_gate_up_swiglu_quant).
 * No workspace: an MX block's scale needs only its own 32 values.
 */
int moe_mxfp4_gate_up_swiglu_quant(const uint8_t* x_q, const uint8_t* x_scale, const int32_t* perm,
                                   const int32_t* offsets, const int32_t* dst_row, const uint8_t* w13_q,
                                   const uint8_t* w13_scale, uint8_t* h_q, uint8_t* h_scale, int64_t T, int64_t H,
                                   int64_t I, int64_t E, int64_t topk, int order, hipStream_t stream);

/*
 * moe_mxfp4_down_combine — grouped down projection and combine:
 *   y[slot, :]  = topk_w[slot] * (h[r] . W2[e]^T)            (sorted row r, float32)
 *   out_bf16[t] = bf16( sum over valid j, in order j = 0, 1, ... of y[t*topk + j] )
 *                 (float32 sum, one rounding)
 *   y_f32 [T*topk, H] is caller-provided float32 scratch.
 *   out_q [T, H/2], out_scale [T, H/32]  optional (both NULL or both set):
 *               mxfp4_quantize(out_bf16), bit for bit, fused into the
 *               combine — the next pass's expert input.
 */
int moe_mxfp4_down_combine(const uint8_t* h_q, const uint8_t* h_scale, const int32_t* perm, const int32_t* offsets,
                           const int32_t* topk_ids, const float* topk_w, const uint8_t* w2_q, const uint8_t* w2_scale,
                           uint16_t* out_bf16, float* y_f32, uint8_t* out_q, uint8_t* out_scale, int64_t T, int64_t H,
                           int64_t I, int64_t E, int64_t topk, int order, hipStream_t stream);

/* Bytes of scratch moe_mxfp4_grouped needs (0 for invalid sizes). */
size_t moe_mxfp4_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk);

/*
 * moe_mxfp4_grouped — one MXFP4 routed-expert pass on buffers carved from
 * `workspace`, all in order 0: moe_route, moe_mxfp4_gate_up_swiglu_quant,
 * moe_mxfp4_down_combine. out_bf16 [T, H]; out_q / out_scale as for
 * moe_mxfp4_down_combine. The second pass of the stack is a second call on
 * the first call's out_q / out_scale.
 */
int moe_mxfp4_grouped(const uint8_t* x_q, const uint8_t* x_scale, const int32_t* topk_ids, const float* topk_w,
                      const uint8_t* w13_q, const uint8_t* w13_scale, const uint8_t* w2_q, const uint8_t* w2_scale,
                      uint16_t* out_bf16, uint8_t* out_q, uint8_t* out_scale, int64_t T, int64_t H, int64_t I,
                      int64_t E, int64_t topk, void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
