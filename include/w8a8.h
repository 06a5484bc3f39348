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
 *   All matrices are dense and row-major. Weights are [out, in] with one
 *   scale per output row (Lernex/Metis-1.6-Praxis-NVFP4, "What is in NVFP4").
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

#define W8A8_ABI_VERSION 1

enum {
  W8A8_OK = 0,
  W8A8_ERR_NULL_ARG = 1,      /* a required pointer is NULL                        */
  W8A8_ERR_BAD_SHAPE = 2,     /* a negative size, or a size product that overflows */
  W8A8_ERR_MISALIGNED = 3,    /* a pointer is not 16-byte aligned                  */
  W8A8_ERR_UNSUPPORTED = 4,   /* a size the kernels do not handle (see each call)  */
  W8A8_ERR_WORKSPACE = 5,     /* workspace smaller than the *_workspace_bytes size */
  W8A8_ERR_DEVICE = 6,        /* the current device is not gfx950, or no device    */
  W8A8_ERR_LAUNCH = 7         /* the HIP runtime refused a launch                  */
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

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
