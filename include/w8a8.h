/*
 * w8a8.h -- C ABI of the MI355X (gfx950) W8A8 quantized projection library.
 *
 * The library implements the quantized decoder projection described on the
 * pages about quantized Clef checkpoints:
 *   - "CLEF Calibrated INT8 ConvRot" model card (Benefits list, notes under the
 *     latency table): activations of the INT8 text projections go through a
 *     rotation-plus-per-token-int8 quantizer, then an integer GEMM whose
 *     epilogue fuses the scales, the bias and the paired gate/up SwiGLU;
 *   - "Loading CLEF INT8" usage page: gate/up weights are packed into a single
 *     matrix when loaded; weights are immutable once loaded; fuse_mlp selects
 *     the paired gate/up epilogue;
 *   - "clef-flash-FP8" card (Quantization table, note after recipe.yaml): the
 *     FP8 W8A8 dynamic scheme, E4M3 weights with per-output-channel scales taken
 *     from the weights and E4M3 activations with per-token scales computed at
 *     run time.
 * Where the pages leave the arithmetic open, the library takes these readings:
 *   int8 scale s = amax/127 (fp32 IEEE division), code = round-half-even(y/s);
 *   fp8 scale s = amax/448, code = nearest OCP E4M3FN of clamp(y/s, +-448);
 *   a zero row has s = 0 and all-zero codes; the rotation is the normalized
 *   Sylvester Walsh-Hadamard transform of order 128 on each block of 128
 *   consecutive K elements, computed exactly and rounded once to fp32;
 *   the epilogue rounds once to bf16 (round half to even).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers on the current HIP device.
 *     Tensors are dense, row-major, with the last dimension contiguous:
 *       x      bf16 [M, K]   (raw uint16 bit patterns)
 *       w      int8 [N, K]   or E4M3FN codes uint8 [N, K] (output-channel rows)
 *       q      int8 [M, K]   or E4M3FN codes uint8 [M, K]
 *       s_tok  fp32 [M],  s_ch fp32 [N]
 *       bias   bf16 [N]   (may be NULL: no bias)
 *       y      bf16 [M, N]
 *   - Every pointer must be 16-byte aligned.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronizes; every call only enqueues kernels on `stream` (NULL is the
 *     default stream) and returns.  Calls are therefore safe to capture into
 *     a HIP graph.  Inputs are never written; outputs are fully overwritten;
 *     outputs must not alias inputs or the workspace.
 *   - All argument checks run on the host before anything is enqueued; on an
 *     error nothing is written and the status says why.  M == 0 is W8A8_OK and
 *     enqueues nothing;
 *     since it touches no memory, its pointers are not checked.  Faults inside
 *     kernels surface at the caller's next synchronization, as with any
 *     asynchronous HIP call.
 *   - Inputs must be finite; results for non-finite inputs are unspecified.
 *   - Shape limits: M >= 0; 1 <= K <= W8A8_MAX_K and K % 128 == 0 for the GEMM
 *     entry points (K % 32 == 0 for the quantizers alone; K % 128 == 0 whenever
 *     rot_block == 128); N >= 1 and N % 8 == 0; rot_block is 0 or 128.
 *     W8A8_MAX_K keeps every int8 accumulator (|acc| <= 127*127*K) inside int32.
 *   - Entry points are reentrant; the only global state is a per-device cache
 *     of the architecture check (the device must be gfx950).
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W8A8_MAX_K 131072

typedef enum {
  W8A8_OK = 0,
  W8A8_ERR_NULL_POINTER = 1,       /* a required pointer is NULL (bias may be NULL) */
  W8A8_ERR_BAD_SHAPE = 2,          /* M < 0, N or K out of range or not a multiple as required */
  W8A8_ERR_MISALIGNED = 3,         /* a pointer is not 16-byte aligned */
  W8A8_ERR_BAD_ARGUMENT = 4,       /* rot_block not 0/128, or the workspace is too small */
  W8A8_ERR_UNSUPPORTED_DEVICE = 5, /* no HIP device, or the current device is not gfx950 */
  W8A8_ERR_LAUNCH = 6,             /* the kernel launch itself failed (hipGetLastError) */
  W8A8_ERR_SCRATCH_TOO_SMALL = 7   /* w8a8_linear_packed_noalloc: the call needs more than
                                      W8A8_NOALLOC_MAX_WORKSPACE bytes of scratch */
} w8a8_status;

/* Human-readable name of a status code (static storage, never NULL). */
const char* w8a8_status_string(w8a8_status s);

/* ---- packed operand layout ---------------------------------------------------
 * A matrix of `rows` rows of K one-byte codes (K % 64 == 0) stored as blocks of
 * 32 rows x 64 bytes: block (r / 32, k / 64) starts at byte
 * ((r / 32) * (K / 64) + k / 64) * 2048 and holds row r % 32 of the block at
 * byte 64 * (r % 32) within it.  The row count is rounded up to a multiple of
 * 32.  Each 32-row, 64-byte piece of a GEMM stage is then one contiguous 2 KiB
 * read.  Weights are immutable once loaded ("Loading CLEF INT8" page, as with
 * the load-time gate/up packing), so a loader packs them once with
 * w8a8_pack_weight and calls the *_packed whole-path entry points. */

/* Bytes of the packed form of `rows` x K codes: ceil(rows / 32) * 32 * K
 * (0 for rows <= 0 or K <= 0). */
size_t w8a8_packed_bytes(int64_t rows, int64_t K);

/* Row-major codes w [rows, K] (int8 or E4M3FN, any one-byte codes) -> the packed
 * layout in w_packed (w8a8_packed_bytes(rows, K) bytes, caller-owned; padding
 * rows are written as zeros).  K % 64 == 0, 64 <= K <= W8A8_MAX_K.  For the
 * SwiGLU entry points pack the whole [2N, K] gate/up matrix in one call. */
w8a8_status w8a8_pack_weight(const void* w, int64_t rows, int64_t K, void* w_packed,
                             hipStream_t stream);

/* Bytes of device workspace the whole-path entry points need for M tokens of
 * K features: the int8 (or E4M3FN) codes of x in the packed layout
 * (w8a8_packed_bytes(M, K) bytes) followed by the fp32 scales [M], each part
 * starting on a 256-byte boundary.  Returns 0 for M <= 0 or K <= 0. */
size_t w8a8_workspace_bytes(int64_t M, int64_t K);

/* ---- stage 1: per-row dynamic symmetric quantizer ----------------------------
 * Per-token activation quantizer of the ConvRot INT8 path (INT8 ConvRot card,
 * latency-table notes) and of the FP8 dynamic scheme (clef-flash-FP8 card,
 * Quantization table).  For each row m of x: optionally rotate each block of
 * 128 (rot_block == 128), take amax = max|y|, s_tok[m] = amax/127 (int8) or
 * amax/448 (fp8), then q = round-half-even(y/s) clamped to +-127 (int8) or
 * the nearest E4M3FN value of clamp(y/s, +-448) (fp8).  Applied to the rows of
 * a weight matrix W [N, K] the same call gives the per-output-channel weight
 * codes and scales (weight scales computed straight from the weights, note
 * after the FP8 card's recipe.yaml). */
w8a8_status w8a8_quantize_act(const uint16_t* x, int64_t M, int64_t K, int rot_block,
                              int8_t* q, float* s_tok, hipStream_t stream);
w8a8_status w8a8_quantize_act_fp8(const uint16_t* x, int64_t M, int64_t K, int rot_block,
                                  uint8_t* q, float* s_tok, hipStream_t stream);
/* The same quantizers writing the codes in the packed layout (K % 64 == 0;
 * q_packed holds w8a8_packed_bytes(M, K) bytes; its padding rows are left
 * untouched).  One set of packed activation codes can feed several packed
 * GEMMs -- e.g. projections that share their input. */
w8a8_status w8a8_quantize_act_packed(const uint16_t* x, int64_t M, int64_t K, int rot_block,
                                     int8_t* q_packed, float* s_tok, hipStream_t stream);
w8a8_status w8a8_quantize_act_fp8_packed(const uint16_t* x, int64_t M, int64_t K, int rot_block,
                                         uint8_t* q_packed, float* s_tok, hipStream_t stream);

/* ---- stage 2 alone: acc[m][n] = sum_k q[m][k] * w[n][k], exact int32 ----------
 * The raw integer contraction (diagnostic / test entry point). acc is int32 [M, N].
 * The _packed form takes both code matrices in the packed layout (q_packed of M
 * rows, w_packed of N rows) and runs the same kernel, tile choice and K loop as
 * w8a8_gemm_dequant_packed, so it exposes the accumulators that epilogue sees. */
w8a8_status w8a8_gemm_i32(const int8_t* q, const int8_t* w, int32_t* acc,
                          int64_t M, int64_t N, int64_t K, hipStream_t stream);
w8a8_status w8a8_gemm_i32_packed(const int8_t* q_packed, const int8_t* w_packed, int32_t* acc,
                                 int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* ---- stages 2+3: integer GEMM with the fused dequant epilogue ---------------
 * y[m][n] = bf16( acc[m][n] * s_tok[m] * s_ch[n] + bias[n] ), computed from the
 * exact int32 accumulator in fp32 with a single final rounding (INT8 ConvRot
 * card, Benefits list: scales and bias fused into the GEMM). */
w8a8_status w8a8_gemm_dequant(const int8_t* q, const float* s_tok, const int8_t* w, const float* s_ch,
                              const uint16_t* bias, uint16_t* y,
                              int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* ---- stages 2+3': integer GEMM with the paired gate/up SwiGLU epilogue -------
 * w is the packed [2N, K] weight (gate rows 0..N-1, up rows N..2N-1, as packed
 * at load time on the "Loading CLEF INT8" page), s_ch and bias (nullable) are
 * [2N].  With g and u the unrounded dequantized values of rows n and N+n,
 * y[m][n] = bf16( silu(g) * u ), y is [M, N]. */
w8a8_status w8a8_gemm_swiglu(const int8_t* q, const float* s_tok, const int8_t* w_gateup,
                             const float* s_ch, const uint16_t* bias, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* ---- fp8 stages 2+3: E4M3FN x E4M3FN GEMM (fp32 accumulation) + dequant ------
 * y[m][n] = bf16( (sum_k dec(q[m][k]) * dec(w[n][k])) * s_tok[m] * s_ch[n] + bias[n] ).
 * The fp32 summation order is fixed per output element and does not depend on
 * M, so results are independent of how rows are batched. */
w8a8_status w8a8_fp8_gemm_dequant(const uint8_t* q, const float* s_tok, const uint8_t* w,
                                  const float* s_ch, const uint16_t* bias, uint16_t* y,
                                  int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* ---- stages 2+3 on packed operands ---------------------------------------------
 * w8a8_gemm_dequant / w8a8_gemm_swiglu / w8a8_fp8_gemm_dequant with both code
 * matrices in the packed layout: q_packed from w8a8_quantize_act*_packed (M
 * rows), the weight from w8a8_pack_weight (N rows, or 2N gate/up rows).  Same
 * arithmetic and results as the row-major forms. */
w8a8_status w8a8_gemm_dequant_packed(const int8_t* q_packed, const float* s_tok, const int8_t* w_packed,
                                     const float* s_ch, const uint16_t* bias, uint16_t* y, int64_t M,
                                     int64_t N, int64_t K, hipStream_t stream);
w8a8_status w8a8_gemm_swiglu_packed(const int8_t* q_packed, const float* s_tok,
                                    const int8_t* w_gateup_packed, const float* s_ch,
                                    const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K,
                                    hipStream_t stream);
w8a8_status w8a8_fp8_gemm_dequant_packed(const uint8_t* q_packed, const float* s_tok,
                                         const uint8_t* w_packed, const float* s_ch,
                                         const uint16_t* bias, uint16_t* y, int64_t M, int64_t N,
                                         int64_t K, hipStream_t stream);

/* ---- unfused gate/up: SwiGLU of separately projected gate and up -------------
 * The "Loading CLEF INT8" page's fuse_mlp=False setting disables the paired
 * gate/up epilogue: gate and up are then ordinary linears (for example one
 * w8a8_linear onto the 2N packed rows, giving [M, 2N]) and this call combines
 * their bf16 outputs: y[m][n] = bf16( silu(gate[m][n]) * up[m][n] ), evaluated
 * in fp32 (g / (1 + exp(-g)) * u) with one round to nearest even.  gate and up
 * are bf16 [M, N] whose rows are `ld` elements apart (ld >= N; ld = 2N and
 * up = gate + N for the halves of a [M, 2N] projection); y is dense [M, N].
 * N % 8 == 0, ld % 8 == 0, pointers 16-byte aligned; y must not overlap the
 * inputs. */
w8a8_status w8a8_swiglu(const uint16_t* gate, const uint16_t* up, int64_t ld, uint16_t* y,
                        int64_t M, int64_t N, hipStream_t stream);

/* ---- whole paths: quantize x into the workspace, then GEMM + epilogue --------
 * `workspace` must hold w8a8_workspace_bytes(M, K) bytes (256-byte aligned is
 * best; 16-byte aligned is required) and is used as scratch for the quantized
 * activations and their scales; its contents afterwards are those codes (in
 * the packed layout) and scales.  Two kernels are enqueued on `stream` (the
 * quantizer, then the GEMM) -- or, for short int8 batches (M <= 512,
 * K <= 1024, at most 256 tiles of 32 tokens x 64 weight rows), one kernel
 * that quantizes each tile's rows itself, with the same codes, scales and
 * outputs.  The plain forms take the
 * row-major weight; the *_packed forms take the weight as written by
 * w8a8_pack_weight (same arithmetic, same results). */
w8a8_status w8a8_linear(const uint16_t* x, const int8_t* w, const float* s_ch, const uint16_t* bias,
                        uint16_t* y, int64_t M, int64_t N, int64_t K, int rot_block,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

w8a8_status w8a8_gateup_swiglu(const uint16_t* x, const int8_t* w_gateup, const float* s_ch,
                               const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K,
                               int rot_block, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

w8a8_status w8a8_fp8_linear(const uint16_t* x, const uint8_t* w, const float* s_ch,
                            const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K,
                            int rot_block, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

w8a8_status w8a8_linear_packed(const uint16_t* x, const int8_t* w_packed, const float* s_ch,
                               const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K,
                               int rot_block, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

w8a8_status w8a8_gateup_swiglu_packed(const uint16_t* x, const int8_t* w_gateup_packed,
                                      const float* s_ch, const uint16_t* bias, uint16_t* y, int64_t M,
                                      int64_t N, int64_t K, int rot_block, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

w8a8_status w8a8_fp8_linear_packed(const uint16_t* x, const uint8_t* w_packed, const float* s_ch,
                                   const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K,
                                   int rot_block, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* ---- the int8 whole path without a workspace ---------------------------------
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): w8a8_linear_packed with
 * its workspace -- the packed activation codes and their scales -- taken from a
 * fixed device array inside the library instead of the caller.  Same kernels,
 * same arguments otherwise, same results byte for byte.  The array holds
 * W8A8_NOALLOC_MAX_WORKSPACE bytes on each device the library runs on, kept until
 * the process ends; a call whose w8a8_workspace_bytes(M, K) exceeds it returns
 * W8A8_ERR_SCRATCH_TOO_SMALL (checked after the shapes, before anything else)
 * and enqueues nothing.  This entry point allocates nothing (no hipMalloc, no
 * library allocation).  Every call on one device shares that device's array:
 * calls that overlap in time on one device (e.g. on two streams) race and give
 * undefined results; calls ordered on one stream are safe.  The array keeps the
 * last call's codes and scales; nothing in it needs clearing between calls. */
#define W8A8_NOALLOC_MAX_WORKSPACE (64u << 20)

w8a8_status w8a8_linear_packed_noalloc(const uint16_t* x, const int8_t* w_packed, const float* s_ch,
                                       const uint16_t* bias, uint16_t* y, int64_t M, int64_t N,
                                       int64_t K, int rot_block, hipStream_t stream);

/* ---- gate/up SwiGLU whose output is quantized for the next linear -----------
 * The down projection that follows the gate/up pair is an INT8 projection too,
 * so its input -- the SwiGLU output h [M, N] -- goes through the same per-token
 * activation quantizer as every INT8 projection's input (INT8 ConvRot card,
 * notes under the latency table), after the paired gate/up epilogue ("Loading
 * CLEF INT8", fuse_mlp):
 *   h = bf16(silu(g) * u)                    as w8a8_gateup_swiglu_packed;
 *   q_packed, s_tok = w8a8_quantize_act_packed(h, rot_out)   bit for bit.
 * Three kernels on `stream`: the quantizer of x (rotation rot_in), the gate/up
 * GEMM with the SwiGLU epilogue writing h into the workspace, the quantizer of
 * h.  The codes are w8a8_packed_bytes(M, N) bytes in the packed layout of a
 * [M, N] activation (padding rows untouched): the A operand of
 * w8a8_gemm_dequant_packed for the down projection (its K = N); s_tok is [M].
 * Shapes: the gate/up GEMM's (K % 128 == 0) and N % 64 == 0, N <= W8A8_MAX_K;
 * rot_out == 128 needs N % 128 == 0; rot_in and rot_out are 0 or 128
 * (W8A8_ERR_BAD_ARGUMENT otherwise). */

/* Workspace of w8a8_gateup_swiglu_quant_packed: w8a8_workspace_bytes(M, K)
 * (the codes and scales of x) followed by h, bf16 [M, N], on a 256-byte
 * boundary.  Afterwards it holds those values.  0 for M, N or K <= 0. */
size_t w8a8_swiglu_quant_workspace_bytes(int64_t M, int64_t N, int64_t K);

w8a8_status w8a8_gateup_swiglu_quant_packed(const uint16_t* x, const int8_t* w_gateup_packed,
                                            const float* s_ch, const uint16_t* bias, int64_t M,
                                            int64_t N, int64_t K, int rot_in, int rot_out,
                                            int8_t* q_packed, float* s_tok, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
