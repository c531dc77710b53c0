/*
 * qlin.h -- C ABI of the fused 4-bit + low-rank-adapter linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is a frozen base weight W[d_out][d_in] stored in 4 bits plus a
 * trainable 16-bit adapter (A, B):
 *
 *     y  = x . dequant(Wq)^T + s . (P . A^T) . B^T          (forward)
 *     P  = x                      (plain adapter, pool = 1)
 *     P  = group sums of x        (QA-LoRA pooled adapter, pool = group)
 *
 * and the backward pass into the adapter and the input only (W is frozen):
 *
 *     du = s . dY . B,   dB = s . dY^T . u,   dA = du^T . P,
 *     dX = dY . dequant(Wq) + expand(du . A)
 *
 * Sources (web pages, cited by title and section):
 *   [QLoRA]   "QLoRA: Efficient Finetuning of Quantized LLMs" explainer
 *             (azimuth.plus), sections "Background: what is quantization?",
 *             "Innovation 1: 4-bit NormalFloat (NF4)", "Background: how LoRA
 *             works", "The QLoRA recipe: quantize, then adapt", "Innovation 2:
 *             Double Quantization", "The complete QLoRA forward pass", "The
 *             same idea in code".
 *   [QA-LoRA] "QA-LoRA: Quantization-Aware Low-Rank Adaptation of Large
 *             Language Models", abstract (group-wise INT4 operators, merge).
 *
 * Conventions for every entry point
 *   - Matrices are dense, row-major, contiguous.  "bf16" and "fp16" buffers
 *     are passed as uint16_t bit patterns.
 *   - Every pointer argument of qlin_quantize_*, qlin_fwd, qlin_bwd and
 *     qlin_dequant_bf16 is DEVICE memory owned by the caller, except where a
 *     comment says "host".  The library never keeps a pointer after a call
 *     returns and never frees caller memory.
 *   - Device pointers must be 16-byte aligned (QLIN_E_ALIGN otherwise).
 *   - Argument errors are reported synchronously, before anything is
 *     enqueued.  qlin_fwd / qlin_bwd / qlin_dequant_bf16 are asynchronous on
 *     `stream`; a device-side fault surfaces at the caller's next
 *     synchronisation.  The two quantizers synchronise `stream` and report
 *     non-finite input.
 *   - Outputs are overwritten, never accumulated into.
 *   - Calls keep no global mutable state: concurrent calls on different
 *     streams are safe provided they do not share a workspace.
 */
#ifndef QLIN_H_
#define QLIN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
typedef enum {
  QLIN_OK = 0,
  QLIN_E_NULL = 1,        /* a required pointer is NULL                        */
  QLIN_E_SHAPE = 2,       /* a size is out of range or not a required multiple */
  QLIN_E_ALIGN = 3,       /* a device pointer is not 16-byte aligned           */
  QLIN_E_NONFINITE = 4,   /* quantizer input holds NaN/Inf (or, for INT4, a
                             value outside the fp16 range)                     */
  QLIN_E_UNSUPPORTED = 5, /* a valid but unimplemented parameter combination   */
  QLIN_E_WORKSPACE = 6,   /* workspace NULL or smaller than qlin_workspace_bytes */
  QLIN_E_HIP = 7          /* the HIP runtime reported an error                 */
} qlin_status;

/* Packed weight formats. */
typedef enum {
  QLIN_FMT_NF4 = 1,        /* NormalFloat-4, blockwise absmax [QLoRA NF4, DQ]  */
  QLIN_FMT_INT4_GROUP = 2  /* asymmetric INT4, per-group fp16 scale and zero
                              [QA-LoRA abstract]                              */
} qlin_format;

/*
 * A packed 4-bit weight W[d_out][d_in] (read-only device memory).
 *
 * codes   uint8[d_out][d_in/2]: two 4-bit indices per byte along each row;
 *         every run of 8 elements of a row fills 4 bytes, and byte j of the
 *         run holds element j in its low nibble and element j + 4 in its
 *         high nibble (so one little-endian 32-bit word holds elements
 *         0..3 in its low nibbles and 4..7 in its high nibbles).
 * NF4 (block = 64): element (n, k) belongs to block b = (n*d_in + k)/64 (64
 *         consecutive elements of one row) and decodes to
 *             bf16( fl32( c[idx] * a_hat_b ) ),   ties-to-even,
 *         with c the 16 NF4 levels (qlin_nf4_codebook).
 *   dq_block = 0:   absmax = float[n_blocks], a_hat_b = absmax[b].
 *   dq_block = 256: absmax = int8[n_blocks] (values 0..127), absmax2 =
 *         float[ceil(n_blocks/256)] and
 *             step_g  = fl32( absmax2[g] * fl32(1/127) ),  g = b/256,
 *             a_hat_b = fl32( absmax[b] * step_g ).
 *         [QLoRA "Innovation 2: Double Quantization"]
 * INT4 (block = group = 32): scale, zero = fp16[d_out][d_in/32]; element
 *         (n, k) with q = its index decodes to
 *             bf16( fl32( scale[n][k/32] * q + zero[n][k/32] ) ).
 *         [QA-LoRA abstract: group-wise quantization]
 */
typedef struct {
  int32_t format;          /* qlin_format                                    */
  int32_t block;           /* NF4: 64; INT4: group size, 32                  */
  int32_t dq_block;        /* NF4: 256 or 0; INT4: 0                         */
  int32_t reserved;        /* must be 0                                      */
  int64_t d_out, d_in;     /* d_in % block == 0                              */
  const uint8_t *codes;    /* uint8[d_out][d_in/2]                           */
  const void *absmax;      /* NF4: int8[n_blocks] (dq) or float[n_blocks]    */
  const float *absmax2;    /* NF4 with dq: float[ceil(n_blocks/dq_block)]    */
  const uint16_t *scale;   /* INT4: fp16[d_out][d_in/group]                  */
  const uint16_t *zero;    /* INT4: fp16[d_out][d_in/group]                  */
} qlin_qweight;

/*
 * The 16 NF4 levels as fp32, ascending, into `out` (HOST memory).  Levels
 * sit at equally spaced probabilities of N(0, 1) on each side of an exact
 * zero (7 below, 8 above), with the outermost at probability 31/32, and are
 * normalised so that c[0] = -1, c[7] = 0, c[15] = +1.  Computed on the host
 * with the library's own inverse normal CDF; needs no GPU.
 * [QLoRA "Innovation 1: 4-bit NormalFloat (NF4)" and the code sketch's
 * quantile table]  Returns QLIN_E_NULL for out == NULL.
 */
int qlin_nf4_codebook(float out[16]);

/*
 * NF4 blockwise quantization with optional double quantization of the
 * absmax constants.  [QLoRA "Background: what is quantization?",
 * "Innovation 2: Double Quantization", "The same idea in code"]
 *
 *   W        fp32[d_out][d_in] (device, read only)
 *   block    must be 64;  d_in % 64 == 0;  d_out >= 1
 *   dq_block 256 (absmax int8[n_blocks], absmax2 float[ceil(n_blocks/256)])
 *            or 0 (absmax float[n_blocks]; absmax2 may be NULL)
 *   codes    uint8[d_out][d_in/2]  (output)
 *
 * Each element takes the index of the level nearest to w/absmax_b (exact
 * comparison; a tie goes to the lower index; an all-zero block encodes to
 * index 7 with absmax 0).  With dq_block = 256 each absmax becomes
 * round_half_even(127 * absmax_b / absmax2_g) and absmax2_g is the group's
 * fp32 maximum.  Synchronises `stream`; returns QLIN_E_NONFINITE if W holds
 * NaN or Inf (outputs are then unspecified).
 */
int qlin_quantize_nf4(const float *W, int64_t d_out, int64_t d_in, int32_t block,
                      int32_t dq_block, uint8_t *codes, void *absmax, float *absmax2,
                      hipStream_t stream);

/*
 * Group-wise asymmetric INT4 quantization.  [QA-LoRA abstract]
 *
 *   W      fp32[d_out][d_in] (device); group must be 32; d_in % 32 == 0
 *   codes  uint8[d_out][d_in/2]; scale, zero fp16[d_out][d_in/32] (outputs)
 *
 * Per (row, group): zero = fp16(min), scale = fp16(fl32(fl32(max-min)/15)),
 * q = 0 if scale == 0 else clamp(round_half_even(fl32(fl32(w-zero)/scale)), 0, 15).
 * Synchronises `stream`; QLIN_E_NONFINITE if W holds NaN/Inf or |w| > 65504.
 */
int qlin_quantize_int4_group(const float *W, int64_t d_out, int64_t d_in, int32_t group,
                             uint8_t *codes, uint16_t *scale, uint16_t *zero,
                             hipStream_t stream);

/*
 * Bytes of device workspace qlin_fwd / qlin_bwd need for this weight, token
 * count M, adapter rank r and pool.  The workspace must be zero-filled once
 * before its first use with the library; every completed call leaves its
 * synchronisation counters at zero again, so it can be reused as is.  Two
 * calls in flight at the same time must not share a workspace.  Returns 0
 * for invalid arguments.  Host only; needs no GPU.
 */
size_t qlin_workspace_bytes(const qlin_qweight *w, int64_t M, int32_t r, int32_t pool);

/*
 * Forward pass of the adapted layer.  [QLoRA "Background: how LoRA works",
 * "The QLoRA recipe" stage 3, "The same idea in code"; QA-LoRA abstract]
 *
 *   w      packed weight (see qlin_qweight)
 *   x      bf16[M][d_in];  1 <= M
 *   A      bf16[r][d_in/pool];  B bf16[d_out][r];  1 <= r <= 128
 *   s      adapter scale (any finite float; 0 disables the adapter term)
 *   pool   1 for a plain adapter, or the INT4 group size (32) for the
 *          QA-LoRA pooled adapter, whose input is the sum of each group of
 *          32 consecutive features of x
 *   y      bf16[M][d_out]  (output): x W_bf16^T + s u B^T, fp32 accumulate,
 *          one rounding to bf16 (ties to even)
 *   u_out  fp32[M][r] (output, may be NULL): u = P A^T, kept in fp32 so the
 *          backward pass can reuse it
 *   workspace, ws_bytes  >= qlin_workspace_bytes(w, M, r, pool)
 * Asynchronous on `stream`.
 */
int qlin_fwd(const qlin_qweight *w, const uint16_t *x, int64_t M, const uint16_t *A,
             const uint16_t *B, int32_t r, float s, int32_t pool, uint16_t *y, float *u_out,
             void *workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Backward pass: gradients of <dY, y> into the input and the adapter.  The
 * frozen weight gets none.  [QLoRA "The QLoRA recipe" stage 3 and the code
 * sketch's closing note; QA-LoRA abstract]
 *
 *   x, A, B, r, s, pool, w  as for qlin_fwd
 *   dy       bf16[M][d_out]
 *   u_saved  fp32[M][r] from qlin_fwd's u_out, or NULL to recompute it
 *   dx       bf16[M][d_in]   (output; NULL skips it)   dY W_bf16 + expand(du A)
 *   dA       bf16[r][d_in/pool] (output)                du^T P
 *   dB       bf16[d_out][r]  (output)                   s dY^T u
 * with du = s dY B held in fp32 inside the workspace.  Asynchronous.
 */
int qlin_bwd(const qlin_qweight *w, const uint16_t *x, int64_t M, const uint16_t *A,
             const uint16_t *B, int32_t r, float s, int32_t pool, const uint16_t *dy,
             const float *u_saved, uint16_t *dx, uint16_t *dA, uint16_t *dB, void *workspace,
             size_t ws_bytes, hipStream_t stream);

/*
 * Test helper: writes the dequantized weight W_bf16 (bf16[d_out][d_in]) using
 * the same in-register lookup-table decode as the fused kernels.  Never
 * called by qlin_fwd / qlin_bwd, which do not materialise W.  Asynchronous.
 */
int qlin_dequant_bf16(const qlin_qweight *w, uint16_t *W_out, hipStream_t stream);

/* Static, human-readable name of a status code (host only). */
const char *qlin_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_H_ */
