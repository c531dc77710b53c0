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
 *   - State the library keeps, per process: the quantizers' non-finite flag
 *     word (one per device; quantizer calls take turns on a mutex), the
 *     profiling hook (qlin_profile_next_launch) and the device array of
 *     qlin_fwd_noalloc.  Otherwise concurrent calls on different streams are
 *     safe provided they do not share a workspace.
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
  QLIN_FMT_INT4_GROUP = 2, /* asymmetric INT4, per-group fp16 scale and zero
                              [QA-LoRA abstract]                              */
  QLIN_FMT_NF = 3          /* NormalFloat-k, k = 2, 3 or 4 bits, blocks of 32,
                              64, 128 or 256, bit-plane codes [LQ-LoRA
                              abstract: bit-width and block size per matrix] */
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
 *         float[ceil(n_blocks/256)] and, with g = b/256,
 *             a_hat_b = RN32( absmax[b] * absmax2[g] / 127 ),
 *         the exact quotient rounded once to fp32 (ties to even), so a code
 *         of 127 reconstructs absmax2[g] itself.
 *         [QLoRA "Innovation 2: Double Quantization"]
 * INT4 (block = group = 32): scale, zero = fp16[d_out][d_in/32]; element
 *         (n, k) with q = its index decodes to
 *             bf16( fl32( scale[n][k/32] * q + zero[n][k/32] ) ).
 *         [QA-LoRA abstract: group-wise quantization]
 * NF (bits = k in 2..4, block in {32, 64, 128, 256}): codes =
 *         uint8[d_out][d_in*k/8] as bit planes: every run of 32 elements of
 *         a row fills k little-endian 32-bit words, word p holding bit p of
 *         element i in its bit i.  Element (n, k) belongs to block
 *         b = (n*d_in + k)/block and decodes to bf16(fl32(c[idx] * a_hat_b))
 *         with c the 2^k levels of qlin_nf_codebook(k) and a_hat_b as for
 *         NF4 (absmax, absmax2, dq_block 0 or 256).  qlin_fwd / qlin_bwd
 *         first transcode such a weight, on their stream, into their
 *         workspace (4-bit indices plus an fp32 scale per 32 elements:
 *         d_in*d_out*(1/2 + 1/8) bytes), then run the same kernels.
 *         [LQ-LoRA abstract; QLoRA "Innovation 1", "Innovation 2"]
 */
typedef struct {
  int32_t format;          /* qlin_format                                    */
  int32_t block;           /* NF4: 64; INT4: group size, 32; NF: 32..256     */
  int32_t dq_block;        /* NF4: 256 or 0; INT4: 0                         */
  int32_t bits;            /* NF: 2, 3 or 4; NF4 and INT4: 0                 */
  int64_t d_out, d_in;     /* d_out % 16 == 0; d_in % 64 == 0 (both formats) */
  const uint8_t *codes;    /* uint8[d_out][d_in/2] (NF: [d_out][d_in*bits/8]) */
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
 *   block    must be 64;  d_in % 64 == 0;  d_out % 16 == 0 (the shapes
 *            qlin_fwd / qlin_bwd accept)
 *   dq_block 256 (absmax int8[n_blocks], absmax2 float[ceil(n_blocks/256)])
 *            or 0 (absmax float[n_blocks]; absmax2 may be NULL)
 *   codes    uint8[d_out][d_in/2]  (output)
 *
 * Each element takes the index of the level nearest to w/absmax_b (exact
 * comparison; a tie goes to the lower index; an all-zero block encodes to
 * index 7 with absmax 0).  With dq_block = 256 each absmax becomes
 * round_half_even(127 * absmax_b / absmax2_g) and absmax2_g is the group's
 * fp32 maximum.  Synchronises `stream`; returns QLIN_E_NONFINITE if W holds
 * NaN or Inf (outputs are then unspecified).  Non-finite input is detected
 * on the GPU and reported through one flag word per device that the
 * library owns; quantizer calls of one process therefore run one at a time
 * (a host mutex), and only the flag word crosses back to the host.
 */
int qlin_quantize_nf4(const float *W, int64_t d_out, int64_t d_in, int32_t block,
                      int32_t dq_block, uint8_t *codes, void *absmax, float *absmax2,
                      hipStream_t stream);

/*
 * The 2^bits NormalFloat levels (bits = 2, 3, 4) as fp32, ascending, into
 * `out` (HOST memory, 2^bits floats): the NF4 construction with 2^(bits-1)
 * levels above and 2^(bits-1) - 1 below an exact zero, the outermost at
 * probability 1 - 1/2^(bits+1); bits = 4 gives qlin_nf4_codebook's levels.
 * [QLoRA "Innovation 1: 4-bit NormalFloat (NF4)"; LQ-LoRA abstract]
 * QLIN_E_NULL for out == NULL, QLIN_E_UNSUPPORTED for other bit counts.
 */
int qlin_nf_codebook(int32_t bits, float *out);

/*
 * NormalFloat-k blockwise quantization (format QLIN_FMT_NF).  [LQ-LoRA
 * abstract: per-matrix bit-width and block size; QLoRA "Background: what is
 * quantization?", "Innovation 2: Double Quantization"]
 *
 *   W        fp32[d_out][d_in] (device);  d_out % 16 == 0; d_in % 64 == 0
 *            and d_in % block == 0
 *   bits     2, 3 or 4;  block 32, 64, 128 or 256;  dq_block 0 or 256
 *   codes    uint8[d_out][d_in*bits/8] bit planes (output);  absmax and
 *            absmax2 as for qlin_quantize_nf4 with n_blocks = d_out*d_in/block
 *
 * Same rules as qlin_quantize_nf4 with the 2^bits levels of
 * qlin_nf_codebook(bits): nearest level of w/absmax_b (exact comparison,
 * ties to the lower index, an all-zero block to the zero level), 8-bit
 * double quantization of the constants.  Synchronous; QLIN_E_NONFINITE as
 * for qlin_quantize_nf4.
 */
int qlin_quantize_nf(const float *W, int64_t d_out, int64_t d_in, int32_t bits, int32_t block,
                     int32_t dq_block, uint8_t *codes, void *absmax, float *absmax2,
                     hipStream_t stream);

/*
 * Group-wise asymmetric INT4 quantization.  [QA-LoRA abstract]
 *
 *   W      fp32[d_out][d_in] (device); group must be 32; d_in % 64 == 0 and
 *          d_out % 16 == 0 (the shapes qlin_fwd / qlin_bwd accept)
 *   codes  uint8[d_out][d_in/2]; scale, zero fp16[d_out][d_in/32] (outputs)
 *
 * Per (row, group), with every rounding taken on the exact real value:
 *   zero  = RN16(min),   scale = RN16((max - min) / 15),
 *   q     = clamp(round_half_even((w - zero) / scale), 0, 15), 0 if scale == 0.
 * Synchronises `stream`; QLIN_E_NONFINITE if W holds NaN/Inf or |w| > 65504
 * (reported as for qlin_quantize_nf4, through the device flag word).
 */
int qlin_quantize_int4_group(const float *W, int64_t d_out, int64_t d_in, int32_t group,
                             uint8_t *codes, uint16_t *scale, uint16_t *zero,
                             hipStream_t stream);

/*
 * Low-rank plus quantized decomposition W ~ Q + B A of an fp32 weight, with
 * Q an NF4 weight (blocks of 64) and B A of rank r.  [LQ-LoRA record,
 * abstract: each pretrained matrix is split iteratively into a quantized
 * component and a high-precision low-rank component; only the latter is
 * trained]
 *
 *   W        fp32[d_out][d_in] (device); shapes as for qlin_quantize_nf4
 *   r        rank, 0 .. 128 (and <= d_out, d_in); 0 gives plain NF4
 *   iters    alternations, >= 1;  power: subspace-iteration steps, >= 0
 *   omega_t  fp32[r][d_in] (device): start of the subspace iteration, drawn
 *            by the caller (NULL when r == 0)
 *   dq_block 0 or 256;  codes, absmax, absmax2: outputs as for
 *            qlin_quantize_nf4
 *   B_out    bf16[d_out][r], A_out bf16[r][d_in] (device outputs; NULL when
 *            r == 0): the layer's adapter with s = 1
 *   err_out  fp32[iters] (device) or NULL: ||W - W_bf16(Q_t) - L_t|| / ||W||
 *            (Frobenius) after each iteration
 *   workspace, ws_bytes: device memory of qlin_lq_workspace_bytes bytes
 *
 * L_0 = 0.  Iteration t: Q_t = NF4(W - L_{t-1}) (the qlin_quantize_nf4
 * rules on the fp32 difference); R = W - W_bf16(Q_t); U = the Q factor of
 * the thin QR (positive diagonal) of R Omega, then `power` times
 * V = QR(R^T U), U = QR(R V); L_t = U (U^T R).  B = U and A = U^T R of the
 * last iteration, rounded to bf16.  All arithmetic is fp32 on the device
 * (the small r x r Cholesky factorisations in fp64).  Synchronises `stream`
 * (once per iteration and at the end); QLIN_E_NONFINITE as for
 * qlin_quantize_nf4; QLIN_E_WORKSPACE if the workspace is too small.
 */
size_t qlin_lq_workspace_bytes(int64_t d_out, int64_t d_in, int32_t r);
int qlin_lq_nf4(const float *W, int64_t d_out, int64_t d_in, int32_t r, int32_t iters, int32_t power,
                const float *omega_t, int32_t dq_block, uint8_t *codes, void *absmax, float *absmax2,
                uint16_t *B_out, uint16_t *A_out, float *err_out, void *workspace, size_t ws_bytes,
                hipStream_t stream);

/*
 * Bytes of device workspace qlin_fwd / qlin_bwd need for this weight, token
 * count M, adapter rank r and pool.  The first 64 KiB of every workspace hold
 * the ticket counters of the split reductions; the workspace must be
 * zero-filled once before its first use with the library.  Every completed
 * call leaves the counters at zero and no call writes anything else into
 * those 64 KiB, so one workspace can be reused by later calls of any shape
 * (given enough bytes).  Two calls in flight at the same time must not share
 * a workspace.  Returns 0 for invalid arguments, and for shapes whose split
 * reductions would need more than 16384 counters (d_in > 2 097 152 or d_out
 * > 262 144 at M <= 16).  Host only; needs no GPU.
 */
size_t qlin_workspace_bytes(const qlin_qweight *w, int64_t M, int32_t r, int32_t pool);

/*
 * Forward pass of the adapted layer.  [QLoRA "Background: how LoRA works",
 * "The QLoRA recipe" stage 3, "The same idea in code"; QA-LoRA abstract]
 *
 *   w      packed weight (see qlin_qweight: d_out % 16 == 0, d_in % 64 == 0)
 *   x      bf16[M][d_in];  1 <= M
 *   A      bf16[r][d_in/pool];  B bf16[d_out][r];  0 <= r <= 128; r = 0 is
 *          the layer without an adapter (A, B may be NULL, u_out must be
 *          NULL), e.g. an INT4 weight whose adapter qlin_qa_merge folded in
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
 * Forward pass that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, or
 * harnesses that forbid hipMalloc.  Same arguments and results as qlin_fwd
 * (bit-identical: the same kernels), without the workspace: the library
 * uses its own 64 MiB device array (one per GPU it runs on, held until the
 * process ends) for ticket counters, u and split partial sums.
 *   - Returns QLIN_E_WORKSPACE, before any HIP call, when the layer needs
 *     more than that array holds (64 KiB of counters + M*r*4 bytes of u +
 *     the forward's split partials; e.g. the 4096 x 11008 INT4 layer at
 *     M = 2048 does not fit, every few-token layer does).
 *   - The first call on each GPU looks up the array's device address and
 *     zeroes its counters with a kernel on `stream`; make that first call
 *     outside graph capture.  Every completed call leaves the counters at
 *     zero again.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (different streams, or threads) race and must not be
 *     issued.
 * Asynchronous on `stream`.
 */
int qlin_fwd_noalloc(const qlin_qweight *w, const uint16_t *x, int64_t M, const uint16_t *A,
                     const uint16_t *B, int32_t r, float s, int32_t pool, uint16_t *y,
                     float *u_out, hipStream_t stream);

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
 * QA-LoRA merge: folds a trained pooled adapter into the INT4 zero points,
 * so that the quantized layer alone computes the adapted layer.  [QA-LoRA
 * abstract, point (ii)]  With the adapter acting on the sum of each group of
 * 32 inputs, s (P A^T) B^T adds s (B A)[n][g] to every weight of group g in
 * row n, i.e. shifts that group's additive zero point:
 *     zero_out[n][g] = RN16( zero[n][g] + s * sum_j B[n][j] A[j][g] ),
 * the exact sum rounded once to fp16 (ties to even; exact whenever the
 * terms span fewer than ~99 bits).  Then qlin_fwd(merged weight, r = 0)
 * equals qlin_fwd(original, adapter, pool = 32) up to that fp16 rounding.
 *
 *   w         INT4 weight (QLIN_FMT_INT4_GROUP, group 32); its zero is read
 *   A         bf16[r][d_in/32];  B bf16[d_out][r];  1 <= r <= 128; s finite
 *   zero_out  fp16[d_out][d_in/32] (output; may be w->zero itself)
 * Asynchronous on `stream`.
 */
int qlin_qa_merge(const qlin_qweight *w, const uint16_t *A, const uint16_t *B, int32_t r,
                  float s, uint16_t *zero_out, hipStream_t stream);

/*
 * Gradients of the INT4 group scales and zero points, for fine-tuning them
 * as parameters.  [LoQA abstract: scale and zero point fine-tuned through a
 * LoRA-compatible operator; QA-LoRA abstract for the INT4 groups]  With
 * W[n][k] = scale[n][g] q[n][k] + zero[n][g] (g = k/32) and y = x W^T, the
 * gradients of <dY, y>, the bf16 rounding of W passed straight through:
 *     dscale[n][g] = sum_{k in g} q[n][k] dW[n][k],
 *     dzero[n][g]  = sum_{k in g} dW[n][k],          dW = dY^T x,
 * dW formed by bf16 MFMAs with fp32 accumulation, tile by tile, never
 * stored.  (The page gives no formula: this is the plain reading.)
 *
 *   w        INT4 weight (QLIN_FMT_INT4_GROUP, group 32); its codes are read
 *   x        bf16[M][d_in];  dy bf16[M][d_out];  1 <= M
 *   dscale, dzero  fp32[d_out][d_in/32] (outputs)
 * Asynchronous on `stream`.
 */
int qlin_int4_scale_zero_grad(const qlin_qweight *w, const uint16_t *x, int64_t M,
                              const uint16_t *dy, float *dscale, float *dzero,
                              hipStream_t stream);

/*
 * Test helper: writes the dequantized weight W_bf16 (bf16[d_out][d_in]) using
 * the same in-register lookup-table decode as the fused kernels.  Never
 * called by qlin_fwd / qlin_bwd, which do not materialise W.  Asynchronous.
 */
int qlin_dequant_bf16(const qlin_qweight *w, uint16_t *W_out, hipStream_t stream);

/*
 * Profiling aid; takes no part in the computation.  Arms a one-shot hook:
 * the next launch of the kernel named `kernel` made by any qlin_* call of
 * this process records `start` on that call's stream just before the launch
 * and `stop` just after it, and the hook disarms itself.  Kernel names:
 * "k_gemv_fwd", "k_fwd_gemm" (forward products), "k_gemv_dx", "k_dx_gemm"
 * (input gradient), "k_nt_skinny", "k_tn2", "k_split_hl", "k_transpose16",
 * "k_qa_pool_u", "k_qa_dA" (adapter products), "k_int4_scale_zero_grad".  `start` and `stop` are HIP
 * events created by the caller; the elapsed time between them is the
 * kernel's duration on the device.  kernel = NULL disarms.  One hook per
 * process (a later call replaces an armed one).  Host only; QLIN_E_NULL for
 * a missing event, QLIN_E_SHAPE for a name of 64 or more characters.
 */
int qlin_profile_next_launch(const char *kernel, hipEvent_t start, hipEvent_t stop);

/* Static, human-readable name of a status code (host only). */
const char *qlin_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_H_ */
