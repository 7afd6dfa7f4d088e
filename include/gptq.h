/*
 * gptq.h -- C ABI of the MI355X (gfx950) GPTQ layer-quantization library.
 *
 * GPTQ quantizes one linear layer at a time with second-order error
 * compensation.  The three calls below are its three stages:
 *
 *   gptq_hessian_accumulate  H += 2 X X^T from calibration activations
 *   gptq_prepare_hinv        damp H and take the upper Cholesky factor U of
 *                            the damped inverse
 *   gptq_quantize_layer      sweep the columns of W in blocks, rounding each
 *                            column, compensating later columns from the rows
 *                            of U, and emitting packed codes, scales and zeros
 *
 * OBQ's greedy-order alternative to the sweep, for small layers:
 *
 *   gptq_quantize_greedy     per row, quantize the weight whose rounding adds
 *                            the least loss, compensate, and downdate that
 *                            row's own copy of the inverse Hessian
 *
 * one call that uses the packed result at run time:
 *
 *   gptq_dequant_matmul      Y = X What^T with the packed codes unpacked and
 *                            dequantized next to 16-bit activations
 *                            (gptq_dequant_matmul_static: the same without a
 *                            workspace, for callers that cannot allocate)
 *
 * and one that prepares a layer for it with a fixed rotation:
 *
 *   gptq_rotate_hadamard     M <- M R (block-diagonal Hadamard), applied to
 *                            the weights and the activations alike
 *
 * and the steps of the network-level loop over transformer blocks that are
 * not products:
 *
 *   gptq_attention, gptq_swiglu, gptq_residual_add
 *
 * Sources (web pages describing the method):
 *   [OBQ]    "Part 2: Adaptive Rounding: Optimal Brain Quantizer (OBQ)"
 *   [GPTQ]   "Part 3: Adaptive Rounding: GPTQ"
 *   [SOQ]    the English post on GPTQ second-order quantization
 *            (hungho77.github.io) and [SOQ-vi], its Vietnamese edition.
 *
 * Conventions for every call:
 *   - Array arguments are DEVICE pointers owned by the caller; the library
 *     allocates no memory and keeps no state between calls.  Scratch memory
 *     is passed in as `workspace`, sized by the matching *_workspace_bytes()
 *     (gptq_dequant_matmul_static alone uses a fixed buffer of its own).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work on it and return without synchronizing.
 *   - Matrices are row-major with an explicit leading dimension.
 *   - Argument errors are detected on the host, before any HIP call, and
 *     returned synchronously; nothing is enqueued then.  Launch failures
 *     return GPTQ_ERR_HIP.  Numerical failure of the factorization is
 *     reported through the device-side `info` word (see gptq_prepare_hinv).
 *   - Concurrent calls on distinct buffers and workspaces are safe.
 *   - NaN or Inf inputs give unspecified (but memory-safe) outputs.
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPTQ_OK = 0,
  GPTQ_ERR_INVALID_ARG = 1,  /* bad size, pointer, dtype, bits, group/block */
  GPTQ_ERR_UNSUPPORTED = 2,  /* valid request this library does not run    */
  GPTQ_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than required     */
  GPTQ_ERR_HIP = 4,          /* a HIP launch or runtime call failed         */
  GPTQ_ERR_SCRATCH_LIMIT = 5 /* needs more than the fixed scratch buffer of
                                gptq_dequant_matmul_static                 */
} gptq_status;

typedef enum { GPTQ_F16 = 0, GPTQ_BF16 = 1, GPTQ_F32 = 2 } gptq_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* gptq_status_string(int32_t status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t gptq_version(void);

/* ------------------------------------------------------------------------
 * Stage 1: Hessian accumulation.
 *
 * Defines H = 2 X X^T, the Hessian of the layer objective ||WX - What X||^2
 * ([SOQ] "The objective is layer output, not weight distance"; [OBQ]
 * "Goal": the input covariance is the proxy Hessian).
 *
 *   H        [n x n] float32, row-major, leading dimension n.  In/out:
 *            H <- H + 2 * sum_t x_t x_t^T over the `tokens` rows of X.
 *            The caller zeroes H before the first call and may call again
 *            for further token chunks; both triangles are valid (and exactly
 *            symmetric) after every call.
 *   X        [tokens x n] activations, token-major (one token per row),
 *            leading dimension ldx >= n, element type x_dtype (fp16, bf16 or
 *            fp32).  Products of fp16/bf16 inputs are exact in fp32; sums
 *            are fp32 in a fixed order, so results are deterministic.
 *   tokens   >= 0 (0 is a no-op).
 *   workspace, ws_bytes: at least gptq_hessian_workspace_bytes(n, tokens).
 * Errors: n < 1, ldx < n, tokens < 0, NULL H/X (tokens > 0), unknown dtype
 * -> GPTQ_ERR_INVALID_ARG; short workspace -> GPTQ_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t gptq_hessian_workspace_bytes(int64_t n, int64_t tokens);
gptq_status gptq_hessian_accumulate(float* H, int64_t n, const void* X, int32_t x_dtype,
                                    int64_t tokens, int64_t ldx,
                                    void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stage 2+3: damping and the inverse-Hessian factor.
 *
 * lambda = damp * mean(diag H) ([SOQ] "3. Cholesky reformulation": about one
 * percent of the average Hessian diagonal; [GPTQ] "Algorithm GPTQ":
 * H + lambda I), then U upper-triangular with (H + lambda I)^{-1} = U^T U
 * ([GPTQ] "Observation 3: The Cholesky Reformulation": factor the inverse
 * once and read its rows; [SOQ-vi] writes the flush with rows R[B, B:] of
 * this upper factor).
 *
 *   H          [n x n] float32 symmetric (both triangles read), leading
 *              dimension n.  Not modified unless U == H (in-place allowed).
 *   damp       relative damping (>= 0), 0.01 for the usual one percent.
 *   U          [n x n] float32 out, leading dimension n; strictly lower part
 *              written as 0.
 *   info       device int32 out: 0 on success; k > 0 if H + lambda I is not
 *              positive definite (numerically), k being the 1-based column
 *              at which the factorization (which runs from the last column
 *              towards the first) broke down.  U is undefined when k > 0.
 *   lambda_out device float32 out: the lambda used.
 *   workspace, ws_bytes: at least gptq_prepare_workspace_bytes(n).
 * Errors: n < 1, damp < 0 or not finite, NULL pointers ->
 * GPTQ_ERR_INVALID_ARG; short workspace -> GPTQ_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t gptq_prepare_workspace_bytes(int64_t n);
gptq_status gptq_prepare_hinv(const float* H, int64_t n, float damp, float* U,
                              int32_t* info, float* lambda_out,
                              void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stage 4: the blocked column sweep with lazy trailing updates.
 *
 * [GPTQ] "Algorithm GPTQ" and "Observation 2: Lazy Batch Updates";
 * [SOQ-vi] "Lazy batch update".  Columns are swept left to right
 * ([GPTQ] "Observation 1").  For each column p, all rows at once:
 *   at the first column of a group: s, z from the current values of the
 *     group: x_lo = min(0, min), x_hi = max(0, max) (x_hi = 1 if both are 0),
 *     s = (x_hi - x_lo)/maxq, z = rint(-x_lo/s), maxq = 2^bits - 1;
 *     per-row mode takes them once from the original row;
 *   q = clamp(rint(v/s) + z, 0, maxq), what = s (q - z);
 *   e = (v - what)/U[p][p];  later columns of the block v_j -= e U[p][j];
 * and the block's errors reach the later columns as V[:, i2:] -= E U[i:i2, i2:]
 * before those columns are swept (the library may apply the errors of two
 * consecutive blocks, or of a 1024-column superblock, in one product; the
 * result differs only in the order of floating-point sums).  Working
 * precision: V and E in float32; for rows of at most 16384 columns, when
 * block_size is a multiple of 64, n a multiple of 4 and the groups fit
 * inside a block (or scales are per row), the products past a pair of
 * blocks or a superblock (K a multiple of 64) take E and U split into
 * bf16 hi and lo parts, E_hi U_hi + E_hi U_lo + E_lo U_hi accumulated in
 * float32 (about 16 bits of every term); otherwise float32 products.
 *
 *   W          [m x n] weights, leading dimension ldw >= n, type w_dtype.
 *              Read; if write_dequant != 0, overwritten by what = s(q - z)
 *              (rounded to w_dtype).
 *   U          [n x n] float32 from gptq_prepare_hinv (only the upper
 *              triangle is read), leading dimension n.
 *   bits       2..8.
 *   group_size <= 0: one (s, z) per row; else g >= 1 with
 *              g % block_size == 0 or block_size % g == 0.
 *   block_size 1..128 (B).  Results do not depend on B except through the
 *              order of floating-point sums.
 *   qcodes     [m x ceil(n*bits/32)] uint32 out: per row a little-endian
 *              bit-stream, code j at bits [j*bits, (j+1)*bits) from bit 0 of
 *              the row's first word (a code may straddle two words; unused
 *              high bits of the last word are 0).
 *   scales     [m x G] float32 out, zeros [m x G] int32 out, G = 1 per-row,
 *              else ceil(n / group_size).
 *   err_sq     optional [m] float32 out (NULL to skip): sum_p e_p^2 per row.
 *   workspace, ws_bytes: at least gptq_quantize_workspace_bytes(m, n, block_size)
 *              (for n <= 16384 it includes 4 n^2 bytes for the split factor).
 * Errors: m < 1, n < 1, ldw < n, bits outside 2..8, block_size outside
 * 1..128, group/block not nesting, NULL required pointers, unknown dtype ->
 * GPTQ_ERR_INVALID_ARG; short workspace -> GPTQ_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t gptq_quantize_workspace_bytes(int64_t m, int64_t n, int64_t block_size);
gptq_status gptq_quantize_layer(void* W, int32_t w_dtype, int64_t m, int64_t n, int64_t ldw,
                                const float* U, int32_t bits, int64_t group_size,
                                int64_t block_size, uint32_t* qcodes, float* scales,
                                int32_t* zeros, float* err_sq, int32_t write_dequant,
                                void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * gptq_quantize_greedy: OBQ's greedy-order quantization of W against the
 * same factor U ([OBQ] "Greedy Search"; "The OBS / GPTQ Trick" for the
 * rank-one downdate of H^-1; "Generalized Weight Update" for the
 * compensation).
 *
 * Each row runs on its own copy of H^-1 = U^T U.  At every step the row's
 * unquantized weight with the smallest dL_p = (what_p - w_p)^2 / [H^-1]_pp
 * (equal scores: the smaller column) is rounded on its group's grid, the other
 * unquantized weights move by (what_p - w_p) [H^-1]_{p,k} / [H^-1]_pp, and
 * weight p leaves H^-1 by H^-1 - H^-1_{:,p} H^-1_{p,:} / [H^-1]_pp.  Since
 * the order jumps across groups, every group's grid (s, z, the quantizer of
 * gptq_quantize_layer) is taken once from the ORIGINAL row.  Work per row is
 * about n^3/3 flops against n^2 for the sweep ([OBQ] "Limitations of OBQ"),
 * so this is for small layers.
 *
 *   W          [m x n] weights (read only), leading dimension ldw >= n,
 *              w_dtype GPTQ_F16 / GPTQ_BF16 / GPTQ_F32.
 *   U          [n x n] float32 upper factor from gptq_prepare_hinv.
 *   bits       2..8.  group_size <= 0: one grid per row; else groups of
 *              group_size columns (the last may be short).
 *   qcodes, scales, zeros: outputs in the layout of gptq_quantize_layer.
 *   order      [m x n] int32 out, optional (NULL): the column quantized at
 *              each step.
 *   loss       [m] float32 out, optional (NULL): the sum of the chosen dL_p,
 *              which equals (w - what)^T H_d (w - what) for the row.
 *   workspace, ws_bytes: at least gptq_quantize_greedy_workspace_bytes(m, n)
 *              bytes (the packed H^-1, and for n > 256 one packed copy per
 *              resident workgroup, at most 256).
 * This version runs n <= 4096 and group_size <= 0 or >= 16; other valid
 * requests return GPTQ_ERR_UNSUPPORTED.  Bad sizes, bits, dtype or NULL
 * required pointers -> GPTQ_ERR_INVALID_ARG; short workspace ->
 * GPTQ_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t gptq_quantize_greedy_workspace_bytes(int64_t m, int64_t n);
gptq_status gptq_quantize_greedy(const void* W, int32_t w_dtype, int64_t m, int64_t n, int64_t ldw,
                                 const float* U, int32_t bits, int64_t group_size, uint32_t* qcodes,
                                 float* scales, int32_t* zeros, int32_t* order, float* loss,
                                 void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * gptq_dequant_matmul: Y = X What^T with What = s (q - z) taken from a packed
 * layer (the codes, scales and zeros gptq_quantize_layer wrote).
 *
 * The weight-only runtime path: activations stay 16-bit and the packed
 * weights are unpacked and dequantized on the fly, so far fewer weight bytes
 * cross HBM ([SOQ] "What the original results established"; [SOQ-vi], closing
 * paragraph: the artifact needs a packed INT4 kernel for the target device).
 * Sums are taken in fp32 with the zero points folded out of the products:
 * per group, s (sum_c (q_c + b) x_c - (z + b) sum_c x_c) for a constant b,
 * every product exact in fp32; Y is rounded once to x_dtype.
 *
 *   X          [tokens x n] activations, leading dimension ldx >= n
 *              (ldx % 8 == 0, X 16-byte aligned), x_dtype GPTQ_F16 or GPTQ_BF16.
 *   qcodes     [m x ceil(n*bits/32)] uint32, the packed layout of
 *              gptq_quantize_layer (16-byte aligned).
 *   scales     [m x G] float32, zeros [m x G] int32 (G as for
 *              gptq_quantize_layer).
 *   bits, group_size: as passed to gptq_quantize_layer.  This version runs
 *              bits == 4 and bits == 3 (any number of tokens), with
 *              n % 32 == 0 and group_size <= 0 (per row) or a multiple of
 *              128; other valid combinations return GPTQ_ERR_UNSUPPORTED.
 *   Y          [tokens x m] out, leading dimension ldy >= m, type x_dtype.
 *   workspace, ws_bytes: at least gptq_dequant_matmul_workspace_bytes(tokens,
 *              m, n) bytes (0 for shapes that need no partial sums; then
 *              workspace may be NULL).
 * tokens == 0 is a no-op.  The result does not depend on the launch shape
 * chosen for (tokens, m, n) except through the order of fp32 sums.
 * Errors: m < 1, n < 1, tokens < 0, ldx < n, ldy < m, bits outside 2..8,
 * x_dtype not 16-bit, NULL required pointers -> GPTQ_ERR_INVALID_ARG; the
 * cases above -> GPTQ_ERR_UNSUPPORTED; short workspace -> GPTQ_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t gptq_dequant_matmul_workspace_bytes(int64_t tokens, int64_t m, int64_t n);
gptq_status gptq_dequant_matmul(const void* X, int32_t x_dtype, int64_t tokens, int64_t ldx,
                                const uint32_t* qcodes, const float* scales, const int32_t* zeros,
                                int64_t m, int64_t n, int32_t bits, int64_t group_size, void* Y,
                                int64_t ldy, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * gptq_dequant_matmul_static: gptq_dequant_matmul without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc).
 *
 * Arguments, results, errors and supported cases are those of
 * gptq_dequant_matmul.  The fp32 partial sums of the K ranges go to a fixed
 * buffer inside the library instead: gptq_static_scratch_bytes() bytes
 * (32 MiB) per GPU, reserved when the library is loaded on that GPU and held
 * until the process ends.  Nothing is allocated by the call.
 *   - A request whose gptq_dequant_matmul_workspace_bytes(tokens, m, n)
 *     exceeds that size returns GPTQ_ERR_SCRATCH_LIMIT (nothing enqueued);
 *     e.g. 16 tokens with m x (number of 1024-column K ranges) up to 131072.
 *   - Every call on one GPU uses the same buffer, and the buffer keeps the
 *     last call's partial sums (each call writes every partial it reads, so
 *     nothing needs clearing).  Calls that overlap in time on one GPU (two
 *     streams, or two host threads) race on it and give wrong results: the
 *     caller serializes them, e.g. on one stream.
 *   - The first call on a GPU looks up the buffer's device address (a host
 *     call, no allocation); later calls reuse it.
 * ---------------------------------------------------------------------- */
size_t gptq_static_scratch_bytes(void);
gptq_status gptq_dequant_matmul_static(const void* X, int32_t x_dtype, int64_t tokens, int64_t ldx,
                                       const uint32_t* qcodes, const float* scales, const int32_t* zeros,
                                       int64_t m, int64_t n, int32_t bits, int64_t group_size, void* Y,
                                       int64_t ldy, void* stream);

/* ------------------------------------------------------------------------
 * Fixed rotation before GPTQ ("OptRot: Mitigating Weight Outliers via
 * Data-Free Rotations for Post-Training Quantization", abstract and Figure 1:
 * a rotation that folds into the previous layer, applied to spread weight
 * outliers; the Hadamard rotation is its baseline).
 *
 * gptq_rotate_hadamard: M <- M R in place, R = blockdiag(H_b, ..., H_b) /
 * sqrt(b), H_b the Sylvester-ordered Hadamard matrix of order b
 * (H_2k = [[H_k, H_k], [H_k, -H_k]]).  Rotate both the weights (W' = W R)
 * and the calibration activations (X' = X R): X' W'^T = X W^T and
 * H' = 2 X'^T X' = R^T H R, so gptq_hessian_accumulate on X' and
 * gptq_quantize_layer on W' quantize the rotated layer, whose run-time input
 * is X R.  Computed in fp32, rounded once to M's dtype.
 *   M       [rows x ld] device, row-major, 16-byte aligned; dtype
 *           GPTQ_F16/BF16/F32; columns [0, n) are rotated, the rest untouched.
 *   rows    >= 0 (0 is a no-op).
 *   n       row length, a multiple of b.
 *   ld      >= n; a multiple of 8 (16-bit) or 4 (fp32) elements.
 *   block   b: a power of two, 16 <= b <= 4096, dividing n; 0 takes the
 *           largest power of two dividing n (at most 4096).
 * Errors: rows < 0, n < 1, ld < n, unknown dtype, block < 0, block not a
 * power of two or not dividing n, NULL M (rows > 0) -> GPTQ_ERR_INVALID_ARG;
 * b < 16 or > 4096, misaligned M or ld -> GPTQ_ERR_UNSUPPORTED.
 * ---------------------------------------------------------------------- */
gptq_status gptq_rotate_hadamard(void* M, int32_t dtype, int64_t rows, int64_t n, int64_t ld,
                                 int64_t block, void* stream);

/* ------------------------------------------------------------------------
 * The network-level loop ("Part 3: Adaptive Rounding: GPTQ", 'Algorithm
 * GPTQ': one layer at a time, each layer's calibration inputs collected from
 * the network as quantized so far; [SOQ] 'Calibration for a multimodal or VLA
 * backbone': later blocks see activations already changed by the earlier
 * quantized blocks).  Over MLP blocks x <- x + W_down (silu(W_gate x) *
 * (W_up x)) the products run in gptq_dequant_matmul; these two calls do the
 * elementwise rest, in fp32 with one rounding to the activations' dtype.
 *
 * gptq_swiglu:       A = silu(G) * Uo, silu(v) = v / (1 + e^-v).
 * gptq_residual_add: X <- X + Y.
 *   G, Uo, A / X, Y  [tokens x f] (resp. [tokens x d]) device, row-major with
 *                    the common leading dimension ld >= f (d); dtype
 *                    GPTQ_F16 or GPTQ_BF16.  A may alias G or Uo.
 * tokens == 0 is a no-op.  Errors: tokens < 0, f (d) < 1, ld too small,
 * dtype not 16-bit, NULL pointers (tokens > 0) -> GPTQ_ERR_INVALID_ARG.
 * ---------------------------------------------------------------------- */
gptq_status gptq_swiglu(const void* G, const void* Uo, void* A, int32_t dtype, int64_t tokens,
                        int64_t f, int64_t ld, void* stream);
gptq_status gptq_residual_add(void* X, const void* Y, int32_t dtype, int64_t tokens, int64_t d,
                              int64_t ld, void* stream);

/* ------------------------------------------------------------------------
 * gptq_attention: the attention of a transformer block in the network-level
 * loop, between its quantized q/k/v and o projections ("Part 3: Adaptive
 * Rounding: GPTQ", 'Algorithm GPTQ': each layer's calibration inputs are
 * computed by the network as quantized so far).  Causal multi-head softmax
 * attention over sequences of seq_len consecutive tokens:
 *   O[i, h] = sum_{j <= i in i's sequence} softmax_j(Q[i,h] . K[j,h] / sqrt(dh)) V[j,h]
 * with head h the columns [h dh, (h + 1) dh).  fp32 arithmetic, one rounding
 * of O to dtype.
 *   Q, K, V, O  [tokens x heads * head_dim] device, row-major, common leading
 *               dimension ld >= heads * head_dim; dtype GPTQ_F16 or
 *               GPTQ_BF16.  O must not alias Q, K or V.
 *   tokens      a multiple of seq_len (0 is a no-op).
 * This version runs head_dim 64 or 128, seq_len a multiple of 64, ld % 8 == 0
 * and 16-byte aligned pointers; other valid requests return
 * GPTQ_ERR_UNSUPPORTED.  Errors: tokens < 0 or not a multiple of seq_len,
 * seq_len / heads / head_dim < 1, ld too small, dtype not 16-bit, NULL
 * pointers (tokens > 0) -> GPTQ_ERR_INVALID_ARG.
 * ---------------------------------------------------------------------- */
gptq_status gptq_attention(const void* Q, const void* K, const void* V, void* O, int32_t dtype,
                           int64_t tokens, int64_t seq_len, int64_t heads, int64_t head_dim,
                           int64_t ld, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
