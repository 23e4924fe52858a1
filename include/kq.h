/*
 * kq.h — C ABI of the KronQ per-layer quantization solver on AMD Instinct MI355X (gfx950).
 *
 * The solver follows the KronQ method (paper review page "KronQ: LLM Quantization via
 * Kronecker-Factored Hessian", sections Background, Method, Key idea; KronQ abstract on the
 * Hugging Face paper page): under the Kronecker-factored Hessian H ~ H_X (x) H_G the layer loss
 * is tr(H_G dW H_X dW^T); bidirectional incoherence processing rotates the input side with a
 * random-sign Hadamard matrix and the output side with a rotation applied after H_G^{1/2}, which
 * turns the loss into a plain GPTQ loss so that the unchanged GPTQ column sweep applies; a
 * per-sublayer score tr(H_G) tr(H_X) drives mixed-precision bit allocation.
 *
 * Conventions shared by every call
 *  - W is o x i (row r = output channel), X is n x i, H_X is i x i, H_G is o x o (or a diagonal,
 *    or o/blk dense blk x blk blocks). All matrices are row-major with a leading dimension
 *    (elements) >= the row length; leading dimensions and base pointers must be multiples of
 *    4 elements / 16 bytes.
 *  - Every pointer is a DEVICE pointer unless stated otherwise. The caller owns every buffer; the
 *    library never allocates device memory (no hipMalloc or allocating library routine). Scratch
 *    memory comes from the caller's workspace (ws, ws_bytes), sized by kq_workspace_bytes(); a call
 *    with a smaller workspace returns KQ_EWORKSPACE and enqueues nothing.
 *  - Calls validate their arguments on the host, enqueue their kernels on `stream` (a
 *    hipStream_t; NULL = the default stream) and return without synchronising the host, except
 *    kq_hg_sqrt (block and full forms) and kq_hg_lowrank: they wait once, after the first
 *    Denman-Beavers step, to read back the number of further steps (counted on the device from
 *    that step's interval bounds) into a 16-byte pinned host buffer of the calling host thread
 *    (allocated on its first such call and kept until the process ends), and they refuse
 *    (KQ_EINVAL) a stream that is capturing a HIP graph. Errors found on the host
 *    are returned; numerical failures found on the device (a matrix that is not positive definite)
 *    are written to a device int32 `info` (0 = success) that the caller reads after synchronising
 *    the stream.
 *  - Results are deterministic: fixed reduction orders, no order-dependent atomics.
 *  - No C++ exception crosses the ABI. Calls keep no data between them and are safe to call from
 *    several host threads on different streams. Per device, the square root's pipelined sweep uses
 *    two queues and nine events of the library's own, and the column sweep of 16384 rows or more
 *    three side queues (row panels beside the caller's stream) with four events, all default
 *    priority, created on the device's first such call and kept until the process ends; they carry
 *    no data from one call to the next, and a mutex per set orders the enqueueing of concurrent calls.
 */
#ifndef KQ_H
#define KQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* kq_stream; /* same type as hipStream_t */

typedef enum {
    KQ_OK = 0,
    KQ_EINVAL = 1,        /* null / misaligned pointer, bad enum, bad scalar */
    KQ_ESHAPE = 2,        /* inconsistent or unsupported sizes */
    KQ_ENOTPD = 3,        /* reserved: host-detected non-PD input */
    KQ_EUNSUPPORTED = 4,  /* dimension without a Hadamard order, bits/group not supported */
    KQ_EHIP = 5,          /* a HIP launch failed; detail in kq_last_error() */
    KQ_EWORKSPACE = 6     /* workspace smaller than kq_workspace_bytes() */
} kq_status;

typedef enum { KQ_F32 = 0, KQ_BF16 = 1 } kq_dtype;

typedef enum {
    KQ_HG_DIAG = 0,   /* o floats */
    KQ_HG_BLOCK = 1,  /* (o/blk) dense blk x blk blocks, stored one after another */
    KQ_HG_FULL = 2    /* o x o dense, leading dimension o */
} kq_hg_form;

typedef enum {
    KQ_OP_HESSIAN = 0,
    KQ_OP_ROTATE_IN = 1,
    KQ_OP_HG_SQRT = 2,
    KQ_OP_ROTATE_OUT = 3,
    KQ_OP_CHOLINV = 4,
    KQ_OP_QUANTIZE = 5,
    KQ_OP_UNROTATE = 6,
    KQ_OP_LOSS = 7,
    KQ_OP_MATVEC = 8,      /* n = number of tokens */
    KQ_OP_HG_LOWRANK = 9,  /* n = gradient rows, o, i = rank k */
    KQ_OP_KFAC_LOSS = 10,  /* o, i, form, blk */
    KQ_OP_CROSS = 11,      /* n tokens, i */
    KQ_OP_DRIFT = 12       /* o, i */
} kq_op;

/* Workspace bytes needed by `op` for a layer of o x i weights, n calibration tokens (X dtype
 * xdt), `bits`, `group` and H_G `form`/`blk`. Arguments an op does not use are ignored. */
size_t kq_workspace_bytes(kq_op op, int64_t o, int64_t i, int64_t n, kq_dtype xdt, int bits, int group,
                          kq_hg_form form, int64_t blk);

/*
 * H_X accumulation (review page, Background: the input activation covariance H_X as the
 * layer-Hessian proxy; Prior limitations: GPTQ's OBS update uses H_X only).
 *     H <- beta * H + alpha * X^T X
 * X: n x d, row-major, leading dimension ldx, fp32 or bf16 (xdt). H: d x d fp64, leading
 * dimension d, written in full (both triangles, exactly symmetric). With alpha = 1/n_total and
 * beta = 0 for the first token batch and 1 for later ones, H becomes X^T X / n_total over all
 * batches. bf16 inputs are multiplied exactly on the bf16 matrix cores; each instruction's
 * 32-product fp32 sum is accumulated in fp64. H stays fp64 through the rotation and the damped
 * factor because R moves with H as cond(H) makes it: rounding H to fp32 alone would shift the
 * sweep's pre-rounding values by up to ~2e-4 grid steps on 4096-wide layers. n = 0 only scales H.
 */
kq_status kq_hessian_accum(const void* X, kq_dtype xdt, int64_t n, int64_t d, int64_t ldx, double alpha,
                           double beta, double* H, void* ws, size_t ws_bytes, kq_stream stream);

/*
 * Input-side incoherence rotation (review page, "Where this paper sits": the QuIP / QuIP#
 * random Hadamard rotations; Method (1)).
 *     U = D_s H_i^T / sqrt(i),   Wout = Win U,   HX <- U^T HX U   (HX may be NULL)
 * Every row w of W becomes H_i (s * w) / sqrt(i). H_i = P_m (x) H_{2^k} with i = m 2^k, H_{2^k}
 * Sylvester's matrix and P_m a Paley type-I matrix of order m = q + 1 (q a prime, 27 or 343,
 * q = 3 mod 4), m the smallest such order dividing i; KQ_EUNSUPPORTED if none exists.
 * Win: o x i, fp32 or bf16 (wdt), leading dimension ldwin. Wout: o x i fp32, leading dimension
 * ldw; Wout may equal Win when wdt = KQ_F32 and ldw = ldwin. sign_in: i int8 values +-1.
 * HX: i x i fp64, leading dimension i, transformed in place (fp64 arithmetic). o = 0 rotates
 * only HX (Win, Wout may then be NULL).
 */
kq_status kq_rotate_in(const void* Win, kq_dtype wdt, int64_t ldwin, float* Wout, int64_t ldw, int64_t o,
                       int64_t i, double* HX, const int8_t* sign_in, void* ws, size_t ws_bytes, kq_stream stream);

/*
 * Output-side factor S = H_G^{1/2}, the principal (symmetric positive definite) square root, and
 * S^{-1} (KronQ abstract and review page Method (1): the output side of bidirectional
 * incoherence processing uses the gradient covariance; S^{-1} H_G S^{-1} = I makes H_G cancel).
 * HG, S and Sinv share the storage form: diag (o floats), block (o/blk blocks of blk x blk), or
 * full (o x o). Diagonal: elementwise square root. Block and full: scaled Denman-Beavers
 * iteration in fp64 whose SPD inverses are symmetric block Gauss-Jordan sweeps, stopped on a
 * device-side convergence test (at most 7 steps; enough for cond(H_G) <= 1e16). When the iterates
 * are already within 8e-5 of convergence before the last step, that step is one Newton-Schulz step
 * instead (E = I - Z Y in fp64, then S = Y + Y E / 2 and S^{-1} = Z + E Z / 2 with fp32 products),
 * which meets the same tolerance (relative eigenvalue error under 1e-8). The sweep runs on
 * the two queues of the device named above, forked from and joined back into `stream`. The call
 * returns only after the first step has completed on the device: it reads back the number of
 * further steps that step's interval bounds imply (counted on the device) and launches exactly
 * those; the rest is asynchronous on `stream`. A stream that is capturing a graph is refused (KQ_EINVAL). The sweep's
 * pivot kernels wait on the device, in a bounded loop, for the other queue's work, through a counter
 * in the call's workspace; where the device runs kernels one at a time (some profilers), that wait
 * runs out in the first step, and the call then redoes its work with queue waits and leaves a notice
 * in kq_last_error() (which the call clears when it starts). Nothing of this is kept for later calls.
 * Sinv may be NULL. info (device int32): 0; k in 1..o if H_G (or an iterate) is not positive
 * definite (k = 1 + index of the failing pivot); o + 1 if the iteration did not converge; -1 if a
 * device-side wait ran out after the first step (the device stopped running the two queues side by
 * side during the call; S is then invalid and the call should be issued again). The caller may free
 * HG once the work has completed in stream order (H_G is only needed transiently).
 */
kq_status kq_hg_sqrt(const float* HG, kq_hg_form form, int64_t o, int64_t blk, float* S, float* Sinv,
                     int32_t* info, void* ws, size_t ws_bytes, kq_stream stream);

/*
 * Output-side transform (review page, Method (1): on the output side the weights are transformed by
 * H_G^{1/2} and then rotated; KronQ abstract: the incoherence rotation extended to the output
 * dimension): W <- V S W with V = H_o D_t / sqrt(o) applied along the output axis (columns of the
 * row-major W), so that the loss tr(H_G dW H_X dW^T) becomes the GPTQ loss of the new coordinates
 * (review page, Key idea). S in the storage form given (from kq_hg_sqrt).
 * W: o x i fp32, leading dimension ldw, in place. sign_out: o int8 values +-1.
 */
kq_status kq_rotate_out(float* W, int64_t o, int64_t i, int64_t ldw, const float* S, kq_hg_form form,
                        int64_t blk, const int8_t* sign_out, void* ws, size_t ws_bytes, kq_stream stream);

/*
 * Damped factor of the inverse Hessian (review page, Prior limitations: GPTQ's column-wise OBS update
 * built on H_X alone, which KronQ keeps unchanged; its Cholesky form of H^{-1} with the usual 1 %
 * damping, the damping the smallest workload states).
 *     lambda = damp * mean(diag HX),   H = HX + lambda I,   R upper-triangular, H^{-1} = R^T R
 * computed without forming H^{-1}: with J the reversal permutation, J H J = L L^T (Cholesky) and
 * R = J L^{-1} J. From a width of 6144 the Cholesky is blocked in two levels (2048-wide panels
 * factored in 128-wide steps, then one deep update of the rest per panel); everything runs on
 * `stream`. The factorisation and the triangular inverse run in fp64 (vector FMA products); R is
 * rounded to fp32, so its error is that rounding rather than sqrt(cond(H)) fp32 steps.
 * HX: i x i fp64 (only its lower triangle is read), leading dimension ldh.
 * R: i x i fp32, leading dimension i, upper triangle written, strict lower triangle zeroed.
 * info (device int32): 0, or k > 0 if H is not positive definite (k = 1 + index, counted from the
 * last row, of the first failing pivot). No automatic re-damping.
 */
kq_status kq_cholinv(const double* HX, int64_t i, int64_t ldh, double damp, float* R, int32_t* info, void* ws,
                     size_t ws_bytes, kq_stream stream);

/*
 * GPTQ column sweep (review page, Prior limitations and Goal: the column-wise OBS update with H_X
 * only, kept unchanged; the H_G factor does not appear). For j = 0 .. i-1 in natural order:
 *     q_j = clamp(rne((W[:,j] - mu) / s), 0, 2^b - 1),  w^_j = mu + s q_j
 *     e = (W[:,j] - w^_j) / R_jj,  W[:, j+1:] -= e R[j, j+1:],  W[:,j] = w^_j,  row_loss += e^2
 * run in column blocks of `block` (128) with lazy trailing updates W[:, b1:] -= E R[b0:b1, b1:].
 * Grid: asymmetric min-max, mu = min v, s = (max v - min v) / (2^b - 1) (s = 0 gives q = 0), over
 * v = the whole row before the sweep (group = 0) or v = W[r, j:j+group] as updated when the sweep
 * reaches j (group > 0; group must divide block or block divide group).
 * W: o x i fp32, leading dimension ldw; in: W'' (rotated weights), out: w^ (dequantized, rotated
 * coordinates). R: i x i upper fp32 from kq_cholinv, leading dimension ldr.
 * codes: o x (i*bits/32) uint32 words, row-major; per row an LSB-first stream of b-bit fields in
 * little-endian words (i*bits must be a multiple of 32). scale, offset: o x (i/group) fp32 (or o
 * when group = 0); dequantize with offset + scale * q. row_loss: o fp32 (may be NULL).
 * bits in 2..8; i must be a multiple of `block`.
 */
kq_status kq_quantize_layer(float* W, int64_t o, int64_t i, int64_t ldw, const float* R, int64_t ldr, int bits,
                            int group, int block, uint32_t* codes, float* scale, float* offset, float* row_loss,
                            void* ws, size_t ws_bytes, kq_stream stream);

/*
 * kq_quantize_layer with a Hessian-aware choice of every grid (H_Z-PTQ page, Weight scales and
 * rounding: the scale of a quantization tile picked by a grid search over candidates for the
 * smallest curvature-weighted rounding error; its experimental settings: 500 candidates over one
 * half to all of the full range). Each grid's [min, max] range (over the row, group = 0, or over the
 * group's current values when the sweep reaches it) is shrunk about its midpoint by the factor
 * alpha_m = 1/2 + m / (2 (candidates - 1)), m = 0 .. candidates-1, and the first alpha minimising
 *     sum_c (w_c - w^_c(alpha))^2 / R_cc^2
 * over the grid's columns is kept: offset = mid - alpha h, scale = 2 alpha h / (2^b - 1), h the half
 * range. alpha = 1 is the min-max grid. candidates = 0 is kq_quantize_layer; 1..4096 otherwise.
 */
kq_status kq_quantize_layer_search(float* W, int64_t o, int64_t i, int64_t ldw, const float* R, int64_t ldr, int bits,
                                   int group, int block, int candidates, uint32_t* codes, float* scale, float* offset,
                                   float* row_loss, void* ws, size_t ws_bytes, kq_stream stream);

/*
 * Trace-sorted block order (H_Z-PTQ page, Weight scales and rounding: the blocks with larger
 * curvature traces are quantized first, as GPTQ's act-order does for columns). H: i x i fp64
 * (leading dimension ldh), i a multiple of width, at most 4096 blocks. order (device int32, 2 i/width
 * entries): order[k] = the block with the k-th largest trace of its diagonal part of H (ties: lower
 * index first), order[i/width + b] = the position of block b (the inverse permutation).
 * Used with width = 128 (the sweep's block), so groups and packed words stay within blocks: permute
 * W'' and H_X' (both axes) forward, factor and sweep, then undo the permutation on W, the codes (4 b
 * words per row and block) and the group scales and offsets (128/group per row and block).
 */
kq_status kq_block_order(const double* H, int64_t i, int64_t ldh, int64_t width, int32_t* order, kq_stream stream);

/*
 * Block permutation for the trace-sorted order above (H_Z-PTQ page, Weight scales and rounding):
 * out block k = in block perm[k], for column blocks (axis 0) or row blocks (axis 1) of a rows x cols
 * row-major matrix of 4- or 8-byte elements (leading dimensions ldi, ldo; in and out must differ).
 * perm: device int32, one entry per block of `width` elements.
 */
kq_status kq_permute_blocks(const void* in, int64_t ldi, void* out, int64_t ldo, int64_t rows, int64_t cols,
                            int64_t width, int axis, int elem_bytes, const int32_t* perm, kq_stream stream);

/*
 * Sublayer sensitivity tr(H_G) * tr(H_X), both undamped (review page, Method (2)). HX: i x i fp64,
 * leading dimension ldh (a rotated H_X gives the same trace up to rounding). HG in its storage
 * form. score: one device double.
 */
kq_status kq_sensitivity(const double* HX, int64_t i, int64_t ldh, const float* HG, kq_hg_form form, int64_t o,
                         int64_t blk, double* score, kq_stream stream);

/*
 * Verification: dequantized weights in the original coordinates (review page, Limitations (3): the
 * stored weights live in the transformed coordinates, and the orthogonal transforms and H_G^{1/2} are
 * reverted to recover the layer; Method (1) for the transforms themselves),
 *     What = S^{-1} V^T Q U^T
 * Q: o x i fp32 (the w^ output of kq_quantize_layer), leading dimension ldq; What: o x i fp32,
 * leading dimension ldw (must not alias Q). Sinv in the storage form of H_G.
 */
kq_status kq_unrotate(const float* Q, int64_t o, int64_t i, int64_t ldq, const int8_t* sign_in,
                      const int8_t* sign_out, const float* Sinv, kq_hg_form form, int64_t blk, float* What,
                      int64_t ldw, void* ws, size_t ws_bytes, kq_stream stream);

/*
 * Inference-side product with the quantized layer, y = W^ x for a block of nt tokens, with
 * W^ = S^{-1} V^T Q'' U^T applied factor by factor instead of materialising W^ (review page,
 * Limitations (3): inference reverts the orthogonal transforms online at Theta(d log d) per layer,
 * which a fused kernel keeps close to the cost of the weight matvec):
 *     x' = U^T x = H_i (s * x) / sqrt(i)         (fast transform per token)
 *     z  = Q'' x'                                 (dequantized on the fly from the packed codes)
 *     y  = S^{-1} V^T z = S^{-1} (t * H_o^T z) / sqrt(o)
 * codes, scale, offset: as written by kq_quantize_layer for this (o, i, bits, group); group must be
 * 0 or a multiple of 32 dividing i; bits in 2..8; o a multiple of 4. sign_in (i), sign_out (o), Sinv (storage
 * form of H_G): as for kq_unrotate. X: nt x i fp32 tokens, leading dimension ldx (16-byte aligned);
 * Y: nt x o fp32, leading dimension ldy (must not alias X). Workspace: kq_workspace_bytes with
 * op KQ_OP_MATVEC and n = nt.
 */
kq_status kq_matvec_quantized(const uint32_t* codes, const float* scale, const float* offset, int64_t o, int64_t i,
                              int bits, int group, const int8_t* sign_in, const int8_t* sign_out, const float* Sinv,
                              kq_hg_form form, int64_t blk, const float* X, int64_t ldx, int64_t nt, float* Y,
                              int64_t ldy, void* ws, size_t ws_bytes, kq_stream stream);

/* Size of the fixed per-device scratch array of kq_matvec_quantized_static (32 MiB). */
#define KQ_MATVEC_STATIC_SCRATCH_BYTES (32u << 20)

/*
 * kq_matvec_quantized without a workspace, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments (minus ws,
 * ws_bytes), same kernels and bit-identical results. The scratch comes from a fixed array of
 * KQ_MATVEC_STATIC_SCRATCH_BYTES per device inside the library, held by every device the library runs
 * on until the process ends; calls whose kq_workspace_bytes(KQ_OP_MATVEC, o, i, nt, ...) exceeds it
 * return KQ_EWORKSPACE and enqueue nothing (the workloads of this library fit with up to 16 tokens).
 * The call allocates nothing. Every call on a device shares that device's array, so calls that overlap
 * on one device (different streams, or host threads) race: order them on one stream. Nothing in the
 * array has to start at zero; it keeps the last call's contents.
 */
kq_status kq_matvec_quantized_static(const uint32_t* codes, const float* scale, const float* offset, int64_t o,
                                     int64_t i, int bits, int group, const int8_t* sign_in, const int8_t* sign_out,
                                     const float* Sinv, kq_hg_form form, int64_t blk, const float* X, int64_t ldx,
                                     int64_t nt, float* Y, int64_t ldy, kq_stream stream);

/*
 * H_G storage forms from an fp64 covariance H (o x o, leading dimension ldh), e.g. H_G = G^T G / n
 * accumulated from gradient rows by kq_hessian_accum (KronQ review page, Method: the gradient
 * covariance from one calibration backward pass; Limitations (2): its full d_out x d_out size).
 * form FULL: HG = H (o x o); BLOCK: the o/blk diagonal blocks (blk x blk each, stored one after
 * another; the 128-block approximation for blk = 128); DIAG: the diagonal (o). Values rounded to
 * fp32 (nearest even).
 */
kq_status kq_hg_extract(const double* H, int64_t o, int64_t ldh, kq_hg_form form, int64_t blk, float* HG,
                        kq_stream stream);

/*
 * Low-rank-plus-isotropic approximation of H_G = G^T G / n from the gradient rows G alone (the o x o
 * covariance is never formed), with its square root and inverse square root (KronQ review page,
 * Sparks: low-rank or blockwise approximations of H_G against the transient d_out^2 memory of the
 * bidirectional preprocessing; the approximation below is this library's reading):
 *     Q = orthonormal basis of range(H^{q+1} Omega)   (randomised range finder, q power steps)
 *     B = Q^T H Q,  sigma = (tr H - tr B) / (o - k)
 *     H^ = Q B Q^T + sigma (I - Q Q^T)                 (same trace as H)
 *     S = H^{1/2} = sqrt(sigma) I + Q (B^{1/2} - sqrt(sigma) I) Q^T,  S^{-1} likewise with B^{-1/2}
 * G: n x o fp32 rows (leading dimension ldg); Omega: o x k fp32 (the caller's Gaussian test
 * matrix); 0 < k < o, k <= n, 0 <= q <= 15. Out (device, fp32 o x o, full storage form): S, and
 * optionally Sinv and HGhat = H^ (may be NULL); sigma (may be NULL): two doubles {sigma, tr H}.
 * info (device int32): 0; 1 the range basis lost rank; 2 sigma <= 0; 3 the k x k square root failed.
 * Work in fp64 (G widened once). Workspace: kq_workspace_bytes(KQ_OP_HG_LOWRANK, o, k, n, ...).
 * The k x k root is kq_hg_sqrt's iteration, so this call too returns only after its first step has
 * completed on the device, and refuses a stream that is capturing a graph (KQ_EINVAL).
 */
kq_status kq_hg_lowrank(const float* G, int64_t n, int64_t o, int64_t ldg, int64_t k, int q, const float* omega,
                        float* S, float* Sinv, float* HGhat, double* sigma, int32_t* info, void* ws, size_t ws_bytes,
                        kq_stream stream);

/*
 * K-FAC layer loss tr(H_G dW H_X dW^T), dW = W^ - W, in the original coordinates (KronQ review page,
 * Background: H ~ H_X (x) H_G; the loss that the bidirectional transforms turn into a GPTQ loss).
 * W: o x i fp32 or bf16 (wdt), leading dimension ldw; What: o x i fp32 (ldq); HX: i x i fp64 (ldh);
 * HG in its storage form. loss: one device double. fp64 throughout (two fp64 GEMMs and a fixed-order
 * reduction). Workspace: kq_workspace_bytes(KQ_OP_KFAC_LOSS, o, i, 0, ..., form, blk).
 */
kq_status kq_kfac_loss(const void* W, kq_dtype wdt, int64_t ldw, const float* What, int64_t ldq, int64_t o, int64_t i,
                       const double* HX, int64_t ldh, const float* HG, kq_hg_form form, int64_t blk, double* loss,
                       void* ws, size_t ws_bytes, kq_stream stream);

/*
 * Cross-covariance of two token matrices (KronQ review page, Prior limitations: GPTAQ's correction of
 * the input drift that quantizing earlier layers causes), C <- beta C + alpha A^T B (d x d fp64,
 * leading dimension d), for the input-drift correction below (A = X the full-precision inputs, B = X~ the drifted ones,
 * alpha = 1/n). A, B: n x d fp32 or bf16 (dt), leading dimensions lda, ldb. fp64 accumulation (rows
 * widened in chunks of 8192). Workspace: kq_workspace_bytes(KQ_OP_CROSS, 0, d, n, ...).
 */
kq_status kq_cross_accum(const void* A, const void* B, kq_dtype dt, int64_t n, int64_t d, int64_t lda, int64_t ldb,
                         double alpha, double beta, double* C, void* ws, size_t ws_bytes, kq_stream stream);

/*
 * Input-drift correction (KronQ review page, Prior limitations: GPTAQ corrects the drift of a layer's
 * input caused by quantizing earlier layers; the pages do not give its formula, so this is this
 * library's reading): the layer should reproduce W X^T from the drifted X~, and
 *     || W^ X~^T - W X^T ||^2 = || (W^ - W*) X~^T ||^2 + const,  W* = W C (H~ + lambda I)^{-1}
 * with C = X^T X~ / n (kq_cross_accum) and H~ = X~^T X~ / n, so the unchanged sweep runs on the
 * target W* with H~ (lambda = damp mean diag H~: the ridge solution). Wt (o x i fp32, ldt) = W C R^T R
 * with R the damped factor of H~ from kq_cholinv ((H~ + lambda I)^{-1} = R^T R). W: fp32 or bf16;
 * C: fp64 (ldc); R: fp32 (ldr). fp64 products. Workspace: kq_workspace_bytes(KQ_OP_DRIFT, o, i, ...).
 */
kq_status kq_drift_target(const void* W, kq_dtype wdt, int64_t ldw, int64_t o, int64_t i, const double* C, int64_t ldc,
                          const float* R, int64_t ldr, float* Wt, int64_t ldt, void* ws, size_t ws_bytes,
                          kq_stream stream);

/*
 * Verification: layer loss in rotated coordinates (review page, Background: the Kronecker-factored
 * loss tr(H_G dW H_X dW^T); Key idea: in the transformed coordinates it is the plain GPTQ loss),
 * sum_r (Q - W2)_r HX2 (Q - W2)_r^T, which equals tr(H_G dW H_X dW^T) in the original coordinates
 * when HX2 is the rotated, undamped H_X.
 * W2, Q: o x i fp32 (leading dimension ldw); HX2: i x i fp64 (leading dimension ldh).
 * row_loss (may be NULL): o doubles; loss: one device double.
 */
kq_status kq_layer_loss(const float* W2, const float* Q, int64_t o, int64_t i, int64_t ldw, const double* HX2,
                        int64_t ldh, double* row_loss, double* loss, void* ws, size_t ws_bytes, kq_stream stream);

/*
 * Sublayer mixed-precision bit allocation (review page, Method (2) and Comparison: the joint score
 * tr(H_G) tr(H_X) orders sublayer upgrades). HOST pointers; runs on the calling thread.
 * Every sublayer starts at bmin bits; repeatedly the single upgrade b -> b + 1 (b < bmax) with the
 * largest scores[l] * (c(b) - c(b + 1)) / sizes[l], c(b) = (2^b - 1)^-2, that keeps
 * sum_l sizes[l] * bits[l] <= budget * sum_l sizes[l] is applied; ties go to the lower index.
 * c(b) is the expected squared rounding error per unit squared range of a b-bit grid (uniform
 * rounding errors of step d have variance d^2 / 12; the range is (2^b - 1) d).
 * scores: count doubles (>= 0); sizes: count weights per sublayer (> 0); bits: count int32 out.
 */
kq_status kq_allocate_bits(const double* scores, const int64_t* sizes, int64_t count, double budget, int bmin,
                           int bmax, int32_t* bits);

/* Text of a status code; thread-local detail of the last error on this host thread. */
const char* kq_strerror(kq_status status);
const char* kq_last_error(void);
/* Hadamard decomposition used for dimension d (review page, "Where this paper sits": the random
 * Hadamard rotations): returns m (and 2^k in *pow2), or 0 if unsupported. */
int64_t kq_hadamard_order(int64_t d, int64_t* pow2);
int kq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KQ_H */
