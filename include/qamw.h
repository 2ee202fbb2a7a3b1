/*
 * qamw.h -- C ABI of the QAM-W weight codec on AMD Instinct MI355X (gfx950).
 *
 * QAM-W ("QAM-W: Joint 2D Codebook Quantization for LLM Weights via Hadamard
 * Rotation and Activation-Aware Scaling"; cited below as "QAM-W, <section>")
 * codes an LLM weight matrix row by row (QAM-W, Methodology: The QAM-W Codec):
 *
 *   s_j      = r_j ^ alpha                       activation-aware channel scale
 *   W'       = W diag(s)
 *   rho_n    = ||W'_n||_2,  u_n = W'_n / rho_n   scale / direction split
 *   y_n      = R_fwd u_n,   R_fwd = (I (x) H_b / sqrt(b)) diag(eps)
 *   z_{n,k}  = (y_{n,2k}, y_{n,2k+1})            pairing
 *   sigma_k  = mean_n |z_{n,k}| / sqrt(pi/2)     per-pair calibration
 *   idx_{n,k}= nearest centroid of z_{n,k}/sigma_k in a 2D Lloyd-Max codebook
 *   packed   = idx at B = ceil(log2 K) bits each, LSB-first per row
 *   decode   : unpack -> C[idx] * sigma_k -> R_fwd^T -> * rho_hat_n -> / s_j
 *
 * Conventions shared by every entry point
 *   - W is row-major [N][ldw]: a row is an output channel, column j is input
 *     channel j (s_j scales columns).  ldw >= d, in elements.
 *   - H_b is the Sylvester-order Hadamard matrix H[i][k] = (-1)^popcount(i&k)
 *     applied to each contiguous block [beta*b, beta*b + b) of a row.
 *   - eps_j = -1 exactly when bit 63 of the j-th output (0-based) of
 *     SplitMix64 seeded with sign_seed is set; one mask per matrix.
 *   - The codebook is K x 2 float32, interleaved (cx, cy).
 *   - Packed indices: row-major [N][qamw_packed_row_words(d, K)] uint32;
 *     bit t of a row's stream is bit (t mod 32) of word t/32; index k holds
 *     bits [k*B, k*B + B); unused bits are 0; rows start on 16-byte boundaries.
 *   - Row norms are stored as IEEE binary16 bits, round-to-nearest-even of the
 *     exact norm.
 *   - Ties between equally distant centroids (equal fp32 scores) go to the
 *     lowest index.
 *
 * Memory and streams
 *   - Every array argument is a DEVICE pointer unless stated otherwise; the
 *     caller allocates and owns all of them, including workspaces.  The
 *     library never allocates, frees or synchronises, and keeps no global
 *     mutable state: calls on different streams are independent.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every compute
 *     call only enqueues kernels on it and returns; results are valid once
 *     the stream has reached that point.  In-place calls are not supported
 *     (outputs must not alias inputs).
 *   - W, W_out, packed, codebook, s and sigma must be 16-byte aligned (a plan
 *     256-byte aligned), and
 *     ldw / ldo rows must keep 16-byte alignment (ldw * element size % 16 == 0).
 *
 * Errors
 *   Arguments are validated on the host before anything is launched; on a
 *   failure nothing is enqueued or written and the status is returned.  A
 *   failed kernel launch returns QAMW_EHIP.  qamw_last_error() gives a
 *   message for the calling thread's last failure.  Device-side contracts the
 *   host cannot check (r_j > 0, finite inputs) are the caller's: violating
 *   them gives unspecified values but no out-of-bounds access.
 */
#ifndef QAMW_H
#define QAMW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QAMW_OK = 0,
  QAMW_EINVAL = -1,        /* bad argument (null pointer, size, stride, alignment) */
  QAMW_EUNSUPPORTED = -2,  /* valid but unsupported (block, K, d, dtype) */
  QAMW_EHIP = -3,          /* HIP runtime error on launch */
  QAMW_EWORKSPACE = -4     /* workspace missing or too small */
} qamw_status;

typedef enum { QAMW_F32 = 0, QAMW_BF16 = 1, QAMW_F16 = 2 } qamw_dtype;

/* ---------------- host-only helpers (pure, no device access) ---------------- */

/* B = ceil(log2 K) for 2 <= K <= 4096; -1 otherwise. */
int32_t qamw_index_bits(int32_t K);

/* uint32 words per packed row: ceil((d/2) * B / 32) rounded up to a multiple
 * of 4; -1 for invalid d or K. */
int64_t qamw_packed_row_words(int64_t d, int32_t K);

/* Bytes of device workspace qamw_calibrate needs for an N x d matrix (row
 * factors 1 / (sqrt(block) rho_n) in fp64, column factors eps_j s_j and
 * per-row-tile partial sums of pair amplitudes). */
size_t qamw_calibrate_workspace_bytes(int64_t N, int64_t d, int32_t block);

/* Bytes of device workspace qamw_encode needs for an N x d matrix (fp64 row
 * factors 1 / (sqrt(block) rho_n), 0 for rho_n = 0; fp32 per-column factors
 * eps_j s_j; fp32 1 / sigma_k). */
size_t qamw_encode_workspace_bytes(int64_t N, int64_t d);

const char* qamw_status_string(int32_t status);
const char* qamw_last_error(void);
const char* qamw_version(void);

/* ---------------- device entry points ---------------- */

/*
 * Calibration (QAM-W, Methodology: Activation-Aware Scaling; Pairing and
 * Calibration).
 *   W         [N][ldw] of wdtype (QAMW_F32 or QAMW_BF16)
 *   chan_rms  [d] float32, r_j > 0: RMS of input channel j's activations
 *   alpha     finite exponent; s_j = r_j ^ alpha (alpha = 0 gives s = 1)
 *   block     Hadamard block b: power of two, 2 <= b <= 1024, d % b == 0; the
 *             row length d must also be a multiple of 16 (QAMW_EUNSUPPORTED
 *             otherwise: the kernels give each lane 16 columns)
 *   s_out     [d] float32 out: s_j
 *   sigma_out [d/2] float32 out: sigma_k = sum_n |z_{n,k}| / (N sqrt(pi/2)),
 *             |z_{n,k}| taken on the normalised rotated row u_n (0 for rho_n = 0)
 *   workspace >= qamw_calibrate_workspace_bytes(N, d, block), 256-byte aligned
 * Deterministic: the column sums use a fixed order, no atomics.
 */
int32_t qamw_calibrate(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw,
                       const float* chan_rms, float alpha, int32_t block, uint64_t sign_seed,
                       float* s_out, float* sigma_out,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Nearest-centroid search plan (QAM-W, Methodology: Joint 2D Quantization).
 * An optional, codebook-specific acceleration structure for qamw_encode: a
 * grid over [-5, 5)^2 and a 128 x 128 grid over [-20, 20)^2 whose cells
 * list, in ascending index order, every centroid that can be the nearest one
 * (under qamw_encode's fp32 scores) for some point of the cell.  For
 * K <= 2048 the inner grid is a table the encode keeps in LDS: cells narrow
 * near the origin and wider away from it (edges on 2048 equal bins per axis),
 * each listing exactly the centroids whose Voronoi region, widened by the fp32
 * scores' error bound, meets the cell; equal lists are stored once.  For
 * larger K it is a uniform 512 x 512 grid of per-cell records.  Encoding with
 * a plan gives the same indices, bit for bit, as encoding without one; pairs
 * beyond both grids and cells with too many candidates fall back to scanning
 * all K centroids.  The outer grid's cells that tile [-5, 5)^2 are never
 * consulted (points there take the inner grid) and are marked "scan all".
 *
 * qamw_plan_bytes(K): bytes of device memory a plan for K centroids takes
 *   (0 for K outside [2, 4096]).  Host-only.
 * qamw_build_plan: enqueue the plan's construction on `stream`.
 *   codebook  [K][2] float32, the codebook later passed to qamw_encode
 *   plan      device buffer of plan_size >= qamw_plan_bytes(K) bytes,
 *             256-byte aligned; caller-owned, written entirely by the call
 * A plan stays valid while the codebook's values do not change; it may be
 * shared by concurrent encodes (they only read it).
 */
size_t qamw_plan_bytes(int32_t K);
int32_t qamw_build_plan(const float* codebook, int32_t K, void* plan, size_t plan_size, void* stream);

/*
 * Encode (QAM-W, Methodology: Separation of Scale and Direction; Deterministic
 * Rotation; Pairing and Calibration; Joint 2D Quantization).
 *   W, wdtype, N, d, ldw, block, sign_seed  as for qamw_calibrate
 *   s          [d] float32: channel scales (normally s_out of qamw_calibrate)
 *   sigma      [d/2] float32: pair scales; sigma_k = 0 codes z~ = 0
 *   codebook   [K][2] float32, 2 <= K <= 4096
 *   plan       NULL (exhaustive search over the codebook) or a plan that
 *              qamw_build_plan built for this codebook and K; same result.
 *              A plan built for another K is detected on the device and the
 *              whole codebook is scanned; one built for another codebook of
 *              the same K gives unspecified (in-range) indices
 *   plan_size  bytes of the plan buffer (ignored when plan is NULL); less than
 *              qamw_plan_bytes(K) is rejected (QAMW_EWORKSPACE) before any launch
 *   packed     [N][qamw_packed_row_words(d, K)] uint32 out
 *   rownorm_f16[N] uint16 out: binary16 bits of rho_n (RNE)
 *   workspace  >= qamw_encode_workspace_bytes(N, d), 256-byte aligned
 * The nearest centroid is decided in fp32 on the expanded score
 * |c|^2/2 - z~ . c (equal to |z~ - c|^2/2 - |z~|^2/2); equal scores go to the
 * lowest index.
 */
int32_t qamw_encode(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw,
                    const float* s, const float* sigma, int32_t block, uint64_t sign_seed,
                    const float* codebook, int32_t K, const void* plan, size_t plan_size,
                    uint32_t* packed, uint16_t* rownorm_f16,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * qamw_encode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The workspace lives in a device array of
 * qamw_encode_noalloc_scratch_bytes() (1 MiB) inside the library, one per GPU,
 * held until the process ends; the call allocates and frees nothing.
 *   arguments  as for qamw_encode, less workspace and workspace_bytes
 *   limit      qamw_encode_workspace_bytes(N, d) <= 1 MiB (every N <= 65536
 *              with d <= 65536 fits); larger sizes return QAMW_EUNSUPPORTED
 *              before anything runs
 * Same results as qamw_encode, bit for bit.  All calls on one GPU share the
 * array: calls that overlap on one GPU (other streams, other host threads)
 * race, so the caller must order them.  Errors as for qamw_encode; QAMW_EHIP
 * also when the array's device address cannot be looked up.
 */
size_t qamw_encode_noalloc_scratch_bytes(void);
int32_t qamw_encode_noalloc(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw,
                            const float* s, const float* sigma, int32_t block, uint64_t sign_seed,
                            const float* codebook, int32_t K, const void* plan, size_t plan_size,
                            uint32_t* packed, uint16_t* rownorm_f16, void* stream);

/*
 * qamw_encode in two phases, for callers that time or reuse them separately.
 *
 * qamw_encode_prepare (QAM-W, Methodology: Separation of Scale and Direction;
 * Pairing and Calibration): row norms rho_n = ||W_n diag(s)||_2 (binary16
 * bits RNE into rownorm_f16 [N]; into the workspace the fp64 row factors
 * 1 / (sqrt(block) rho_n)), the per-column factors eps_j s_j and the pair
 * factors 1 / sigma_k (into the workspace).
 * Arguments as for qamw_encode.
 *
 * qamw_encode_indices (QAM-W, Methodology: Deterministic Rotation; Joint 2D
 * Quantization): rotation, normalisation, nearest centroid and packing of W
 * into packed, reading the factors from a workspace that qamw_encode_prepare
 * filled for the same W, s, sigma, block and sign_seed, earlier on the same
 * stream (or otherwise ordered before this call).  The workspace is only
 * read.  Arguments as for qamw_encode.
 *
 * qamw_encode is exactly qamw_encode_prepare followed by qamw_encode_indices.
 */
int32_t qamw_encode_prepare(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw,
                            const float* s, const float* sigma, int32_t block, uint64_t sign_seed,
                            uint16_t* rownorm_f16, void* workspace, size_t workspace_bytes, void* stream);
int32_t qamw_encode_indices(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw, int32_t block,
                            const float* codebook, int32_t K, const void* plan, size_t plan_size,
                            uint32_t* packed, const void* workspace, size_t workspace_bytes, void* stream);

/*
 * Calibration and encode in one call (QAM-W, Methodology: Activation-Aware
 * Scaling; Separation of Scale and Direction; Deterministic Rotation; Pairing
 * and Calibration; Joint 2D Quantization): exactly qamw_calibrate followed by
 * qamw_encode -- s_out, sigma_out, packed and rownorm_f16 are bit-identical
 * to theirs -- but the row norms, column factors and 1 / sigma of the
 * calibration pass are kept for the encode, which saves the encode's own pass
 * over W for the row norms.
 *   arguments  as for qamw_calibrate and qamw_encode
 *   workspace  >= qamw_calibrate_encode_workspace_bytes(N, d), 256-byte aligned
 */
size_t qamw_calibrate_encode_workspace_bytes(int64_t N, int64_t d);
/*
 * qamw_calibrate_prepare: the calibration half of qamw_calibrate_encode.
 * Writes s_out, sigma_out and rownorm_f16 and leaves in the workspace (the
 * same size and alignment as above) what qamw_encode_prepare would: a
 * following qamw_encode_indices with this workspace gives qamw_calibrate_encode's
 * packed words, bit for bit.  It does not read a codebook or a plan, so a
 * caller may build the plan on another stream meanwhile and join before
 * qamw_encode_indices.  Errors as for qamw_calibrate_encode.
 */
int32_t qamw_calibrate_prepare(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw,
                               const float* chan_rms, float alpha, int32_t block, uint64_t sign_seed,
                               float* s_out, float* sigma_out, uint16_t* rownorm_f16,
                               void* workspace, size_t workspace_bytes, void* stream);
int32_t qamw_calibrate_encode(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw,
                              const float* chan_rms, float alpha, int32_t block, uint64_t sign_seed,
                              const float* codebook, int32_t K, const void* plan, size_t plan_size,
                              float* s_out, float* sigma_out, uint32_t* packed, uint16_t* rownorm_f16,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Codebook refinement on a matrix's own pairs (QAM-W, Significance and
 * Claims: the codebook is trained on the unit circular Gaussian, and a
 * codebook learned from a checkpoint's own distribution may do better).
 * Lloyd rounds on the normalised pairs z~ the encoder quantises.
 *
 * qamw_lloyd_update: one round's update.  packed must hold the indices that
 *   qamw_encode (or qamw_encode_indices) produced for this W, codebook and
 *   encode workspace (filled by qamw_encode_prepare or qamw_calibrate_encode,
 *   only read here).  Writes codebook_out[c] = the mean of the pairs coded c
 *   (sums in 64-bit fixed point of 2^-28, so independent of summation
 *   order; the mean rounded to fp32), or codebook[c] when no pair is coded c,
 *   and *distortion_out = the mean of |z~ - codebook[idx]|^2 (fp64, fixed
 *   order) of the given assignment.  codebook_out must not alias codebook.
 *   workspace >= qamw_lloyd_workspace_bytes(K), 256-byte aligned.
 *   Deterministic.
 *
 * qamw_learn_codebook: iters >= 1 rounds of (qamw_build_plan for the current
 *   codebook, the planned encode into packed, qamw_lloyd_update) from
 *   codebook_init; the result goes to codebook_out and round t's distortion
 *   (of its assignment to its starting codebook) to distortion_out[t].
 *   plan (>= qamw_plan_bytes(K)) and packed ([N][qamw_packed_row_words(d, K)])
 *   are scratch; the encode workspace as above.
 */
size_t qamw_lloyd_workspace_bytes(int32_t K);
int32_t qamw_lloyd_update(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw, int32_t block,
                          const uint32_t* packed, const float* codebook, int32_t K,
                          const void* enc_workspace, size_t enc_workspace_bytes,
                          float* codebook_out, double* distortion_out,
                          void* workspace, size_t workspace_bytes, void* stream);
int32_t qamw_learn_codebook(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw, int32_t block,
                            const void* enc_workspace, size_t enc_workspace_bytes,
                            const float* codebook_init, int32_t K, int32_t iters,
                            float* codebook_out, double* distortion_out,
                            void* plan, size_t plan_size, uint32_t* packed,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Polar-code baseline (QAM-W, Methodology: Joint 2D Quantization, and the
 * Experiments' joint-versus-polar ablation): the same transform as
 * qamw_encode, but amplitude and phase of each normalised pair z~ = (x, y)
 * are quantised independently.
 *   levels  [Ka] float32 amplitude levels, >= 0 and strictly ascending
 *   dirs    [Kp][2] float32 unit directions (cos, sin); 2 <= Ka Kp <= 4096
 *   index   ia * Kp + ip, packed with B = ceil(log2(Ka Kp)) bits exactly as
 *           qamw_encode packs (qamw_packed_row_words(d, Ka * Kp) words a row)
 *   ia      the lowest i minimising |r - a_i|, r = sqrt(x*x + y*y), all fp32
 *   ip      the lowest j maximising x c_j + y s_j in fp32
 * Other arguments as for qamw_encode.  The result decodes with qamw_decode
 * (and qamw_decode_matmul) given the Ka Kp-entry table whose entry
 * ia * Kp + ip is a_ia (c_ip, s_ip).
 */
int32_t qamw_encode_polar(const void* W, int32_t wdtype, int64_t N, int64_t d, int64_t ldw,
                          const float* s, const float* sigma, int32_t block, uint64_t sign_seed,
                          const float* levels, int32_t Ka, const float* dirs, int32_t Kp,
                          uint32_t* packed, uint16_t* rownorm_f16,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Activation statistics and the layer-output error (QAM-W, Methodology:
 * Activation-Aware Scaling; the trace identity of the composite bound
 * chain, || X dW^T ||_F^2 = Tr(dW M dW^T) with M = X^T X).
 *
 * qamw_channel_rms: r_j = sqrt(sum_t X[t][j]^2 / T), the chan_rms input of
 *   qamw_calibrate, from T activation rows.
 *   X        [T][ldx] of xdtype (QAMW_F32 or QAMW_BF16), 16-byte aligned rows
 *   d        a multiple of 8
 *   r_out    [d] float32 out, 16-byte aligned
 *   workspace >= qamw_channel_rms_workspace_bytes(T, d), 256-byte aligned
 *   Squares are summed in fp32 over tiles of 64 rows and the tiles in fp64,
 *   in a fixed order: deterministic.
 *
 * qamw_output_error: E = sum_{t, n} (sum_j X[t][j] (W[n][j] - W_hat[n][j]))^2,
 *   the layer-output error of replacing W by W_hat for the activations X
 *   (equal to Tr(dW X^T X dW^T)).
 *   X        [T][ldx] as above; W [N][ldw] of wdtype and W_hat [N][ldh] of
 *            hdtype (QAMW_F32 or QAMW_BF16 each), 16-byte aligned rows
 *   d        a multiple of 16
 *   err_out  one double on the device, written by the call
 *   workspace >= qamw_output_error_workspace_bytes(T, N, d), 256-byte
 *            aligned (holds bf16 copies of dW and, for fp32 X, of X)
 *   Arithmetic: dW = W - W_hat in fp32, then dW and X rounded to bf16 and
 *   multiplied on bf16 MFMA with fp32 accumulation; squares summed in fp64 in
 *   a fixed order (deterministic).  Relative error of E: about 2^-8 in the
 *   worst case, far less for unstructured rounding errors.
 */
size_t qamw_channel_rms_workspace_bytes(int64_t T, int64_t d);
int32_t qamw_channel_rms(const void* X, int32_t xdtype, int64_t T, int64_t d, int64_t ldx, float* r_out,
                         void* workspace, size_t workspace_bytes, void* stream);
size_t qamw_output_error_workspace_bytes(int64_t T, int64_t N, int64_t d);
int32_t qamw_output_error(const void* X, int32_t xdtype, int64_t T, int64_t d, int64_t ldx,
                          const void* W, int32_t wdtype, int64_t N, int64_t ldw,
                          const void* W_hat, int32_t hdtype, int64_t ldh,
                          double* err_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode (QAM-W, Methodology: Decoding).
 *   packed, rownorm_f16, N, d, block, sign_seed, codebook, K  as produced by
 *             qamw_encode; indices >= K (never produced) are clamped to K - 1
 *   s          [d] float32 or NULL.  With s the output approximates W; with
 *              NULL it approximates W' = W diag(s) (scales folded elsewhere)
 *   sigma      [d/2] float32
 *   W_out      [N][ldo] of out_dtype (QAMW_F32, QAMW_BF16 or QAMW_F16; bf16
 *              is rounded to nearest even from the fp32 value, fp16 from the
 *              exact product of the last fp32 scale, in one rounding, which
 *              can differ from rounding the fp32 value by one unit at ties)
 * Arithmetic is fp32.
 */
int32_t qamw_decode(const uint32_t* packed, const uint16_t* rownorm_f16, int64_t N, int64_t d,
                    const float* s, const float* sigma, int32_t block, uint64_t sign_seed,
                    const float* codebook, int32_t K,
                    void* W_out, int32_t out_dtype, int64_t ldo, void* stream);

/*
 * Decoded-weight matmul, Y = X W^^T, without materialising W^ (QAM-W,
 * Methodology: Decoding; the pages dequantise to BF16 before the matmul and
 * name the fused kernel as the missing piece).  A decoded row is
 * W^_n = rho^_n (R_fwd^T y^_n) / s with y^_{n,2k:2k+2} = sigma_k C[idx_{n,k}],
 * and R_fwd is orthogonal, so Y[t][n] = rho^_n <R_fwd (X_t / s), y^_n>:
 * the activations are rotated once, and the matmul needs per weight only an
 * index unpack, a codebook lookup and a scale by sigma_k.
 *
 * qamw_rotate_activations: Xr_bf16[t] = bf16_RNE(R_fwd (X[t] / s)).
 *   X          [T][ldx] of xdtype (QAMW_F32 or QAMW_BF16), activations
 *   s          [d] float32 channel scales of the matrix, or NULL (s = 1: use
 *              with a matrix decoded as W diag(s), see qamw_decode)
 *   block, sign_seed  those the matrix was encoded with
 *   Xr_bf16    [T][ldr] bf16 bits out, rows 16-byte aligned (ldr % 8 == 0)
 *
 * qamw_decode_matmul: Y[t][n] = rho^_n sum_k Xr[t][k] y^_n[k].
 *   Xr_bf16    [T][ldr] from qamw_rotate_activations
 *   packed, rownorm_f16, N, sigma, codebook, K  as for qamw_decode
 *   Y          [T][ldy] of ydtype (QAMW_F32 or QAMW_BF16), ldy >= N
 * Products use bf16 operands (the looked-up y^ and Xr, rounded to nearest
 * even) on bf16 MFMA with fp32 accumulation; each output is within
 * 2^-7 rho^_n sum_k |Xr[t][k] y^_n[k]| of the exact product.  With T = 1 the
 * product runs as a GEMV in fp32 (y^ not rounded; Xr is bf16), inside the
 * same bound.  The sum over columns is split into a fixed number of parts
 * added in a fixed order, so results are deterministic.
 */
int32_t qamw_rotate_activations(const void* X, int32_t xdtype, int64_t T, int64_t d, int64_t ldx,
                                const float* s, int32_t block, uint64_t sign_seed,
                                uint16_t* Xr_bf16, int64_t ldr, void* stream);
int32_t qamw_decode_matmul(const uint16_t* Xr_bf16, int64_t T, int64_t d, int64_t ldr,
                           const uint32_t* packed, const uint16_t* rownorm_f16, int64_t N,
                           const float* sigma, const float* codebook, int32_t K,
                           void* Y, int32_t ydtype, int64_t ldy, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QAMW_H */
