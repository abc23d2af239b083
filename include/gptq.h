/*
 * gptq.h -- C ABI of the MI355X (gfx950) GPTQ layer quantizer.
 *
 * GPTQ quantizes one linear layer at a time against calibration data
 * (glossary entry "gptq", paragraph "Method"): it builds the Hessian of the
 * layer's reconstruction loss from calibration activations, then quantizes
 * the weights column by column, pushing each column's rounding error onto
 * the columns not yet quantized using the inverse Hessian (same entry,
 * paragraphs "Key innovation" and "Algorithm").  The three calls below are
 * that pipeline for one layer:
 *
 *   gptq_hessian_accumulate   H += 2 X^T X          (once per calibration chunk)
 *   gptq_prepare              damp, order, factor   -> Hinv_chol, perm
 *   gptq_quantize_layer       sweep + pack          -> qweight, scales, zeros, g_idx
 *
 * and around it:
 *   gptq_dequant_matmul       Y = X W^T from the packed layer (dequantized on the fly)
 *   gptq_dequant_matmul_noalloc  the same without a workspace (fixed scratch)
 *   gptq_dequant_group_order  act-order layer -> group-sorted copy + x_order (once)
 *   gptq_silu_mul             gated activation between the MLP layers of a block
 *   gptq_attention_forward    attention between the q/k/v and o projections of a block
 *   gptq_residual_rmsnorm     residual add + RMS norm between the attention and the MLP
 *   gptq_export_params        fp16 scales + b-bit packed zeros, for saving
 *   gptq_unpack_zeros         zeros from their packed form, after loading
 *
 * Conventions shared by every call
 *   - Every array argument is DEVICE memory owned by the caller (HIP device
 *     pointers), row-major, densely packed unless a leading dimension is given.
 *     The library never allocates or frees device memory; scratch space comes
 *     from the caller's workspace, sized by the *_workspace_bytes queries
 *     (gptq_dequant_matmul_noalloc: a fixed per-device array instead).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work on it and return; nothing is synchronised.  Results are valid once
 *     the stream has reached that point.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failing check returns a nonzero gptq_status_t and leaves every output
 *     untouched.  gptq_last_error_message() then names the failing argument.
 *   - Conditions found on the device (a non-positive or non-finite Cholesky
 *     pivot) are reported through a device int32 `info`, as LAPACK does.
 *   - There is no CPU fallback.
 *   - Calls are safe on different streams concurrently as long as they use
 *     different workspaces and outputs.
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
  GPTQ_ERR_INVALID_ARG = 1, /* a pointer, size or parameter is out of range      */
  GPTQ_ERR_UNSUPPORTED = 2, /* a valid request this library does not implement   */
  GPTQ_ERR_WORKSPACE = 3,   /* workspace_bytes below the size the query returned */
  GPTQ_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed        */
} gptq_status_t;

typedef enum { GPTQ_F16 = 0, GPTQ_BF16 = 1, GPTQ_F32 = 2 } gptq_dtype_t;

/* Maximum matrix order accepted by gptq_prepare (one row of H is staged in
 * the 160 KiB LDS of a gfx950 compute unit during the column gather). */
#define GPTQ_MAX_PREPARE_N 32768

/* Workspace (bytes) gptq_hessian_accumulate can use for order n on the
 * current device: 256 x 256 fp32 partial tiles for the schedules that split
 * tiles along the tokens, which run when the 256 x 256 tiles of H cannot
 * fill the compute units in whole rounds (e.g. 335 MiB at n = 4096 on a
 * 256-CU device); 0 where whole tiles are always used (e.g. n = 11008) or
 * n < 1. */
size_t gptq_hessian_workspace_bytes(int64_t n);

/*
 * Hessian accumulation:  H += 2 * X^T X   (upper triangle only).
 *
 * Glossary entry "gptq", paragraph "Algorithm" step (1): the Hessian of the
 * layer loss with respect to the layer weights, approximated from the
 * calibration data.  For the reconstruction loss sum_t ||(W - W^) x_t||^2 it
 * is exactly 2 * sum_t x_t x_t^T; the sum (not the mean) is accumulated, so
 * calibration data can be streamed in chunks of any size.
 *
 *   H      fp32 [n x n], row-major.  Entries H[i][j] with i <= j are read and
 *          updated; entries below the diagonal are never touched.  The caller
 *          zero-initialises H before the first chunk.
 *   n      number of input features (columns of the layer's W), n >= 1.
 *   X      calibration activations, [ntok x n] (tokens x features), row-major
 *          with leading dimension ldx >= n, dtype GPTQ_F16 or GPTQ_BF16.
 *   ntok   tokens in this chunk; ntok == 0 is a no-op returning GPTQ_OK.
 *   workspace  NULL, or device memory of at least
 *          gptq_hessian_workspace_bytes(n).  With a workspace, a layer too
 *          small to fill the GPU with whole 256 x 256 tiles is split over all
 *          compute units along the tokens (partial tiles are combined in a
 *          fixed order: results do not depend on timing).  Calls that share a
 *          workspace must not overlap.  Long calls (all calibration tokens
 *          at once) let the library choose the token blocks; chunks of any
 *          size give the same sum up to fp32 rounding order.
 *
 * Products of fp16/bf16 values are exact in fp32; accumulation is fp32.
 * Errors: INVALID_ARG (null pointers, n < 1, ntok < 0, ldx < n),
 *         UNSUPPORTED (x_dtype not F16/BF16), WORKSPACE, HIP.
 */
int gptq_hessian_accumulate(float* H, int64_t n, const void* X, int x_dtype,
                            int64_t ntok, int64_t ldx, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Workspace (bytes) gptq_prepare needs for order n (0 if n is out of range). */
size_t gptq_prepare_workspace_bytes(int64_t n);

/*
 * Damping, column order and the factor that drives the sweep.
 *
 *   - Damping ("GPTQ > Using AutoGPTQ in Practice", Key Parameters,
 *     damp_percent): mu = mean(diag H); H_d = H + damp_percent * mu * I.
 *     A feature whose diagonal entry is exactly 0 is given H_ii = 1 before
 *     the mean is taken (it never fired; its weights cannot change the loss).
 *   - Column order (same list, desc_act): with desc_act != 0 the columns are
 *     processed by decreasing diag(H) (the raw diagonal; ties keep the lower
 *     original index first); otherwise in natural order.
 *   - Factor (same page, introduction: "Cholesky factorization"; glossary
 *     "Algorithm" step (2): compensation "using H^-1"): Hinv_chol is U, the
 *     upper-triangular Cholesky factor of (P H_d P^T)^-1, U^T U = H_p^-1,
 *     computed as the inverse of the reverse Cholesky factor of H_p.
 *
 *   H          fp32 [n x n]; only the upper triangle (i <= j) is read.
 *   n          1 <= n <= GPTQ_MAX_PREPARE_N.
 *   damp_percent  >= 0 (0.01 means 1 %).
 *   Hinv_chol  out: fp32 [n x n], row-major; upper triangle = U, strictly
 *              lower triangle = 0.  Row/column j refers to the j-th column in
 *              quantization order.
 *   perm       out: int32 [n]; perm[j] = original column quantized j-th
 *              (the identity when desc_act == 0).
 *   info       out: device int32; 0 on success, k > 0 if the pivot of
 *              quantization-order column k-1 was non-positive or not finite
 *              (then Hinv_chol is not meaningful).
 *   workspace  device memory of at least gptq_prepare_workspace_bytes(n).
 *
 * The factorization runs on the caller's stream and on two helper streams
 * the library creates once per device (default priority): they wait for the
 * caller's earlier work and the caller's stream waits for them before the
 * call returns, so on the caller's stream the call behaves as one ordered
 * operation.  Calls on one device enqueue one after the other (a host-side
 * lock); calls that share a workspace must not overlap.
 * Errors: INVALID_ARG, UNSUPPORTED (n > GPTQ_MAX_PREPARE_N), WORKSPACE, HIP.
 */
int gptq_prepare(const float* H, int64_t n, float damp_percent, int desc_act,
                 float* Hinv_chol, int32_t* perm, int32_t* info,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace (bytes) gptq_quantize_layer needs (0 if the arguments are invalid). */
size_t gptq_quantize_workspace_bytes(int64_t out, int64_t in, int bits,
                                     int group_size, int block);

/*
 * The column sweep and the packing.
 *
 * Glossary "gptq", "Algorithm" step (2) and "Key innovation": each weight, in
 * quantization order, is quantized, its error computed, and the remaining
 * weights of its row adjusted to compensate:  w_k -= (e / U_jj) * U_jk for
 * k > j.  Groups (agent skill page "gptq", "Group-wise quantization"; handbook
 * Key Parameters, group_size): group_size consecutive columns in quantization
 * order share one scale and zero-point per output row; group_size == -1 means
 * one group per row.  A group's scale and zero are taken when its first
 * column comes up, from the group's current values:
 *     lo = min(0, min w), hi = max(0, max w)
 *     sym:   hi = max(-lo, hi), lo = -hi, zero = 2^(bits-1)
 *     lo == hi  ->  lo = -1, hi = +1
 *     scale = (hi - lo) / (2^bits - 1),   asym: zero = rint(-lo / scale)
 *     code  = clamp(rint(w / scale) + zero, 0, 2^bits - 1)
 * in IEEE fp32 with round-half-to-even.  Columns are swept in lazy blocks of
 * `block` columns; the update of the columns right of a block is applied as a
 * matrix product on the matrix cores (the set of updates is the same): in
 * fp32 for fewer than 512 columns of errors, above that with each error
 * (its row scaled by a power of two) split into two fp16 parts times the
 * factor U_jk / U_jj in fp16, fp32 sums: the factor rounded once to fp16
 * for in <= 16384 (pre-rounding values move by a few 1e-4 code units
 * against exact arithmetic), as two fp16 parts for wider layers (~1e-5).
 *
 *   W          [out x in] row-major, dtype F16 / BF16 / F32, ORIGINAL column
 *              order; not modified.
 *   Hinv_chol  fp32 [in x in] upper triangle, as written by gptq_prepare
 *              (any upper-triangular matrix with a positive diagonal is
 *              accepted; the strictly lower triangle is ignored).
 *   perm       int32 [in] from gptq_prepare, or NULL for the identity.
 *   bits       2, 3, 4 or 8 (glossary "Quantization targets"; catalogue page).
 *   group_size -1, or a positive divisor of `block`.
 *   sym        0 = asymmetric, 1 = symmetric.
 *   block      lazy block width: 32, 64 or 128.
 *   in         a positive multiple of 32 (3-bit packs 32 codes in 3 words).
 * Outputs (caller-allocated device memory, fully overwritten):
 *   qweight    int32 [in*bits/32 x out]: for output row r, the codes of input
 *              columns 0..in-1 (original order) form a little-endian bit
 *              stream, column k at bits [k*bits, (k+1)*bits); word w of that
 *              stream is qweight[w][r].
 *   scales     fp32  [n_groups x out], n_groups = group_size == -1 ? 1
 *              : ceil(in / group_size); group g = quantization-order columns
 *              [g*group_size, (g+1)*group_size).
 *   zeros      int32 [n_groups x out], values in [0, 2^bits - 1].
 *   g_idx      int32 [in]: g_idx[k] = group of original column k.
 * Errors: INVALID_ARG, UNSUPPORTED (bits, block), WORKSPACE, HIP.
 */
int gptq_quantize_layer(const void* W, int w_dtype, int64_t out, int64_t in,
                        const float* Hinv_chol, const int32_t* perm,
                        int bits, int group_size, int sym, int block,
                        int32_t* qweight, float* scales, int32_t* zeros,
                        int32_t* g_idx, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Workspace (bytes) gptq_dequant_matmul needs for M token rows, in inputs and
 * out outputs, with (has_order != 0) or without an x_order: the fp32 partial
 * sums when the input range is split over several workgroups (always for
 * M <= 8, e.g. 16 x 1 x 4096 for one token of a 4096 x 4096 layer; for
 * M > 8 when the output tiles alone would not fill the GPU), plus, for
 * M >= 256 with out a multiple of 4, a table of one int per 32 inputs (the
 * group of each 32-position chunk, or -1 where it mixes groups), plus, for
 * M > 8 with an x_order, the gathered copy of X (M x in fp16).  0 when
 * none applies (e.g. M = 64 on a 4096 x 4096 layer needs only partial sums;
 * M = 8192 on it needs only the 512-byte table). */
size_t gptq_dequant_matmul_workspace_bytes(int64_t M, int64_t in, int64_t out, int has_order);

/*
 * Dequantize-on-the-fly matmul: Y = X W^T for a layer quantized by
 * gptq_quantize_layer.
 *
 * Glossary entry "gptq", paragraph "Inference": the quantized weights are
 * dequantized during the computation and multiplied.  Here
 *     W[r][p] = scales[g_idx[p]][r] * (code[r][p] - zeros[g_idx[p]][r]),
 * code[r][p] the p-th b-bit field of row r's little-endian bit stream
 * (qweight[j][r] is word j of it), and
 *     Y[t][r] = sum_p X[t][x_order[p]] W[r][p]
 * (x_order NULL: x_order[p] = p, the layer as gptq_quantize_layer writes it;
 * with the outputs of gptq_dequant_group_order, the same product).
 *
 *   X        fp16 [M x in], row-major, leading dimension ldx >= in, ldx a
 *            multiple of 8, X 16-byte aligned.  M == 0 is a no-op.
 *   qweight  int32 [in * bits / 32 x out]; scales fp32 and zeros int32
 *            [n_groups x out]; g_idx int32 [in] with values in
 *            [0, n_groups) (not checked: device data).
 *   x_order  int32 [in], a permutation of 0..in-1 (not checked), or NULL.
 *   in       a positive multiple of 32; out >= 1; bits 2, 3, 4 or 8.
 *   Y        out: [M x out], row-major, ldy >= out, y_dtype GPTQ_F32 or
 *            GPTQ_F16 (the fp32 sum rounded to nearest).
 *   workspace  device memory of gptq_dequant_matmul_workspace_bytes(M, in,
 *            out, x_order != NULL) bytes, or NULL when that is 0.
 *
 * Arithmetic: M <= 8 (HBM-bound on qweight) takes each weight exactly:
 * q - z as an fp16 integer times the fp16 activation, summed in fp32 over a
 * 32-input chunk, times the group's fp32 scale (s (q - z) in fp32 per
 * weight where a chunk mixes groups), fp32 accumulation; larger M rounds
 * each dequantized weight to fp16 (the scale split into two fp16 parts and
 * the weight formed in one fused rounding, close to the fp16 rounding of the
 * exact s (q - z)) and multiplies on the fp16 matrix cores with fp32
 * accumulation.  Results do
 * not depend on timing.  Calls that share a workspace must not overlap.
 * A chunk of 32 positions whose g_idx entries are all equal is dequantized
 * with one scale and zero; chunks that mix groups (act-order layers as
 * packed) read them per position and run several times slower:
 * gptq_dequant_group_order turns such a layer into one without them (from
 * 256 tokens on the check is per 16 positions).
 * Errors: INVALID_ARG, UNSUPPORTED (x_dtype not F16, bits, alignment;
 *         qweight, scales or zeros of 2 GiB or more; ldx above 2^22 with
 *         M > 8), WORKSPACE, HIP.
 */
int gptq_dequant_matmul(const void* X, int x_dtype, int64_t M, int64_t in, int64_t ldx,
                        const int32_t* qweight, const float* scales, const int32_t* zeros,
                        const int32_t* g_idx, const int32_t* x_order, int64_t n_groups,
                        int64_t out, int bits, void* Y, int y_dtype, int64_t ldy,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Scratch (bytes) of gptq_dequant_matmul_noalloc: one fixed array per device. */
#define GPTQ_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * gptq_dequant_matmul without a workspace, for callers that cannot allocate
 * device memory: code under HIP stream capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * Same arguments (minus the workspace), kernels and results, bit for bit, as
 * gptq_dequant_matmul.  Its scratch is a fixed device array of
 * GPTQ_NOALLOC_SCRATCH_BYTES (16 MiB) that each device holds until the
 * process ends.  Every product with M <= 8 fits; a larger M fits while
 * gptq_dequant_matmul_workspace_bytes(M, in, out, x_order != NULL) is at
 * most that size, otherwise the call returns GPTQ_ERR_WORKSPACE before
 * anything is enqueued.  The call allocates nothing (its first call on a
 * device looks up that device's array address, once).  The stream must
 * belong to the current device (else INVALID_ARG).  Calls that overlap on
 * one device (two streams, two host threads) share its array and race:
 * serialise them.
 * Errors: as gptq_dequant_matmul; WORKSPACE when the scratch is too small.
 */
int gptq_dequant_matmul_noalloc(const void* X, int x_dtype, int64_t M, int64_t in, int64_t ldx,
                                const int32_t* qweight, const float* scales, const int32_t* zeros,
                                const int32_t* g_idx, const int32_t* x_order, int64_t n_groups,
                                int64_t out, int bits, void* Y, int y_dtype, int64_t ldy,
                                void* stream);

/* Workspace (bytes) of gptq_dequant_group_order for in input positions. */
size_t gptq_dequant_group_order_workspace_bytes(int64_t in);

/*
 * Group order of a packed layer, for gptq_dequant_matmul.
 *
 * With desc_act ("desc_act", Key Parameters of "GPTQ > Using AutoGPTQ in
 * Practice") the groups follow the permuted column order, so g_idx of the
 * packed layer (original order) jumps between groups from one position to
 * the next.  This call sorts the input positions by group, ties by position
 * (stable): x_order[p] = the position of rank p, g_idx_sorted[p] =
 * g_idx[x_order[p]] (non-decreasing) and qweight_sorted the codes re-packed
 * in that order (code_sorted[r][p] = code[r][x_order[p]]).  Scales and zeros
 * are unchanged.  gptq_dequant_matmul(..., qweight_sorted, scales, zeros,
 * g_idx_sorted, x_order, ...) then computes the same Y as with the layer as
 * packed, the input column of each term being the same.  Meant to run once
 * per layer when it is loaded.
 *
 *   qweight, g_idx   the packed layer as above (device); in a positive
 *                    multiple of 32; out >= 1; bits 2, 3, 4 or 8.
 *   qweight_sorted   out: int32 [in * bits / 32 x out] (not aliasing qweight).
 *   g_idx_sorted, x_order  out: int32 [in].
 *   workspace        gptq_dequant_group_order_workspace_bytes(in) bytes.
 * Errors: INVALID_ARG, UNSUPPORTED (bits), WORKSPACE, HIP.
 */
int gptq_dequant_group_order(const int32_t* qweight, const int32_t* g_idx, int64_t in,
                             int64_t out, int bits, int32_t* qweight_sorted,
                             int32_t* g_idx_sorted, int32_t* x_order, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Gated activation of a Llama-style MLP block: A = SiLU(G) * U elementwise,
 * SiLU(g) = g / (1 + e^-g).
 *
 * The layer-wise method takes each layer's calibration inputs from the
 * block with its earlier layers already quantized (glossary entry "gptq",
 * paragraph "Method" (1)); the down projection's input is this product of
 * the gate and up projections' outputs.  The pages name the Llama layers but
 * not the activation: SiLU gating is the Llama MLP's (a reading).
 *
 *   G, U   fp16 [rows x cols], row-major, leading dimensions ldg, ldu >= cols
 *          (they may be the two halves of one [rows x 2 cols] matrix).
 *   A      out: fp16 [rows x cols], lda >= cols; may alias G or U exactly.
 * Arithmetic in fp32 (expf), one rounding to fp16.  rows or cols == 0 is a
 * no-op.  Errors: INVALID_ARG, HIP.
 */
int gptq_silu_mul(const void* G, int64_t ldg, const void* U, int64_t ldu, int64_t rows,
                  int64_t cols, void* A, int64_t lda, void* stream);

/*
 * Multi-head attention of a Llama-style decoder block, per sequence:
 *     O[t][h] = sum_{s} softmax_s(Q[t][h] . K[s][h] / sqrt(head_dim)) V[s][h],
 * s over the keys of t's own sequence (s <= t when causal != 0).
 *
 * The layer-wise method quantizes one layer at a time from calibration
 * activations computed through the block (glossary entry "gptq", paragraph
 * "Method" (1) and (3)); the output projection's calibration inputs are
 * this attention of the query, key and value projections.  The pages do not
 * give the block's arithmetic: causal softmax attention without positional
 * rotation is a reading (rotation changes the inputs, not the method).
 *
 *   Q, K, V  fp16 [seqs * seq_len x >= heads * head_dim], row-major with
 *            leading dimensions ldq, ldk, ldv; sequence b is rows
 *            b * seq_len .. b * seq_len + seq_len - 1; head h is columns
 *            h * head_dim .. + head_dim - 1 (they may be the three parts of
 *            one [tokens x 3 d] matrix).
 *   O        out: fp16, same layout, leading dimension ldo.
 *   head_dim 64 or 128; heads <= 65535; seqs <= 65535 per call.
 *   Pointers 16-byte aligned, leading dimensions multiples of 8.
 * Arithmetic: fp32 scores, softmax (exp2) and accumulation; the softmax
 * weights enter the value product as fp16; O rounded once to fp16.  seqs or
 * seq_len == 0 is a no-op.  Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
int gptq_attention_forward(const void* Q, int64_t ldq, const void* K, int64_t ldk, const void* V,
                           int64_t ldv, void* O, int64_t ldo, int64_t seqs, int64_t seq_len,
                           int heads, int head_dim, int causal, void* stream);

/*
 * Residual add and RMS normalization between the attention and MLP halves of
 * a Llama-style decoder block, per row r:
 *     Hs[r] = X[r] + A[r]                         (the residual stream, fp16)
 *     U[r]  = Hs[r] / sqrt(mean_c Hs[r][c]^2 + eps) * gamma
 *
 * The MLP's calibration inputs are computed through the block with the
 * attention layers already quantized (glossary entry "gptq", paragraph
 * "Method" (1)); the normalization is the Llama block's (a reading).
 *
 *   X, A     fp16 [rows x d] (leading dimensions ldx, lda >= d).
 *   gamma    fp16 [d].
 *   Hs, U    out: fp16 [rows x d] (ldh, ldu >= d).
 *   eps      finite, >= 0.
 * Sums in fp32 over the fp16 Hs; one rounding of each output.  rows == 0 is
 * a no-op.  Errors: INVALID_ARG, HIP.
 */
int gptq_residual_rmsnorm(const void* X, int64_t ldx, const void* A, int64_t lda,
                          const void* gamma, int64_t rows, int64_t d, float eps, void* Hs,
                          int64_t ldh, void* U, int64_t ldu, void* stream);

/*
 * Storage form of a layer's group parameters, for saving it.
 *
 * The pages save quantized models as safetensors files with a
 * quantize_config.json ("AutoGPTQ" catalogue page, Safetensors Support;
 * "GPTQ > Using AutoGPTQ in Practice", saving).  The layout of the stored
 * tensors is not given there; the reading taken: scales as fp16, and the
 * zero-points packed like the codes, as a dense little-endian b-bit stream,
 * here along the output channels: qzeros[g][w] is word w of the stream of
 * zeros[g][0 .. out-1] (zero r at bits [r b, (r+1) b)); zero-points are
 * stored as they are (no offset).
 *
 *   scales   fp32 [n_groups x out]; zeros int32 [n_groups x out], values in
 *            [0, 2^bits) (higher bits are dropped).
 *   scales_f16  out: fp16 [n_groups x out] (round to nearest).
 *   qzeros   out: int32 [n_groups x out * bits / 32].
 *   out * bits must be a multiple of 32; bits 2, 3, 4 or 8.
 * Errors: INVALID_ARG, UNSUPPORTED (bits, out * bits % 32), HIP.
 */
int gptq_export_params(const float* scales, const int32_t* zeros, int64_t n_groups, int64_t out,
                       int bits, void* scales_f16, int32_t* qzeros, void* stream);

/* zeros int32 [n_groups x out] from qzeros as gptq_export_params writes it
 * (the same conditions; errors as there). */
int gptq_unpack_zeros(const int32_t* qzeros, int64_t n_groups, int64_t out, int bits,
                      int32_t* zeros, void* stream);

/* Static text for a gptq_status_t value. */
const char* gptq_status_string(int status);

/* Detail of the last failing call on the calling host thread ("" if none). */
const char* gptq_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
