/*
 * gptq.h - C ABI of libgptq.so, a one-shot GPTQ quantizer for one linear
 * layer on AMD Instinct MI355X (gfx950).
 *
 * The method (GPTQ knowledge note, "How It Works"): record the layer's
 * inputs X, form the Hessian H = 2 X X^T of the layer-output reconstruction
 * loss, quantize the weight matrix one column at a time in one column order
 * shared by every row, adjust the still-unquantized columns with
 * inverse-Hessian information after each column, batch those corrections in
 * 128-column blocks before one global update, and take the correction rows
 * from a damped Cholesky formulation.  The result is a low-bit grid with
 * per-group scales (Wiki "GPTQ", "Technical Approach") and packed weights
 * (GPTQ knowledge note, "Tradeoffs": packed-weight kernels).
 *
 * Conventions for every call:
 *  - Pointers marked "device" point to device memory on the current HIP
 *    device; "host" pointers to host memory.  The caller owns and allocates
 *    every buffer, including the workspace (sized by the *_ws_bytes query of
 *    the call).  The library keeps no device allocation between calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls are asynchronous and stream-ordered, except
 *    gptq_prepare_hinv, gptq_lowrank_basis and gptq_lowrank_hessian, which
 *    synchronise `stream` once to report whether a matrix they factor was
 *    positive definite.
 *  - Row-major storage; `ld*` are leading dimensions in elements.
 *  - Every argument is validated on the host before anything is launched; a
 *    failed check returns an error and touches no memory.  Device data is
 *    not validated (NaN/Inf inputs propagate; codes >= 2^bits handed to
 *    gptq_pack are undefined).  A failed HIP call returns GPTQ_ERR_HIP.
 *  - Calls on distinct streams with distinct buffers may run concurrently.
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
  GPTQ_ERR_INVALID_ARG = 1,  /* null pointer, bad size or leading dimension */
  GPTQ_ERR_UNSUPPORTED = 2,  /* valid request the library does not implement */
  GPTQ_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the query */
  GPTQ_ERR_NOT_PD = 4,       /* damped Hessian not positive definite */
  GPTQ_ERR_HIP = 5           /* a HIP runtime call or kernel launch failed */
} gptq_status;

typedef enum { GPTQ_F32 = 0, GPTQ_F16 = 1, GPTQ_BF16 = 2 } gptq_dtype;

/* Human-readable name of a status code (static string). */
const char* gptq_status_string(int status);

/* ------------------------------------------------------------------------
 * Stage 1: Hessian accumulation.
 * GPTQ knowledge note, "How It Works": H = 2 X X^T over the recorded inputs
 * of the layer.  X is stored tokens x n (activation layout), so
 *     H <- (reset ? 0 : H) + alpha * X^T X ,  alpha = 2 gives the pages' H.
 *   H       device, n x n float32, leading dimension n.  Full symmetric on
 *           return (the upper triangle is computed and mirrored; with
 *           reset = 0 the upper triangle of the incoming H is the one used).
 *   X       device, tokens x n, element type x_dtype, leading dimension
 *           ldx >= n.  Any alignment; rows 16-byte aligned take the fast path.
 *   tokens  >= 0 (0 with reset = 0 leaves H unchanged).
 *   ws      device workspace of at least gptq_hessian_ws_bytes(n, tokens,
 *           x_dtype) bytes (NULL allowed when that is 0).
 * Arithmetic: products of 16-bit inputs are exact in float32.  The tokens
 * are cut into splits of at most 32768 tokens; within a split every entry of
 * the upper triangle is summed in one float32 matrix-core accumulator (16
 * tokens per instruction), and the splits' sums are added in float64 (with alpha and the
 * incoming H when reset = 0) before the one rounding to float32.  The
 * workspace holds the split sums: splits x upper 256 x 256 tiles x 256 KB
 * (about 2.4 GB for n = 12288 over 262144 tokens); it is written and read
 * back within the call.
 * ---------------------------------------------------------------------- */
size_t gptq_hessian_ws_bytes(int64_t n, int64_t tokens, int x_dtype);
gptq_status gptq_hessian_accumulate(float* H, int64_t n, const void* X, int x_dtype,
                                    int64_t tokens, int64_t ldx, float alpha, int reset,
                                    void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * H as gptq_hessian_accumulate (up to the float32 accumulation order), with
 * no workspace argument and no allocation.  The token-split partial sums
 * live in a static device array of GPTQ_HESSIAN_NOALLOC_SCRATCH_BYTES bytes
 * that the library holds on every device it runs on until the process ends.
 * When one split's partial tiles fill more than that (n > 12800) the call
 * returns GPTQ_ERR_UNSUPPORTED; otherwise the tokens are taken in passes of
 * as many splits as the array holds, each pass adding its float64 sum into H.
 * Calls on one device share the array: calls that overlap on one device
 * (concurrent streams or threads) race and give undefined results.  A failed
 * lookup of the array's device address returns GPTQ_ERR_HIP.  Arguments as
 * for gptq_hessian_accumulate. */
#define GPTQ_HESSIAN_NOALLOC_SCRATCH_BYTES (320u * 1024u * 1024u)
gptq_status gptq_hessian_accumulate_noalloc(float* H, int64_t n, const void* X, int x_dtype,
                                            int64_t tokens, int64_t ldx, float alpha, int reset,
                                            void* stream);

/* The two blocks asymmetric calibration needs (GPTAQ / GPTQv2 abstract, see
 * gptq_asym_target) from one pass over Xcat = [Xq | Xf] (tokens x 2n, Xq in
 * columns 0..n-1, Xf in n..2n-1): H2 (2n x 2n, row-major) receives
 * alpha Xq^T Xq (rows and columns 0..n-1) and alpha Xq^T Xf (rows 0..n-1,
 * columns n..2n-1), with their mirror images below the diagonal, as
 * gptq_hessian_accumulate on Xcat would (up to the float32 accumulation
 * order: the token splits may differ).  The block
 * alpha Xf^T Xf (rows and columns n..2n-1) is unspecified on return: when n
 * is a multiple of 2048 its tiles are not computed (a third of the work).
 * Arguments as for gptq_hessian_accumulate with 2n columns (ldx >= 2n);
 * n <= 32768.  Workspace: gptq_hessian_pair_ws_bytes(n, tokens, x_dtype)
 * bytes, which never exceeds gptq_hessian_ws_bytes(2n, tokens, x_dtype)
 * (0 for invalid arguments). */
size_t gptq_hessian_pair_ws_bytes(int64_t n, int64_t tokens, int x_dtype);
gptq_status gptq_hessian_pair_accumulate(float* H2, int64_t n, const void* Xcat, int x_dtype,
                                         int64_t tokens, int64_t ldx, float alpha, int reset,
                                         void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stage 2: damping, act-order and the inverse-Hessian factor.
 * GPTQ knowledge note, "How It Works": a damped Cholesky formulation
 * supplies the correction rows.  Computes
 *   lambda = damp_rel * mean(diag H)
 *   perm   = identity, or (act_order != 0) the columns sorted by descending
 *            diag H with ties kept in ascending index (stable)
 *   H_d    = H[perm][:, perm] + lambda * I
 *   U      = the upper-triangular factor with positive diagonal such that
 *            U^T U = H_d^{-1}   (row j of U / U_jj is column j's correction row)
 * U is obtained as R^{-1} where H_d = R R^T with R upper (a Cholesky
 * factorisation run from the last index to the first), in float64.
 *   H        device, n x n float32 (symmetric), read only.
 *   U        device, n x n float32 output, leading dimension n; lower
 *            triangle set to 0.
 *   perm     device, n int32 output (processing position -> original column).
 *   info_out host, may be NULL: 0, or the 1-based position k at which the
 *            factorisation of the index-reversed H_d met a non-positive (or
 *            non-finite) pivot, i.e. the trailing block H_d[n-k:, n-k:] is not
 *            positive definite.  Then GPTQ_ERR_NOT_PD is returned and U is
 *            undefined.
 *   ws       device workspace of gptq_prepare_ws_bytes(n) bytes.
 * Synchronises `stream` once, at the end.
 * ---------------------------------------------------------------------- */
size_t gptq_prepare_ws_bytes(int64_t n);
gptq_status gptq_prepare_hinv(const float* H, int64_t n, float damp_rel, int act_order,
                              float* U, int32_t* perm, int32_t* info_out,
                              void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stage 3: the column sweep with lazy block updates.
 * GPTQ knowledge note, "How It Works" (one column order for all rows,
 * 128-column blocks that accumulate corrections before a global update);
 * Wiki "GPTQ", "Technical Approach" (low-bit grid, group-wise scales).
 * For processing position j (original column perm[j]) of every row r:
 *   at a group start: xmin = min(0, min w), xmax = max(0, max w) over the
 *     current values of the group's columns (whole original row when
 *     group_size = 0); an all-zero range is taken as [-1, 1];
 *     s = fl32(fl32(xmax - xmin) / maxq), z = clamp(rint(fl32(-xmin/s)), 0, maxq)
 *   c = clamp(rint(fl32(w_rj / s)) + z, 0, maxq)      (float32, IEEE division,
 *                                                     round half to even)
 *   e = (w_rj - s*(c - z)) / U_jj
 *   w_rk -= e * U_jk for the later columns k of the block; the later blocks
 *   receive the block's corrections as one matrix product.
 * maxq = levels - 1.  Groups are group_size consecutive processing
 * positions; "current values" at a group start include every correction of
 * the columns before it (also for groups wider than a block).
 *   W          device, m x n, element type w_dtype, leading dimension ldw
 *              >= n; read only.
 *   U          device, n x n float32 from gptq_prepare_hinv (processing order).
 *   perm       device, n int32 processing order (a permutation of 0..n-1),
 *              or NULL for the identity.
 *   levels     3 (ternary), 4 (2-bit), 8 (3-bit) or 16 (4-bit).
 *   group_size 0 (one grid per row), a divisor of 128 (1, 2, 4, ..., 128)
 *              or a multiple of 128; others return GPTQ_ERR_UNSUPPORTED.
 *   block_size 128.
 * Outputs (original column order unless noted):
 *   codes      device, m x n uint8 (leading dimension n): codes[r*n + k] is the
 *              code of original column k.
 *   scales     device, m x G float32, G = 1 if group_size = 0 else
 *              ceil(n / group_size); group g covers processing positions
 *              [g*group_size, (g+1)*group_size).
 *   zeros      device, m x G uint8.
 *   g_idx      device, n int32 or NULL: the group of original column k,
 *              g_idx[perm[j]] = j / group_size (all 0 when group_size = 0).
 *   row_loss   device, m float32 = sum_j e_rj^2 / 2 per row, or NULL.
 *   Wq         device, m x n (leading dimension n) dequantized weights in
 *              w_dtype, or NULL: Wq[r][k] = fl_w(fl32(s (c - z))) with the
 *              scale and zero of column k's group, rounded to nearest even.
 *   ws         device workspace of gptq_quantize_ws_bytes(m, n, block_size)
 *              bytes (0 for invalid arguments).
 * Every row is independent: running a subset of rows gives those rows'
 * results exactly.  With m = 0 only g_idx is written.
 * ---------------------------------------------------------------------- */
size_t gptq_quantize_ws_bytes(int64_t m, int64_t n, int block_size);
gptq_status gptq_quantize_layer(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw,
                                const float* U, const int32_t* perm,
                                int levels, int group_size, int block_size,
                                uint8_t* codes, float* scales, uint8_t* zeros, int32_t* g_idx,
                                float* row_loss, void* Wq, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stage 4: pack (GPTQ knowledge note, "Tradeoffs": packed weights; Wiki
 * "GPTQ", "Performance and Accuracy": 4 bits per weight).
 *   codes      device, m x n uint8 in original column order (as
 *              gptq_quantize_layer writes them), values < 2^bits.
 *   bits       2, 3 or 4.
 *   packed     device, m x ld_packed uint32 output; ld_packed >=
 *              ceil(n*bits/32).  Row r's codes form a little-endian bit
 *              stream: code of column k occupies bits [k*bits, (k+1)*bits)
 *              of the row; unused tail bits are 0; words beyond
 *              ceil(n*bits/32) are not written.
 * ---------------------------------------------------------------------- */
gptq_status gptq_pack(const uint8_t* codes, int64_t m, int64_t n, int bits, uint32_t* packed,
                      int64_t ld_packed, void* stream);

/* ------------------------------------------------------------------------
 * Asymmetric calibration (GPTAQ / GPTQv2 abstract, Daily Papers and mlsanity
 * pages: the quantized layer's output on the quantized model's inputs Xq is
 * matched to the full-precision output on the full-precision inputs Xf).
 * Because ||Xq Q^T - Xf W^T||^2 = ||Xq (Q - W')^T||^2 + const for the
 * least-squares target W' (a derivation: the pages give no closed form), the
 * method is GPTQ with H = 2 Xq^T Xq applied to W'.  This call forms
 *   W' = W Hc^T H_d^{-1},   Hc = 2 Xq^T Xf,   H_d^{-1} = U^T U,
 * with GPTQ's own damping inside U.  Typical use: one
 * gptq_hessian_accumulate over [Xq | Xf] (tokens x 2n, side by side) gives
 * H (top-left n x n block, prepared as usual) and Hc (top-right block);
 * then gptq_quantize_layer(W', U, perm).
 *   W      device, m x n (ldw >= n), element type w_dtype; read only.
 *   Hc     device, n x n float32, leading dimension ldhc >= n.
 *   U, perm  from gptq_prepare_hinv on H (perm NULL for the identity).
 *   Wt     device, m x n float32 output (ldwt >= n), original column order.
 *   ws     device workspace of gptq_asym_target_ws_bytes(m, n) bytes.
 * float32 products (matrix cores), float32 rounding of W Hc^T, of the product
 * with U^T and with U.
 * ---------------------------------------------------------------------- */
size_t gptq_asym_target_ws_bytes(int64_t m, int64_t n);
gptq_status gptq_asym_target(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw,
                             const float* Hc, int64_t ldhc, const float* U, const int32_t* perm,
                             float* Wt, int64_t ldwt, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Low-rank correction folded into the GPTQ pass (GPTQ-intrinsic LoRA
 * abstract, Daily Papers page): W is approximated as Q + (L R)^T with L
 * n x r and R r x m, judged by ||(W - Q - R^T L^T) X^T||^2, with the choice
 * L = V_r (top-r right singular vectors of X).  The page prints no formula
 * for its Hessian augmentation; the one used here follows from the
 * objective: for a fixed L the least-squares R is
 *   R* = K^T (W - Q)^T,   K = H L M^{-1},   M = L^T H L,
 * and what is left to minimise over Q is GPTQ's objective with
 *   H_L = H - H L M^{-1} L^T H.
 * Sequence: gptq_hessian_accumulate (H) -> gptq_lowrank_basis (L) ->
 * gptq_lowrank_hessian (H_L, K) -> gptq_prepare_hinv(H_L) ->
 * gptq_quantize_layer -> gptq_pack -> gptq_lowrank_compensation (R*).
 * H_L and R* depend on L only through its column span.
 * Float64 arithmetic throughout; H and H_L are float32, R float32.
 * Matrices with r columns (Omega, L, K) are device float64, row-major
 * n x r (leading dimension r).  1 <= r <= GPTQ_LOWRANK_MAX_RANK, r <= n.
 * ---------------------------------------------------------------------- */
#define GPTQ_LOWRANK_MAX_RANK 64

/* Workspace for all three calls below on a layer of m rows (m may be 0 for
 * the first two); 0 for an invalid n or r. */
size_t gptq_lowrank_ws_bytes(int64_t m, int64_t n, int64_t r);

/* L = V_r by subspace iteration: Q_0 = orth(Omega), Q_{t+1} = orth(H Q_t)
 * for `iters` steps, orthonormalised by Cholesky-QR, plus one final
 * Cholesky-QR pass.  The span converges to that of V_r at the rate
 * (lambda_{r+1} / lambda_r)^iters of H's eigenvalues.
 *   H      device, n x n float32 symmetric (ldh >= n), e.g. from
 *          gptq_hessian_accumulate; rows are read as columns.
 *   Omega  device, n x r float64 starting block (random numbers drawn by
 *          the caller); read only.
 *   iters  >= 0.
 *   L      device, n x r float64 output, orthonormal columns.
 * Synchronises `stream` once; returns GPTQ_ERR_NOT_PD if a Cholesky-QR
 * Gram matrix was not positive definite (a rank-deficient block). */
gptq_status gptq_lowrank_basis(const float* H, int64_t n, int64_t ldh, int64_t r, const double* Omega,
                               int iters, double* L, void* ws, size_t ws_bytes, void* stream);

/* H_L = H - Z Z^T and K = Z C^{-1}, where Z = H L C^{-T} and C C^T = L^T H L
 * (Cholesky).
 *   H      device, n x n float32 symmetric (ldh >= n).
 *   L      device, n x r float64 (any basis of the correction's span).
 *   H_L    device, n x n float32 output (ldhl >= n), symmetric; must not
 *          alias H.  Pass it to gptq_prepare_hinv (act-order and damping
 *          then apply to H_L).
 *   K      device, n x r float64 output (for gptq_lowrank_compensation).
 * Synchronises `stream` once; returns GPTQ_ERR_NOT_PD if L^T H L is not
 * positive definite. */
gptq_status gptq_lowrank_hessian(const float* H, int64_t n, int64_t ldh, const double* L, int64_t r,
                                 float* H_L, int64_t ldhl, double* K, void* ws, size_t ws_bytes,
                                 void* stream);

/* R[a][i] = sum_c K[c][a] (W[i][c] - W^[i][c]): the least-squares R for the
 * quantized weights W^[i][c] = scales[i][g(c)] (codes[i][c] -
 * zeros[i][g(c)]), g(c) = g_idx[c], or c / group_size when g_idx is NULL
 * (0 when group_size = 0).
 *   W, w_dtype, m, n, ldw   the layer as given to gptq_quantize_layer.
 *   codes, scales, zeros    gptq_quantize_layer's outputs (codes in original
 *                           column order), group_size as given to it.
 *   g_idx                   gptq_quantize_layer's g_idx output (needed with
 *                           act-order), or NULL.
 *   K      device, n x r float64 from gptq_lowrank_hessian.
 *   R      device, r x m float32 output (ldr >= m).
 * Does not synchronise. */
gptq_status gptq_lowrank_compensation(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw,
                                      const uint8_t* codes, const float* scales, const uint8_t* zeros,
                                      int group_size, const int32_t* g_idx, const double* K, int64_t r,
                                      float* R, int64_t ldr, void* ws, size_t ws_bytes, void* stream);

/* Fixed-grid refinement of the codes, to alternate with
 * gptq_lowrank_compensation (Daily Papers page, GPTQ-intrinsic LoRA abstract:
 * "Bid-Up", a refinement on the fixed grid that alternates with the optimal
 * low-rank compensation and never increases the layer-wise error; the page
 * prints no algorithm).  Reading implemented: cyclic coordinate descent.
 * With the grid (scales, zeros) and the correction C = (L R)^T held fixed,
 * row i's error 1/2 d H d^T, d = W_i - C_i - W^_i, is lowered one column at
 * a time in original column order: column j's code becomes the one whose
 * grid value s (c - z) is nearest to W^_ij + g_j / H_jj, g = H d, when that
 * lowers the error (a tie keeps the code; columns with H_jj <= 0 keep
 * theirs).  The error never increases.  Float64 throughout.
 * Two uses with the compensation: H = 2 X^T X with the current (L, R) held
 * fixed (the literal alternation), or H = H_L from gptq_lowrank_hessian
 * with r = 0: min over R of the joint error is 1/2 d H_L d^T with
 * d = W - W^, so every move is then optimal over the code and R together
 * (recompute R with gptq_lowrank_compensation afterwards).
 *   W, w_dtype, m, n, ldw   the layer (float32, float16 or bfloat16), m, n >= 1.
 *   H      device, n x n float32 (ldh >= n), exactly symmetric: the
 *          undamped calibration Hessian (as gptq_hessian_accumulate writes
 *          it) or H_L (as gptq_lowrank_hessian writes it).
 *   L, R   the correction: L device n x r float64 (leading dimension r), R
 *          device r x m float32 (ldr >= m), as gptq_lowrank_basis and
 *          gptq_lowrank_compensation write them; r = 0 for none (L, R may
 *          then be NULL).  0 <= r <= GPTQ_LOWRANK_MAX_RANK, r <= n.
 *   scales, zeros, group_size, g_idx   the fixed grid, as for
 *          gptq_lowrank_compensation (m x G, G = ceil(n / group_size) or 1).
 *   levels 2 .. 256 (codes stay in [0, levels - 1]).
 *   sweeps >= 0 passes over all columns (0: nothing is launched).
 *   codes  device, m x n uint8, original column order: read, and
 *          overwritten with the refined codes.
 *   moves  device int64[sweeps] output (the number of codes changed in each
 *          pass), or NULL.
 * Workspace gptq_refine_ws_bytes(m, n) (0 for sizes it does not take: m or n
 * outside 1 .. 2^31 - 1, or m n > 2^48).  Does not synchronise. */
size_t gptq_refine_ws_bytes(int64_t m, int64_t n);
gptq_status gptq_refine_codes(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw, const float* H,
                              int64_t ldh, const double* L, const float* R, int64_t r, int64_t ldr,
                              const float* scales, const uint8_t* zeros, int group_size, const int32_t* g_idx,
                              int levels, int sweeps, uint8_t* codes, int64_t* moves, void* ws, size_t ws_bytes,
                              void* stream);

/* ------------------------------------------------------------------------
 * Reading the packed weights back: matrix-vector product for decode
 * (GPTQ knowledge note, "Tradeoffs": the speed of a quantized model rests on
 * kernels that consume the packed weights, inference being limited by weight
 * memory traffic; anthology record SOTA-185, "The scope worth holding onto":
 * decode is bandwidth-bound).
 *   Y[b, r] = sum_k scales[r, g(k)] * (c[r, k] - zeros[r, g(k)]) * X[b, k]
 * for b < batch, r < m, where c[r, k] is column k's code in row r of `packed`.
 *   packed     device, m x ld_packed uint32 in the layout gptq_pack writes
 *              (bits 2, 3 or 4; ld_packed >= ceil(n*bits/32)).
 *   scales     device, m x G float32; zeros device, m x G uint8 (G >= 1).
 *   g_idx      device, n int32 (the group of each column, < G) or NULL: then
 *              g(k) = k / group_size, or 0 when group_size = 0.
 *              gptq_quantize_layer's g_idx output (act-order) can be passed
 *              as is.
 *   X          device, batch x ldx IEEE binary16 (ldx >= n).
 *   Y          device, batch x ldy float32 output (ldy >= m), overwritten.
 *   batch      >= 1 (GPTQ_ERR_INVALID_ARG otherwise).
 * Accumulation is float32; the rounding error of Y[b, r] is bounded by a
 * small multiple of (n/32 + 64) 2^-24 sum_k s (c + z) |X[b, k]|.  Group
 * indices in g_idx are not validated (an index >= G reads out of bounds).
 * Batches of 3 or more with g_idx NULL and group_size 0 or a multiple of 128
 * run on the matrix cores (as gptq_dequant_gemm); otherwise a VALU kernel
 * takes GPTQ_GEMV_MAX_BATCH rows of X per pass (each pass reads the packed
 * weights once).  No workspace.
 * ---------------------------------------------------------------------- */
#define GPTQ_GEMV_MAX_BATCH 8
gptq_status gptq_dequant_gemv(const uint32_t* packed, int64_t m, int64_t n, int64_t ld_packed,
                              int bits, const float* scales, const uint8_t* zeros, int64_t G,
                              int group_size, const int32_t* g_idx, const uint16_t* X,
                              int64_t batch, int64_t ldx, float* Y, int64_t ldy, void* stream);

/* ------------------------------------------------------------------------
 * Reading the packed weights back on the matrix cores, for any batch
 * (batched decode and prefill; same sources as gptq_dequant_gemv): the same
 * Y as gptq_dequant_gemv for batch >= 0 rows of X (batch 0 is a no-op), with
 * the same arguments and rounding bound.  Groups that are contiguous and 0
 * or a multiple of 128 columns wide (g_idx NULL) run on the matrix cores;
 * act-order (g_idx given) or narrower groups run on the VALU kernel, eight
 * rows of X per pass.  No workspace.
 * ---------------------------------------------------------------------- */
gptq_status gptq_dequant_gemm(const uint32_t* packed, int64_t m, int64_t n, int64_t ld_packed,
                              int bits, const float* scales, const uint8_t* zeros, int64_t G,
                              int group_size, const int32_t* g_idx, const uint16_t* X, int64_t batch,
                              int64_t ldx, float* Y, int64_t ldy, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
