/*
 * lh.h - C ABI of the Local-Hessian NVFP4 weight-scale calibration library
 *        (liblh.so, HIP kernels for AMD Instinct MI355X / gfx950).
 *
 * The method (pages cited by title and section):
 *   "Local-Hessian weight-scale guide" (xxmr.cn/news/266017)
 *     - "What is Local-Hessian": NVFP4 stores FP4 E2M1 values, 16 weights
 *       share one FP8 E4M3 block scale, a block scale maps the block into
 *       the E2M1 range [-6, 6]; the scale sweep tries all 126 positive
 *       non-zero FP8 values.
 *     - "Algorithm principle": linear layer Y = W X with W [C_out x C_in]
 *       and calibration input X [C_in x N]; Q(W, s) = Cast(W / s) * s,
 *       Delta = Q - W; output error E(s) = ||Delta X||_F^2 =
 *       tr(Delta X X^T Delta^T); block-diagonal approximation per 16-weight
 *       block b: E_b(s_b) = Delta_b (X_b X_b^T) Delta_b^T; the sweep kernel
 *       takes weights [N_BLOCKS, 16] in (cout, cin // 16) order, the global
 *       FP32 amax and per-block Hessians [cin // 16, 16, 16], minimises
 *       dw^T H dw over the 126 E4M3 candidates and outputs the per-block
 *       best amax; candidate generation is bit-consistent with fake-quant.
 *     - "Entry API and calibration flow", phase 2: H accumulates the sum of
 *       X^T X over calibration batches; phase 3 passes the normalised
 *       per-block Hessian to the search.
 *     - "Combining with GPTQ": the cast rounds to nearest (RTN).
 *   "ModelOpt overview" (linlog.top/article/1517), "Local-Hessian": 126
 *     candidate scales per block, each block optimised independently.
 *
 * Readings taken where the pages leave a step open:
 *   - candidates: the 126 positive finite OCP E4M3FN values (codes
 *     0x01..0x7E, max 448); candidate index k <-> E4M3 code k + 1;
 *   - S_g = fl32(g / 2688) (2688 = 6 * 448), s_k = fl32(c_k * S_g);
 *   - Cast: x = fl32(|w| / s_k) (IEEE division), nearest E2M1 magnitude
 *     {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, saturation at 6;
 *     Q = fl32(sign(w) * r * s_k), -0 written as +0; s_k = 0 gives Q = 0;
 *   - "normalised" = divided by the token count N (alpha = 1 / N);
 *   - equal errors resolve to the lowest candidate index.
 *
 * Conventions for every entry point:
 *   - all data pointers are DEVICE pointers (hipMalloc'd or a framework's
 *     device tensor); the caller owns and frees every buffer;
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream);
 *     every call only enqueues work on it and returns; the library never
 *     synchronises the device, never allocates, keeps no state between
 *     calls and is safe to call from several host threads;
 *   - arguments are validated on the host before anything is launched; a
 *     non-zero lh_status means nothing was enqueued (LH_ERR_HIP: a launch
 *     failed; lh_last_error_message() holds the HIP error text);
 *   - sizes are element counts; strides / leading dimensions are in
 *     elements of the buffer's own dtype;
 *   - empty problems (a zero size) are valid and enqueue nothing, except the
 *     Hessian with n_tokens = 0, which still applies h = beta * h;
 *   - non-finite inputs give unspecified (but memory-safe) results.
 */
#ifndef LH_H
#define LH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lh_status {
    LH_OK = 0,
    LH_ERR_NULL = 1,      /* a required pointer is NULL                      */
    LH_ERR_SHAPE = 2,     /* negative size, c_in % 16 != 0, ld / stride too small */
    LH_ERR_DTYPE = 3,     /* unknown dtype code                               */
    LH_ERR_LAYOUT = 4,    /* unknown layout code                              */
    LH_ERR_WORKSPACE = 5, /* workspace non-empty but smaller than required    */
    LH_ERR_ARG = 6,       /* other invalid argument (e.g. no output requested) */
    LH_ERR_HIP = 7        /* a HIP launch failed (see lh_last_error_message)  */
} lh_status;

typedef enum lh_dtype {
    LH_DTYPE_F32 = 0,  /* IEEE binary32                                       */
    LH_DTYPE_BF16 = 1  /* bfloat16 (upper half of binary32), RNE-rounded data */
} lh_dtype;

typedef enum lh_layout {
    LH_LAYOUT_CHANNEL_MAJOR = 0, /* x[c * ld_x + t]: X as [C_in][N] (the pages' X) */
    LH_LAYOUT_TOKEN_MAJOR = 1    /* x[t * ld_x + c]: X^T as [N][C_in] (hooked activations) */
} lh_layout;

typedef enum lh_rule {
    LH_RULE_SWEEP = 0,         /* all 126 E4M3 candidates (the Local-Hessian sweep) */
    LH_RULE_MAX = 1,           /* max scaling: the block's amax maps to 6           */
    LH_RULE_FOUR_OVER_SIX = 2, /* best of amax -> 6 and amax -> 4                   */
    LH_RULE_AMAX_SEARCH = 3    /* amax multipliers 0.25, 0.35, ..., 3.95            */
} lh_rule;

/* Library ABI version (this header describes version 1). */
int lh_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char *lh_status_string(int status);

/* Message of the last failing call on this host thread ("" if none). */
const char *lh_last_error_message(void);

/*
 * Global amax per group:  amax[g] = max |w[g][r][c]| over r < rows, c < cols.
 * The per-tensor FP32 amax the sweep derives its candidates from ("Algorithm
 * principle": the kernel receives the global FP32 amax).
 *   w        [n_groups] x [rows][ld_w] elements of w_dtype, group stride
 *            group_stride_w (>= 0).
 *   amax     [n_groups] fp32, written (device).
 * ld_w >= cols.  rows, cols, n_groups >= 0 (rows * cols == 0 writes 0).
 * Result is exact (a max), independent of launch shape.
 */
lh_status lh_absmax(const void *w, int w_dtype, int64_t rows, int64_t cols, int64_t ld_w,
                    int64_t n_groups, int64_t group_stride_w, float *amax, void *stream);

/*
 * The normalisation factor that lh_accumulate_hessian and lh_full_hessian
 * apply for a given alpha: alpha itself, or for alpha = NaN the normalised
 * Hessian's factor 1/N of "Entry API and calibration flow", phase 3 (the
 * per-block Hessian normalised by the token count), as fl32(1/n_tokens), and 0
 * for n_tokens <= 0.  Pure host function; lh_calibrate_* use the same factor.
 */
float lh_hessian_alpha(float alpha, int64_t n_tokens);

/*
 * Scratch bytes that let lh_accumulate_hessian split the token dimension of
 * each block over several workgroups and reduce the partial sums in a fixed
 * order (deterministic).  0 bytes is always accepted (one workgroup per
 * block); the value depends only on the three sizes.
 */
size_t lh_hessian_workspace_bytes(int64_t c_in, int64_t n_tokens, int64_t n_groups);

/*
 * Local-Hessian accumulation ("Algorithm principle": local Hessian
 * X_b X_b^T, 16 x 16 per input block; "Entry API and calibration flow",
 * phase 2: H is the sum of X^T X, normalised before the search):
 *
 *   h[g][b][i][j] = beta * h[g][b][i][j]
 *                 + alpha * sum_{t < n_tokens} X[g][16b+i][t] * X[g][16b+j][t]
 *
 * for every group g < n_groups, input block b < c_in / 16, 0 <= i, j < 16.
 * alpha = NaN asks for the normalised Hessian's factor: the library uses
 * lh_hessian_alpha(NaN, n_tokens) = fl32(1/n_tokens) (0 when n_tokens = 0).
 * alpha = 1/n_tokens (or NaN), beta = 0 gives the normalised one-shot
 * Hessian; alpha = 1, beta = 1 streams further token chunks into h.  beta == 0 never
 * reads h (so h may be uninitialised).  Products are exact (bf16 x bf16 or
 * fp32 x fp32 on matrix cores), sums are fp32.
 *   x        activations, x_dtype, `layout` (see lh_layout), leading
 *            dimension ld_x (channel-major: >= n_tokens; token-major:
 *            >= c_in), group stride group_stride_x (>= 0).
 *   h        [n_groups][c_in/16][16][16] fp32, group stride group_stride_h
 *            (>= (c_in/16)*256 when n_groups > 1), read (beta != 0) and written.
 *   workspace, workspace_bytes: NULL/0, or a device buffer of at least
 *            lh_hessian_workspace_bytes(c_in, n_tokens, n_groups) bytes,
 *            4-byte aligned; contents on entry are ignored.
 * c_in % 16 == 0.  Errors: LH_ERR_NULL, LH_ERR_SHAPE, LH_ERR_DTYPE,
 * LH_ERR_LAYOUT, LH_ERR_WORKSPACE, LH_ERR_HIP.
 */
lh_status lh_accumulate_hessian(const void *x, int x_dtype, int layout, int64_t c_in,
                                int64_t n_tokens, int64_t ld_x, int64_t n_groups,
                                int64_t group_stride_x, float alpha, float beta, float *h,
                                int64_t group_stride_h, void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * Scratch bytes lh_accumulate_hessian_ragged can use for its deterministic
 * split of each group's rows (0 = it runs one pass per block).  Depends only
 * on the arguments (max_group_rows as passed to the accumulation).
 */
size_t lh_hessian_ragged_workspace_bytes(int64_t c_in, int64_t n_rows, int64_t n_groups,
                                         int64_t max_group_rows);

/*
 * Ragged / streaming local Hessians ("Entry API and calibration flow",
 * phase 2: forward hooks capture each layer's token-major inputs batch by
 * batch and accumulate X^T X; MoE experts receive only their routed tokens,
 * so their token counts differ and may be zero; phase 3 normalises by the
 * token count).
 *
 * x is token-major, x[t * ld_x + c] for rows t < n_rows; rows
 * token_offsets[g] .. token_offsets[g+1]-1 belong to group g (expert g),
 * n_g = their count.  With S_g[b] = sum over those rows of x_b x_b^T:
 *   token_counts == NULL:  h[g] = S_g / n_g for groups with n_g > 0.
 *   token_counts != NULL:  running mean over calls,
 *                          h[g] = (n_old h[g] + S_g) / (n_old + n_g),
 *                          n_old = token_counts[g]; then token_counts[g] += n_g.
 * A group that receives no row keeps h[g] unchanged (the caller's fallback,
 * e.g. the identity, which makes the sweep the plain weight-error sweep).
 *   x             fp32 or bf16 (x_dtype), ld_x >= c_in.
 *   token_offsets device int64 [n_groups + 1], 8-byte aligned; expected
 *                 non-decreasing within [0, n_rows].  Offsets are clamped to
 *                 [0, n_rows] and a decreasing pair gives an empty group, so
 *                 no offset can make the kernels read outside x.
 *   h             fp32 [n_groups][c_in/16][16][16], group stride
 *                 group_stride_h (>= (c_in/16)*256 when n_groups > 1).
 *   max_group_rows  host-side bound on any group's row count, or 0 if
 *                 unknown.  It only shapes the work split (with it, the rows
 *                 of the largest group spread over many workgroups in 1024-row
 *                 slices; without it, the split follows the average group);
 *                 results are correct whatever it is.
 *   token_counts  NULL, or device int64 [n_groups] (8-byte aligned), read
 *                 and updated on the stream.
 *   workspace     NULL/0, or at least lh_hessian_ragged_workspace_bytes(c_in,
 *                 n_rows, n_groups, max_group_rows) bytes (4-byte aligned).
 * Results are deterministic (fixed reduction order).
 * Errors: LH_ERR_NULL, LH_ERR_SHAPE, LH_ERR_DTYPE, LH_ERR_WORKSPACE,
 * LH_ERR_ARG, LH_ERR_HIP.
 */
lh_status lh_accumulate_hessian_ragged(const void *x, int x_dtype, int64_t c_in, int64_t ld_x,
                                       int64_t n_rows, const int64_t *token_offsets,
                                       int64_t n_groups, int64_t max_group_rows, float *h,
                                       int64_t group_stride_h,
                                       int64_t *token_counts, void *workspace,
                                       size_t workspace_bytes, void *stream);

/*
 * Scratch bytes that let lh_scale_sweep skip provably worse candidates with a
 * tight per-block certificate (a lower bound on the smallest eigenvalue of
 * the block's correlation matrix, one fp32 per block).  0 bytes is always
 * accepted: the sweep then uses a weaker certificate computed on the fly.
 * Results are identical either way; only the speed differs.
 */
size_t lh_sweep_workspace_bytes(int64_t c_in, int64_t n_groups);

/*
 * Local-Hessian scale sweep ("Algorithm principle": per 16-weight block,
 * all 126 FP8 E4M3 candidate scales derived from the global FP32 amax,
 * minimise dw^T H_b dw with dw = Q(w, s) - w; "ModelOpt overview",
 * "Local-Hessian": blocks are independent).
 *
 * For every group g, output row r < c_out and input block b < c_in/16, with
 * w_b = w[g][r][16b .. 16b+15], H_b = h[g][b] and global amax amax[g]:
 *   k*  = the lowest k in [0, 125] minimising E_k = dw_k^T H_b dw_k
 *   best_idx [g][r][b] = k*              (E4M3 block-scale code = k* + 1)
 *   best_err [g][r][b] = E_k* (fp32)     (optional)
 *   best_amax[g][r][b] = fl32(6 * s_k*)  (optional; the per-block amax)
 * The minimum is exact over all 126 candidates: a candidate is only skipped
 * when a certified lower bound proves it worse than one already evaluated.
 *   w         weights, w_dtype, row stride ld_w >= c_in, group stride
 *             group_stride_w (>= 0).
 *   h         fp32 [n_groups][c_in/16][16][16], 16-byte aligned (any square
 *             matrix is used as given; the output of lh_accumulate_hessian
 *             fits), group stride group_stride_h (>= 0, multiple of 4).
 *   amax      fp32 [n_groups] (device), e.g. from lh_absmax.
 *   best_idx  uint8 [n_groups][c_out][c_in/16], required.
 *   best_err, best_amax  fp32, same shape, NULL to skip.
 *   workspace, workspace_bytes: NULL/0, or a device buffer of at least
 *             lh_sweep_workspace_bytes(c_in, n_groups) bytes, 4-byte
 *             aligned; contents on entry are ignored.
 * Errors: LH_ERR_NULL, LH_ERR_SHAPE, LH_ERR_DTYPE, LH_ERR_WORKSPACE,
 * LH_ERR_ARG, LH_ERR_HIP.
 */
lh_status lh_scale_sweep(const void *w, int w_dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                         int64_t n_groups, int64_t group_stride_w, const float *h,
                         int64_t group_stride_h, const float *amax, uint8_t *best_idx,
                         float *best_err, float *best_amax, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * The sweep and the fake-quant with its result in one pass ("Algorithm
 * principle": the candidate scales are bit-consistent with fake-quant, and
 * Q(W, s) = Cast(W / s) * s is the path's end product).  Writes exactly what
 * lh_scale_sweep followed by lh_fake_quant_nvfp4 with the chosen indices
 * writes, from one sweep launch that also emits the quantised blocks (each
 * lane quantises the rows it has just swept, so the weights are read again
 * from cache rather than by a second pass over the layer).
 *   Arguments up to workspace_bytes: as lh_scale_sweep (best_idx required).
 *   w_q, packed_e2m1, scale_e4m3, global_scale: as lh_fake_quant_nvfp4
 *             (dense layouts, each optional; w_q 16-byte aligned,
 *             packed_e2m1 8-byte aligned).
 * Errors: LH_ERR_NULL, LH_ERR_SHAPE, LH_ERR_DTYPE, LH_ERR_WORKSPACE,
 * LH_ERR_ARG, LH_ERR_HIP.
 */
lh_status lh_scale_sweep_fake_quant(const void *w, int w_dtype, int64_t c_out, int64_t c_in,
                                    int64_t ld_w, int64_t n_groups, int64_t group_stride_w,
                                    const float *h, int64_t group_stride_h, const float *amax,
                                    uint8_t *best_idx, float *best_err, float *best_amax,
                                    float *w_q, uint8_t *packed_e2m1, uint8_t *scale_e4m3,
                                    float *global_scale, void *workspace, size_t workspace_bytes,
                                    void *stream);

/*
 * Scratch bytes lh_calibrate_nvfp4 needs: the per-block skip certificates
 * and the Hessian's per-slice partial sums (and partial amax values).
 */
size_t lh_calibrate_workspace_bytes(int64_t c_out, int64_t c_in, int64_t n_tokens, int64_t n_groups);

/*
 * The first half of lh_calibrate_nvfp4: amax and h (as lh_absmax and
 * lh_accumulate_hessian with alpha = fl32(1/N), beta = 0), and the sweep's
 * skip certificates, which stay in the workspace for lh_calibrate_sweep.
 * Arguments as lh_calibrate_nvfp4.  With channel-major X and a contiguous W
 * (ld_w == c_in), both 16-byte aligned, this is two launches (amax and the
 * Hessian's token slices in one, the Hessian's finalisation with the
 * certificates in the other).
 * Errors: LH_ERR_NULL, LH_ERR_SHAPE, LH_ERR_DTYPE, LH_ERR_LAYOUT,
 * LH_ERR_WORKSPACE, LH_ERR_ARG, LH_ERR_HIP.
 */
lh_status lh_calibrate_prologue(const void *w, int w_dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                                int64_t n_groups, int64_t group_stride_w, const void *x, int x_dtype,
                                int x_layout, int64_t n_tokens, int64_t ld_x, int64_t group_stride_x,
                                float *amax, float *h, int64_t group_stride_h, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * The second half of lh_calibrate_nvfp4: lh_scale_sweep_fake_quant with the
 * certificates that lh_calibrate_prologue left in the workspace (same
 * workspace, same h and w, in stream order; no other call may write the
 * workspace in between).  Arguments as lh_scale_sweep_fake_quant; the
 * workspace is required.
 * Errors: LH_ERR_NULL, LH_ERR_SHAPE, LH_ERR_DTYPE, LH_ERR_WORKSPACE,
 * LH_ERR_ARG, LH_ERR_HIP.
 */
lh_status lh_calibrate_sweep(const void *w, int w_dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                             int64_t n_groups, int64_t group_stride_w, const float *h,
                             int64_t group_stride_h, const float *amax, uint8_t *best_idx,
                             float *best_err, float *best_amax, float *w_q, uint8_t *packed_e2m1,
                             uint8_t *scale_e4m3, float *global_scale, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * The whole calibration path for a layer in one call: the global amax of W
 * ("Algorithm principle": the kernel receives the global FP32 amax), the
 * normalised local Hessians H_b = X_b X_b^T / N ("Entry API and calibration
 * flow", phase 3), the 126-candidate sweep and the fake-quant of its result
 * (as lh_scale_sweep_fake_quant).  Every output equals what lh_absmax,
 * lh_accumulate_hessian (alpha = fl32(1/N), beta = 0), lh_scale_sweep and
 * lh_fake_quant_nvfp4 write, bit for bit.
 *   w, w_dtype, c_out, c_in, ld_w, n_groups, group_stride_w: as lh_scale_sweep.
 *   x, x_dtype, x_layout, n_tokens, ld_x, group_stride_x: as
 *             lh_accumulate_hessian (N = n_tokens; N = 0 gives H = 0).
 *   amax      fp32 [n_groups] output.
 *   h         fp32 [n_groups][c_in/16][16][16] output, 16-byte aligned,
 *             group stride group_stride_h (multiple of 4).
 *   best_idx (required), best_err, best_amax, w_q, packed_e2m1, scale_e4m3,
 *   global_scale: as lh_scale_sweep_fake_quant.
 *   workspace: at least lh_calibrate_workspace_bytes(c_out, c_in, n_tokens,
 *             n_groups) bytes, 256-byte aligned, required.
 * It is lh_calibrate_prologue followed by lh_calibrate_sweep: three
 * launches with channel-major X and a contiguous W, both 16-byte aligned;
 * other layouts run the separate calls' kernels in turn.
 * Errors: LH_ERR_NULL, LH_ERR_SHAPE, LH_ERR_DTYPE, LH_ERR_LAYOUT,
 * LH_ERR_WORKSPACE, LH_ERR_ARG, LH_ERR_HIP.
 */
lh_status lh_calibrate_nvfp4(const void *w, int w_dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                             int64_t n_groups, int64_t group_stride_w, const void *x, int x_dtype,
                             int x_layout, int64_t n_tokens, int64_t ld_x, int64_t group_stride_x,
                             float *amax, float *h, int64_t group_stride_h, uint8_t *best_idx,
                             float *best_err, float *best_amax, float *w_q, uint8_t *packed_e2m1,
                             uint8_t *scale_e4m3, float *global_scale, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * lh_calibrate_nvfp4 for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without the workspace, the same outputs
 * bit for bit.  Its scratch is a device array inside the library, 32 MiB on
 * each GPU the library runs on, held until the process ends; the call
 * allocates nothing.  Layers whose lh_calibrate_workspace_bytes(c_out, c_in,
 * n_tokens, n_groups) exceeds 32 MiB are rejected with LH_ERR_WORKSPACE
 * before anything is enqueued (mlp-down 5120 x 17408 with 16384 tokens needs
 * 17 MiB).  The stream must belong to the current device.  Every call on a
 * GPU uses that GPU's one array: calls that overlap on one GPU (other
 * streams, other host threads) race and must be ordered by the caller.  No
 * part of the array needs to start at zero: each call writes the scratch it
 * reads before reading it.
 * Errors: as lh_calibrate_nvfp4 (LH_ERR_WORKSPACE: layer too large for the
 * array; LH_ERR_ARG: stream of another device).
 */
lh_status lh_calibrate_nvfp4_noalloc(const void *w, int w_dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                                     int64_t n_groups, int64_t group_stride_w, const void *x, int x_dtype,
                                     int x_layout, int64_t n_tokens, int64_t ld_x, int64_t group_stride_x,
                                     float *amax, float *h, int64_t group_stride_h, uint8_t *best_idx,
                                     float *best_err, float *best_amax, float *w_q, uint8_t *packed_e2m1,
                                     uint8_t *scale_e4m3, float *global_scale, void *stream);

/*
 * Block-scale selection by rule: the scale rules the Local-Hessian guide
 * compares against ("What is Local-Hessian": max scaling takes the block
 * scale from the block's largest |w|; Four-Over-Six picks one of two
 * candidate scales by the in-block error; the MSE method sweeps all 126
 * positive FP8 values by the weight error; "Entry API and calibration
 * flow": with the 126-value sweep off, the amax is searched from
 * multiplier 0.25 to 4.0 in steps of 0.1).
 *
 * Objective: E_k = dw_k^T H_b dw_k when h is given (the local Hessian),
 * else the plain weight error sum_i dw_i^2 (H = I, the "MSE" rule).
 * Candidate set per block, with a = max |w_b| and S_g = fl32(amax[g]/2688);
 * a wanted scale value t is stored as the nearest positive finite E4M3
 * value (ties to the even code, above 448 -> 448, never zero):
 *   LH_RULE_SWEEP          all 126 candidates (with h: identical to
 *                          lh_scale_sweep; without h: the MSE sweep)
 *   LH_RULE_MAX            t = fl32(fl32(a / 6) / S_g)
 *   LH_RULE_FOUR_OVER_SIX  that t and t = fl32(fl32(a / 4) / S_g)
 *   LH_RULE_AMAX_SEARCH    t_i = fl32(fl32(fl32(m_i a) / 6) / S_g),
 *                          m_i = fl32((25 + 10 i) / 100), i = 0..37
 * Each block gets the candidate of lowest E_k in its set, lowest index on
 * ties; S_g = 0 gives candidate 0.  Outputs, layouts and arguments are
 * those of lh_scale_sweep, except:
 *   rule      an lh_rule value (else LH_ERR_ARG).
 *   h         may be NULL (plain weight error); group_stride_h is then
 *             ignored.
 *   workspace used only by LH_RULE_SWEEP with a Hessian (same contract
 *             as lh_scale_sweep); may be NULL/0.
 * Errors: LH_ERR_NULL, LH_ERR_SHAPE, LH_ERR_DTYPE, LH_ERR_WORKSPACE,
 * LH_ERR_ARG, LH_ERR_HIP.
 */
lh_status lh_select_scales(int rule, const void *w, int w_dtype, int64_t c_out, int64_t c_in,
                           int64_t ld_w, int64_t n_groups, int64_t group_stride_w,
                           const float *h, int64_t group_stride_h, const float *amax,
                           uint8_t *best_idx, float *best_err, float *best_amax, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * NVFP4 fake-quant with chosen block scales ("Algorithm principle":
 * Q(W, s) = Cast(W / s) * s; the candidate scales match the sweep bit for
 * bit; "What is Local-Hessian": two-level format = E2M1 values, E4M3 block
 * scale, FP32 per-tensor scale).  For every weight of block (g, r, b) with
 * s = s_{best_idx[g][r][b]}:
 *   w_q[g][r][c]               = Q(w, s) (fp32, exactly the Q of the sweep)
 *   packed_e2m1[g][r][c/2]     = E2M1 nibble (bit 3 = sign, bits 0-2 =
 *                                magnitude code); low nibble = even column
 *   scale_e4m3[g][r][b]        = best_idx + 1 (OCP E4M3FN byte)
 *   global_scale[g]            = S_g = fl32(amax[g] / 2688)
 * Every output is optional (NULL to skip) but at least one must be given.
 * Output layouts are dense ([n_groups][c_out][c_in], [.][.][c_in/2],
 * [.][.][c_in/16], [n_groups]).  best_idx entries must be < 126.
 * Errors: LH_ERR_NULL, LH_ERR_SHAPE, LH_ERR_DTYPE, LH_ERR_ARG, LH_ERR_HIP.
 */
lh_status lh_fake_quant_nvfp4(const void *w, int w_dtype, int64_t c_out, int64_t c_in,
                              int64_t ld_w, int64_t n_groups, int64_t group_stride_w,
                              const uint8_t *best_idx, const float *amax, float *w_q,
                              uint8_t *packed_e2m1, uint8_t *scale_e4m3, float *global_scale,
                              void *stream);

/*
 * ---------------------------------------------------------------------------
 * Approximation diagnostics ("Algorithm principle": the layer's output error
 * is ||Delta X||_F^2 = tr(Delta X X^T Delta^T), and Local-Hessian keeps only
 * the 16 x 16 diagonal blocks of X X^T; "How scaling reshapes the weight
 * distribution": the histogram of W/s, the values fed to the E2M1 rounding).
 * ---------------------------------------------------------------------------
 */

/*
 * Full Hessian h_full[g] = alpha * X_g X_g^T (C_in x C_in, fp32 accumulation
 * on matrix cores), X channel-major x[g][c * ld_x + t] (fp32 or bf16),
 * h_full[g][i * ld_h + j], ld_h >= c_in, group strides >= 0 (h groups must not
 * overlap).  With alpha = 1/N (or NaN, which the library replaces by
 * lh_hessian_alpha(NaN, n_tokens) = fl32(1/N)) its diagonal 16 x 16 blocks are
 * the local Hessians.  n_tokens = 0 writes zeros.  For bf16 layers with at
 * least 128 output tiles of 256 x 256 (16-byte aligned rows), only the lower
 * triangle of 256 x 256 or 192 x 192 tiles is computed and each off-diagonal
 * tile is also written transposed, so entries outside the diagonal tiles are
 * exact mirrors; otherwise h_full[i][j] and h_full[j][i] are computed
 * separately.
 * Errors: LH_ERR_NULL, LH_ERR_SHAPE, LH_ERR_DTYPE, LH_ERR_ARG, LH_ERR_HIP.
 */
lh_status lh_full_hessian(const void *x, int x_dtype, int64_t c_in, int64_t n_tokens, int64_t ld_x,
                          int64_t n_groups, int64_t group_stride_x, float alpha, float *h_full,
                          int64_t ld_h, int64_t group_stride_h, void *stream);

/* Scratch bytes lh_output_error needs (one fp32 per row and 64-column tile). */
size_t lh_output_error_workspace_bytes(int64_t c_out, int64_t c_in, int64_t n_groups);

/*
 * Layer output error per output row with quantised weights w_q:
 *   err[g][r] = d H d^T,  d = w_q[g][r] - w[g][r] (fp32),  H = h_full[g]
 * (fp32 matrix cores; the row dot and the sum over column tiles run in a
 * fixed order, so results are deterministic).  With h_full = X X^T / N the
 * sum over rows is ||(W_q - W) X||_F^2 / N, to compare with the sum of the
 * sweep's block errors (the block-diagonal part).  H is used as given and
 * must be symmetric (h_full[j][i] stands in for h_full[i][j]).
 *   w (w_dtype, ld_w), w_q fp32 (ld_q), both [n_groups][c_out][.] with group
 *   strides; h_full [n_groups][c_in][ld_h]; err fp32 [n_groups][c_out].
 *   workspace: at least lh_output_error_workspace_bytes(c_out, c_in,
 *   n_groups) bytes, 4-byte aligned, required when there is work.
 * Errors: LH_ERR_NULL, LH_ERR_SHAPE, LH_ERR_DTYPE, LH_ERR_WORKSPACE,
 * LH_ERR_ARG, LH_ERR_HIP.
 */
lh_status lh_output_error(const void *w, int w_dtype, const float *w_q, int64_t c_out, int64_t c_in,
                          int64_t ld_w, int64_t ld_q, int64_t n_groups, int64_t group_stride_w,
                          int64_t group_stride_q, const float *h_full, int64_t ld_h,
                          int64_t group_stride_h, float *err, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Histogram of W/s: for every weight, x = fl32(|w| / s_k) with its block's
 * candidate k = best_idx (the quotient the cast rounds) and s_k from
 * amax[g]; bin = floor(fl32(x * bins_per_unit)), values at or beyond n_bins
 * go to the overflow bin n_bins; s = 0 gives x = 0.  counts (uint64
 * [n_groups][n_bins + 1], 8-byte aligned) is overwritten.  n_bins in
 * [1, 4096], bins_per_unit positive and finite.
 * Errors: LH_ERR_NULL, LH_ERR_SHAPE, LH_ERR_DTYPE, LH_ERR_ARG, LH_ERR_HIP.
 */
lh_status lh_scaled_histogram(const void *w, int w_dtype, int64_t c_out, int64_t c_in,
                              int64_t ld_w, int64_t n_groups, int64_t group_stride_w,
                              const uint8_t *best_idx, const float *amax, int n_bins,
                              float bins_per_unit, uint64_t *counts, void *stream);

/*
 * ---------------------------------------------------------------------------
 * GPTQ rounding with fixed Local-Hessian scales ("Combining with GPTQ":
 * Local-Hessian sets the block scales, GPTQ then replaces round-to-nearest
 * to minimise the layer output error).  The GPTQ steps are the published
 * method's (Frantar et al., ICLR 2023).  One layer (group) per call.
 * ---------------------------------------------------------------------------
 */

/* Scratch bytes for lh_gptq_prepare (c_in) and lh_gptq_quantize (c_out, c_in). */
size_t lh_gptq_workspace_bytes(int64_t c_out, int64_t c_in);

/*
 * u = the upper Cholesky factor of H'^-1, H' = H + damp * mean(diag H) * I
 * (the identity when the diagonal is all zero): H'^-1 = u^T u, u upper with
 * a positive diagonal, zeros below.  h_full: fp32 [c_in][ld_h] (e.g. from
 * lh_full_hessian; any positive factor gives the same rounding); u: fp32
 * [c_in][ld_u].  The damped Hessian must be numerically positive definite,
 * else u holds non-finite values.  damp = 0.01 is the method's usual value.
 * workspace: lh_gptq_workspace_bytes(c_out, c_in) bytes, 16-byte aligned.
 * Errors: LH_ERR_NULL, LH_ERR_SHAPE, LH_ERR_WORKSPACE, LH_ERR_ARG, LH_ERR_HIP.
 */
lh_status lh_gptq_prepare(const float *h_full, int64_t c_in, int64_t ld_h, float damp, float *u,
                          int64_t ld_u, void *workspace, size_t workspace_bytes, void *stream);

/*
 * GPTQ quantisation of w [c_out][ld_w] (w_dtype) with the fixed block scales
 * best_idx [c_out][c_in/16] (candidate indices, e.g. from lh_scale_sweep)
 * and the global amax (device fp32 scalar): per row, for i = 0..c_in-1,
 *   q_i = Q(w_i, s_block(i))  (the cast of lh_fake_quant_nvfp4),
 *   e = (w_i - q_i) / u_ii,   w_j = fma(-e, u_ij, w_j) for j > i (fp32),
 * each w_j receiving its updates in increasing i.  w_q [c_out][ld_q] fp32
 * receives the q_i (dequantised values on each block's E2M1 grid; their
 * codes are what lh_fake_quant_nvfp4 would pack).  w is not modified.
 * workspace: lh_gptq_workspace_bytes(c_out, c_in) bytes, 16-byte aligned.
 * Errors: LH_ERR_NULL, LH_ERR_SHAPE, LH_ERR_DTYPE, LH_ERR_WORKSPACE,
 * LH_ERR_ARG, LH_ERR_HIP.
 */
lh_status lh_gptq_quantize(const void *w, int w_dtype, int64_t c_out, int64_t c_in, int64_t ld_w,
                           const uint8_t *best_idx, const float *amax, const float *u,
                           int64_t ld_u, float *w_q, int64_t ld_q, void *workspace,
                           size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LH_H */
