/*
 * fusedrow — fused, single-pass, memory-bound row kernels for AMD MI355X
 * (gfx950, CDNA4): online softmax, Welford LayerNorm, residual-add + RMSNorm
 * and softmax cross-entropy forward + backward.
 *
 * Every operation reads each input element from HBM once and writes each
 * output element once; the row stays in registers between its reduction and
 * its normalisation, and no intermediate is written to memory.
 *   ("Engineering a CUDA Machine Learning Framework from Scratch", §2.1 The
 *    Memory Bandwidth Bottleneck: fusing normalisations and loss gradients
 *    into registers removes intermediate DRAM traffic; "GPU Programming for
 *    Machine Learning", Key Concepts, Why Fusion Matters.)
 *
 * Conventions shared by all entry points
 * --------------------------------------
 * Layout     Row-major, contiguous: element (r, c) of a [rows, cols] buffer is
 *            at base + (r * cols + c) * element_size. Per-column vectors
 *            (gamma, beta, weight) are [cols]; per-row outputs are [rows].
 * Pointers   Device pointers (hipMalloc / torch CUDA tensors), each aligned to
 *            its element size. Any such alignment is accepted; 16-byte
 *            aligned rows take the 128-bit vector path, misaligned rows are
 *            split into a scalar head, a 128-bit body and a scalar tail.
 * Ownership  The caller owns every buffer, workspaces included. The library
 *            keeps no pointer after the call returns and allocates no
 *            memory. Inputs are read-only.
 *            Every output element is written.
 * Aliasing   An output may coincide exactly with a row input of the same
 *            shape and dtype (in-place): each row is read completely before
 *            any of it is written. Any other overlap involving an output is
 *            rejected with FR_E_ALIAS.
 * Stream     `stream` is a hipStream_t passed as void*; NULL is the default
 *            stream. Calls are asynchronous: nothing synchronises the host,
 *            nothing allocates, so calls may be captured into HIP graphs.
 * Errors     Argument errors are returned before any HIP call is made.
 *            FR_E_LAUNCH reports a failed kernel launch. Faults during kernel
 *            execution surface at the caller's next synchronisation.
 * Sizes      rows >= 0 (rows == 0 is a no-op returning FR_OK, pointers may
 *            then be NULL; the norm backward calls still zero their
 *            parameter gradients); 1 <= cols <= FR_MAX_COLS (less for the
 *            backward calls).
 * Threads    Entry points are re-entrant. fr_debug_force_variant,
 *            fr_debug_set_split_batch_bytes, fr_debug_set_split_one_pass
 *            and fr_debug_set_coop_spin_limit are the only global settings.
 *
 * Arithmetic is fp32 throughout (bf16 inputs are widened exactly, bf16
 * outputs are rounded to nearest-even once, at the store).
 */
#ifndef FUSEDROW_H
#define FUSEDROW_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef FR_API
#define FR_API __attribute__((visibility("default")))
#endif

typedef enum { FR_F32 = 0, FR_BF16 = 1 } fr_dtype_t;

/* Operations, for the workspace query and the variant controls below. */
typedef enum {
  FR_OP_SOFTMAX = 0,
  FR_OP_LAYERNORM = 1,
  FR_OP_RMSNORM = 2,
  FR_OP_XENT = 3,
  FR_OP_SOFTMAX_BWD = 4,
  FR_OP_RMSNORM_BWD = 5,
  FR_OP_LAYERNORM_BWD = 6,
  FR_OP_SOFTMAX_SPLIT = 7,
  FR_OP_XENT_SPLIT = 8,
  FR_OP_LAYERNORM_SPLIT = 9,
  FR_OP_RMSNORM_SPLIT = 10,
  FR_OP_SOFTMAX_BWD_SPLIT = 11
} fr_op_t;

typedef enum {
  FR_OK = 0,
  FR_E_NULL = 1,    /* a required pointer is NULL */
  FR_E_SHAPE = 2,   /* rows < 0, cols < 1, cols above the op's limit, size overflow,
                       or a workspace smaller than the op needs */
  FR_E_DTYPE = 3,   /* unsupported dtype or dtype combination */
  FR_E_ALIAS = 4,   /* an output partially overlaps another buffer */
  FR_E_LAUNCH = 5,  /* the kernel launch failed (hipGetLastError) */
  FR_E_ALIGN = 6,   /* a pointer is not aligned to its element size */
  FR_E_VALUE = 7,   /* an invalid scalar argument (eps negative or not finite) */
  FR_E_VARIANT = 8  /* a forced variant does not exist or cannot hold the row */
} fr_status_t;

/* Widest row any entry point accepts (the whole row is held in registers). */
#define FR_MAX_COLS 65536

/* Row softmax.
 *   p_j = exp(x_j - m) / s,  m = max_j x_j,  s = sum_j exp(x_j - m).
 * Computed in one pass over memory: each lane reduces its register-resident
 * values to a (max, sum) pair and the pairs are combined with the online
 * normaliser merge (m, s) (+) (m', s') = (M, s e^(m-M) + s' e^(m'-M)).
 *   ("Engineering a CUDA Machine Learning Framework from Scratch", §3.1
 *    Mathematical Recurrence: Online FlashSoftmax.)
 * x   [rows, cols] in x_dtype;  y [rows, cols] in y_dtype (may equal x when
 *     the dtypes match).
 * dtypes: any combination of FR_F32 / FR_BF16.
 * A row whose entries are all -inf yields NaN; a row containing NaN yields NaN. */
FR_API fr_status_t fr_softmax_fwd(const void* x, void* y, int64_t rows, int64_t cols,
                           fr_dtype_t x_dtype, fr_dtype_t y_dtype, void* stream);

/* LayerNorm forward.
 *   mu = mean_j x_j,  var = mean_j (x_j - mu)^2 (biased),
 *   rstd = 1 / sqrt(var + eps),  y_j = (x_j - mu) * rstd * gamma_j + beta_j.
 * Moments are merged as (count, mean, M2) triples with the pairwise Welford
 * update, so the row is read once.
 *   ("Engineering a CUDA Machine Learning Framework from Scratch", §3.2
 *    Mathematical Recurrence: Welford Single-Pass Normalization.)
 * x, y [rows, cols] and gamma, beta [cols] in `dtype` (FR_F32 or FR_BF16);
 * mean, rstd [rows] fp32 (each may be NULL to skip it); y may equal x.
 * eps must be finite and >= 0. */
FR_API fr_status_t fr_layernorm_fwd(const void* x, const void* gamma, const void* beta,
                             void* y, float* mean, float* rstd,
                             int64_t rows, int64_t cols, float eps, fr_dtype_t dtype,
                             void* stream);

/* Residual add + RMSNorm forward.
 *   h_j = x_j + residual_j (fp32),  residual_out_j = round(h_j),
 *   rstd = 1 / sqrt(mean_j h_j^2 + eps),  y_j = round(h_j * rstd * weight_j).
 * The unrounded fp32 h is what is normalised.
 *   ("NexusGrad", Core Capabilities: RMSNorm among the transformer
 *    components, residual blocks in the layer stack; fused elementwise work,
 *    Kernel Fusion.)
 * x, residual, y, residual_out [rows, cols] and weight [cols] in `dtype`
 * (FR_F32 or FR_BF16). residual_out may be NULL (not written); it may equal
 * residual (the in-place "updated residual") or x; y may equal x or residual.
 * eps must be finite and >= 0. */
FR_API fr_status_t fr_add_rmsnorm_fwd(const void* x, const void* residual, const void* weight,
                               void* y, void* residual_out,
                               int64_t rows, int64_t cols, float eps, fr_dtype_t dtype,
                               void* stream);

/* Softmax cross-entropy, forward and backward in one pass.
 *   loss_r = m + ln(s) - x[label_r]     (log-sum-exp minus the label logit),
 *   grad_j = exp(x_j - m) / s - [j == label_r],  per row, no reduction over
 *   rows and no 1/rows scaling (upstream gradient 1).
 *   argmax_r = the smallest j with x_j == m (optional output).
 *   ("Engineering a CUDA Machine Learning Framework from Scratch", §2.1:
 *    loss gradients fused into registers; "GPU Programming for Machine
 *    Learning", Module 3: Cross-entropy loss.)
 * logits, grad [rows, cols] fp32; labels [rows] int32; loss [rows] fp32;
 * argmax [rows] int32 or NULL. grad may equal logits. bf16 logits, and the
 * options of training code, are fr_softmax_xent_ex's.
 * A label outside [0, cols) is a data error, not an API error: that row's
 * loss is NaN and its grad is the softmax row; no out-of-bounds access. */
FR_API fr_status_t fr_softmax_xent_fwd_bwd(const float* logits, const int32_t* labels,
                                           float* loss, float* grad, int32_t* argmax,
                                           int64_t rows, int64_t cols, void* stream);

/* ---- cross-entropy variants ---- */

typedef enum { FR_REDUCE_NONE = 0, FR_REDUCE_SUM = 1, FR_REDUCE_MEAN = 2 } fr_reduction_t;

/* Options of fr_softmax_xent_ex (NULL: all defaults, in brackets). */
typedef struct {
  int32_t use_ignore_index; /* nonzero: rows whose label == ignore_index are ignored [0] */
  int32_t ignore_index;     /* e.g. -100 [0] */
  float label_smoothing;    /* eps in [0, 1] [0] */
  float grad_scale;         /* finite; multiplies the gradient [1] */
  int32_t reduction;        /* fr_reduction_t [FR_REDUCE_NONE] */
} fr_xent_options_t;

/* Softmax cross-entropy forward + backward with the options of training code.
 *   target q_j = (1 - eps) [j == label] + eps / C,
 *   loss_r = sum_j q_j (lse - x_j) = lse - (1 - eps) x[label] - eps mean_j x_j,
 *   grad_rj = g (p_j - q_j),  g = grad_scale, or grad_scale / n_valid for
 *   FR_REDUCE_MEAN (n_valid = rows not ignored),
 *   loss_total = sum_r loss_r (SUM) or that sum / n_valid (MEAN; NaN when
 *   every row is ignored), accumulated in double in a fixed order.
 * Ignored rows: loss 0 and a zero gradient row. A label outside [0, cols)
 * that is not ignored: loss NaN, grad_j = g (p_j - eps / C).
 *   ("GPU Programming for Machine Learning", Module 3: cross-entropy loss;
 *    "Engineering a CUDA Machine Learning Framework from Scratch", §2.1.)
 * logits, grad [rows, cols] in `dtype` (FR_F32 or FR_BF16, grad in the
 * logits' dtype; grad may equal logits); labels [rows] int32; loss [rows]
 * fp32 (always written: the per-row losses the total is summed from); argmax
 * [rows] int32 or NULL; loss_total [1] fp32, required for SUM and MEAN (NULL
 * allowed for NONE); during a MEAN call it first holds the row count. One
 * to three kernels on `stream` (count, row pass, total). rows == 0: SUM
 * writes 0, MEAN writes NaN, NONE does nothing. Options out of range
 * (eps outside [0, 1], scale not finite, unknown reduction) give FR_E_VALUE. */
FR_API fr_status_t fr_softmax_xent_ex(const void* logits, const int32_t* labels, float* loss,
                               void* grad, int32_t* argmax, float* loss_total,
                               int64_t rows, int64_t cols, fr_dtype_t dtype,
                               const fr_xent_options_t* options, void* stream);

/* ---- split rows: any width up to FR_SPLIT_MAX_COLS ---- */

/* Widest row of the split entry points (the argmax column is carried as an
 * exact fp32 integer). */
#define FR_SPLIT_MAX_COLS (1 << 24)
/* Smallest segment the split kernels use (the workspace bound below). */
#define FR_SPLIT_MIN_SEGMENT 8192

/* Bytes of workspace the split entry points need for [rows, cols]:
 * rows * ceil(cols / FR_SPLIT_MIN_SEGMENT) * 16 + 16 (one 16-byte partial
 * state per row segment, and 16 bytes more), 0 for rows = 0. -1 for an
 * invalid shape. */
FR_API int64_t fr_split_workspace_bytes(int64_t rows, int64_t cols);

/* Softmax for rows of any width (and for few rows: several workgroups share
 * a row). Same result definition as fr_softmax_fwd. A row is cut into
 * segments, one workgroup per segment; each segment's partial state (max,
 * exponential sum) is taken, the row's states are merged in segment order
 * with the online normaliser merge, and each segment's outputs are written.
 *   ("Engineering a CUDA Machine Learning Framework from Scratch", §3.1:
 *    the merge of partial (max, sum) states.)
 * One-pass form, when the rows give at least 4 segments of 32768 columns per
 * compute unit and a row has at most 64 of them (fr_debug_set_split_one_pass):
 * a kernel zeroing the workspace's counter and slots, then one launch in
 * which a row's workgroups hold their segments in registers, exchange their
 * states through the workspace (each waits for the others of its row; rows
 * are handed out in the order workgroups start, so the waits need no more
 * of the device than one row's workgroups) and write from the registers: x
 * is read once. A workgroup that waits too long (fr_debug_set_coop_spin_limit;
 * not reached in a correct run) writes NaN for its row (the cross-entropy's
 * argmax: -1). Otherwise two passes
 * over segments of 8192 columns (16384 for bf16 input): pass 1 writes each
 * segment's state to `workspace`, pass 2 merges and re-reads its segment (x
 * read twice), over one batch of rows, at most 256 MiB of input, before the
 * next, so that the second read can come from the last-level cache
 * (fr_debug_set_split_batch_bytes): on `stream`, pass 1 of the first batch,
 * one kernel per further batch running pass 2 of the batch before together
 * with pass 1 of this one, then pass 2 of the last (batches + 1 kernels).
 * Other segment shapes via fr_debug_force_variant.
 * x, y as for fr_softmax_fwd (y may equal x); 1 <= cols <= FR_SPLIT_MAX_COLS.
 * workspace: device memory of >= fr_split_workspace_bytes(rows, cols) bytes,
 * 16-byte aligned, not overlapping any other buffer; contents on entry do not
 * matter. Results are bitwise reproducible for a given form and shape. */
FR_API fr_status_t fr_softmax_fwd_split(const void* x, void* y, int64_t rows, int64_t cols,
                                 fr_dtype_t x_dtype, fr_dtype_t y_dtype, void* workspace,
                                 int64_t workspace_bytes, void* stream);

/* Cross-entropy (with the options of fr_softmax_xent_ex) for rows of any
 * width, split as fr_softmax_fwd_split (the partials also carry the sum of
 * the logits and the column of the maximum). Arguments and results as
 * fr_softmax_xent_ex, plus the workspace as fr_softmax_fwd_split. */
FR_API fr_status_t fr_softmax_xent_split(const void* logits, const int32_t* labels, float* loss,
                                  void* grad, int32_t* argmax, float* loss_total,
                                  int64_t rows, int64_t cols, fr_dtype_t dtype,
                                  const fr_xent_options_t* options, void* workspace,
                                  int64_t workspace_bytes, void* stream);

/* LayerNorm for rows of any width, split as fr_softmax_fwd_split: pass 1
 * writes each segment's exact (count, mean, M2) to `workspace`, pass 2 merges
 * a row's partials in segment order with the pairwise (Chan) merge of the
 * Welford moments and writes the segment's y (and, from the row's first
 * segment, mean and rstd). Reads x twice, writes y once. fp32 also in the
 * one-pass form of fr_softmax_fwd_split (segments of 16384 columns); bf16
 * only with fr_debug_set_split_one_pass(2) (no faster there: the apply
 * step reads gamma and beta for every row segment).
 *   ("Engineering a CUDA Machine Learning Framework from Scratch", §3.2
 *    Welford Single-Pass Normalization: partial moments merged pairwise.)
 * Arguments and results as fr_layernorm_fwd, with 1 <= cols <=
 * FR_SPLIT_MAX_COLS, plus the workspace as fr_softmax_fwd_split. */
FR_API fr_status_t fr_layernorm_fwd_split(const void* x, const void* gamma, const void* beta,
                                          void* y, float* mean, float* rstd, int64_t rows,
                                          int64_t cols, float eps, fr_dtype_t dtype,
                                          void* workspace, int64_t workspace_bytes, void* stream);

/* Residual add + RMSNorm for rows of any width, split as
 * fr_softmax_fwd_split, in one pass or two: each segment's sum of h^2
 * (h = x + residual in fp32) is taken, a row's sums are added in segment
 * order, and residual_out and y are written — in the one-pass form from the
 * registers (x and residual read once), in two passes after a second read.
 *   ("NexusGrad", Core Capabilities: RMSNorm, residual blocks.)
 * Arguments and results as fr_add_rmsnorm_fwd (residual_out may equal
 * residual, y may equal x), with 1 <= cols <= FR_SPLIT_MAX_COLS, plus the
 * workspace as fr_softmax_fwd_split. */
FR_API fr_status_t fr_add_rmsnorm_fwd_split(const void* x, const void* residual,
                                            const void* weight, void* y, void* residual_out,
                                            int64_t rows, int64_t cols, float eps,
                                            fr_dtype_t dtype, void* workspace,
                                            int64_t workspace_bytes, void* stream);

/* Softmax backward for rows of any width, split as fr_softmax_fwd_split,
 * in one pass or two: each segment's sum of p * dy is taken, a row's sums
 * are added in segment order and dx = p (dy - s) is written — in the
 * one-pass form from the registers (p and dy read once), in two passes
 * after a second read.
 *   ("NexusGrad", Verified VJP Operators: the softmax vector-Jacobian
 *    product.)
 * Arguments and results as fr_softmax_bwd (dx may equal p or dy), with
 * 1 <= cols <= FR_SPLIT_MAX_COLS, plus the workspace as
 * fr_softmax_fwd_split. */
FR_API fr_status_t fr_softmax_bwd_split(const void* p, const void* dy, void* dx, int64_t rows,
                                        int64_t cols, fr_dtype_t dtype, void* workspace,
                                        int64_t workspace_bytes, void* stream);

/* ---- the online softmax inside attention ---- */

/* Scaled dot-product attention forward (the online normaliser fused into
 * attention, "Engineering a CUDA Machine Learning Framework from Scratch",
 * §3.1), on the bf16 matrix cores:
 *   s_ij = scale * q_i . k_j over the keys visible to query i (all, or
 *   j <= i + seq_k - seq_q when causal: queries aligned to the end of the
 *   keys), lse_i = ln sum_j exp(s_ij), o_i = sum_j exp(s_ij - lse_i) v_j.
 * No score or probability is written to memory. A query with no visible key
 * gets o = 0 and lse = -inf.
 * q, o [batch, heads, seq_q, head_dim]; k, v [batch, heads, seq_k, head_dim];
 * bf16 (FR_BF16 only), row-major, each pointer 16-byte aligned; lse
 * [batch, heads, seq_q] fp32 or NULL. head_dim 64 or 128; batch * heads
 * <= 65535. o may equal q; any other overlap with an output is FR_E_ALIAS.
 * Arithmetic: fp32 accumulation; probabilities enter the value product
 * rounded to bf16; o rounded to bf16 once. scale must be finite (commonly
 * 1/sqrt(head_dim)). */
FR_API fr_status_t fr_attention_fwd(const void* q, const void* k, const void* v, void* o,
                             float* lse, int64_t batch, int64_t heads, int64_t seq_q,
                             int64_t seq_k, int64_t head_dim, int causal, float scale,
                             fr_dtype_t dtype, void* stream);

/* ---- backward of the row operations ---- */

/* Widest row of the backward entry points (their working set per element is
 * larger: two row operands and, for the norms, per-column partial sums). */
#define FR_BWD_MAX_COLS 16384
/* Most partial rows a norm backward call leaves in its workspace. */
#define FR_BWD_PARTIALS 512

/* Softmax backward (vector-Jacobian product) from the stored forward output.
 *   s = sum_k p_k dy_k,  dx_j = p_j (dy_j - s)   per row.
 *   ("NexusGrad", Verified VJP Operators: softmax.)
 * p, dy, dx [rows, cols] in `dtype` (FR_F32 or FR_BF16); dx may equal p or
 * dy. cols <= FR_BWD_MAX_COLS. Rows whose p, dy and dx share their
 * address modulo 16 take the 128-bit path. */
FR_API fr_status_t fr_softmax_bwd(const void* p, const void* dy, void* dx, int64_t rows,
                           int64_t cols, fr_dtype_t dtype, void* stream);

/* Bytes of device workspace fr_add_rmsnorm_bwd (op FR_OP_RMSNORM_BWD) or
 * fr_layernorm_bwd (FR_OP_LAYERNORM_BWD) needs for a [rows, cols] problem:
 * min(rows, FR_BWD_PARTIALS) * cols * 4 per parameter gradient (one for
 * RMSNorm, two for LayerNorm). -1 for another op or an invalid shape. */
FR_API int64_t fr_norm_bwd_workspace_bytes(fr_op_t op, int64_t rows, int64_t cols);

/* Backward of residual add + RMSNorm (fr_add_rmsnorm_fwd).
 *   r = 1 / sqrt(mean_j h_j^2 + eps),  c = r^2 mean_k(dy_k weight_k h_k),
 *   dh_j = r (weight_j dy_j - h_j c) + dres_j,
 *   dweight_j = sum over rows of dy_j h_j r.
 * h is the stored updated residual (residual_out of the forward); dres is the
 * gradient reaching h through that output (NULL: none). dh is the gradient
 * of both x and residual.
 *   ("NexusGrad", Verified VJP Operators; Core Capabilities: RMSNorm,
 *    residual blocks.)
 * h, dy, dres, dh [rows, cols] and weight [cols] in `dtype`; dweight [cols]
 * fp32, overwritten with the sum over all rows. dh may equal h, dy or dres.
 * workspace: device memory of at least fr_norm_bwd_workspace_bytes bytes,
 * 16-byte aligned, not overlapping any other buffer; its contents on entry
 * do not matter and it holds partial sums afterwards. Both kernels run on
 * `stream`, so a workspace may be reused by the next call on that stream.
 * dweight is bitwise reproducible: fixed reduction order, no atomics.
 * cols <= FR_BWD_MAX_COLS. rows == 0 sets dweight to zero (the other
 * pointers may then be NULL). Rows on the 16-byte grid (every pointer
 * 16-byte aligned and cols * element size a multiple of 16) take the 128-bit
 * path. eps must be finite and >= 0. */
FR_API fr_status_t fr_add_rmsnorm_bwd(const void* h, const void* dy, const void* dres,
                               const void* weight, void* dh, float* dweight,
                               void* workspace, int64_t workspace_bytes,
                               int64_t rows, int64_t cols, float eps, fr_dtype_t dtype,
                               void* stream);

/* fr_add_rmsnorm_bwd without a workspace: for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). The dweight partial rows go to a device array the library
 * holds, FR_NOALLOC_SCRATCH_BYTES per GPU (allocated with the library's code
 * on each GPU it runs on, kept until the process ends); a call whose partial
 * rows (min(rows, 256) or fewer, times cols * 4 bytes) exceed it returns
 * FR_E_SHAPE — any row count up to 8192 columns fits. Nothing is allocated
 * and nothing has to be cleared: each call overwrites the partials it reads.
 * All calls on one GPU share its array, so calls that overlap in time on one
 * GPU (on different streams) race and give wrong dweight: serialise them.
 * Arguments, results and errors otherwise as fr_add_rmsnorm_bwd (the same
 * kernels, so the results are bitwise those of fr_add_rmsnorm_bwd). */
#define FR_NOALLOC_SCRATCH_BYTES (8 << 20)
FR_API fr_status_t fr_add_rmsnorm_bwd_noalloc(const void* h, const void* dy, const void* dres,
                                              const void* weight, void* dh, float* dweight,
                                              int64_t rows, int64_t cols, float eps,
                                              fr_dtype_t dtype, void* stream);

/* Backward of LayerNorm (fr_layernorm_fwd) at its saved statistics.
 *   n_j = (x_j - mean) rstd,  g_j = dy_j gamma_j,
 *   dx_j = rstd (g_j - mean_k g_k - n_j mean_k(g_k n_k)),
 *   dgamma_j = sum over rows of dy_j n_j,  dbeta_j = sum over rows of dy_j.
 *   ("NexusGrad", Verified VJP Operators; "Engineering a CUDA Machine
 *    Learning Framework from Scratch", §3.2 for mean and rstd.)
 * x, dy, dx [rows, cols] and gamma [cols] in `dtype`; mean, rstd [rows] fp32
 * as written by fr_layernorm_fwd; dgamma, dbeta [cols] fp32, overwritten.
 * dx may equal x or dy. workspace, reproducibility, rows == 0 (dgamma and
 * dbeta set to zero), cols limit and vector path as for fr_add_rmsnorm_bwd. */
FR_API fr_status_t fr_layernorm_bwd(const void* x, const void* dy, const void* gamma,
                             const float* mean, const float* rstd, void* dx,
                             float* dgamma, float* dbeta, void* workspace,
                             int64_t workspace_bytes, int64_t rows, int64_t cols,
                             fr_dtype_t dtype, void* stream);

/* ---- backward of the norms for rows of any width ---- */

/* Bytes of device workspace fr_add_rmsnorm_bwd_split (op FR_OP_RMSNORM_BWD)
 * or fr_layernorm_bwd_split (FR_OP_LAYERNORM_BWD) needs for [rows, cols]:
 * the per-segment row sums (rows * ceil(cols / 8192) * 16 + 16 bytes,
 * padded to a multiple of 256; none for rows = 0) plus G * cols * 4 per
 * parameter gradient, G =
 * min(rows, max(1, min(512, 1024 / ceil(cols / 8192)))) partial rows. -1 for
 * another op or an invalid shape (1 <= cols <= FR_SPLIT_MAX_COLS). */
FR_API int64_t fr_norm_bwd_split_workspace_bytes(fr_op_t op, int64_t rows, int64_t cols);

/* fr_add_rmsnorm_bwd for rows of any width (cols up to FR_SPLIT_MAX_COLS).
 * A row is cut into segments of 8192 columns: pass 1 writes each segment's
 * two partial row sums (sum h^2, sum dy weight h); pass 2 — workgroup
 * (segment, row group) over rows g, g + G, ... — adds a row's partials in
 * segment order, writes the segment's dh and accumulates its columns'
 * dweight partials, one partial row per row group; a third kernel adds the
 * G partial rows in order. Reads h, dy (and dres) twice. One-pass form (fp32,
 * rows giving at least 4 workgroups per compute unit;
 * fr_debug_set_split_one_pass): a kernel zeroing the workspace's slots,
 * then one launch in which the row group's segment workgroups walk their
 * rows together, exchange each row's sums through the workspace and write
 * dh from the registers (h, dy and dres read once), then the column sums.
 * Arguments and results as fr_add_rmsnorm_bwd, with the workspace of
 * fr_norm_bwd_split_workspace_bytes. Results are bitwise reproducible. */
FR_API fr_status_t fr_add_rmsnorm_bwd_split(const void* h, const void* dy, const void* dres,
                                            const void* weight, void* dh, float* dweight,
                                            void* workspace, int64_t workspace_bytes,
                                            int64_t rows, int64_t cols, float eps,
                                            fr_dtype_t dtype, void* stream);

/* fr_layernorm_bwd for rows of any width, split as
 * fr_add_rmsnorm_bwd_split (the partial row sums are sum g and sum g n).
 * Arguments and results as fr_layernorm_bwd, with the workspace of
 * fr_norm_bwd_split_workspace_bytes. */
FR_API fr_status_t fr_layernorm_bwd_split(const void* x, const void* dy, const void* gamma,
                                          const float* mean, const float* rstd, void* dx,
                                          float* dgamma, float* dbeta, void* workspace,
                                          int64_t workspace_bytes, int64_t rows, int64_t cols,
                                          fr_dtype_t dtype, void* stream);

/* Human-readable name of a status code (static storage). */
FR_API const char* fr_status_str(fr_status_t s);

/* Library version string (static storage). */
FR_API const char* fr_version(void);

/* ---- measurement and tuning (not part of the row-operation contract) ---- */

/* Memory-system probes: what HBM sustains for reads alone, writes alone and
 * a copy, with the access pattern of the row kernels and no arithmetic (the
 * ceilings the row kernels' bandwidth is compared with, "Engineering a CUDA
 * Machine Learning Framework from Scratch", §2.1 The Memory Bandwidth
 * Bottleneck; also the known-size references for scaling hardware byte
 * counters). A workgroup of `threads` lanes owns a contiguous row of up to
 * threads * vecs 16-byte chunks (lane t: chunks t, t + threads, ...; 64 lanes
 * = one row per wavefront, four per workgroup); rows follow each other
 * without gaps. A copy issues all of a row's loads and waits for them (and
 * for the workgroup barrier) before its first store, as a row kernel's
 * stores wait for the row's reduction. The compiled shapes (threads, vecs) are 64 x {2, 4, 8,
 * 16}, 128 x 4, 256 x {1, 2, 4, 8, 16}, 512 x {1, 2, 4, 8} and 1024 x {1, 2, 4,
 * 8, 13, 16}. The cache policy is a mask: FR_PROBE_NT_LOADS makes the loads
 * non-temporal, FR_PROBE_NT_STORES the stores (else ordinary cached ones). */
typedef enum { FR_PROBE_READ = 0, FR_PROBE_WRITE = 1, FR_PROBE_COPY = 2 } fr_probe_t;
#define FR_PROBE_NT_LOADS 1
#define FR_PROBE_NT_STORES 2
/* Shape and policy of fr_stream_read, fr_stream_write and fr_stream_copy. */
#define FR_STREAM_THREADS 256
#define FR_STREAM_VECS 8
#define FR_STREAM_POLICY (FR_PROBE_NT_LOADS | FR_PROBE_NT_STORES)

/* Device-to-device copy of `bytes` bytes: the probe's copy in its default
 * shape and policy when both pointers are 16-byte aligned and bytes is a
 * multiple of 16; a plain byte loop otherwise. src and dst must not overlap. */
FR_API fr_status_t fr_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Read `bytes` bytes of src (16-byte aligned, bytes a multiple of 16), in the
 * default shape and policy; each row's XOR of its 32-bit words goes to
 * sink[row] (fr_stream_probe_rows(bytes, FR_STREAM_THREADS * FR_STREAM_VECS
 * * 16) words, 4-byte aligned, not overlapping src): the only writes. */
FR_API fr_status_t fr_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* Set every 32-bit word of dst (16-byte aligned, bytes a multiple of 16) to
 * `value`, in the default shape and policy; reads nothing. */
FR_API fr_status_t fr_stream_write(void* dst, int64_t bytes, uint32_t value, void* stream);

/* Rows of row_bytes over `bytes` bytes (the last one may be partial): the
 * sink words a read probe writes. -1 for bytes < 0 or row_bytes not a
 * positive multiple of 16. */
FR_API int64_t fr_stream_probe_rows(int64_t bytes, int64_t row_bytes);

/* Any probe in any compiled shape: FR_PROBE_READ reads src and writes sink,
 * FR_PROBE_WRITE writes `value` to every word of dst, FR_PROBE_COPY copies
 * src to dst (no overlap). row_bytes: the row each row owner handles, a
 * multiple of 16 up to threads * vecs * 16 (0: exactly that; FR_E_SHAPE
 * otherwise), so that a probe can take a workload's own row length.
 * policy: a mask of FR_PROBE_NT_LOADS and FR_PROBE_NT_STORES (FR_E_VALUE
 * otherwise). Pointers 16-byte aligned (sink 4-byte), bytes a multiple of
 * 16; unused pointers may be NULL. FR_E_VARIANT for a shape that is not
 * compiled. */
FR_API fr_status_t fr_stream_probe(fr_probe_t kind, const void* src, void* dst, int64_t bytes,
                                   int64_t row_bytes, uint32_t value, uint32_t* sink, int threads,
                                   int vecs, int policy, void* stream);

/* Matrix-core probe: what the bf16 matrix cores sustain when nothing else
 * competes for the issue slots (no operand loads, no vector work) — the
 * ceiling the attention forward's flop rate is compared with beside the
 * published dense peak, which assumes the top clock ("Engineering a CUDA
 * Machine Learning Framework from Scratch", §6.4 Multi-Head Attention &
 * FlashAttention-2 Extension: attention's two matrix products). Runs
 * `workgroups` workgroups of 256 lanes (1 .. 2^20); each wavefront issues
 * `iters` (1 .. 2^19) rounds of 8 v_mfma_f32_32x32x16_bf16 on four
 * independent accumulators, 2^15 flops each, so a call is
 * workgroups * 4 * iters * 8 * 32768 flops. The rate depends on the operand
 * data (the clock the chip holds does): pattern 0 takes every operand
 * element 1/8, and each lane's sum of its accumulators, written to sink, is
 * exactly 32 * iters; pattern 1 takes pseudo-random bf16 elements in [-1, 1)
 * (full mantissas, as real data), the same in every wavefront, and every
 * wavefront writes the same 64 sums. sink: workgroups * 256 floats, 4-byte
 * aligned, caller-owned device memory. FR_E_SHAPE for counts out of range,
 * FR_E_VALUE for another pattern, FR_E_NULL / FR_E_ALIGN for sink. */
FR_API fr_status_t fr_mfma_probe(int workgroups, int iters, int pattern, float* sink,
                                 void* stream);

/* Force the kernel variant used by later calls of `op`: `threads` lanes per
 * row (64 = one wavefront per row, 256..1024 = one workgroup per row) and
 * `vecs` 128-bit vectors (or scalars, on the scalar path) per lane.
 * threads == 0 restores automatic selection. A forced variant that does not
 * exist, or cannot hold a given row, makes those calls return FR_E_VARIANT.
 * Process-wide setting meant for tests and tuning; not synchronised with
 * concurrent calls. */
FR_API fr_status_t fr_debug_force_variant(fr_op_t op, int threads, int vecs);

/* Row batching of the two-pass (split) entry points: both passes run over
 * one batch of rows before the next, a batch holding at most `bytes` of the
 * rows' inputs (at least one row), so that the second read of a batch can be
 * served by the memory-side last-level cache. bytes == 0: no batching (one
 * batch of all rows); bytes < 0: the built-in default (256 MiB). Results do
 * not depend on it. Returns the previous setting. Process-wide setting meant
 * for tests and tuning; not synchronised with concurrent calls. */
FR_API int64_t fr_debug_set_split_batch_bytes(int64_t bytes);

/* The one-pass form of the split entry points (fr_softmax_fwd_split,
 * fr_softmax_xent_split, fr_add_rmsnorm_fwd_split, fr_softmax_bwd_split,
 * fr_layernorm_fwd_split, fr_add_rmsnorm_bwd_split and fr_layernorm_bwd_split
 * in fp32; their bf16 forms in mode 2 only): mode 0
 * always runs the two passes; mode 1 (the default) takes the one-pass form
 * where it applies and the rows give at least 4 work items per compute
 * unit; mode 2 takes it wherever it applies (any row count, and with a
 * forced variant, whose shape it keeps); other values mean 1.
 * Results do not depend on it beyond rounding (both merge the same kind of
 * segment states in segment order, the one-pass form by a fixed DPP tree).
 * Returns the previous setting. Process-wide setting meant for tests and
 * tuning; not synchronised with concurrent calls. */
FR_API int fr_debug_set_split_one_pass(int mode);

/* Bound on the polls a workgroup of the one-pass split form makes for the
 * partial states of its row's other segments before it gives up and writes
 * NaN for that row (the others always arrive in a correct run: rows are
 * handed out in start order). polls < 0 restores the default (2^18);
 * polls = 0 gives up whenever one poll does not find all states. Returns the
 * previous setting. Process-wide setting meant for tests; not synchronised
 * with concurrent calls. */
FR_API int fr_debug_set_coop_spin_limit(int polls);

/* hipError_t code of the last failed kernel launch on this thread (0 if
 * none), to explain an FR_E_LAUNCH. */
FR_API int fr_debug_last_launch_error(void);

/* Describe the variant automatic selection would pick (or the forced one)
 * for a row of `cols` elements: writes lanes per row, vectors per lane and
 * elements per vector (1 on the scalar path). in/out dtypes as for the op
 * (softmax: x and y; the others: their one dtype in both). vector_path is 1
 * when the call's buffers qualify for 128-bit access, 0 otherwise. */
FR_API fr_status_t fr_debug_select_variant(fr_op_t op, int64_t cols, fr_dtype_t in_dtype,
                                    fr_dtype_t out_dtype, int vector_path,
                                    int* threads, int* vecs, int* elems_per_vec);

/* As fr_debug_select_variant, for a call over `rows` rows (>= 0): the
 * cross-entropy entry points may then take a 256-lane shape instead of a
 * 1024-lane one when the rows fill the device's compute units once but not
 * twice (two rows per compute unit resident instead of one). */
FR_API fr_status_t fr_debug_select_variant_for(fr_op_t op, int64_t rows, int64_t cols,
                                        fr_dtype_t in_dtype, fr_dtype_t out_dtype,
                                        int vector_path, int* threads, int* vecs,
                                        int* elems_per_vec);

#ifdef __cplusplus
}
#endif
#endif /* FUSEDROW_H */
