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
 * Ownership  The caller owns every buffer. The library keeps no pointer after
 *            the call returns and allocates no memory. Inputs are read-only.
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
 *            then be NULL); 1 <= cols <= FR_MAX_COLS.
 * Threads    Entry points are re-entrant. fr_debug_force_variant is the only
 *            global setting.
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

typedef enum {
  FR_OK = 0,
  FR_E_NULL = 1,    /* a required pointer is NULL */
  FR_E_SHAPE = 2,   /* rows < 0, cols < 1, cols > FR_MAX_COLS, or size overflow */
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
 * logits, grad [rows, cols] in `dtype` (FR_F32); labels [rows] int32;
 * loss [rows] fp32; argmax [rows] int32 or NULL. grad may equal logits.
 * A label outside [0, cols) is a data error, not an API error: that row's
 * loss is NaN and its grad is the softmax row; no out-of-bounds access. */
FR_API fr_status_t fr_softmax_xent_fwd_bwd(const void* logits, const int32_t* labels,
                                    float* loss, void* grad, int32_t* argmax,
                                    int64_t rows, int64_t cols, fr_dtype_t dtype,
                                    void* stream);

/* Human-readable name of a status code (static storage). */
FR_API const char* fr_status_str(fr_status_t s);

/* Library version string (static storage). */
FR_API const char* fr_version(void);

/* ---- measurement and tuning (not part of the row-operation contract) ---- */

/* Plain device-to-device streaming copy of `bytes` bytes (128-bit accesses
 * where aligned). Used as the bandwidth ceiling and as the known-size
 * reference when scaling hardware byte counters. src and dst must not
 * overlap. */
FR_API fr_status_t fr_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);

typedef enum { FR_OP_SOFTMAX = 0, FR_OP_LAYERNORM = 1, FR_OP_RMSNORM = 2, FR_OP_XENT = 3 } fr_op_t;

/* Force the kernel variant used by later calls of `op`: `threads` lanes per
 * row (64 = one wavefront per row, 256..1024 = one workgroup per row) and
 * `vecs` 128-bit vectors (or scalars, on the scalar path) per lane.
 * threads == 0 restores automatic selection. A forced variant that does not
 * exist, or cannot hold a given row, makes those calls return FR_E_VARIANT.
 * Process-wide setting meant for tests and tuning; not synchronised with
 * concurrent calls. */
FR_API fr_status_t fr_debug_force_variant(fr_op_t op, int threads, int vecs);

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

#ifdef __cplusplus
}
#endif
#endif /* FUSEDROW_H */
