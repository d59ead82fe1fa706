/*
 * Double-precision CPU oracle for the fused row operations.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link or
 * call this library; only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no source with the GPU kernels.
 *
 * Every routine computes the plain definition of the operation in double
 * precision, row by row, in the order the definition states. Inputs are
 * converted exactly to double (fp32 and bf16 are subsets of double). Outputs
 * are returned in double; rounding to bf16 for comparison is a separate,
 * explicit step (oracle_round_bf16).
 *
 * Row-major layout: element (r, c) of a [rows, cols] buffer is at r*cols + c.
 * Rows are independent; OpenMP runs them in parallel without changing any
 * row's arithmetic.
 */
#ifndef FUSEDROW_ORACLE_H
#define FUSEDROW_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Stored input dtypes. F64 exists for the pins (finite differences in double). */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

int oracle_threads(void);
void oracle_set_threads(int n);

/* double -> bf16, round to nearest, ties to even, directly from double
 * (never through fp32). NaN -> quiet NaN with the input's sign; values at or
 * beyond the overflow threshold -> +/-inf; gradual underflow to bf16
 * subnormals (smallest 2^-133). */
uint16_t oracle_round_bf16(double v);
void oracle_round_bf16_array(const double* in, uint16_t* out, int64_t n);

/* Exact decode of stored inputs to double. */
void oracle_decode(const void* in, int dtype, double* out, int64_t n);

/* Row softmax: m = max_j x_j; s = sum_j exp(x_j - m); p_j = exp(x_j - m) / s. */
void oracle_softmax(const void* x, int dtype, int64_t rows, int64_t cols, double* p);

/* LayerNorm, biased variance, eps inside the root:
 * mu = mean(x); var = mean((x - mu)^2); rstd = 1/sqrt(var + eps);
 * y_j = (x_j - mu) * rstd * gamma_j + beta_j.  gamma/beta are in `dtype`.
 * mean/rstd may be NULL. eps is the fp32 value the kernels receive. */
void oracle_layernorm(const void* x, const void* gamma, const void* beta, int dtype,
                      int64_t rows, int64_t cols, float eps,
                      double* y, double* mean, double* rstd);

/* Residual add + RMSNorm:
 * h_j = x_j + r_j (exact in double); ms = mean(h^2); rstd = 1/sqrt(ms + eps);
 * y_j = h_j * rstd * w_j. Returns y and h (the updated residual before
 * rounding) in double. rstd may be NULL. */
void oracle_add_rmsnorm(const void* x, const void* res, const void* w, int dtype,
                        int64_t rows, int64_t cols, float eps,
                        double* y, double* h, double* rstd);

/* Softmax cross-entropy, forward and backward, per row:
 * m, s as in softmax; loss = m + ln(s) - x[label];
 * grad_j = exp(x_j - m)/s - [j == label];
 * argmax = smallest j with x_j == m.
 * A label outside [0, cols) gives loss = NaN and grad = the softmax row.
 * argmax may be NULL. */
void oracle_softmax_xent(const void* logits, int dtype, const int32_t* labels,
                         int64_t rows, int64_t cols,
                         double* loss, double* grad, int32_t* argmax);

/* Cross-entropy with ignore_index, label smoothing, reduction and a gradient
 * scale. target q_j = (1 - smoothing) [j == label] + smoothing / C;
 * loss_r = sum_j q_j (lse - x_j), lse = m + ln s;
 * grad_rj = g (p_j - q_j), g = grad_scale (reduction 0 none, 1 sum) or
 * grad_scale / n_valid (2 mean), n_valid = rows not ignored.
 * use_ignore: rows with label == ignore_index have loss 0 and grad 0.
 * A label outside [0, cols) that is not ignored: loss NaN, grad = g (p - smoothing/C).
 * total (reduction 1, 2; may be NULL): sum of loss_r in row order, / n_valid for mean.
 * argmax may be NULL. */
void oracle_softmax_xent_ex(const void* logits, int dtype, const int32_t* labels, int64_t rows,
                            int64_t cols, int use_ignore, int32_t ignore_index, double smoothing,
                            int reduction, double grad_scale, double* loss, double* grad,
                            int32_t* argmax, double* total);

/* Scaled dot-product attention per (batch, head):
 * s_ij = scale * q_i . k_j over the visible keys (causal: j <= i + Sk - Sq);
 * lse_i = log-sum-exp_j s_ij; o_i = sum_j exp(s_ij - lse_i) v_j.
 * No visible key: o_i = 0, lse_i = -inf. Layouts [B, H, S, D] row-major;
 * lse [B, H, Sq] may be NULL. */
void oracle_attention(const void* q, const void* k, const void* v, int dtype, int64_t B, int64_t H,
                      int64_t Sq, int64_t Sk, int64_t D, int causal, double scale, double* o,
                      double* lse);

/* ---- backward of the row operations (vector-Jacobian products) ---- */

/* Softmax backward from the stored forward output p and the upstream
 * gradient dy: dx_j = p_j * (dy_j - sum_k p_k dy_k). */
void oracle_softmax_bwd(const void* p, const void* dy, int dtype, int64_t rows, int64_t cols,
                        double* dx);

/* Backward of residual add + RMSNorm, y = h * r * w with h = x + residual and
 * r = 1/sqrt(mean(h^2) + eps), from the stored h (the updated residual), w,
 * dy, and dres, the gradient that reaches h through the updated residual
 * (NULL: none):
 * dh_j = r * (w_j dy_j - h_j r^2 mean_k(dy_k w_k h_k)) + dres_j;
 * dw_j = sum_rows dy_j h_j r.  dh is the gradient of both x and residual.
 * dw is [cols]. */
void oracle_rmsnorm_bwd(const void* h, const void* dy, const void* dres, const void* w, int dtype,
                        int64_t rows, int64_t cols, float eps, double* dh, double* dw);

/* LayerNorm backward for y = n * gamma + beta, n = (x - mean) * rstd, using
 * the given per-row mean and rstd (as saved by the forward):
 * g = dy * gamma;  dx_j = rstd * (g_j - mean(g) - n_j mean(g n));
 * dgamma_j = sum_rows dy_j n_j;  dbeta_j = sum_rows dy_j. */
void oracle_layernorm_bwd(const void* x, const void* dy, const void* gamma, const double* mean,
                          const double* rstd, int dtype, int64_t rows, int64_t cols,
                          double* dx, double* dgamma, double* dbeta);

/* The methods' recurrences, in double, used to pin the definitions above. */

/* Online normaliser: sequential running (max, rescaled sum) over x[0..n). */
void oracle_online_softmax_stats(const double* x, int64_t n, double* m, double* d);
/* Merge of two partial (max, sum) states; a state with max -inf is empty. */
void oracle_softmax_stats_merge(double ma, double da, double mb, double db,
                                double* m, double* d);
/* Welford's sequential update over x[0..n): count, mean, M2. */
void oracle_welford(const double* x, int64_t n, double* count, double* mean, double* m2);
/* Pairwise merge of two (count, mean, M2) states; an empty state has count 0. */
void oracle_chan_merge(double na, double mua, double m2a, double nb, double mub, double m2b,
                       double* n, double* mu, double* m2);

#ifdef __cplusplus
}
#endif
#endif
