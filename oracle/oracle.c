/*
 * Double-precision CPU oracle for the fused row operations.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product path. It shares no
 * source, header, table or helper with the GPU library.
 *
 * Sources of the definitions (web pages on the subject):
 *  - "Engineering a CUDA Machine Learning Framework from Scratch" (page 1),
 *    §3.1 "Online FlashSoftmax": softmax as max, exponential sum, normalise;
 *    the online (running max, rescaled sum) recurrence.
 *    §3.2 "Welford Single-Pass Normalization": LayerNorm moments by
 *    Welford's update.
 *    §2.1 "The Memory Bandwidth Bottleneck": loss gradients fused with the
 *    softmax (cross-entropy forward + backward in one pass).
 *  - "NexusGrad" (page 3), "Core Capabilities": RMSNorm and residual blocks
 *    among the transformer components.
 *  - "GPU Programming for Machine Learning" (page 2), "Module 3": cross-entropy
 *    loss as a network component.
 * The pages state the recurrences in words only (the equations did not
 * survive); the standard published forms are used: the online normaliser of
 * Milakov & Gimelshein (2018) and Welford (1962) with the pairwise merge of
 * Chan, Golub & LeVeque (1979).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp (no fast-math), so every
 * operation below is one IEEE double operation in source order.
 */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

int oracle_threads(void) { return omp_get_max_threads(); }
void oracle_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }

/* ---------------------------------------------------------------- decoding */

static double dec_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16; /* bf16 is the top half of an fp32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load(const void* p, int dtype, int64_t i) {
    if (dtype == ORACLE_BF16) return dec_bf16(((const uint16_t*)p)[i]);
    if (dtype == ORACLE_F64) return ((const double*)p)[i];
    return (double)((const float*)p)[i];
}

void oracle_decode(const void* in, int dtype, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = load(in, dtype, i);
}

/* ------------------------------------------------------ double -> bf16 RNE */

uint16_t oracle_round_bf16(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    /* a in [2^E, 2^(E+1)). bf16 keeps 8 significant bits for normals
     * (E >= -126); below that the spacing is fixed at 2^-133. */
    int e;
    (void)frexp(a, &e);
    int E = e - 1;
    int q = (E < -126 ? -126 : E) - 7;      /* exponent of one unit in the last place */
    double n = nearbyint(ldexp(a, -q));     /* exact scaling, then round to nearest even */
    double r = ldexp(n, q);                 /* exact */
    if (r >= 0x1p128) return (uint16_t)(sign | 0x7F80u);
    float f = (float)r;                     /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

void oracle_round_bf16_array(const double* in, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_bf16(in[i]);
}

/* ------------------------------------------------------------------ softmax */

/* Page 1 §3.1: (1) max, (2) normaliser sum of exp(x - max), (3) normalise. */
static void softmax_row(const void* x, int dtype, int64_t base, int64_t C, double* p) {
    double m = -INFINITY;
    for (int64_t j = 0; j < C; ++j) {
        double v = load(x, dtype, base + j);
        if (v > m || j == 0) m = v;
    }
    double s = 0.0;
    for (int64_t j = 0; j < C; ++j) s += exp(load(x, dtype, base + j) - m);
    for (int64_t j = 0; j < C; ++j) p[j] = exp(load(x, dtype, base + j) - m) / s;
}

void oracle_softmax(const void* x, int dtype, int64_t rows, int64_t cols, double* p) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) softmax_row(x, dtype, r * cols, cols, p + r * cols);
}

/* ---------------------------------------------------------------- LayerNorm */

void oracle_layernorm(const void* x, const void* gamma, const void* beta, int dtype,
                      int64_t rows, int64_t cols, float eps,
                      double* y, double* mean, double* rstd) {
    const double e = (double)eps;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t b = r * cols;
        double sum = 0.0;
        for (int64_t j = 0; j < cols; ++j) sum += load(x, dtype, b + j);
        const double mu = sum / (double)cols;
        double ss = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            double d = load(x, dtype, b + j) - mu;
            ss += d * d;
        }
        const double var = ss / (double)cols;        /* biased */
        const double rs = 1.0 / sqrt(var + e);
        for (int64_t j = 0; j < cols; ++j)
            y[b + j] = (load(x, dtype, b + j) - mu) * rs * load(gamma, dtype, j) + load(beta, dtype, j);
        if (mean) mean[r] = mu;
        if (rstd) rstd[r] = rs;
    }
}

/* ----------------------------------------------------- residual add + RMSNorm */

void oracle_add_rmsnorm(const void* x, const void* res, const void* w, int dtype,
                        int64_t rows, int64_t cols, float eps,
                        double* y, double* h, double* rstd) {
    const double e = (double)eps;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t b = r * cols;
        double ss = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            double hj = load(x, dtype, b + j) + load(res, dtype, b + j);
            h[b + j] = hj;
            ss += hj * hj;
        }
        const double rs = 1.0 / sqrt(ss / (double)cols + e);
        for (int64_t j = 0; j < cols; ++j) y[b + j] = h[b + j] * rs * load(w, dtype, j);
        if (rstd) rstd[r] = rs;
    }
}

/* ------------------------------------------------ softmax cross-entropy fwd+bwd */

void oracle_softmax_xent(const void* logits, int dtype, const int32_t* labels,
                         int64_t rows, int64_t cols,
                         double* loss, double* grad, int32_t* argmax) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t b = r * cols;
        double m = -INFINITY;
        int64_t am = 0;
        for (int64_t j = 0; j < cols; ++j) {
            double v = load(logits, dtype, b + j);
            if (v > m || j == 0) { m = v; am = j; }   /* strict >: first index wins ties */
        }
        double s = 0.0;
        for (int64_t j = 0; j < cols; ++j) s += exp(load(logits, dtype, b + j) - m);
        const int32_t lab = labels[r];
        const int valid = lab >= 0 && (int64_t)lab < cols;
        for (int64_t j = 0; j < cols; ++j) {
            double pj = exp(load(logits, dtype, b + j) - m) / s;
            grad[b + j] = (valid && j == (int64_t)lab) ? pj - 1.0 : pj;
        }
        loss[r] = valid ? m + log(s) - load(logits, dtype, b + lab) : NAN;
        if (argmax) argmax[r] = (int32_t)am;
    }
}

/* Cross-entropy with the options of training code ("GPU Programming for
 * Machine Learning", Module 3: cross-entropy loss; the variants of the
 * cross-entropy row). Per row, straight from the definitions:
 * lse = m + ln s; target q_j = (1 - eps) [j == label] + eps / C;
 * loss_r = sum_j q_j (lse - x_j); p_j = exp(x_j - m) / s;
 * grad_rj = g (p_j - q_j) with g = grad_scale (reduction none or sum) or
 * grad_scale / n_valid (mean), n_valid = rows not ignored.
 * Ignored rows (use_ignore and label == ignore_index): loss 0, grad 0.
 * Other labels outside [0, C): loss NaN, grad_j = g (p_j - eps / C).
 * total (sum / mean) = sum of loss_r in row order (/ n_valid).
 * Terms of zero weight q_j are absent from the sum (a -inf logit, e.g. a
 * masked class, would otherwise give 0 * inf). */
void oracle_softmax_xent_ex(const void* logits, int dtype, const int32_t* labels, int64_t rows,
                            int64_t cols, int use_ignore, int32_t ignore_index, double smoothing,
                            int reduction, double grad_scale, double* loss, double* grad,
                            int32_t* argmax, double* total) {
    int64_t n_valid = 0;
    for (int64_t r = 0; r < rows; ++r)
        if (!(use_ignore && labels[r] == ignore_index)) ++n_valid;
    const double g = reduction == 2 ? grad_scale / (double)n_valid : grad_scale;
    const double off = smoothing / (double)cols;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t b = r * cols;
        double m = -INFINITY;
        int64_t am = 0;
        for (int64_t j = 0; j < cols; ++j) {
            double v = load(logits, dtype, b + j);
            if (v > m || j == 0) { m = v; am = j; }
        }
        if (argmax) argmax[r] = (int32_t)am;
        const int32_t lab = labels[r];
        if (use_ignore && lab == ignore_index) {
            loss[r] = 0.0;
            for (int64_t j = 0; j < cols; ++j) grad[b + j] = 0.0;
            continue;
        }
        double s = 0.0;
        for (int64_t j = 0; j < cols; ++j) s += exp(load(logits, dtype, b + j) - m);
        const double lse = m + log(s);
        const int valid = lab >= 0 && (int64_t)lab < cols;
        double l = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            const double q = (valid && j == (int64_t)lab ? 1.0 - smoothing : 0.0) + off;
            if (q != 0.0) l += q * (lse - load(logits, dtype, b + j));  /* weight 0: no term */
            const double pj = exp(load(logits, dtype, b + j) - m) / s;
            grad[b + j] = g * (pj - q);
        }
        loss[r] = valid ? l : NAN;
    }
    if (total && reduction != 0) {
        double t = 0.0;
        for (int64_t r = 0; r < rows; ++r) t += loss[r];
        *total = reduction == 2 ? t / (double)n_valid : t;
    }
}

/* --------------------------------------------------------------- attention */
/* Scaled dot-product attention per (batch, head), the plain definition the
 * online softmax is fused into ("Engineering a CUDA Machine Learning
 * Framework from Scratch", §3.1: the online normaliser inside attention):
 * s_ij = scale * sum_d q_id k_jd over the keys j visible to query i (all j,
 * or j <= i + (Sk - Sq) when causal: queries aligned to the end of the keys);
 * lse_i = m_i + ln sum_j exp(s_ij - m_i); o_id = sum_j exp(s_ij - lse_i) v_jd.
 * A query with no visible key: o = 0 and lse = -inf. q [B, H, Sq, D],
 * k, v [B, H, Sk, D], o [B, H, Sq, D], lse [B, H, Sq] (may be NULL). */
void oracle_attention(const void* q, const void* k, const void* v, int dtype, int64_t B, int64_t H,
                      int64_t Sq, int64_t Sk, int64_t D, int causal, double scale, double* o,
                      double* lse) {
    const int64_t BH = B * H;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
#pragma omp for schedule(static) collapse(2)
        for (int64_t bh = 0; bh < BH; ++bh)
            for (int64_t i = 0; i < Sq; ++i) {
                const int64_t qb = (bh * Sq + i) * D;
                int64_t nk = Sk;
                if (causal) {
                    nk = i + (Sk - Sq) + 1;
                    if (nk < 0) nk = 0;
                    if (nk > Sk) nk = Sk;
                }
                double m = -INFINITY;
                for (int64_t j = 0; j < nk; ++j) {
                    const int64_t kb = (bh * Sk + j) * D;
                    double acc = 0.0;
                    for (int64_t d = 0; d < D; ++d) acc += load(q, dtype, qb + d) * load(k, dtype, kb + d);
                    s[j] = scale * acc;
                    if (s[j] > m) m = s[j];
                }
                double z = 0.0;
                for (int64_t j = 0; j < nk; ++j) z += exp(s[j] - m);
                const double l = nk > 0 ? m + log(z) : -INFINITY;
                if (lse) lse[bh * Sq + i] = l;
                for (int64_t d = 0; d < D; ++d) o[qb + d] = 0.0;
                for (int64_t j = 0; j < nk; ++j) {
                    const double p = exp(s[j] - l);
                    const int64_t vb = (bh * Sk + j) * D;
                    for (int64_t d = 0; d < D; ++d) o[qb + d] += p * load(v, dtype, vb + d);
                }
            }
        free(s);
    }
}

/* ---------------------------------------------------------------- backward */
/* The vector-Jacobian products of the row operations above (the backward
 * pipelines "NexusGrad" verifies against finite differences, Verified VJP
 * Operators; the analytical backward of page 1 §2.2). Per-column parameter
 * gradients are sums over all rows, accumulated in row order. */

void oracle_softmax_bwd(const void* p, const void* dy, int dtype, int64_t rows, int64_t cols,
                        double* dx) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t b = r * cols;
        double s = 0.0;
        for (int64_t j = 0; j < cols; ++j) s += load(p, dtype, b + j) * load(dy, dtype, b + j);
        for (int64_t j = 0; j < cols; ++j)
            dx[b + j] = load(p, dtype, b + j) * (load(dy, dtype, b + j) - s);
    }
}

void oracle_rmsnorm_bwd(const void* h, const void* dy, const void* dres, const void* w, int dtype,
                        int64_t rows, int64_t cols, float eps, double* dh, double* dw) {
    const double e = (double)eps;
    double* rr = (double*)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1));
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t b = r * cols;
        double ss = 0.0, sg = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            double hj = load(h, dtype, b + j);
            ss += hj * hj;
            sg += load(dy, dtype, b + j) * load(w, dtype, j) * hj;
        }
        const double rs = 1.0 / sqrt(ss / (double)cols + e);
        rr[r] = rs;
        const double c = rs * rs * sg / (double)cols;
        for (int64_t j = 0; j < cols; ++j) {
            dh[b + j] = rs * (load(w, dtype, j) * load(dy, dtype, b + j) - load(h, dtype, b + j) * c);
            if (dres) dh[b + j] += load(dres, dtype, b + j);
        }
    }
    for (int64_t j = 0; j < cols; ++j) dw[j] = 0.0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j)
            dw[j] += load(dy, dtype, r * cols + j) * load(h, dtype, r * cols + j) * rr[r];
    free(rr);
}

void oracle_layernorm_bwd(const void* x, const void* dy, const void* gamma, const double* mean,
                          const double* rstd, int dtype, int64_t rows, int64_t cols,
                          double* dx, double* dgamma, double* dbeta) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t b = r * cols;
        double sg = 0.0, sgn = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            double n = (load(x, dtype, b + j) - mean[r]) * rstd[r];
            double g = load(dy, dtype, b + j) * load(gamma, dtype, j);
            sg += g;
            sgn += g * n;
        }
        const double mg = sg / (double)cols, mgn = sgn / (double)cols;
        for (int64_t j = 0; j < cols; ++j) {
            double n = (load(x, dtype, b + j) - mean[r]) * rstd[r];
            double g = load(dy, dtype, b + j) * load(gamma, dtype, j);
            dx[b + j] = rstd[r] * (g - mg - n * mgn);
        }
    }
    for (int64_t j = 0; j < cols; ++j) { dgamma[j] = 0.0; dbeta[j] = 0.0; }
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j) {
            double d = load(dy, dtype, r * cols + j);
            dgamma[j] += d * (load(x, dtype, r * cols + j) - mean[r]) * rstd[r];
            dbeta[j] += d;
        }
}

/* ------------------------------------------------------ recurrences (for pins) */

/* Online normaliser: m_j = max(m_{j-1}, x_j);
 * d_j = d_{j-1} * exp(m_{j-1} - m_j) + exp(x_j - m_j). */
void oracle_online_softmax_stats(const double* x, int64_t n, double* m, double* d) {
    double mm = -INFINITY, dd = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double mn = x[j] > mm ? x[j] : mm;
        double carried = (mm == -INFINITY) ? 0.0 : dd * exp(mm - mn);
        dd = carried + exp(x[j] - mn);
        mm = mn;
    }
    *m = mm;
    *d = dd;
}

void oracle_softmax_stats_merge(double ma, double da, double mb, double db,
                                double* m, double* d) {
    double mx = ma > mb ? ma : mb;
    double ta = (ma == -INFINITY) ? 0.0 : da * exp(ma - mx);
    double tb = (mb == -INFINITY) ? 0.0 : db * exp(mb - mx);
    *m = mx;
    *d = ta + tb;
}

/* Welford: n += 1; delta = x - mu; mu += delta / n; M2 += delta * (x - mu). */
void oracle_welford(const double* x, int64_t n, double* count, double* mean, double* m2) {
    double c = 0.0, mu = 0.0, q = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        c += 1.0;
        double delta = x[j] - mu;
        mu += delta / c;
        q += delta * (x[j] - mu);
    }
    *count = c;
    *mean = mu;
    *m2 = q;
}

/* n = na + nb; delta = mub - mua; mu = mua + delta * nb / n;
 * M2 = M2a + M2b + delta^2 * na * nb / n. */
void oracle_chan_merge(double na, double mua, double m2a, double nb, double mub, double m2b,
                       double* n, double* mu, double* m2) {
    double nn = na + nb;
    if (nn == 0.0) { *n = 0.0; *mu = 0.0; *m2 = 0.0; return; }
    double delta = mub - mua;
    *n = nn;
    *mu = mua + delta * (nb / nn);
    *m2 = m2a + m2b + delta * delta * (na * nb / nn);
}
