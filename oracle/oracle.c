/*
 * CPU oracle for CSR SpMM, CSR SDDMM and CSR softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * GPU library is checked against.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it; the library never does.  It
 * shares no code, header, table or helper with the GPU path.
 *
 * Everything is accumulated in double precision, one row at a time, in the
 * order the definitions are written, with no blocking or reordering:
 *
 *  - SpMM (AutoSAGE page, Abstract: CSR SpMM aggregation): for row i,
 *    Y[i, f] = sum over the row's stored entries e, in storage order, of
 *    a_e * X[col_e, f].  A missing value array means a_e = 1.
 *  - SDDMM (AutoSAGE page, Abstract: CSR SDDMM): for every stored entry e of
 *    row i, out_e = sum over k of U[i, k] * V[col_e, k].
 *  - Attention (AutoSAGE page, Abstract: the pipeline SDDMM -> row-softmax ->
 *    SpMM; POPCORNBENCH trace page, task statement: softmax over the scores of
 *    the edges coming into each destination, then aggregation of the source
 *    values with those weights; its kernels: the row maximum is subtracted
 *    before exponentiation, and a destination with no incoming edge keeps a
 *    zero output).  Two passes over the scores (maximum, then the sum of
 *    exponentials), then the weighted sum with p_e = exp(t_e - m) / l.
 *  - Multi-head attention: the same per head h, with the score of edge e
 *    t_e = scale * sum_d Q[i, h, d] * K[col_e, h, d] from bfloat16 inputs read
 *    exactly, or from fp32 inputs (the scores computed from queries and keys
 *    rather than given).
 *
 *  - Backward (the gradients of the three products; prior art's GNN training,
 *    SparseTIR page, Abstract): the softmax backward over a row's entries,
 *    ds_e = scale * p_e * (g_e - sum over the row of p g), which is the chain
 *    rule through p_e = exp(t_e - m) / l with t = scale * s; the attention's
 *    score gradient from its inputs (probabilities by the two-pass softmax
 *    above, dp_e = sum_f dOut[i, f] V[col_e, f], then the softmax backward);
 *    and the product with the transpose, dX[j, f] = sum over the entries e
 *    with col_e = j of a_e * dY[row_e, f], accumulated row by row in storage
 *    order.
 *
 * Besides each value the oracle returns its magnitude, the same sum taken over
 * absolute values (sum |a_e| |X[col_e, f]|, sum |U| |V|, sum p_e |V|).  Tests
 * divide the GPU's error by it, which stays meaningful where random signs
 * cancel the value itself.
 *
 * All functions work on the row range [r0, r1) and write results relative to
 * r0, so callers can run disjoint ranges on several threads.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Y, mag: [r1 - r0, F] row-major.  mag may be NULL. */
void oracle_spmm(const int32_t *row_ptr, const int32_t *col_idx, const float *vals,
                 const float *X, int64_t F, int64_t ldx, int64_t r0, int64_t r1,
                 double *Y, double *mag)
{
    for (int64_t i = r0; i < r1; ++i) {
        double *y = Y + (i - r0) * F;
        double *g = mag ? mag + (i - r0) * F : 0;
        for (int64_t f = 0; f < F; ++f) {
            y[f] = 0.0;
            if (g) g[f] = 0.0;
        }
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            double a = vals ? (double)vals[e] : 1.0;
            const float *x = X + (int64_t)col_idx[e] * ldx;
            for (int64_t f = 0; f < F; ++f) {
                y[f] += a * (double)x[f];
                if (g) g[f] += fabs(a) * fabs((double)x[f]);
            }
        }
    }
}

/* out, mag: indexed by the stored entry, for entries row_ptr[r0] .. row_ptr[r1]
 * (relative to row_ptr[r0]).  mag may be NULL. */
void oracle_sddmm(const int32_t *row_ptr, const int32_t *col_idx,
                  const float *U, int64_t ldu, const float *V, int64_t ldv, int64_t K,
                  int64_t r0, int64_t r1, double *out, double *mag)
{
    int64_t base = row_ptr[r0];
    for (int64_t i = r0; i < r1; ++i) {
        const float *u = U + i * ldu;
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            const float *v = V + (int64_t)col_idx[e] * ldv;
            double s = 0.0, m = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                s += (double)u[k] * (double)v[k];
                m += fabs((double)u[k]) * fabs((double)v[k]);
            }
            out[e - base] = s;
            if (mag) mag[e - base] = m;
        }
    }
}

/* Scores given.  out, mag: [r1 - r0, F]; probs (may be NULL): per stored entry
 * relative to row_ptr[r0]. */
void oracle_attention(const int32_t *row_ptr, const int32_t *col_idx, const float *scores,
                      const float *Vv, int64_t F, int64_t ldv, double scale,
                      int64_t r0, int64_t r1, double *out, double *mag, double *probs)
{
    int64_t base = row_ptr[r0];
    for (int64_t i = r0; i < r1; ++i) {
        double *y = out + (i - r0) * F;
        double *g = mag ? mag + (i - r0) * F : 0;
        for (int64_t f = 0; f < F; ++f) {
            y[f] = 0.0;
            if (g) g[f] = 0.0;
        }
        int64_t b = row_ptr[i], end = row_ptr[i + 1];
        if (end == b) continue; /* no incoming edge: the output row stays zero */

        double m = scale * (double)scores[b];
        for (int64_t e = b + 1; e < end; ++e) {
            double t = scale * (double)scores[e];
            if (t > m) m = t;
        }
        double l = 0.0;
        for (int64_t e = b; e < end; ++e) l += exp(scale * (double)scores[e] - m);

        for (int64_t e = b; e < end; ++e) {
            double p = exp(scale * (double)scores[e] - m) / l;
            if (probs) probs[e - base] = p;
            const float *v = Vv + (int64_t)col_idx[e] * ldv;
            for (int64_t f = 0; f < F; ++f) {
                y[f] += p * (double)v[f];
                if (g) g[f] += p * fabs((double)v[f]);
            }
        }
    }
}

/* Q, K, V: bfloat16 bit patterns, [n, H, D] with node stride H * D.
 * out, mag: [r1 - r0, H, D]; probs (may be NULL): [entry - row_ptr[r0]][H]. */
void oracle_mha(const int32_t *row_ptr, const int32_t *col_idx,
                const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                int64_t H, int64_t D, double scale, int64_t r0, int64_t r1,
                double *out, double *mag, double *probs)
{
    int64_t base = row_ptr[r0];
    int64_t HD = H * D;
    for (int64_t i = r0; i < r1; ++i) {
        double *y = out + (i - r0) * HD;
        double *g = mag ? mag + (i - r0) * HD : 0;
        for (int64_t f = 0; f < HD; ++f) {
            y[f] = 0.0;
            if (g) g[f] = 0.0;
        }
        int64_t b = row_ptr[i], end = row_ptr[i + 1];
        if (end == b) continue;

        for (int64_t h = 0; h < H; ++h) {
            const uint16_t *q = Q + i * HD + h * D;
            double m = -INFINITY;
            for (int64_t e = b; e < end; ++e) {
                const uint16_t *k = K + (int64_t)col_idx[e] * HD + h * D;
                double t = 0.0;
                for (int64_t d = 0; d < D; ++d) t += bf16_to_double(q[d]) * bf16_to_double(k[d]);
                t *= scale;
                if (t > m) m = t;
            }
            double l = 0.0;
            for (int64_t e = b; e < end; ++e) {
                const uint16_t *k = K + (int64_t)col_idx[e] * HD + h * D;
                double t = 0.0;
                for (int64_t d = 0; d < D; ++d) t += bf16_to_double(q[d]) * bf16_to_double(k[d]);
                l += exp(scale * t - m);
            }
            for (int64_t e = b; e < end; ++e) {
                const uint16_t *k = K + (int64_t)col_idx[e] * HD + h * D;
                const uint16_t *v = V + (int64_t)col_idx[e] * HD + h * D;
                double t = 0.0;
                for (int64_t d = 0; d < D; ++d) t += bf16_to_double(q[d]) * bf16_to_double(k[d]);
                double p = exp(scale * t - m) / l;
                if (probs) probs[(e - base) * H + h] = p;
                for (int64_t d = 0; d < D; ++d) {
                    y[h * D + d] += p * bf16_to_double(v[d]);
                    if (g) g[h * D + d] += p * fabs(bf16_to_double(v[d]));
                }
            }
        }
    }
}

/* fp32 queries and keys (SDDMM -> row-softmax -> SpMM from Q, K, V): the same
 * as oracle_mha with float inputs.  Q: [n_rows, H, D], K, V: [n_cols, H, D],
 * node stride H * D.  Per head h of row i: t_e = scale * sum_d Q[i, h, d] *
 * K[col_e, h, d]; the row maximum, then the sum of exponentials, then
 * out[i, h, :] = sum_e p_e V[col_e, h, :].  out, mag: [r1 - r0, H, D]; probs
 * (may be NULL): [entry - row_ptr[r0]][H]. */
void oracle_attention_qk(const int32_t *row_ptr, const int32_t *col_idx,
                         const float *Q, const float *K, const float *V,
                         int64_t H, int64_t D, double scale, int64_t r0, int64_t r1,
                         double *out, double *mag, double *probs)
{
    int64_t base = row_ptr[r0];
    int64_t HD = H * D;
    for (int64_t i = r0; i < r1; ++i) {
        double *y = out + (i - r0) * HD;
        double *g = mag ? mag + (i - r0) * HD : 0;
        for (int64_t f = 0; f < HD; ++f) {
            y[f] = 0.0;
            if (g) g[f] = 0.0;
        }
        int64_t b = row_ptr[i], end = row_ptr[i + 1];
        if (end == b) continue;

        for (int64_t h = 0; h < H; ++h) {
            const float *q = Q + i * HD + h * D;
            double m = -INFINITY;
            for (int64_t e = b; e < end; ++e) {
                const float *kq = K + (int64_t)col_idx[e] * HD + h * D;
                double t = 0.0;
                for (int64_t d = 0; d < D; ++d) t += (double)q[d] * (double)kq[d];
                t *= scale;
                if (t > m) m = t;
            }
            double l = 0.0;
            for (int64_t e = b; e < end; ++e) {
                const float *kq = K + (int64_t)col_idx[e] * HD + h * D;
                double t = 0.0;
                for (int64_t d = 0; d < D; ++d) t += (double)q[d] * (double)kq[d];
                l += exp(scale * t - m);
            }
            for (int64_t e = b; e < end; ++e) {
                const float *kq = K + (int64_t)col_idx[e] * HD + h * D;
                const float *vq = V + (int64_t)col_idx[e] * HD + h * D;
                double t = 0.0;
                for (int64_t d = 0; d < D; ++d) t += (double)q[d] * (double)kq[d];
                double p = exp(scale * t - m) / l;
                if (probs) probs[(e - base) * H + h] = p;
                for (int64_t d = 0; d < D; ++d) {
                    y[h * D + d] += p * (double)vq[d];
                    if (g) g[h * D + d] += p * fabs((double)vq[d]);
                }
            }
        }
    }
}

/* Softmax backward from given probabilities and incoming gradient (fp32 arrays
 * read exactly): out_e = scale * p_e * (g_e - S_i), S_i = sum over row i of
 * p g; mag_e = |scale| * p_e * (|g_e| + sum over the row of p |g|).  out and
 * mag are indexed from row_ptr[r0]. */
void oracle_softmax_backward(const int32_t *row_ptr, const float *probs, const float *grad, double scale,
                             int64_t r0, int64_t r1, double *out, double *mag)
{
    const int64_t base = row_ptr[r0];
    for (int64_t i = r0; i < r1; ++i) {
        double S = 0.0, A = 0.0;
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            S += (double)probs[e] * (double)grad[e];
            A += (double)probs[e] * fabs((double)grad[e]);
        }
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            double p = (double)probs[e];
            out[e - base] = scale * p * ((double)grad[e] - S);
            if (mag) mag[e - base] = fabs(scale) * p * (fabs((double)grad[e]) + A);
        }
    }
}

/* Gradient of the scores-given attention out = softmax_row(scale * s) V with
 * respect to the scores, for the incoming gradient dOut [n_rows, F]:
 * ds_e = scale * p_e * (dp_e - sum over the row of p dp), dp_e = <dOut_i,
 * V[col_e]>.  Probabilities by the two-pass softmax.  mag_e = |scale| * p_e *
 * (|dp|_e + sum over the row of p |dp|), |dp|_e = sum_f |dOut| |V|.  ds and
 * mag are indexed from row_ptr[r0]. */
void oracle_attention_backward(const int32_t *row_ptr, const int32_t *col_idx, const float *scores,
                               const float *Vv, const float *dOut, int64_t F, double scale, int64_t r0,
                               int64_t r1, double *ds, double *mag)
{
    const int64_t base = row_ptr[r0];
    for (int64_t i = r0; i < r1; ++i) {
        const int64_t b = row_ptr[i], end = row_ptr[i + 1];
        if (b == end) continue;
        double m = -INFINITY;
        for (int64_t e = b; e < end; ++e) {
            double t = scale * (double)scores[e];
            if (t > m) m = t;
        }
        double l = 0.0;
        for (int64_t e = b; e < end; ++e) l += exp(scale * (double)scores[e] - m);
        const float *go = dOut + i * F;
        double S = 0.0, A = 0.0;
        for (int64_t e = b; e < end; ++e) {
            const float *v = Vv + (int64_t)col_idx[e] * F;
            double dp = 0.0, ap = 0.0;
            for (int64_t f = 0; f < F; ++f) {
                dp += (double)go[f] * (double)v[f];
                ap += fabs((double)go[f]) * fabs((double)v[f]);
            }
            double p = exp(scale * (double)scores[e] - m) / l;
            ds[e - base] = dp;  /* dp for now */
            if (mag) mag[e - base] = ap;
            S += p * dp;
            A += p * ap;
        }
        for (int64_t e = b; e < end; ++e) {
            double p = exp(scale * (double)scores[e] - m) / l;
            ds[e - base] = scale * p * (ds[e - base] - S);
            if (mag) mag[e - base] = fabs(scale) * p * (mag[e - base] + A);
        }
    }
}

/* dX = A^T dY over the whole matrix: dX[j, f] = sum over entries e with
 * col_e = j of a_e dY[row_e, f] (a_e = vals[e], double; vals NULL means 1),
 * visiting the rows in order and each row's entries in storage order.
 * dX, mag: [n_cols, F], zeroed here. */
void oracle_spmm_transpose(const int32_t *row_ptr, const int32_t *col_idx, const double *vals, const float *dY,
                           int64_t n_rows, int64_t n_cols, int64_t F, double *dX, double *mag)
{
    for (int64_t k = 0; k < n_cols * F; ++k) {
        dX[k] = 0.0;
        if (mag) mag[k] = 0.0;
    }
    for (int64_t i = 0; i < n_rows; ++i) {
        const float *y = dY + i * F;
        for (int64_t e = row_ptr[i]; e < row_ptr[i + 1]; ++e) {
            double a = vals ? vals[e] : 1.0;
            double *x = dX + (int64_t)col_idx[e] * F;
            double *g = mag ? mag + (int64_t)col_idx[e] * F : 0;
            for (int64_t f = 0; f < F; ++f) {
                x[f] += a * (double)y[f];
                if (g) g[f] += fabs(a) * fabs((double)y[f]);
            }
        }
    }
}
