/*
 * osm_oracle.c -- CPU reference ("oracle") for exact softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * loads this file.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may use it.  It shares no code, header, table or helper
 * with the GPU path.
 *
 * Everything here is plain fp64 and follows the definitions on the pages
 * literally: no blocking, no fusion, no reordering beyond what a definition
 * states.  Rows are independent, so OpenMP spreads rows over host cores; the
 * arithmetic inside a row is the same sequential loop with or without it.
 *
 * Sources (titles of the three web pages, and the sections used):
 *   [P1] "Online softmax: how FlashAttention skips the N x N matrix" (dev.to)
 *   [P2] "Online softmax" (guide.dupenodi.dev, inference guide)
 *   [P3] "Online softmax" (zerotofrontier.app, efficient-attention chapter)
 *
 * Readings taken where the pages are silent:
 *   - A row with no unmasked score (all -inf, or zero length) gives output 0,
 *     maximum -inf and sum 0; for attention, O = 0 and LSE = -inf.
 *     ([P3] "Precision, and what can still go wrong": a fully masked row ends
 *     with l = 0 and must be handled explicitly; [P3] "Merging partial
 *     results": the empty set's summary is (-inf, 0, 0).)
 *   - A masked score does not enter the sums at all (it contributes exactly
 *     zero), and masked keys' K/V values are never read.  ([P2] "Walking
 *     through it", the paragraph on masks; [P2] "Common mistakes".)
 *   - Causal means key j is visible to query i iff j <= i (top-left aligned).
 *   - Lengths are valid prefixes (right padding); a NULL length array means
 *     the full extent.
 *   - Grouped heads: query head h reads key/value head h / (Hq / Hkv).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* Return codes. */
#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

/* ---------------------------------------------------------------------------
 * Safe softmax of one row: [P3] "Three passes, and why that is a problem"
 * (the displayed safe-softmax definition): m = max_j s_j,
 * l = sum_j exp(s_j - m), y_i = exp(s_i - m) / l.  Three passes: max, sum,
 * divide.  Inputs are widened to double exactly.
 * ------------------------------------------------------------------------- */
static void safe_softmax_row(const double *s, int64_t n, double *y,
                             double *m_out, double *l_out) {
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j)            /* pass 1: the maximum */
        if (s[j] > m) m = s[j];
    if (m == -INFINITY) {                      /* empty or fully masked row */
        for (int64_t j = 0; j < n; ++j) y[j] = 0.0;
        *m_out = -INFINITY;
        *l_out = 0.0;
        return;
    }
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j)            /* pass 2: the normalizer */
        l += exp(s[j] - m);
    for (int64_t j = 0; j < n; ++j)            /* pass 3: divide */
        y[j] = exp(s[j] - m) / l;
    *m_out = m;
    *l_out = l;
}

/*
 * oracle_softmax_rows: safe softmax of selected rows of an fp32 matrix.
 *   x       fp32, row r starts at x + r*ld, `cols` valid entries
 *   sel     row indices to compute (nsel of them); NULL means rows 0..nsel-1
 *   y       double [nsel][cols]
 *   row_max, row_sum  double [nsel], may be NULL
 */
int oracle_softmax_rows(const float *x, int64_t ld, int64_t cols,
                        const int64_t *sel, int64_t nsel, double *y,
                        double *row_max, double *row_sum) {
    if (!x || !y || cols < 0 || nsel < 0 || ld < cols) return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(cols > 0 ? cols : 1));
        if (!s) {
#pragma omp atomic write
            err = ORACLE_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < nsel; ++t) {
                int64_t r = sel ? sel[t] : t;
                const float *xr = x + r * ld;
                for (int64_t j = 0; j < cols; ++j) s[j] = (double)xr[j];
                double m, l;
                safe_softmax_row(s, cols, y + t * cols, &m, &l);
                if (row_max) row_max[t] = m;
                if (row_sum) row_sum[t] = l;
            }
            free(s);
        }
    }
    return err;
}

/*
 * oracle_online_normalizer: the scalar recurrence of [P3] "The recurrence,
 * and a proof that it is right", run one score at a time from m_0 = -inf,
 * l_0 = 0:  m_j = max(m_{j-1}, s_j),  l_j = l_{j-1} exp(m_{j-1} - m_j)
 * + exp(s_j - m_j).  Writes (m_j, l_j) after every step j = 1..n.
 * Used by the tests to check the worked example of [P3] "Two numbers that
 * can be updated" and the theorem's identity at every step; it is the
 * method's iteration, not the definition the GPU results are checked against.
 * exp(-inf - (-inf)) is taken as 0 (the empty running sum is discarded), as
 * the proof and [P2]'s cell do.
 */
int oracle_online_normalizer(const double *s, int64_t n, double *m_steps,
                             double *l_steps) {
    if ((!s && n > 0) || n < 0) return ORACLE_ERR_ARG;
    double m = -INFINITY, l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double m_new = s[j] > m ? s[j] : m;
        double alpha = (m == -INFINITY) ? 0.0 : exp(m - m_new);
        double term = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m_new);
        l = l * alpha + term;
        m = m_new;
        if (m_steps) m_steps[j] = m;
        if (l_steps) l_steps[j] = l;
    }
    return ORACLE_OK;
}

/*
 * oracle_summary: the triple that summarizes a set of scores and values,
 * [P3] "Merging partial results" (the displayed triple):
 *   m = max_i s_i,  l = sum_i exp(s_i - m),  o~ = sum_i exp(s_i - m) v_i.
 *   s double [n], v double [n][d]; outputs m, l (scalars) and o_tilde [d].
 * The empty set (or all -inf) gives the identity (-inf, 0, 0).
 */
int oracle_summary(const double *s, const double *v, int64_t n, int64_t d,
                   double *m_out, double *l_out, double *o_tilde) {
    if (n < 0 || d < 0 || !m_out || !l_out || (d > 0 && !o_tilde)) return ORACLE_ERR_ARG;
    double m = -INFINITY;
    for (int64_t i = 0; i < n; ++i)
        if (s[i] > m) m = s[i];
    for (int64_t k = 0; k < d; ++k) o_tilde[k] = 0.0;
    *m_out = m;
    *l_out = 0.0;
    if (m == -INFINITY) return ORACLE_OK;
    double l = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        if (s[i] == -INFINITY) continue;
        double w = exp(s[i] - m);
        l += w;
        for (int64_t k = 0; k < d; ++k) o_tilde[k] += w * v[i * d + k];
    }
    *l_out = l;
    return ORACLE_OK;
}

/*
 * The merge of two summaries, [P3] "Merging partial results" (displayed
 * definition of the merge): bring both to the common reference
 * m = max(m_A, m_B), then add:
 *   l = l_A exp(m_A - m) + l_B exp(m_B - m),  o~ likewise.
 * The identity (-inf, 0, 0) changes nothing (property 2 of that section);
 * it is handled first so that exp(-inf - (-inf)) never arises.
 * Result is written over (ma, la, oa).
 */
static void merge_into(double *ma, double *la, double *oa, double mb,
                       double lb, const double *ob, int64_t d) {
    if (mb == -INFINITY) return;               /* B is the empty set */
    if (*ma == -INFINITY) {                    /* A is the empty set */
        *ma = mb;
        *la = lb;
        for (int64_t k = 0; k < d; ++k) oa[k] = ob[k];
        return;
    }
    double m = *ma > mb ? *ma : mb;
    double wa = exp(*ma - m), wb = exp(mb - m);
    *la = *la * wa + lb * wb;
    for (int64_t k = 0; k < d; ++k) oa[k] = oa[k] * wa + ob[k] * wb;
    *ma = m;
}

/*
 * oracle_merge: fold the merge left to right over `splits` partial
 * summaries of each row, then finish as [P3] "From weights to outputs"
 * does: o = o~ / l and lse = m + log l ([P3], the log-sum-exp paragraph).
 *   part_m, part_l  fp32 [rows][splits]   (m in natural-log units)
 *   part_o          fp32 [rows][splits][d]
 *   o               double [rows][d];  lse double [rows]
 * A row whose pieces are all the identity gives o = 0 and lse = -inf.
 */
int oracle_merge(const float *part_m, const float *part_l, const float *part_o,
                 int64_t rows, int64_t splits, int64_t d, double *o,
                 double *lse) {
    if (!part_m || !part_l || !part_o || !o || !lse || rows < 0 || splits < 0 || d < 1)
        return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
#pragma omp parallel
    {
        double *ob = (double *)malloc(sizeof(double) * (size_t)d);
        if (!ob) {
#pragma omp atomic write
            err = ORACLE_ERR_NOMEM;
        } else {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < rows; ++r) {
                double m = -INFINITY, l = 0.0;
                double *acc = o + r * d;
                for (int64_t k = 0; k < d; ++k) acc[k] = 0.0;
                for (int64_t c = 0; c < splits; ++c) {
                    int64_t pc = r * splits + c;
                    for (int64_t k = 0; k < d; ++k) ob[k] = (double)part_o[pc * d + k];
                    merge_into(&m, &l, acc, (double)part_m[pc], (double)part_l[pc], ob, d);
                }
                if (m == -INFINITY || l == 0.0) {
                    for (int64_t k = 0; k < d; ++k) acc[k] = 0.0;
                    lse[r] = -INFINITY;
                } else {
                    for (int64_t k = 0; k < d; ++k) acc[k] /= l;
                    lse[r] = m + log(l);
                }
            }
            free(ob);
        }
    }
    return err;
}

static int64_t clamp_len(const int32_t *lens, int64_t b, int64_t full) {
    if (!lens) return full;
    int64_t L = lens[b];
    if (L < 0) L = 0;
    if (L > full) L = full;
    return L;
}

/*
 * oracle_attention: naive attention that materializes each score row.
 * [P1] "What problem does online softmax actually solve?" and [P3]
 * "From weights to outputs": s_j = scale * (q . k_j) ([P3] "Blocks, the
 * bridge to FlashAttention" divides Q K^T by sqrt(d_k); the caller passes
 * the scale), y = safe softmax of the unmasked scores, o = sum_j y_j v_j,
 * lse = m + log l ([P3], the log-sum-exp paragraph).
 *
 * Layouts (contiguous): q [B][Hq][Nq][d], k and v [B][Hkv][Nk][d],
 * o double [nsel][d], lse double [nsel].  Row id t (or sel[t]) names
 * query row ((b*Hq + h)*Nq + i).  Mask: key j is visible to query i iff
 * i < Lq_b and j < Lk_b and (not causal or j <= i).  Only visible keys are
 * read and enter the sums.  A row with no visible key gives o = 0,
 * lse = -inf.  Inputs are fp32 (bf16 inputs are widened exactly by the
 * caller); the arithmetic is fp64.
 */
int oracle_attention(const float *q, const float *k, const float *v,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                     int64_t d, const int32_t *seqlens_q, const int32_t *seqlens_k,
                     double scale, int causal, const int64_t *sel, int64_t nsel,
                     double *o, double *lse) {
    if (!q || !k || !v || !o || !lse || B < 0 || Hq < 1 || Hkv < 1 || Nq < 0 ||
        Nk < 0 || d < 1 || Hq % Hkv != 0 || nsel < 0)
        return ORACLE_ERR_ARG;
    const int64_t group = Hq / Hkv;
    int err = ORACLE_OK;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        double *y = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        if (!s || !y) {
#pragma omp atomic write
            err = ORACLE_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < nsel; ++t) {
                int64_t row = sel ? sel[t] : t;
                int64_t i = row % Nq;
                int64_t h = (row / Nq) % Hq;
                int64_t b = row / (Nq * Hq);
                int64_t g = h / group;
                int64_t Lq = clamp_len(seqlens_q, b, Nq);
                int64_t Lk = clamp_len(seqlens_k, b, Nk);
                double *orow = o + t * d;
                /* visible keys are j < n_vis */
                int64_t n_vis = (i < Lq) ? Lk : 0;
                if (causal && n_vis > i + 1) n_vis = i + 1;
                if (n_vis == 0) {
                    for (int64_t c = 0; c < d; ++c) orow[c] = 0.0;
                    lse[t] = -INFINITY;
                    continue;
                }
                const float *qr = q + ((b * Hq + h) * Nq + i) * d;
                const float *kh = k + (b * Hkv + g) * Nk * d;
                const float *vh = v + (b * Hkv + g) * Nk * d;
                for (int64_t j = 0; j < n_vis; ++j) {       /* S row */
                    double dot = 0.0;
                    for (int64_t c = 0; c < d; ++c)
                        dot += (double)qr[c] * (double)kh[j * d + c];
                    s[j] = scale * dot;
                }
                double m, l;
                safe_softmax_row(s, n_vis, y, &m, &l);
                for (int64_t c = 0; c < d; ++c) orow[c] = 0.0;
                for (int64_t j = 0; j < n_vis; ++j)          /* O = P V */
                    for (int64_t c = 0; c < d; ++c)
                        orow[c] += y[j] * (double)vh[j * d + c];
                lse[t] = m + log(l);
            }
        }
        free(s);
        free(y);
    }
    return err;
}

/*
 * oracle_merge_lse: combine two (o, lse) results of disjoint key sets,
 * [P3] "The same merge, in log-sum-exp form": lse = log(e^lse_A + e^lse_B),
 * computed as max + log(e^(lse_A - max) + e^(lse_B - max)), and
 * o = e^(lse_A - lse) o_A + e^(lse_B - lse) o_B.  A piece with lse = -inf is
 * the empty set and drops out.  o_* double [rows][d], lse_* double [rows].
 */
int oracle_merge_lse(const double *o_a, const double *lse_a, const double *o_b,
                     const double *lse_b, int64_t rows, int64_t d, double *o,
                     double *lse) {
    if (!o_a || !lse_a || !o_b || !lse_b || !o || !lse || rows < 0 || d < 1)
        return ORACLE_ERR_ARG;
    for (int64_t r = 0; r < rows; ++r) {
        double la = lse_a[r], lb = lse_b[r];
        if (la == -INFINITY && lb == -INFINITY) {
            for (int64_t c = 0; c < d; ++c) o[r * d + c] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        double mx = la > lb ? la : lb;
        double L = mx + log(exp(la - mx) + exp(lb - mx));
        double wa = exp(la - L), wb = exp(lb - L);
        for (int64_t c = 0; c < d; ++c)
            o[r * d + c] = wa * o_a[r * d + c] + wb * o_b[r * d + c];
        lse[r] = L;
    }
    return ORACLE_OK;
}

/*
 * oracle_attention_bwd: gradients of naive attention with respect to Q, K
 * and V, given the gradient dO of the output.  The pages define only the
 * forward ([P3] "From weights to outputs"; the log-sum-exp paragraph there
 * notes that lse is what a backward pass keeps to rebuild the weights, as
 * y_j = exp(s_j - lse)); the gradient is the derivative of that definition,
 * written out by the chain rule for one query row with visible keys j:
 *   s_j  = scale * (q . k_j),   y = safe softmax of s,   o = sum_j y_j v_j
 *   dv_j += y_j * dO                        (o is linear in v_j)
 *   g_j   = dO . v_j                        (dL/dy_j)
 *   ds_j  = y_j * (g_j - sum_k y_k g_k)     (the softmax Jacobian
 *                                            dy_k/ds_j = y_k (delta_kj - y_j))
 *   dq   += scale * sum_j ds_j k_j,   dk_j += scale * ds_j q
 * The weights y are the safe softmax of the materialized scores, not rebuilt
 * from an lse.  Masks, lengths and grouped heads are those of
 * oracle_attention; a row with no visible key contributes nothing, and
 * rows past the valid lengths get zero gradients.  dK and dV of a key/value
 * head sum over the query heads that read it.
 *
 * Layouts as oracle_attention; dout [B][Hq][Nq][d] fp32; outputs double:
 * dq [B][Hq][Nq][d], dk and dv [B][Hkv][Nk][d].
 */
int oracle_attention_bwd(const float *q, const float *k, const float *v,
                         const float *dout, int64_t B, int64_t Hq, int64_t Hkv,
                         int64_t Nq, int64_t Nk, int64_t d,
                         const int32_t *seqlens_q, const int32_t *seqlens_k,
                         double scale, int causal, double *dq, double *dk,
                         double *dv) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv || B < 0 || Hq < 1 || Hkv < 1 ||
        Nq < 0 || Nk < 0 || d < 1 || Hq % Hkv != 0)
        return ORACLE_ERR_ARG;
    const int64_t group = Hq / Hkv;
    int err = ORACLE_OK;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        double *y = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        double *gy = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        if (!s || !y || !gy) {
#pragma omp atomic write
            err = ORACLE_ERR_NOMEM;
        } else {
            /* one (batch, key/value head) per iteration: it owns its dK, dV
             * rows and the dQ rows of the query heads that read it */
#pragma omp for schedule(dynamic, 1)
            for (int64_t bg = 0; bg < B * Hkv; ++bg) {
                int64_t b = bg / Hkv, g = bg % Hkv;
                int64_t Lq = clamp_len(seqlens_q, b, Nq);
                int64_t Lk = clamp_len(seqlens_k, b, Nk);
                const float *kh = k + (b * Hkv + g) * Nk * d;
                const float *vh = v + (b * Hkv + g) * Nk * d;
                double *dkh = dk + (b * Hkv + g) * Nk * d;
                double *dvh = dv + (b * Hkv + g) * Nk * d;
                for (int64_t c = 0; c < Nk * d; ++c) {
                    dkh[c] = 0.0;
                    dvh[c] = 0.0;
                }
                for (int64_t h = g * group; h < (g + 1) * group; ++h) {
                    for (int64_t i = 0; i < Nq; ++i) {
                        const float *qr = q + ((b * Hq + h) * Nq + i) * d;
                        const float *dor = dout + ((b * Hq + h) * Nq + i) * d;
                        double *dqr = dq + ((b * Hq + h) * Nq + i) * d;
                        for (int64_t c = 0; c < d; ++c) dqr[c] = 0.0;
                        int64_t n_vis = (i < Lq) ? Lk : 0;
                        if (causal && n_vis > i + 1) n_vis = i + 1;
                        if (n_vis == 0) continue;
                        for (int64_t j = 0; j < n_vis; ++j) {   /* scores */
                            double dot = 0.0;
                            for (int64_t c = 0; c < d; ++c)
                                dot += (double)qr[c] * (double)kh[j * d + c];
                            s[j] = scale * dot;
                        }
                        double m, l;
                        safe_softmax_row(s, n_vis, y, &m, &l);
                        double yg = 0.0;                         /* sum_k y_k g_k */
                        for (int64_t j = 0; j < n_vis; ++j) {
                            double dot = 0.0;
                            for (int64_t c = 0; c < d; ++c)
                                dot += (double)dor[c] * (double)vh[j * d + c];
                            gy[j] = dot;
                            yg += y[j] * dot;
                        }
                        for (int64_t j = 0; j < n_vis; ++j) {
                            double ds = y[j] * (gy[j] - yg);
                            for (int64_t c = 0; c < d; ++c) {
                                dvh[j * d + c] += y[j] * (double)dor[c];
                                dqr[c] += scale * ds * (double)kh[j * d + c];
                                dkh[j * d + c] += scale * ds * (double)qr[c];
                            }
                        }
                    }
                }
            }
        }
        free(s);
        free(y);
        free(gy);
    }
    return err;
}
