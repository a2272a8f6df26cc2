/*
 * ref_attn.c -- plain, slow, fp64 CPU oracle for the attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the bench use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes (the plain definition, one query row at a time):
 *
 *   s_j = scale * (q . k_j)                  for every visible key j
 *   a_j = exp(s_j) / sum_t exp(s_t)          softmax weights, sum to 1
 *   o   = sum_j a_j v_j                      the attention output
 *   lse = log(sum_j exp(s_j))                natural log, of the scaled scores
 *
 *   -- "The math of FlashAttention" (aicassindra), section "What we must
 *      compute, and why storage is the problem".
 *
 * How: the three-pass safe softmax over a stored score row -- one pass for the
 * maximum m, one for the denominator l = sum exp(s_j - m), one for the weighted
 * sum -- which is the shift-invariant form of the same definition.
 *   -- same page, "Safe softmax: the max-subtraction we cannot give up";
 *      "2.2b: FlashAttention -- Online Softmax", sections "The Numerical
 *      Stability Problem" and "The Sum of Exponentials: What 'l' Represents".
 * The score row is materialised in full (the "textbook route" the method
 * avoids); there is no blocking and no online update here.
 *
 * Visibility: key j is visible to query i when (mask is NULL or mask[b, j] is
 * nonzero) and (not causal or j <= i).  Masked keys contribute nothing
 * (tiled-attention interview answer, second paragraph).  A row with no
 * visible key gets o = 0 and lse = -inf: the pages ask for a defined
 * convention for that case and give none; this is the one the library
 * documents.
 *
 * Inputs are fp32 (bf16 inputs are widened to fp32 exactly by the caller);
 * every product and sum is done in double; `scale` is the caller's value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * Three-pass safe softmax of one stored score row, followed by the weighted
 * sum of value rows.  s[0..n) are the scores, vis[j] != 0 marks visible keys
 * (vis == NULL: all visible), v is n rows of dv fp32 values with row stride
 * ldv (v == NULL: weights only).
 * Writes o[0..dv) and *lse.  Returns the number of visible keys.
 * If p is not NULL the softmax weights are stored there (0 for masked keys),
 * and m_out / l_out receive m and l when not NULL.
 */
int64_t ref_softmax_weighted_sum(const double *s, const uint8_t *vis, int64_t n,
                                 const float *v, int64_t ldv, int64_t dv,
                                 double *o, double *lse, double *p,
                                 double *m_out, double *l_out)
{
    int64_t n_vis = 0;
    double m = -INFINITY;

    /* pass 1: the maximum over visible scores */
    for (int64_t j = 0; j < n; ++j) {
        if (vis && !vis[j]) continue;
        ++n_vis;
        if (s[j] > m) m = s[j];
    }

    if (n_vis == 0) {
        for (int64_t c = 0; c < dv; ++c) o[c] = 0.0;
        *lse = -INFINITY;
        if (p) for (int64_t j = 0; j < n; ++j) p[j] = 0.0;
        if (m_out) *m_out = -INFINITY;
        if (l_out) *l_out = 0.0;
        return 0;
    }

    /* pass 2: the denominator l = sum_j exp(s_j - m) */
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        if (vis && !vis[j]) continue;
        l += exp(s[j] - m);
    }

    /* pass 3: weights a_j = exp(s_j - m) / l and the weighted sum of values */
    for (int64_t c = 0; c < dv; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        if (vis && !vis[j]) {
            if (p) p[j] = 0.0;
            continue;
        }
        double a = exp(s[j] - m) / l;
        if (p) p[j] = a;
        if (v) {
            const float *vj = v + j * ldv;
            for (int64_t c = 0; c < dv; ++c) o[c] += a * (double)vj[c];
        }
    }

    *lse = m + log(l);
    if (m_out) *m_out = m;
    if (l_out) *l_out = l;
    return n_vis;
}

/*
 * Attention forward for selected query rows of q[B,H,Nq,d], k[B,H,Nk,d],
 * v[B,H,Nk,d] (contiguous, row-major, fp32).  rows[t] is the flat row index
 * (b*H + h)*Nq + i; rows == NULL means every row in order (nrows must then be
 * B*H*Nq).  Output row t goes to o[t*d .. t*d+d) and lse[t] (double).
 * threads > 0 sets the OpenMP thread count; 0 keeps the default.
 * Returns the number of threads used, or a negative value on a bad argument.
 */
int ref_attn_rows(const float *q, const float *k, const float *v,
                  int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                  double scale, int causal, const uint8_t *mask,
                  const int64_t *rows, int64_t nrows,
                  double *o, double *lse, int threads)
{
    if (!q || !k || !v || !o || !lse) return -1;
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || d <= 0 || nrows < 0) return -2;
    if (!rows && nrows != B * H * Nq) return -3;
    int used = 1;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
    used = omp_get_max_threads();
#endif
    int bad = 0;

#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)Nk * sizeof(double));
        uint8_t *vis = (uint8_t *)malloc((size_t)Nk);
        if (!s || !vis) {
#pragma omp atomic write
            bad = 1;
        }

#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < nrows; ++t) {
            if (!s || !vis) continue;
            int64_t r = rows ? rows[t] : t;
            if (r < 0 || r >= B * H * Nq) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            int64_t i = r % Nq;
            int64_t bh = r / Nq;
            int64_t b = bh / H;
            const float *qi = q + r * d;
            const float *kb = k + bh * Nk * d;
            const float *vb = v + bh * Nk * d;

            /* the stored score row: s_j = scale * (q_i . k_j) */
            for (int64_t j = 0; j < Nk; ++j) {
                int visible = (!mask || mask[b * Nk + j]) && (!causal || j <= i);
                vis[j] = (uint8_t)visible;
                if (!visible) {
                    s[j] = 0.0;
                    continue;
                }
                const float *kj = kb + j * d;
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c) dot += (double)qi[c] * (double)kj[c];
                s[j] = scale * dot;
            }

            ref_softmax_weighted_sum(s, vis, Nk, vb, d, d, o + t * d, lse + t,
                                     NULL, NULL, NULL);
        }
        free(s);
        free(vis);
    }
    return bad ? -4 : used;
}
