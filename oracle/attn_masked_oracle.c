/*
 * Test infrastructure, not product code.
 *
 * fp64 attention with a general mask and an additive bias, written out from
 * the definition.  The pages warn that custom attention biases and unusual
 * masks take a computation off the fused fast path ("Attention Is
 * Memory-Bound, and Nobody Noticed for Five Years", the paragraph on why the
 * result matters in practice); they define neither, so this file takes the
 * plainest reading, the one common attention libraries use:
 *
 *   key j is allowed for query i iff
 *       (causal == 0 or j <= i)
 *       and (window_left  < 0 or j >= i - window_left)
 *       and (window_right < 0 or j <= i + window_right);
 *   s_ij = scale * q_i . k_j + bias_ij          (bias added after scaling;
 *                                                a bias of -inf removes the key);
 *   p_ij = exp(s_ij - m_i) / sum_j exp(s_ij - m_i) over allowed j with finite
 *          s_ij, m_i their maximum;
 *   o_i  = sum_j p_ij v_j,   lse_i = m_i + ln sum_j exp(s_ij - m_i).
 *
 * A row with no allowed key of finite score has o_i = 0 and lse_i = -inf
 * (the empty sum), a reading: the pages say nothing about it.
 *
 * Bias layout: element (b, h, i, j) of a [B, H, N, N] view at
 * bias[b * sb + h * sh + i * si + j] (strides in elements, 0 to broadcast).
 *
 * IEEE double, sums in increasing key order, -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int allowed(int64_t i, int64_t j, int causal, int64_t wl, int64_t wr)
{
    if (causal && j > i)
        return 0;
    if (wl >= 0 && j < i - wl)
        return 0;
    if (wr >= 0 && j > i + wr)
        return 0;
    return 1;
}

/*
 * oracle_attn_masked_f64
 *
 *   q, k, v : [B*H, N, d] row-major doubles
 *   bias    : NULL, or doubles addressed as described above
 *   rows    : NULL for every row, else n_rows row indices (every slice)
 *   o, lse  : [B*H, R, d] and [B*H, R] (lse may be NULL)
 *
 * Returns 0, 1 for invalid arguments, 2 when out of memory.
 */
int oracle_attn_masked_f64(const double *q, const double *k, const double *v, const double *bias,
                           int64_t sb, int64_t sh, int64_t si, double *o, double *lse,
                           int64_t B, int64_t H, int64_t N, int64_t d, double scale, int causal,
                           int64_t window_left, int64_t window_right,
                           const int64_t *rows, int64_t n_rows, int threads)
{
    if (B < 0 || H < 0 || N < 0 || d < 1)
        return 1;
    if (B == 0 || H == 0 || N == 0)
        return 0;
    if (!q || !k || !v || !o)
        return 1;
    const int64_t R = rows ? n_rows : N;
    if (R < 0)
        return 1;
    for (int64_t r = 0; rows && r < R; ++r)
        if (rows[r] < 0 || rows[r] >= N)
            return 1;
    int failed = 0;
#ifdef _OPENMP
    if (threads <= 0)
        threads = omp_get_max_threads();
#pragma omp parallel num_threads(threads)
#endif
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        if (!s) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
        for (int64_t t = 0; t < B * H * R; ++t) {
            if (!s)
                continue;
            const int64_t slice = t / R, b = slice / H, h = slice % H;
            const int64_t i = rows ? rows[t % R] : t % R;
            const double *qi = q + (slice * N + i) * d;
            const double *ks = k + slice * N * d, *vs = v + slice * N * d;
            double *oi = o + t * d;
            /* Scores of allowed keys; -inf marks a key that takes no part. */
            double top = -INFINITY;
            for (int64_t j = 0; j < N; ++j) {
                s[j] = -INFINITY;
                if (!allowed(i, j, causal, window_left, window_right))
                    continue;
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    dot += qi[c] * ks[j * d + c];
                double sc = scale * dot;
                if (bias)
                    sc += bias[b * sb + h * sh + i * si + j];
                s[j] = sc;
                if (sc > top)
                    top = sc;
            }
            for (int64_t c = 0; c < d; ++c)
                oi[c] = 0.0;
            if (top == -INFINITY) {   /* no allowed key with a finite score */
                if (lse)
                    lse[t] = -INFINITY;
                continue;
            }
            double total = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                s[j] = exp(s[j] - top);  /* exp(-inf) = 0 for keys that take no part */
                total += s[j];
            }
            for (int64_t j = 0; j < N; ++j) {
                const double p = s[j] / total;
                for (int64_t c = 0; c < d; ++c)
                    oi[c] += p * vs[j * d + c];
            }
            if (lse)
                lse[t] = top + log(total);
        }
        free(s);
    }
    (void)threads;
    return failed ? 2 : 0;
}
