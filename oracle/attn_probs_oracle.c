/*
 * Test infrastructure, not product code.
 *
 * The attention probabilities themselves, for selected query rows: the
 * row-wise softmax of the scaled query-key scores (grasp.study lesson on
 * standard self-attention, section "The Computational Steps of Standard
 * Self-Attention": the scores are the query-key dot products and a softmax
 * over each row turns them into weights).  The forward oracle applies these
 * weights to V; this file returns them, so that a test can bound errors that
 * depend on each weight separately (for instance the rounding of every weight
 * to an 8-bit float).
 *
 *   w_ij = exp(scale * q_i . k_j - M_i) / sum_{allowed j'} exp(scale * q_i . k_j' - M_i)
 *
 * with M_i the largest allowed score of row i (an identity that keeps exp()
 * in range), allowed j = every key, or j <= i when causal; disallowed keys
 * get weight 0.  IEEE double, sums in increasing key order, built with
 * -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * oracle_attn_probs_f64
 *
 *   q, k    : [S, N, d] row-major doubles
 *   rows    : NULL for every query row, else n_rows indices in [0, N)
 *   w       : output [S, R, N] (R = N or n_rows)
 *   threads : OpenMP threads (<= 0: the runtime default)
 *
 * Returns 0, or 1 for invalid arguments.
 */
int oracle_attn_probs_f64(const double *q, const double *k, double *w, int64_t S, int64_t N, int64_t d,
                          double scale, int causal, const int64_t *rows, int64_t n_rows, int threads)
{
    if (S < 0 || N < 0 || d < 1)
        return 1;
    if (S == 0 || N == 0)
        return 0;
    if (!q || !k || !w)
        return 1;
    const int64_t R = rows ? n_rows : N;
    if (R < 0)
        return 1;
    for (int64_t r = 0; rows && r < R; ++r)
        if (rows[r] < 0 || rows[r] >= N)
            return 1;
#ifdef _OPENMP
    if (threads <= 0)
        threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 4) num_threads(threads)
#endif
    for (int64_t t = 0; t < S * R; ++t) {
        const int64_t slice = t / R, i = rows ? rows[t % R] : t % R;
        const double *qi = q + (slice * N + i) * d;
        const double *keys = k + slice * N * d;
        double *wr = w + t * N;
        const int64_t last = causal ? i : N - 1;  /* last allowed key */
        double top = -INFINITY;
        for (int64_t j = 0; j < N; ++j) {
            if (j > last) {
                wr[j] = 0.0;
                continue;
            }
            double acc = 0.0;
            for (int64_t c = 0; c < d; ++c)
                acc += qi[c] * keys[j * d + c];
            wr[j] = scale * acc;
            top = wr[j] > top ? wr[j] : top;
        }
        double total = 0.0;
        for (int64_t j = 0; j <= last; ++j) {
            wr[j] = exp(wr[j] - top);
            total += wr[j];
        }
        for (int64_t j = 0; j <= last; ++j)
            wr[j] /= total;
    }
    (void)threads;
    return 0;
}
