/*
 * Test infrastructure, not product code.
 *
 * Plain, slow, obviously correct fp64 CPU reference for scaled dot-product
 * attention.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may call it; the HIP library never links or calls it, and this
 * file includes nothing from the HIP library.
 *
 * What it computes (the definition, written out, no tiling and no
 * reordering beyond it):
 *
 *   scores  s_ij = scale * sum_c q[i,c] * k[j,c]        for allowed j
 *   probs   p_ij = exp(s_ij - m_i) / sum_j' exp(s_ij' - m_i),  m_i = max_j s_ij
 *   output  o[i,c] = sum_j p_ij * v[j,c]
 *   lse_i   = m_i + ln(sum_j exp(s_ij - m_i))   (natural log-sum-exp of the scores)
 *
 * Sources:
 *  - grasp.study lesson on standard self-attention, section "The Computational
 *    Steps of Standard Self-Attention": scores are the query-key dot products
 *    (a matrix product), a row-wise softmax turns them into probabilities, and
 *    the output is the probability matrix times the value matrix.  The scale
 *    1/sqrt(d) of "scaled dot-product attention" is passed in by the caller.
 *  - "The Attention Bottleneck -- and How FlashAttention Fixed It", section
 *    "Why naive attention is a memory monster": every token looks at every
 *    other token; softmax the N x N scores and use them to weight the values.
 *  - "Attention Is Memory-Bound, and Nobody Noticed for Five Years", the
 *    exactness paragraphs: the fused method computes the same function as
 *    this standard attention, up to floating-point reassociation.  That is why
 *    the reference is the plain definition and not the tiled algorithm.
 *
 * Readings where the pages are silent:
 *  - causal: key j is allowed for query i iff j <= i (diagonal included);
 *  - lse is not on the pages; it is the natural-log log-sum-exp of the
 *    scaled, masked scores, i.e. the row normaliser, reported for checking;
 *  - subtracting the row maximum m_i before exp() is an identity in exact
 *    arithmetic; it only keeps exp() in range.
 *
 * Arithmetic: IEEE double throughout, sums taken in increasing index order,
 * built with -ffp-contract=off so that no multiply-add is fused.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Return codes. */
#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

/*
 * One query row of one slice.
 *   q_row   : d values of query i
 *   k, v    : N x d (row-major) keys and values of the slice
 *   n_allow : number of allowed keys (N, or i+1 when causal); keys 0..n_allow-1
 *   s       : scratch of at least n_allow doubles
 *   o_row   : d outputs;  lse_out: one output
 */
static void attend_one_row(const double *q_row, const double *k, const double *v,
                           int64_t n_allow, int64_t d, double scale,
                           double *s, double *o_row, double *lse_out)
{
    /* Scores: s_j = scale * (q . k_j). */
    for (int64_t j = 0; j < n_allow; ++j) {
        const double *k_row = k + j * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += q_row[c] * k_row[c];
        s[j] = scale * dot;
    }

    /* Row maximum. */
    double m = -INFINITY;
    for (int64_t j = 0; j < n_allow; ++j)
        if (s[j] > m)
            m = s[j];

    /* Unnormalised weights e_j = exp(s_j - m) and their sum. */
    double sum = 0.0;
    for (int64_t j = 0; j < n_allow; ++j) {
        s[j] = exp(s[j] - m);
        sum += s[j];
    }

    /* Output: o = sum_j (e_j / sum) * v_j. */
    for (int64_t c = 0; c < d; ++c)
        o_row[c] = 0.0;
    for (int64_t j = 0; j < n_allow; ++j) {
        const double p = s[j] / sum;
        const double *v_row = v + j * d;
        for (int64_t c = 0; c < d; ++c)
            o_row[c] += p * v_row[c];
    }

    *lse_out = m + log(sum);
}

/*
 * oracle_attn_f64
 *
 *   q, k, v : [S, N, d] row-major doubles (S independent slices, e.g. B*H)
 *   rows    : NULL for every query row, else n_rows row indices in [0, N)
 *             that are computed for every slice
 *   o       : [S, R, d] with R = N (rows == NULL) or R = n_rows
 *   lse     : [S, R] or NULL
 *   causal  : 0 = all keys, 1 = keys j <= i only
 *   threads : OpenMP threads to use (<= 0: the runtime default)
 *
 * Returns ORACLE_OK, ORACLE_EINVAL (bad sizes, null pointers or a row index
 * out of range) or ORACLE_ENOMEM.
 */
int oracle_attn_f64(const double *q, const double *k, const double *v,
                    double *o, double *lse,
                    int64_t S, int64_t N, int64_t d, double scale, int causal,
                    const int64_t *rows, int64_t n_rows, int threads)
{
    if (S < 0 || N < 0 || d < 1)
        return ORACLE_EINVAL;
    if (S == 0 || N == 0)
        return ORACLE_OK;
    if (!q || !k || !v || !o)
        return ORACLE_EINVAL;
    const int64_t R = rows ? n_rows : N;
    if (R < 0)
        return ORACLE_EINVAL;
    if (rows)
        for (int64_t r = 0; r < R; ++r)
            if (rows[r] < 0 || rows[r] >= N)
                return ORACLE_EINVAL;

    const int64_t total = S * R;
    int failed = 0;
#ifdef _OPENMP
    if (threads <= 0)
        threads = omp_get_max_threads();
#pragma omp parallel num_threads(threads)
#endif
    {
        double *scratch = (double *)malloc((size_t)N * sizeof(double));
        if (!scratch) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
        for (int64_t t = 0; t < total; ++t) {
            if (!scratch)
                continue;
            const int64_t sl = t / R;
            const int64_t r = t % R;
            const int64_t i = rows ? rows[r] : r;
            const double *qs = q + (sl * N + i) * d;
            const double *ks = k + sl * N * d;
            const double *vs = v + sl * N * d;
            const int64_t n_allow = causal ? i + 1 : N;
            double l_val;
            attend_one_row(qs, ks, vs, n_allow, d, scale, scratch,
                           o + (sl * R + r) * d, &l_val);
            if (lse)
                lse[sl * R + r] = l_val;
        }
        free(scratch);
    }
    (void)threads;
    return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/* Threads the runtime would use by default (for reporting). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
