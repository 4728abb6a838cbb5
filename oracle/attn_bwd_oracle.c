/*
 * Test infrastructure, not product code.
 *
 * Plain, slow, obviously correct fp64 CPU gradient of scaled dot-product
 * attention.  Only the test suite and the benchmark's CPU baseline may call
 * it; the HIP library never links or calls it, and this file includes nothing
 * from the HIP library.
 *
 * The forward function is the one the forward oracle computes (grasp.study
 * lesson on standard self-attention, section "The Computational Steps of
 * Standard Self-Attention": scores are the query-key dot products, a row-wise
 * softmax gives the probabilities, the output is probabilities times
 * values), with the scale passed in and the optional causal restriction
 * j <= i.  The pages describe training only by its results ("Attention Is
 * Memory-Bound, and Nobody Noticed for Five Years", the results paragraph:
 * GPT-2 training speed, memory linear in sequence length) and never write
 * out the gradient, so this file is the chain rule applied to that
 * definition, step by step, for an upstream gradient dO of the output:
 *
 *   s_ij  = scale * q_i . k_j                 (allowed j)
 *   p_ij  = exp(s_ij - m_i) / l_i,  m_i = max_j s_ij,  l_i = sum_j exp(s_ij - m_i)
 *   dv_j  = sum_i p_ij dO_i                   (o_i = sum_j p_ij v_j)
 *   dp_ij = dO_i . v_j
 *   D_i   = sum_j p_ij dp_ij                  (softmax Jacobian: dp -> ds)
 *   ds_ij = p_ij (dp_ij - D_i)
 *   dq_i  = scale * sum_j ds_ij k_j
 *   dk_j  = scale * sum_i ds_ij q_i
 *
 * Arithmetic: IEEE double, sums in increasing index order, built with
 * -ffp-contract=off.  Nothing here reorganises the computation into tiles.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

static double dot(const double *a, const double *b, int64_t d)
{
    double acc = 0.0;
    for (int64_t c = 0; c < d; ++c)
        acc += a[c] * b[c];
    return acc;
}

/*
 * Row statistics of slice `sl`, query row i: m_i, l_i and D_i (see above).
 */
static void row_stats(const double *q, const double *k, const double *v, const double *dout,
                      int64_t N, int64_t d, double scale, int causal, int64_t i,
                      double *m_out, double *l_out, double *D_out)
{
    const int64_t n_allow = causal ? i + 1 : N;
    const double *qi = q + i * d;
    double m = -INFINITY;
    for (int64_t j = 0; j < n_allow; ++j) {
        const double s = scale * dot(qi, k + j * d, d);
        if (s > m)
            m = s;
    }
    double l = 0.0;
    for (int64_t j = 0; j < n_allow; ++j)
        l += exp(scale * dot(qi, k + j * d, d) - m);
    double D = 0.0;
    const double *doi = dout + i * d;
    for (int64_t j = 0; j < n_allow; ++j) {
        const double p = exp(scale * dot(qi, k + j * d, d) - m) / l;
        D += p * dot(doi, v + j * d, d);
    }
    *m_out = m;
    *l_out = l;
    *D_out = D;
}

static int check_index(const int64_t *idx, int64_t n, int64_t N)
{
    if (!idx)
        return 1;
    for (int64_t r = 0; r < n; ++r)
        if (idx[r] < 0 || idx[r] >= N)
            return 0;
    return 1;
}

/*
 * oracle_attn_bwd_f64
 *
 *   q, k, v, dout : [S, N, d] row-major doubles (S independent slices)
 *   qrows         : NULL for every query row, else n_q row indices; dq is
 *                   [S, Rq, d] with Rq = N or n_q
 *   krows         : NULL for every key, else n_k key indices; dk and dv are
 *                   [S, Rk, d] with Rk = N or n_k
 *   dq, dk, dv    : outputs; any of them may be NULL to skip it
 *   causal        : 0 = all keys, 1 = keys j <= i only
 *   threads       : OpenMP threads (<= 0: the runtime default)
 *
 * Returns ORACLE_OK, ORACLE_EINVAL or ORACLE_ENOMEM.
 */
int oracle_attn_bwd_f64(const double *q, const double *k, const double *v, const double *dout,
                        double *dq, double *dk, double *dv,
                        int64_t S, int64_t N, int64_t d, double scale, int causal,
                        const int64_t *qrows, int64_t n_q, const int64_t *krows, int64_t n_k,
                        int threads)
{
    if (S < 0 || N < 0 || d < 1)
        return ORACLE_EINVAL;
    if (S == 0 || N == 0)
        return ORACLE_OK;
    if (!q || !k || !v || !dout)
        return ORACLE_EINVAL;
    const int64_t Rq = qrows ? n_q : N, Rk = krows ? n_k : N;
    if (Rq < 0 || Rk < 0 || !check_index(qrows, Rq, N) || !check_index(krows, Rk, N))
        return ORACLE_EINVAL;

    double *m = (double *)malloc((size_t)(S * N) * sizeof(double));
    double *l = (double *)malloc((size_t)(S * N) * sizeof(double));
    double *D = (double *)malloc((size_t)(S * N) * sizeof(double));
    if (!m || !l || !D) {
        free(m);
        free(l);
        free(D);
        return ORACLE_ENOMEM;
    }
#ifdef _OPENMP
    if (threads <= 0)
        threads = omp_get_max_threads();
#endif
    (void)threads;

    /* 1. Per-row statistics over every query row. */
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 8) num_threads(threads)
#endif
    for (int64_t t = 0; t < S * N; ++t) {
        const int64_t sl = t / N, i = t % N;
        const int64_t off = sl * N * d;
        row_stats(q + off, k + off, v + off, dout + off, N, d, scale, causal, i, &m[t], &l[t], &D[t]);
    }

    /* 2. dq_i = scale * sum_j p_ij (dp_ij - D_i) k_j. */
    if (dq) {
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 8) num_threads(threads)
#endif
        for (int64_t t = 0; t < S * Rq; ++t) {
            const int64_t sl = t / Rq, r = t % Rq;
            const int64_t i = qrows ? qrows[r] : r;
            const int64_t off = sl * N * d;
            const double *qi = q + off + i * d, *doi = dout + off + i * d;
            const int64_t n_allow = causal ? i + 1 : N;
            double *out = dq + t * d;
            for (int64_t c = 0; c < d; ++c)
                out[c] = 0.0;
            for (int64_t j = 0; j < n_allow; ++j) {
                const double *kj = k + off + j * d;
                const double p = exp(scale * dot(qi, kj, d) - m[sl * N + i]) / l[sl * N + i];
                const double ds = p * (dot(doi, v + off + j * d, d) - D[sl * N + i]);
                for (int64_t c = 0; c < d; ++c)
                    out[c] += ds * kj[c];
            }
            for (int64_t c = 0; c < d; ++c)
                out[c] *= scale;
        }
    }

    /* 3. dv_j = sum_i p_ij dO_i and dk_j = scale * sum_i ds_ij q_i over the
     *    rows i that see key j. */
    if (dk || dv) {
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 8) num_threads(threads)
#endif
        for (int64_t t = 0; t < S * Rk; ++t) {
            const int64_t sl = t / Rk, r = t % Rk;
            const int64_t j = krows ? krows[r] : r;
            const int64_t off = sl * N * d;
            const double *kj = k + off + j * d, *vj = v + off + j * d;
            double *okk = dk ? dk + t * d : NULL;
            double *ovv = dv ? dv + t * d : NULL;
            for (int64_t c = 0; c < d; ++c) {
                if (okk)
                    okk[c] = 0.0;
                if (ovv)
                    ovv[c] = 0.0;
            }
            for (int64_t i = causal ? j : 0; i < N; ++i) {
                const double *qi = q + off + i * d, *doi = dout + off + i * d;
                const double p = exp(scale * dot(qi, kj, d) - m[sl * N + i]) / l[sl * N + i];
                if (ovv)
                    for (int64_t c = 0; c < d; ++c)
                        ovv[c] += p * doi[c];
                if (okk) {
                    const double ds = p * (dot(doi, vj, d) - D[sl * N + i]);
                    for (int64_t c = 0; c < d; ++c)
                        okk[c] += ds * qi[c];
                }
            }
            if (okk)
                for (int64_t c = 0; c < d; ++c)
                    okk[c] *= scale;
        }
    }
    free(m);
    free(l);
    free(D);
    return ORACLE_OK;
}
