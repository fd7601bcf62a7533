/*
 * oracle.c -- plain, slow, fp64 CPU reference for the exact attention forward
 * pass O = softmax(scale * Q K^T [+ causal mask]) V and its per-row
 * log-sum-exp.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library; it is its own definition of the result.
 *
 * What it computes is the textbook definition, not the tiled algorithm:
 *   - "解析 FlashAttention（2）", section 1.1: S = Q K^T, P = softmax(S),
 *     O = P V, with the 1/sqrt(d) factor (here: any finite `scale`).
 *   - same page, section 2.1, eq. (2)-(5): the numerically safe softmax in
 *     three passes -- row maximum m, shifted exponentials f = e^(x - m), their
 *     sum l, and p = f / l.
 *   - same page, section 3.2: o_i = (1 / l_i) * sum_t e^(s_it - m_i) v_t.
 *   - "在线 Softmax 与 FlashAttention" (formulas-to-systems unit 12), causal
 *     mask lesson: position i may not see key j > i; masked scores are -inf,
 *     so their probabilities are exactly 0.
 * The log-sum-exp is not defined on the pages; the reading used here is the
 * natural-log LSE_i = m_i + ln(l_i) of the scaled, masked logits.
 *
 * Layout: Q, K, V, O are contiguous [B, H, N, d] row-major doubles; LSE is
 * [B, H, N].  Every sum runs left to right in index order.  No blocking, no
 * fusion, no fast-math.  OpenMP only distributes independent rows.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Safe softmax of one vector x[0..n), eq. (2)-(5).  Entries equal to -inf are
 * masked and receive probability exactly 0.  Writes p[0..n) and returns the
 * natural log-sum-exp m + ln(l).  If every entry is -inf the row has no valid
 * key: p is left all zero and -inf is returned. */
double oracle_softmax(const double *x, long n, double *p)
{
    /* pass 1: m(x) = max_j x_j */
    double m = -INFINITY;
    for (long j = 0; j < n; ++j)
        if (x[j] > m)
            m = x[j];
    if (m == -INFINITY) {
        for (long j = 0; j < n; ++j)
            p[j] = 0.0;
        return -INFINITY;
    }
    /* pass 2: f(x)_j = e^(x_j - m), l(x) = sum_j f(x)_j */
    double l = 0.0;
    for (long j = 0; j < n; ++j) {
        p[j] = (x[j] == -INFINITY) ? 0.0 : exp(x[j] - m);
        l += p[j];
    }
    /* pass 3: softmax(x) = f(x) / l(x) */
    for (long j = 0; j < n; ++j)
        p[j] = p[j] / l;
    return m + log(l);
}

/* One row of scores: s[j] = scale * (q_i . k_j), or -inf when the causal mask
 * hides key j from query i (j > i). */
static void score_row(const double *q_row, const double *k_head, long i, long N,
                      long d, double scale, int causal, double *s)
{
    for (long j = 0; j < N; ++j) {
        if (causal && j > i) {
            s[j] = -INFINITY;
            continue;
        }
        const double *k_row = k_head + j * d;
        double dot = 0.0;
        for (long t = 0; t < d; ++t)
            dot += q_row[t] * k_row[t];
        s[j] = scale * dot;
    }
}

/* o_row[t] = sum_j p[j] * v[j][t] */
static void weighted_sum(const double *p, const double *v_head, long N, long d,
                         double *o_row)
{
    for (long t = 0; t < d; ++t)
        o_row[t] = 0.0;
    for (long j = 0; j < N; ++j) {
        const double *v_row = v_head + j * d;
        for (long t = 0; t < d; ++t)
            o_row[t] += p[j] * v_row[t];
    }
}

/* Full forward pass, the standard materialised form: for each (b, h) the whole
 * N x N score matrix S and probability matrix P exist in memory at once.
 * Returns 0 on success, -1 if memory for S runs out. */
int oracle_attention(const double *q, const double *k, const double *v,
                     long B, long H, long N, long d, double scale, int causal,
                     double *o, double *lse)
{
    double *S = (double *)malloc((size_t)N * (size_t)N * sizeof(double));
    double *P = (double *)malloc((size_t)N * (size_t)N * sizeof(double));
    if (!S || !P) {
        free(S);
        free(P);
        return -1;
    }
    for (long bh = 0; bh < B * H; ++bh) {
        const double *qh = q + bh * N * d;
        const double *kh = k + bh * N * d;
        const double *vh = v + bh * N * d;
        double *oh = o + bh * N * d;
        double *lh = lse + bh * N;
        /* S = scale * Q K^T with the mask applied */
#pragma omp parallel for schedule(dynamic, 16)
        for (long i = 0; i < N; ++i)
            score_row(qh + i * d, kh, i, N, d, scale, causal, S + i * N);
        /* P = softmax(S) row by row; LSE from the same statistics */
#pragma omp parallel for schedule(dynamic, 16)
        for (long i = 0; i < N; ++i)
            lh[i] = oracle_softmax(S + i * N, N, P + i * N);
        /* O = P V */
#pragma omp parallel for schedule(dynamic, 16)
        for (long i = 0; i < N; ++i)
            weighted_sum(P + i * N, vh, N, d, oh + i * d);
    }
    free(S);
    free(P);
    return 0;
}

/* The same definition evaluated for a chosen set of rows only, so that single
 * outputs of very large problems can be checked one by one.  rows holds
 * nrows triples (b, h, i).  o_rows is [nrows, d], lse_rows is [nrows].
 * Returns 0 on success, -1 on a bad index or when memory runs out. */
int oracle_attention_rows(const double *q, const double *k, const double *v,
                          long B, long H, long N, long d, double scale,
                          int causal, const long *rows, long nrows,
                          double *o_rows, double *lse_rows)
{
    for (long r = 0; r < nrows; ++r) {
        long b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= N)
            return -1;
    }
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)N * sizeof(double));
        double *p = (double *)malloc((size_t)N * sizeof(double));
        if (!s || !p) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long r = 0; r < nrows; ++r) {
            if (!s || !p)
                continue;
            long b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
            long bh = b * H + h;
            const double *qh = q + bh * N * d;
            const double *kh = k + bh * N * d;
            const double *vh = v + bh * N * d;
            score_row(qh + i * d, kh, i, N, d, scale, causal, s);
            lse_rows[r] = oracle_softmax(s, N, p);
            weighted_sum(p, vh, N, d, o_rows + r * d);
        }
        free(s);
        free(p);
    }
    return failed ? -1 : 0;
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
