/*
 * oracle.c -- plain, slow, fp64 CPU reference for the exact attention forward
 * pass O = softmax(scale * Q K^T [+ causal mask]) V, its per-row log-sum-exp,
 * and the gradients dQ, dK, dV of that forward pass (end of the file).
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

/* ---------------------------------------------------------------------------
 * Queries and keys of different lengths (decode).  The unit-12 causal lesson
 * notes that a single-token decode step computes only the newest query, which
 * may attend to every existing key.  Reading used here for Nq queries and Nk
 * keys (Nq <= Nk): the queries are the LAST Nq positions of the sequence, so
 * under the causal mask query i (0-based) sits at position Nk - Nq + i and
 * sees keys j <= Nk - Nq + i; with Nq = Nk this is the top-left mask above,
 * and with Nq = 1 every key is visible.  Same definition otherwise.
 * q, o: [B, H, Nq, d]; k, v: [B, H, Nk, d]; lse: [B, H, Nq].
 * ------------------------------------------------------------------------- */
int oracle_attention_qk(const double *q, const double *k, const double *v, long B, long H,
                        long Nq, long Nk, long d, double scale, int causal, double *o,
                        double *lse)
{
    if (Nq < 1 || Nk < Nq)
        return -1;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)Nk * sizeof(double));
        double *p = (double *)malloc((size_t)Nk * sizeof(double));
        if (!s || !p) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (long r = 0; r < B * H * Nq; ++r) {
            if (!s || !p)
                continue;
            const long bh = r / Nq, i = r % Nq;
            /* the mask of score_row with the query at position Nk - Nq + i */
            score_row(q + r * d, k + bh * Nk * d, Nk - Nq + i, Nk, d, scale, causal, s);
            lse[r] = oracle_softmax(s, Nk, p);
            weighted_sum(p, v + bh * Nk * d, Nk, d, o + r * d);
        }
        free(s);
        free(p);
    }
    return failed ? -1 : 0;
}

/* ---------------------------------------------------------------------------
 * Backward pass.  The pages say only that the backward pass recomputes S and P
 * from Q, K and the statistics the forward pass keeps, instead of storing the
 * N x N matrices ("解析 FlashAttention（2）", section 1.2 item (3) and the
 * remark after Algorithm 1 that m and l are kept for the backward pass;
 * Triton page section 5.1: dQ, dK and dV are all needed).  They give no
 * formulas, so this is the derivative of the forward definition above by the
 * chain rule, for a loss whose gradient with respect to O is dO:
 *   dV = P^T dO                        (O = P V)
 *   dP = dO V^T
 *   dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)   (Jacobian of each softmax row)
 *   dQ = scale * dS K,  dK = scale * dS^T Q   (S = scale * Q K^T)
 * Masked entries have P_ij = 0 exactly and so contribute nothing.  Sums run
 * left to right in index order.
 * ------------------------------------------------------------------------- */

/* dP row i and its softmax-Jacobian product: given the probability row p and
 * dO row i, writes ds[j] = p_j (dp_j - sum_k p_k dp_k), dp_j = dO_i . v_j. */
static void grad_score_row(const double *p, const double *do_row, const double *v_head,
                           long N, long d, double *ds)
{
    double dsum = 0.0;
    for (long j = 0; j < N; ++j) {
        double dp = 0.0;
        if (p[j] != 0.0) {
            const double *v_row = v_head + j * d;
            for (long t = 0; t < d; ++t)
                dp += do_row[t] * v_row[t];
        }
        ds[j] = dp; /* dP, turned into dS below */
        dsum += p[j] * dp;
    }
    for (long j = 0; j < N; ++j)
        ds[j] = p[j] * (ds[j] - dsum);
}

/* Full backward pass with S, P and dS materialised per (b, h).  dout is
 * [B, H, N, d]; dq, dk, dv receive [B, H, N, d].  Returns 0, or -1 when memory
 * for the N x N matrices runs out. */
int oracle_attention_backward(const double *q, const double *k, const double *v,
                              const double *dout, long B, long H, long N, long d,
                              double scale, int causal, double *dq, double *dk,
                              double *dv)
{
    double *P = (double *)malloc((size_t)N * (size_t)N * sizeof(double));
    double *dS = (double *)malloc((size_t)N * (size_t)N * sizeof(double));
    if (!P || !dS) {
        free(P);
        free(dS);
        return -1;
    }
    for (long bh = 0; bh < B * H; ++bh) {
        const double *qh = q + bh * N * d;
        const double *kh = k + bh * N * d;
        const double *vh = v + bh * N * d;
        const double *doh = dout + bh * N * d;
        double *dqh = dq + bh * N * d;
        double *dkh = dk + bh * N * d;
        double *dvh = dv + bh * N * d;
        /* P = softmax(scale * Q K^T + mask), row by row (dS holds S meanwhile) */
#pragma omp parallel for schedule(dynamic, 16)
        for (long i = 0; i < N; ++i) {
            score_row(qh + i * d, kh, i, N, d, scale, causal, dS + i * N);
            oracle_softmax(dS + i * N, N, P + i * N);
        }
        /* dS = P o (dP - rowsum(P o dP)), dP = dO V^T */
#pragma omp parallel for schedule(dynamic, 16)
        for (long i = 0; i < N; ++i)
            grad_score_row(P + i * N, doh + i * d, vh, N, d, dS + i * N);
        /* dQ = scale * dS K */
#pragma omp parallel for schedule(dynamic, 16)
        for (long i = 0; i < N; ++i) {
            for (long t = 0; t < d; ++t) {
                double acc = 0.0;
                for (long j = 0; j < N; ++j)
                    acc += dS[i * N + j] * kh[j * d + t];
                dqh[i * d + t] = scale * acc;
            }
        }
        /* dK = scale * dS^T Q and dV = P^T dO, one key j at a time */
#pragma omp parallel for schedule(dynamic, 16)
        for (long j = 0; j < N; ++j) {
            for (long t = 0; t < d; ++t) {
                double ak = 0.0, av = 0.0;
                for (long i = 0; i < N; ++i) {
                    ak += dS[i * N + j] * qh[i * d + t];
                    av += P[i * N + j] * doh[i * d + t];
                }
                dkh[j * d + t] = scale * ak;
                dvh[j * d + t] = av;
            }
        }
    }
    free(P);
    free(dS);
    return 0;
}

/* dQ for chosen rows only (triples (b, h, i) in rows): the same definition,
 * one score row at a time, so that single rows of very large problems can be
 * checked.  dq_rows is [nrows, d].  Returns 0, or -1 on a bad index or when
 * memory runs out. */
int oracle_attention_backward_dq_rows(const double *q, const double *k, const double *v,
                                      const double *dout, long B, long H, long N,
                                      long d, double scale, int causal, const long *rows,
                                      long nrows, double *dq_rows)
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
            const double *kh = k + bh * N * d;
            score_row(q + (bh * N + i) * d, kh, i, N, d, scale, causal, s);
            oracle_softmax(s, N, p);
            grad_score_row(p, dout + (bh * N + i) * d, v + bh * N * d, N, d, s);
            for (long t = 0; t < d; ++t) {
                double acc = 0.0;
                for (long j = 0; j < N; ++j)
                    acc += s[j] * kh[j * d + t];
                dq_rows[r * d + t] = scale * acc;
            }
        }
        free(s);
        free(p);
    }
    return failed ? -1 : 0;
}

/* dK and dV for chosen keys of ONE head (q, k, v, dout are that head's
 * [N, d] matrices), from the same definition: every query row i that can see
 * one of the keys (i >= the smallest key under the causal mask, all rows
 * otherwise) gets its probability row and its dS row once; then
 * dV_j = sum_i P_ij dO_i and dK_j = scale * sum_i dS_ij Q_i over those rows
 * (rows that cannot see key j have P_ij = dS_ij = 0).  dk_rows and dv_rows
 * are [nkeys, d].  Returns 0, or -1 on a bad key or when memory runs out. */
int oracle_attention_backward_kv_keys(const double *q, const double *k, const double *v,
                                      const double *dout, long N, long d, double scale,
                                      int causal, const long *keys, long nkeys,
                                      double *dk_rows, double *dv_rows)
{
    long i0 = causal ? N : 0;
    for (long r = 0; r < nkeys; ++r) {
        if (keys[r] < 0 || keys[r] >= N)
            return -1;
        if (causal && keys[r] < i0)
            i0 = keys[r];
    }
    if (nkeys == 0)
        return 0;
    const long rows = N - i0;
    double *P = (double *)malloc((size_t)rows * (size_t)N * sizeof(double));
    double *dS = (double *)malloc((size_t)rows * (size_t)N * sizeof(double));
    if (!P || !dS) {
        free(P);
        free(dS);
        return -1;
    }
#pragma omp parallel for schedule(dynamic, 4)
    for (long i = i0; i < N; ++i) {
        double *p = P + (i - i0) * N, *ds = dS + (i - i0) * N;
        score_row(q + i * d, k, i, N, d, scale, causal, ds);
        oracle_softmax(ds, N, p);
        grad_score_row(p, dout + i * d, v, N, d, ds);
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (long r = 0; r < nkeys; ++r) {
        const long j = keys[r];
        for (long t = 0; t < d; ++t) {
            double ak = 0.0, av = 0.0;
            for (long i = i0; i < N; ++i) {
                ak += dS[(i - i0) * N + j] * q[i * d + t];
                av += P[(i - i0) * N + j] * dout[i * d + t];
            }
            dk_rows[r * d + t] = scale * ak;
            dv_rows[r * d + t] = av;
        }
    }
    free(P);
    free(dS);
    return 0;
}

/* Sets the number of OpenMP threads of later parallel regions (n >= 1). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
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
