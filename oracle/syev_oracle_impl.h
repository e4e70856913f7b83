/*
 * CPU oracle for the fused small-n dense symmetric eigensolver (syev):
 * Householder reduction to tridiagonal form, the tridiagonal solve of
 * steqr_oracle_impl.h with back-transformation, eigenvalues ascending.
 *
 * TEST INFRASTRUCTURE ONLY, like steqr_oracle_impl.h (included after it by
 * steqr_oracle.c, once per precision). The pages name the stages of the
 * fused kernel (BatchLAS syev routing and tuning page, CTA-family paragraph:
 * reduction sytrd, the steqr solve, the back-transformation, one problem
 * resident from load to store) but not the reduction's arithmetic; it is
 * written here as the textbook Householder tridiagonalization (Golub and
 * Van Loan, "Householder tridiagonalization"; the reflector in the LAPACK
 * larfg convention), one plain step at a time.
 */

/* Householder reflector for x = (alpha, x_1..x_m): H = I - tau v v^T with
 * v = (1, v_1..v_m) and H x = (beta, 0, .., 0). With xnorm = ||(x_1..x_m)||:
 * xnorm = 0 gives tau = 0 and beta = alpha (H = I); otherwise
 * beta = -sign(alpha) ||(alpha, xnorm)||, tau = (beta - alpha) / beta and
 * v_i = x_i / (alpha - beta). x is overwritten with v_1..v_m. */
void SFX(oracle_larfg)(int m, REAL alpha, REAL *x, REAL *beta, REAL *tau)
{
    REAL xnorm = (REAL)0;
    for (int i = 0; i < m; ++i)
        xnorm = R_HYPOT(xnorm, x[i]);
    if (xnorm == (REAL)0) {
        *tau = (REAL)0;
        *beta = alpha;
        return;
    }
    REAL b = -R_COPYSIGN(R_HYPOT(alpha, xnorm), alpha);
    *tau = (b - alpha) / b;
    REAL scal = (REAL)1 / (alpha - b);
    for (int i = 0; i < m; ++i)
        x[i] = x[i] * scal;
    *beta = b;
}

/* Reduce the dense symmetric n x n matrix whose lower triangle is read from
 * row-major A (the strict upper triangle is ignored) to tridiagonal form
 * T = Q^T A Q. Step k = 0..n-2 takes the reflector H_k of column k below
 * the diagonal, records d_k = a_kk and e_k = beta, and applies H_k from both
 * sides to the trailing block by the symmetric rank-2 update
 *   p = tau W v,  w = p - (tau (p^T v) / 2) v,  W <- W - v w^T - w v^T.
 * Q (if non-NULL) receives H_0 H_1 ... H_{n-2}, accumulated from the
 * identity by right-multiplication, row by row. */
void SFX(oracle_sytrd)(int n, const REAL *A, REAL *d, REAL *e, REAL *Q)
{
    if (n <= 0)
        return;
    REAL *W = (REAL *)malloc(sizeof(REAL) * (size_t)n * (size_t)n);
    REAL *v = (REAL *)malloc(sizeof(REAL) * (size_t)n);
    REAL *p = (REAL *)malloc(sizeof(REAL) * (size_t)n);
    for (int i = 0; i < n; ++i)
        for (int j = 0; j <= i; ++j) {
            W[i * n + j] = A[i * n + j];
            W[j * n + i] = A[i * n + j];
        }
    if (Q) {
        for (int i = 0; i < n * n; ++i)
            Q[i] = (REAL)0;
        for (int i = 0; i < n; ++i)
            Q[i * n + i] = (REAL)1;
    }
    for (int k = 0; k + 1 < n; ++k) {
        /* x = column k below the diagonal: alpha = w_{k+1,k}, then the rest */
        for (int i = 0; i <= k; ++i)
            v[i] = (REAL)0;
        for (int i = k + 2; i < n; ++i)
            v[i] = W[i * n + k];
        REAL beta, tau;
        SFX(oracle_larfg)(n - k - 2, W[(k + 1) * n + k], v + k + 2, &beta, &tau);
        v[k + 1] = (REAL)1;
        d[k] = W[k * n + k];
        e[k] = beta;
        if (tau == (REAL)0)
            continue;
        for (int i = k + 1; i < n; ++i) {
            REAL s = (REAL)0;
            for (int j = k + 1; j < n; ++j)
                s = s + W[i * n + j] * v[j];
            p[i] = tau * s;
        }
        REAL pv = (REAL)0;
        for (int i = k + 1; i < n; ++i)
            pv = pv + p[i] * v[i];
        REAL half = tau * pv / (REAL)2;
        for (int i = k + 1; i < n; ++i)
            p[i] = p[i] - half * v[i]; /* p now holds w */
        for (int i = k + 1; i < n; ++i)
            for (int j = k + 1; j < n; ++j)
                W[i * n + j] = W[i * n + j] - v[i] * p[j] - p[i] * v[j];
        if (Q)
            for (int r = 0; r < n; ++r) {
                REAL t = (REAL)0;
                for (int j = k + 1; j < n; ++j)
                    t = t + Q[r * n + j] * v[j];
                t = tau * t;
                for (int j = k + 1; j < n; ++j)
                    Q[r * n + j] = Q[r * n + j] - t * v[j];
            }
    }
    d[n - 1] = W[(n - 1) * n + n - 1];
    free(W);
    free(v);
    free(p);
}

/* Batched reduction: A [batch][n][n] (lower triangle read), d [batch][n],
 * e [batch][n-1], Q [batch][n][n] or NULL. Returns 0, or -1 if n is out of
 * range. */
int SFX(oracle_sytrd_batched)(const REAL *A, REAL *d, REAL *e, REAL *Q, int n, long batch)
{
    if (n < 0 || n > 256)
        return -1;
    if (n == 0)
        return 0;
    REAL *ew = (REAL *)malloc(sizeof(REAL) * (size_t)n);
    for (long b = 0; b < batch; ++b) {
        SFX(oracle_sytrd)(n, A + b * (long)n * n, d + b * n, ew,
                          Q ? Q + b * (long)n * n : 0);
        for (int i = 0; i < n - 1; ++i)
            e[b * (n - 1) + i] = ew[i];
    }
    free(ew);
    return 0;
}

/* Dense symmetric eigensolver: for each A_b (lower triangle read) the
 * reduction above, then the tridiagonal solve with the reduction's Q as the
 * basis of the back-transformation (Q = NULL: eigenvalues only). lam
 * [batch][n] ascending, Q [batch][n][n] row-major with eigenvector k in
 * column k, info [batch] or NULL as in oracle_steqr_batched. */
int SFX(oracle_syev_batched)(const REAL *A, REAL *lam, REAL *Q, int *info, int n, long batch,
                             int max_sweeps_per_n, int sort, int scheme, int shift)
{
    if (n < 0 || n > 256)
        return -1;
    if (n == 0)
        return 0;
    REAL *dw = (REAL *)malloc(sizeof(REAL) * (size_t)n);
    REAL *ew = (REAL *)malloc(sizeof(REAL) * (size_t)n);
    for (long b = 0; b < batch; ++b) {
        REAL *Qb = Q ? Q + b * (long)n * n : 0;
        SFX(oracle_sytrd)(n, A + b * (long)n * n, dw, ew, Qb);
        int inf = SFX(oracle_solve_one)(n, dw, ew, Qb, lam + b * n, max_sweeps_per_n, sort,
                                        scheme, shift, 1, 0);
        if (info)
            info[b] = inf;
    }
    free(dw);
    free(ew);
    return 0;
}
