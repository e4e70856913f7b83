/*
 * CPU oracle for the eigenvalue-only bisection solve of a symmetric
 * tridiagonal matrix (values mode).
 *
 * TEST INFRASTRUCTURE ONLY, like steqr_oracle_impl.h (included after it by
 * steqr_oracle.c, once per precision). The pages describe the values-only
 * path as stebz bisection for the indices 0..n-1 in ascending order, run
 * straight off the tridiagonal, with three exits: the tolerance met, the
 * iteration budget exhausted, the midpoint no longer advancing (BatchLAS
 * syev routing and tuning page: the values-only blocked solve and its
 * open-debts paragraph). They give no formulas; the steps below are the
 * textbook Sturm-count bisection (the LDL^T inertia count of T - x I, as in
 * LAPACK's stebz/laebz), one eigenvalue index at a time:
 *
 *   count(x) = #{i : q_i < 0},  q_1 = d_1 - x,
 *              q_i = (d_i - x) - e_{i-1}^2 / q_{i-1},
 *              each |q_i| < pivmin replaced by -pivmin,
 *   pivmin   = safmin * max(1, max e_i^2),
 *   [gl, gu] = the Gershgorin interval, widened by 2 n ulp ||T|| + 2 pivmin,
 *   eigenvalue k: lo = gl, hi = gu; while hi - lo > max(ulp ||T||,
 *              2 ulp max(|lo|, |hi|)): mid = (lo + hi) / 2, stop if mid
 *              equals lo or hi, count(mid) <= k ? lo = mid : hi = mid;
 *              at most itmax = floor(log2((||T|| + pivmin) / pivmin)) + 2
 *              halvings; lambda_k = (lo + hi) / 2.
 *
 * Readings (the pages leave them open): ||T|| is the Gershgorin norm
 * max_i |e_{i-1}| + |d_i| + |e_i|; the band is first scaled by the power of
 * two 2^-ceil(log2 ||T||) (exact, so lambda(2^j T) = 2^j lambda(T) bit for
 * bit, and e^2 cannot overflow) and lambda is scaled back; a NaN anywhere
 * gives NaN eigenvalues; T = 0 gives zeros; the status is the number of
 * eigenvalues that ran out of halvings (the pages note that stebz records
 * none and needs one).
 */

/* Sturm count: the number of eigenvalues of T smaller than x (above). */
int SFX(oracle_sturm_count)(int n, const REAL *d, const REAL *e2, REAL x, REAL pivmin)
{
    int c = 0;
    REAL q = (REAL)0;
    for (int i = 0; i < n; ++i) {
        if (i == 0)
            q = d[0] - x;
        else
            q = (d[i] - x) - e2[i - 1] / q;
        if (R_FABS(q) < pivmin)
            q = -pivmin;
        c += q < (REAL)0;
    }
    return c;
}

/* All eigenvalues of one tridiagonal, ascending, by bisection (above).
 * Returns the number of indices that exhausted the halving budget; *counts
 * (if non-NULL) receives the number of Sturm counts evaluated. */
int SFX(oracle_stebz_one)(int n, const REAL *d, const REAL *e, REAL *lam, long long *counts)
{
    if (counts)
        *counts = 0;
    const REAL ulp = (REAL)2 * R_EPS;
    REAL tn = (REAL)0;
    int hasnan = 0;
    for (int i = 0; i < n; ++i) {
        REAL r = R_FABS(d[i]);
        if (i > 0)
            r = r + R_FABS(e[i - 1]);
        if (i < n - 1)
            r = r + R_FABS(e[i]);
        hasnan |= r != r;
        if (r > tn)
            tn = r;
    }
    if (hasnan) {
        for (int k = 0; k < n; ++k)
            lam[k] = R_SQRT((REAL)-1); /* NaN */
        return n;
    }
    if (tn == (REAL)0) {
        for (int k = 0; k < n; ++k)
            lam[k] = (REAL)0;
        return 0;
    }
    int ex;
    (void)frexp((double)tn, &ex); /* tn = f * 2^ex, f in [0.5, 1) */
    const REAL s = (REAL)ldexp(1.0, -ex), us = (REAL)ldexp(1.0, ex);
    REAL *ds = (REAL *)malloc(sizeof(REAL) * (size_t)n);
    REAL *e2 = (REAL *)malloc(sizeof(REAL) * (size_t)(n > 1 ? n : 1));
    REAL e2max = (REAL)0;
    for (int i = 0; i < n; ++i)
        ds[i] = d[i] * s;
    for (int i = 0; i < n - 1; ++i) {
        REAL es = e[i] * s;
        e2[i] = es * es;
        if (e2[i] > e2max)
            e2max = e2[i];
    }
    const REAL pivmin = R_SAFMIN * (e2max > (REAL)1 ? e2max : (REAL)1);
    /* Gershgorin interval and norm of the scaled band */
    REAL gl = ds[0], gu = ds[0], tns = (REAL)0;
    for (int i = 0; i < n; ++i) {
        REAL rad = (REAL)0;
        if (i > 0)
            rad = rad + R_FABS(e[i - 1] * s);
        if (i < n - 1)
            rad = rad + R_FABS(e[i] * s);
        if (ds[i] - rad < gl)
            gl = ds[i] - rad;
        if (ds[i] + rad > gu)
            gu = ds[i] + rad;
        if (R_FABS(ds[i]) + rad > tns)
            tns = R_FABS(ds[i]) + rad;
    }
    const REAL widen = (REAL)2 * (REAL)n * ulp * tns + (REAL)2 * pivmin;
    gl = gl - widen;
    gu = gu + widen;
    const REAL atol = ulp * tns;
    int lg;
    (void)frexp(((double)tns + (double)pivmin) / (double)pivmin, &lg);
    const int itmax = (lg - 1) + 2; /* floor(log2(r)) = lg - 1 exactly */
    int info = 0;
    for (int k = 0; k < n; ++k) {
        REAL lo = gl, hi = gu;
        int it = 0, done = 0;
        while (!done) {
            REAL big = R_FABS(lo) > R_FABS(hi) ? R_FABS(lo) : R_FABS(hi);
            REAL tol = (REAL)2 * ulp * big;
            if (atol > tol)
                tol = atol;
            if (hi - lo <= tol)
                break; /* tolerance met */
            if (it == itmax) {
                ++info; /* budget exhausted */
                break;
            }
            REAL mid = (lo + hi) / (REAL)2;
            if (mid == lo || mid == hi)
                break; /* midpoint no longer advances */
            if (SFX(oracle_sturm_count)(n, ds, e2, mid, pivmin) <= k)
                lo = mid;
            else
                hi = mid;
            ++it;
            if (counts)
                ++*counts;
        }
        lam[k] = ((lo + hi) / (REAL)2) * us;
    }
    free(ds);
    free(e2);
    return info;
}

/* Batched values-only bisection: d [batch][n], e [batch][n-1], lam
 * [batch][n] ascending, info [batch] or NULL, counts [batch] (Sturm counts
 * evaluated per item) or NULL. Returns 0, or -1 if n is out of range. */
int SFX(oracle_stebz_batched)(const REAL *d, const REAL *e, REAL *lam, int *info,
                              long long *counts, int n, long batch)
{
    if (n < 0 || n > 512)
        return -1;
    for (long b = 0; b < batch && n > 0; ++b) {
        int inf = SFX(oracle_stebz_one)(n, d + b * n, e + b * (n - 1), lam + b * n,
                                        counts ? counts + b : 0);
        if (info)
            info[b] = inf;
    }
    return 0;
}
