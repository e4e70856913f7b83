/*
 * CPU oracle body for the batched symmetric tridiagonal eigensolver.
 *
 * TEST INFRASTRUCTURE ONLY. This file is included twice by steqr_oracle.c,
 * once with REAL = float and once with REAL = double; it is never linked
 * into the GPU library and shares no code with it. Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load it.
 *
 * It is a plain, slow, step-by-step implicit shifted QR/QL solver written
 * from the BatchLAS steqr algorithm page (its opening summary: batched
 * symmetric tridiagonal eigenvalue problems by the implicit shifted QR or
 * QL iteration with deflation). Each function names the passage it follows.
 * Compile with -ffp-contract=off and without fast-math: every operation is
 * one IEEE operation in precision REAL, in the order written.
 *
 * Macros expected from the includer:
 *   REAL          float or double
 *   SFX(name)     name suffixed with _f32 or _f64
 *   R_EPS         relative machine precision (unit roundoff) of REAL
 *   R_SAFMIN      smallest normal number of REAL
 *   R_SQRT, R_FABS, R_HYPOT, R_COPYSIGN   libm functions for REAL
 */

/* Constants of the scaling step (algorithm page, scaling paragraph: a block
 * whose norm exceeds the safe range is multiplied by ssfmax/||T||, one with a
 * nonzero norm below it by ssfmin/||T||). The page names ssfmax and ssfmin
 * without defining them; we take the LAPACK definitions sqrt(safmax)/3 and
 * sqrt(safmin)/eps^2 with safmax = 1/safmin. */
static REAL SFX(c_eps)(void) { return R_EPS; }
static REAL SFX(c_eps2)(void) { return R_EPS * R_EPS; }
static REAL SFX(c_safmin)(void) { return R_SAFMIN; }
static REAL SFX(c_ssfmax)(void) { return R_SQRT((REAL)1 / R_SAFMIN) / (REAL)3; }
static REAL SFX(c_ssfmin)(void) { return R_SQRT(R_SAFMIN) / (R_EPS * R_EPS); }

/* Givens rotation lartg(f, g) (algorithm page, "G(c,s)" paragraph): find
 * c, s, r with G(c,s) = [[c,-s],[s,c]], c^2 + s^2 = 1 and
 * G^T (f, g)^T = (r, 0)^T, i.e. c*f + s*g = r and -s*f + c*g = 0.
 * Conventions the page leaves open (sign of r, the zero cases) follow the
 * safe-scaling Givens of Anderson (ACM TOMS Algorithm 978): r carries the
 * sign of f, so c >= 0. g = 0 gives (1, 0, f), as the CTA page's Givens
 * paragraph states; f = 0 gives (0, sign g, |g|). */
void SFX(oracle_lartg)(REAL f, REAL g, REAL *c, REAL *s, REAL *r)
{
    if (g == (REAL)0) {
        *c = (REAL)1;
        *s = (REAL)0;
        *r = f;
    } else if (f == (REAL)0) {
        *c = (REAL)0;
        *s = R_COPYSIGN((REAL)1, g);
        *r = R_FABS(g);
    } else {
        REAL h = R_HYPOT(f, g);
        REAL rr = R_COPYSIGN(h, f);
        *c = R_FABS(f) / h;
        *s = g / rr;
        *r = rr;
    }
}

/* Shift from the trailing 2x2 block (algorithm page, shift paragraph, the
 * form with g = (d2 - d1)/(2 e1), r = sqrt(g^2 + 1),
 * mu = d1 - e1/(g + copysign(r, g))). d1 is the diagonal entry at the
 * converging end, d2 its neighbour inside the block and e1 the coupling
 * between them. The result is the eigenvalue of [[d2, e1], [e1, d1]]
 * nearest d1. r uses hypot so that g^2 cannot overflow. */
REAL SFX(oracle_shift)(REAL d1, REAL d2, REAL e1)
{
    REAL g = (d2 - d1) / ((REAL)2 * e1);
    REAL r = R_HYPOT(g, (REAL)1);
    return d1 - e1 / (g + R_COPYSIGN(r, g));
}

/* Shift in the closed form of the algorithm page's shift paragraph: for the
 * trailing block B = [[a, b], [b, c]] (a = d2, b = e1, c = d1 the entry at
 * the converging end), lambda+- = (a+c)/2 +- sqrt(((a-c)/2)^2 + b^2) and mu
 * is lambda+ when |lambda+ - c| < |lambda- - c|, else lambda-. The square
 * root of the sum is taken with hypot (equal in exact arithmetic, and it
 * cannot overflow). */
REAL SFX(oracle_shift_closed)(REAL d1, REAL d2, REAL e1)
{
    REAL a = d2, b = e1, c = d1;
    REAL h = (a + c) / (REAL)2;
    REAL r = R_HYPOT((a - c) / (REAL)2, b);
    REAL lp = h + r, lm = h - r;
    return (R_FABS(lp - c) < R_FABS(lm - c)) ? lp : lm;
}

/* Analytic solve of a deflated 2x2 block [[a, b], [b, c]] (algorithm page,
 * 2x2 block paragraph: such a block is diagonalised in closed form): returns
 * its eigenvalues rt1 (replacing a) and rt2 (replacing c) and a rotation
 * (cs, sn) such that J^T B J = diag(rt1, rt2) with J = [[cs, sn], [-sn, cs]].
 * The rotation is the symmetric 2x2 Schur decomposition of Golub and Van
 * Loan (Matrix Computations, Jacobi chapter): tau = (c - a)/(2b),
 * t = sign(tau)/(|tau| + sqrt(1 + tau^2)) with sign(0) = +1,
 * cs = 1/sqrt(1 + t^2), sn = t*cs, rt1 = a - t*b, rt2 = c + t*b. */
void SFX(oracle_sym2x2)(REAL a, REAL b, REAL c, REAL *rt1, REAL *rt2,
                        REAL *cs, REAL *sn)
{
    if (b == (REAL)0) {
        *rt1 = a;
        *rt2 = c;
        *cs = (REAL)1;
        *sn = (REAL)0;
        return;
    }
    REAL tau = (c - a) / ((REAL)2 * b);
    REAL den = R_FABS(tau) + R_HYPOT((REAL)1, tau);
    REAL t = (tau >= (REAL)0) ? (REAL)1 / den : (REAL)-1 / den;
    REAL cc = (REAL)1 / R_SQRT((REAL)1 + t * t);
    *cs = cc;
    *sn = t * cc;
    *rt1 = a - t * b;
    *rt2 = c + t * b;
}

/* Deflation test (algorithm page, deflation paragraph): e_i is negligible
 * when |e_i|^2 <= eps^2 |d_i| |d_{i+1}| + safmin. A NaN never passes. */
static int SFX(negligible)(REAL ei, REAL di, REAL dj)
{
    REAL lhs = ei * ei;
    REAL rhs = SFX(c_eps2)() * R_FABS(di) * R_FABS(dj) + SFX(c_safmin)();
    return lhs <= rhs;
}

/* Right-multiply columns (k, k+1) of the row-major n x n matrix Q by
 * G(c, s) = [[c, -s], [s, c]] (algorithm page, eigenvector accumulation:
 * Q_{:,{k,k+1}} <- Q_{:,{k,k+1}} G(c,s)). */
static void SFX(rot_cols)(REAL *Q, int n, int k, REAL c, REAL s)
{
    for (int row = 0; row < n; ++row) {
        REAL qa = Q[row * n + k];
        REAL qb = Q[row * n + k + 1];
        Q[row * n + k] = c * qa + s * qb;
        Q[row * n + k + 1] = -s * qa + c * qb;
    }
}

/* One implicit shifted QR sweep on the unreduced block [s, m] with shift mu
 * (algorithm page: QR/QL paragraph, where the QR sweep runs in storage order;
 * the Givens/adjacent similarity paragraphs and the bulge paragraph). The
 * first rotation comes
 * from (d_s - mu, e_s); each later one from (e_{i-1}, bulge) and annihilates
 * the bulge, storing r in e_{i-1}. Each rotation is applied as the
 * congruence G^T B G of the 2x2 block at (i, i+1):
 *   d_i'     = c^2 d_i + 2 c s e_i + s^2 d_{i+1}
 *   d_{i+1}' = s^2 d_i - 2 c s e_i + c^2 d_{i+1}
 *   e_i'     = c s (d_{i+1} - d_i) + (c^2 - s^2) e_i
 * and moves the bulge down: bulge = s e_{i+1}, e_{i+1} <- c e_{i+1}.
 * (The page prints these updates with the opposite sign of s; with the
 * page's own definition of G and lartg the signs above are the consistent
 * ones.) Returns the number of rotations. */
long SFX(oracle_sweep)(REAL *d, REAL *e, REAL *Q, int n, int s, int m, REAL mu)
{
    REAL x = d[s] - mu;
    REAL y = e[s];
    long rots = 0;
    for (int i = s; i < m; ++i) {
        REAL c, sn, r;
        SFX(oracle_lartg)(x, y, &c, &sn, &r);
        if (i > s)
            e[i - 1] = r;
        REAL a = d[i], b = e[i], dd = d[i + 1];
        REAL cc = c * c, ss = sn * sn, cs = c * sn;
        d[i] = cc * a + (REAL)2 * cs * b + ss * dd;
        d[i + 1] = ss * a - (REAL)2 * cs * b + cc * dd;
        e[i] = cs * (dd - a) + (cc - ss) * b;
        REAL bulge = (REAL)0;
        if (i + 1 <= m - 1) {
            bulge = sn * e[i + 1];
            e[i + 1] = c * e[i + 1];
        }
        if (Q)
            SFX(rot_cols)(Q, n, i, c, sn);
        x = e[i];
        y = bulge;
        ++rots;
    }
    return rots;
}

/* One implicit QR sweep on [s, m] in the Parlett-Gray (PG) form of the
 * algorithm page (update-scheme paragraph): four running scalars (g, p, c, s)
 * pass from step to step in place of the written-out 2x2 congruence.
 * Step i (QR form, as the page writes it):
 *   f_i = s_{i-1} e_i,  (c_i, s_i, r_i) = lartg(g_{i-1}, f_i),
 *   g*_i = d_i - p_{i-1},  r*_i = (d_{i+1} - g*_i) s_i + 2 c_i c_{i-1} e_i,
 *   p_i = s_i r*_i,  d_i <- g*_i + p_i,  g_i = c_i r*_i - c_{i-1} e_i,
 * with e_{i-1} <- r_i for i > s. The page leaves the start and the end
 * implicit; read plainly: g_{s-1} = d_s - mu (the shifted corner that the
 * first rotation annihilates), s_{s-1} = c_{s-1} = 1, p_{s-1} = 0, and
 * after the last step d_m <- d_m - p_{m-1}, e_{m-1} <- g_{m-1}. Q receives
 * the same rotations as in the EXP form. Returns the number of rotations. */
long SFX(oracle_sweep_pg)(REAL *d, REAL *e, REAL *Q, int n, int s, int m, REAL mu)
{
    REAL g = d[s] - mu;
    REAL p = (REAL)0, cprev = (REAL)1, sprev = (REAL)1;
    long rots = 0;
    for (int k = s; k < m; ++k) {
        REAL f = sprev * e[k];
        REAL c, sn, r;
        SFX(oracle_lartg)(g, f, &c, &sn, &r);
        if (k > s)
            e[k - 1] = r;
        REAL gs = d[k] - p;
        REAL rs = (d[k + 1] - gs) * sn + (REAL)2 * c * cprev * e[k];
        p = sn * rs;
        d[k] = gs + p;
        g = c * rs - cprev * e[k];
        if (Q)
            SFX(rot_cols)(Q, n, k, c, sn);
        cprev = c;
        sprev = sn;
        ++rots;
    }
    d[m] = d[m] - p;
    e[m - 1] = g;
    return rots;
}

/* Reverse the block [l, hi] in place: d~_k = d_{l+hi-k}, e~_k = e_{l+hi-1-k}
 * and reverse Q's columns l..hi (algorithm page, QR/QL paragraph: the QL
 * sweep is the QR sweep with the local indices reversed). Applying it twice restores the block. */
static void SFX(reverse_block)(REAL *d, REAL *e, REAL *Q, int n, int l, int hi)
{
    for (int i = l, j = hi; i < j; ++i, --j) {
        REAL t = d[i];
        d[i] = d[j];
        d[j] = t;
    }
    for (int i = l, j = hi - 1; i < j; ++i, --j) {
        REAL t = e[i];
        e[i] = e[j];
        e[j] = t;
    }
    if (Q) {
        for (int row = 0; row < n; ++row) {
            for (int i = l, j = hi; i < j; ++i, --j) {
                REAL t = Q[row * n + i];
                Q[row * n + i] = Q[row * n + j];
                Q[row * n + j] = t;
            }
        }
    }
}

/* The QR procedure on one split block [l, hi] whose bottom end converges
 * first (algorithm page: deflation paragraph, where each step repeats the
 * test and finds the last new zero from the converging end; the 2x2, shift
 * and sweep paragraphs). Loop:
 *  (i)   scan from the bottom for the largest s in (l, m] with e_{s-1}
 *        negligible, zero that e_{s-1}; no such s gives s = l;
 *  (ii)  s == m: d_m has converged, m <- m - 1;
 *  (iii) s == m - 1: solve the 2x2 analytically, m <- m - 2;
 *  (iv)  otherwise, if the sweep budget is spent, fail; else count a sweep,
 *        take mu from the trailing 2x2 and sweep [s, m].
 * Returns 1 when the block converged, 0 when the budget ran out. */
static int SFX(qr_block)(REAL *d, REAL *e, REAL *Q, int n, int l, int hi,
                         int *jtot, int nmaxit, int scheme, int shift, long long *stats)
{
    int m = hi;
    while (m > l) {
        int s = l;
        for (int k = m; k > l; --k) {
            if (SFX(negligible)(e[k - 1], d[k - 1], d[k])) {
                e[k - 1] = (REAL)0;
                s = k;
                break;
            }
        }
        if (s == m) {
            m -= 1;
            continue;
        }
        if (s == m - 1) {
            REAL rt1, rt2, cs, sn;
            SFX(oracle_sym2x2)(d[m - 1], e[m - 1], d[m], &rt1, &rt2, &cs, &sn);
            d[m - 1] = rt1;
            d[m] = rt2;
            e[m - 1] = (REAL)0;
            if (Q) /* J = [[cs, sn], [-sn, cs]] = G(cs, -sn) */
                SFX(rot_cols)(Q, n, m - 1, cs, -sn);
            if (stats)
                stats[2] += 1;
            m -= 2;
            continue;
        }
        if (*jtot >= nmaxit)
            return 0;
        *jtot += 1;
        REAL mu = shift ? SFX(oracle_shift_closed)(d[m], d[m - 1], e[m - 1])
                        : SFX(oracle_shift)(d[m], d[m - 1], e[m - 1]);
        long rots = scheme ? SFX(oracle_sweep_pg)(d, e, Q, n, s, m, mu)
                           : SFX(oracle_sweep)(d, e, Q, n, s, m, mu);
        if (stats) {
            stats[0] += 1;
            stats[1] += rots;
        }
    }
    return 1;
}

/* Strict total order used by the sort: ascending value, ties broken by
 * index (stable); a NaN sorts after every number, NaNs by index. */
static int SFX(before)(REAL a, int ia, REAL b, int ib)
{
    int na = a != a, nb = b != b;
    if (na || nb) {
        if (na && nb)
            return ia < ib;
        return nb; /* a is a number and b a NaN */
    }
    if (a < b)
        return 1;
    if (a == b)
        return ia < ib;
    return 0;
}

/* Solve one matrix. d[n], e[n-1] are overwritten (d with the eigenvalues in
 * converged order, e with the final off-diagonal). Q (n x n row-major, may be
 * NULL) receives the eigenvectors as columns. lam receives the eigenvalues,
 * sorted ascending when sort != 0 and the solve converged (algorithm page,
 * last paragraph before the summary: sort ascending and permute Q's columns
 * the same way). Returns info: 0 on success, else the number of nonzero
 * off-diagonal entries left when the sweep budget (max_sweeps_per_n * n
 * implicit sweeps) ran out; then lam = d unsorted and Q unsorted.
 *
 * Split bookkeeping (algorithm page, steqr_cta paragraph on the running left
 * boundary): b_begin <- b_next, e_{b_begin-1} <- 0, b_end = first i >= b_begin
 * with e_i = 0 (n-1 if none), b_next <- b_end + 1. Each block is scaled
 * (scaling paragraph), its direction chosen so the end of smaller |d|
 * converges first ("QL if |D_l| <= |D_lend|", CTA page, micro-structure
 * list), run as a QR procedure on the possibly reversed block, then
 * unscaled. */
int SFX(oracle_solve_one)(int n, REAL *d, REAL *e, REAL *Q, REAL *lam,
                          int max_sweeps_per_n, int sort, int scheme, int shift,
                          int back_transform, long long *stats)
{
    const REAL ssfmax = SFX(c_ssfmax)();
    const REAL ssfmin = SFX(c_ssfmin)();
    int info = 0;
    /* Eigenvector accumulation (algorithm page, eigenvector paragraph):
     * without back-transformation Q starts as the identity; with it, Q
     * holds the caller's basis on entry and every rotation right-multiplies
     * it, so the result is that basis times the product of the rotations. */
    if (Q && !back_transform) {
        for (int i = 0; i < n * n; ++i)
            Q[i] = (REAL)0;
        for (int i = 0; i < n; ++i)
            Q[i * n + i] = (REAL)1;
    }
    int jtot = 0;
    const int nmaxit = max_sweeps_per_n * n;
    int l1 = 0;
    while (l1 < n) {
        if (l1 > 0)
            e[l1 - 1] = (REAL)0;
        int hi = l1;
        while (hi < n - 1 && e[hi] != (REAL)0)
            ++hi;
        int l = l1;
        l1 = hi + 1;
        if (hi == l)
            continue;
        /* block norm: max |d_i|, |e_i| over the block, NaN-propagating */
        REAL anorm = (REAL)0;
        for (int i = l; i <= hi; ++i) {
            REAL a = R_FABS(d[i]);
            if (a != a || a > anorm)
                anorm = a;
            if (anorm != anorm)
                break;
        }
        for (int i = l; i < hi && anorm == anorm; ++i) {
            REAL a = R_FABS(e[i]);
            if (a != a || a > anorm)
                anorm = a;
        }
        if (anorm == (REAL)0)
            continue;
        int mode = 0;
        REAL sigma = (REAL)1;
        if (anorm > ssfmax) {
            mode = 1;
            sigma = ssfmax / anorm;
        } else if (anorm < ssfmin) {
            mode = 2;
            sigma = ssfmin / anorm;
        }
        if (mode) {
            for (int i = l; i <= hi; ++i)
                d[i] = d[i] * sigma;
            for (int i = l; i < hi; ++i)
                e[i] = e[i] * sigma;
        }
        /* converge the end of smaller magnitude first; a tie (or a NaN)
         * converges the top end first, which is done by reversal */
        int rev = !(R_FABS(d[hi]) < R_FABS(d[l]));
        if (rev)
            SFX(reverse_block)(d, e, Q, n, l, hi);
        int ok = SFX(qr_block)(d, e, Q, n, l, hi, &jtot, nmaxit, scheme, shift, stats);
        if (rev)
            SFX(reverse_block)(d, e, Q, n, l, hi);
        if (mode) {
            REAL undo = (mode == 1) ? anorm / ssfmax : anorm / ssfmin;
            for (int i = l; i <= hi; ++i)
                d[i] = d[i] * undo;
            if (!ok)
                for (int i = l; i < hi; ++i)
                    e[i] = e[i] * undo;
        }
        if (!ok) {
            for (int i = 0; i < n - 1; ++i)
                info += (e[i] != (REAL)0);
            if (info == 0)
                info = 1;
            break;
        }
    }
    if (info != 0 || !sort) {
        for (int i = 0; i < n; ++i)
            lam[i] = d[i];
        return info;
    }
    /* stable ascending sort: rank_j = #{k : (d_k, k) before (d_j, j)} */
    int rank_buf[512];
    int *rank = rank_buf;
    REAL *qtmp = 0;
    for (int j = 0; j < n; ++j) {
        int rk = 0;
        for (int k = 0; k < n; ++k)
            rk += SFX(before)(d[k], k, d[j], j);
        rank[j] = rk;
        lam[rk] = d[j];
    }
    if (Q) {
        qtmp = (REAL *)malloc(sizeof(REAL) * (size_t)n * (size_t)n);
        for (int i = 0; i < n * n; ++i)
            qtmp[i] = Q[i];
        for (int row = 0; row < n; ++row)
            for (int j = 0; j < n; ++j)
                Q[row * n + rank[j]] = qtmp[row * n + j];
        free(qtmp);
    }
    return info;
}

/* Batched entry: d [batch][n], e [batch][n-1] (read only), lam [batch][n],
 * Q [batch][n][n] row-major or NULL, info [batch] or NULL, stats
 * [batch][3] or NULL (implicit sweeps, sweep rotations, analytic 2x2
 * solves per item); scheme 0 = EXP sweeps, 1 = PG sweeps; shift 0 = the
 * LAPACK form, 1 = the closed form lambda+-; back_transform 0 = Q is
 * output only (starts as I), 1 = Q holds a basis Z on entry and receives
 * Z times the rotations. Returns 0, or -1 if n is out of range. */
int SFX(oracle_steqr_batched)(const REAL *d, const REAL *e, REAL *lam,
                              REAL *Q, int *info, long long *stats, int n,
                              long batch, int max_sweeps_per_n, int sort, int scheme,
                              int shift, int back_transform)
{
    if (n < 0 || n > 512)
        return -1;
    if (n == 0)
        return 0;
    REAL *dw = (REAL *)malloc(sizeof(REAL) * (size_t)n);
    REAL *ew = (REAL *)malloc(sizeof(REAL) * (size_t)(n > 1 ? n : 1));
    for (long b = 0; b < batch; ++b) {
        for (int i = 0; i < n; ++i)
            dw[i] = d[b * n + i];
        for (int i = 0; i < n - 1; ++i)
            ew[i] = e[b * (n - 1) + i];
        long long *st = stats ? stats + 3 * b : 0;
        if (st)
            st[0] = st[1] = st[2] = 0;
        int inf = SFX(oracle_solve_one)(n, dw, ew, Q ? Q + b * (long)n * n : 0,
                                        lam + b * n, max_sweeps_per_n, sort, scheme, shift,
                                        back_transform, st);
        if (info)
            info[b] = inf;
    }
    free(dw);
    free(ew);
    return 0;
}
