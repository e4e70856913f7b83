"""Anti-vacuity: plausible mistakes planted in a copy of the oracle source
must each fail at least one pin.

Each mutant is the oracle's C source with one textual change (a dropped
term, a flipped sign, a wrong index, a transposed operand, a missing step),
compiled into a temporary directory on the CPU. The real oracle is never
modified.
"""
import os
import shutil
import subprocess

import pytest

import oracle
import oracle_pins as P

MUTANTS = [
    ("drop_cross_term", "d[i] = cc * a + (REAL)2 * cs * b + ss * dd;",
     "d[i] = cc * a + ss * dd;"),
    ("bulge_sign", "bulge = sn * e[i + 1];", "bulge = -sn * e[i + 1];"),
    ("r_wrong_index", "e[i - 1] = r;", "e[i] = r;"),
    ("e_update_sign", "e[i] = cs * (dd - a) + (cc - ss) * b;",
     "e[i] = cs * (dd - a) + (cc + ss) * b;"),
    ("q_rotation_transposed", "Q[row * n + k] = c * qa + s * qb;",
     "Q[row * n + k] = c * qa - s * qb;"),
    ("shift_sign", "return d1 - e1 / (g + R_COPYSIGN(r, g));",
     "return d1 + e1 / (g + R_COPYSIGN(r, g));"),
    ("shift_operands_swapped", "REAL g = (d2 - d1) / ((REAL)2 * e1);",
     "REAL g = (d1 - d2) / ((REAL)2 * e1);"),
    ("lartg_s_unsigned", "*s = g / rr;", "*s = g / h;"),
    ("sym2x2_sign", "*rt1 = a - t * b;", "*rt1 = a + t * b;"),
    ("sym2x2_q_transposed", "SFX(rot_cols)(Q, n, m - 1, cs, -sn);",
     "SFX(rot_cols)(Q, n, m - 1, cs, sn);"),
    ("chase_short", "for (int i = s; i < m; ++i) {", "for (int i = s; i < m - 1; ++i) {"),
    ("bulge_not_moved", "e[i + 1] = c * e[i + 1];", "e[i + 1] = e[i + 1];"),
    ("scale_inverted", "sigma = ssfmax / anorm;", "sigma = anorm / ssfmax;"),
    ("unscale_wrong", "REAL undo = (mode == 1) ? anorm / ssfmax : anorm / ssfmin;",
     "REAL undo = (mode == 1) ? anorm / ssfmax : ssfmin / anorm;"),
    ("no_sort", "lam[rk] = d[j];", "lam[j] = d[j];"),
    ("sort_q_not_permuted", "Q[row * n + rank[j]] = qtmp[row * n + j];",
     "Q[row * n + j] = qtmp[row * n + j];"),
    ("reverse_e_off_by_one", "for (int i = l, j = hi - 1; i < j; ++i, --j) {",
     "for (int i = l, j = hi; i < j; ++i, --j) {"),
    # the choice of the converging end (CTA page, QL versus QR) and the
    # closed-form solve of 2x2 blocks (algorithm page, 2x2 block paragraph)
    ("direction_inverted", "int rev = !(R_FABS(d[hi]) < R_FABS(d[l]));",
     "int rev = (R_FABS(d[hi]) < R_FABS(d[l]));"),
    ("direction_never_reversed", "int rev = !(R_FABS(d[hi]) < R_FABS(d[l]));", "int rev = 0;"),
    ("direction_always_reversed", "int rev = !(R_FABS(d[hi]) < R_FABS(d[l]));", "int rev = 1;"),
    ("no_analytic_2x2", "if (s == m - 1) {", "if (0) {"),
    ("deflation_wrong_pair", "if (SFX(negligible)(e[k - 1], d[k - 1], d[k])) {",
     "if (SFX(negligible)(e[k - 1] * (REAL)1e-3, d[k - 1], d[k])) {"),
    # the PG form of the sweep
    ("pg_drop_factor2", "REAL rs = (d[k + 1] - gs) * sn + (REAL)2 * c * cprev * e[k];",
     "REAL rs = (d[k + 1] - gs) * sn + c * cprev * e[k];"),
    ("pg_g_sign", "g = c * rs - cprev * e[k];", "g = c * rs + cprev * e[k];"),
    ("pg_no_end_fixup", "d[m] = d[m] - p;", "d[m] = d[m];"),
    ("pg_p_not_carried", "REAL gs = d[k] - p;", "REAL gs = d[k];"),
    ("pg_f_unscaled", "REAL f = sprev * e[k];", "REAL f = e[k];"),
    ("pg_q_skipped", "SFX(rot_cols)(Q, n, k, c, sn);", "(void)0;"),
    # the closed-form shift
    ("closed_shift_farther", "return (R_FABS(lp - c) < R_FABS(lm - c)) ? lp : lm;",
     "return (R_FABS(lp - c) < R_FABS(lm - c)) ? lm : lp;"),
    ("closed_shift_radius", "REAL r = R_HYPOT((a - c) / (REAL)2, b);",
     "REAL r = R_HYPOT((a - c), b);"),
    # back-transformation: the basis on entry ignored (Q reset to I)
    ("basis_ignored", "if (Q && !back_transform) {", "if (Q) {"),
    # the dense front end (Householder reduction)
    ("larfg_beta_sign", "REAL b = -R_COPYSIGN(R_HYPOT(alpha, xnorm), alpha);",
     "REAL b = R_COPYSIGN(R_HYPOT(alpha, xnorm), alpha);"),
    ("larfg_tau_inverted", "*tau = (b - alpha) / b;", "*tau = (b - alpha) / alpha;"),
    ("larfg_v_scale", "REAL scal = (REAL)1 / (alpha - b);", "REAL scal = (REAL)1 / (alpha + b);"),
    ("sytrd_no_w_correction", "p[i] = p[i] - half * v[i]; /* p now holds w */",
     "p[i] = p[i]; /* p now holds w */"),
    ("sytrd_rank1_only", "W[i * n + j] = W[i * n + j] - v[i] * p[j] - p[i] * v[j];",
     "W[i * n + j] = W[i * n + j] - v[i] * p[j];"),
    ("sytrd_q_left_applied", "t = t + Q[r * n + j] * v[j];", "t = t + Q[j * n + r] * v[j];"),
    ("sytrd_reads_upper", "W[i * n + j] = A[i * n + j];\n            W[j * n + i] = A[i * n + j];",
     "W[i * n + j] = A[j * n + i];\n            W[j * n + i] = A[j * n + i];"),
    ("sytrd_e_is_alpha", "e[k] = beta;", "e[k] = W[(k + 1) * n + k];"),
    ("syev_no_back_transform", "scheme, shift, 1, 0);", "scheme, shift, 0, 0);"),
    # values-only bisection
    ("sturm_count_sign", "c += q < (REAL)0;", "c += q > (REAL)0;"),
    ("sturm_drop_coupling", "q = (d[i] - x) - e2[i - 1] / q;", "q = (d[i] - x);"),
    ("sturm_wrong_e_index", "q = (d[i] - x) - e2[i - 1] / q;", "q = (d[i] - x) - e2[i] / q;"),
    ("bisect_update_inverted", "if (SFX(oracle_sturm_count)(n, ds, e2, mid, pivmin) <= k)",
     "if (SFX(oracle_sturm_count)(n, ds, e2, mid, pivmin) > k)"),
    ("bisect_index_off_by_one", "if (SFX(oracle_sturm_count)(n, ds, e2, mid, pivmin) <= k)",
     "if (SFX(oracle_sturm_count)(n, ds, e2, mid, pivmin) <= k + 1)"),
    ("gershgorin_no_radius", "if (ds[i] - rad < gl)", "if (ds[i] < gl)"),
    ("stebz_not_unscaled", "lam[k] = ((lo + hi) / (REAL)2) * us;", "lam[k] = ((lo + hi) / (REAL)2);"),
]


def _build_mutant(tmp, old, new):
    src = os.path.join(tmp, "src")
    os.makedirs(src)
    for f in ("steqr_oracle.c", "steqr_oracle_impl.h", "syev_oracle_impl.h",
              "stebz_oracle_impl.h"):
        shutil.copy(os.path.join(oracle.HERE, f), src)
    hits = []
    for f in ("steqr_oracle_impl.h", "syev_oracle_impl.h", "stebz_oracle_impl.h"):
        impl = os.path.join(src, f)
        text = open(impl).read()
        if old in text:
            hits.append((impl, text))
    assert len(hits) == 1 and hits[0][1].count(old) == 1, \
        "mutation anchor not unique/absent: %r" % old
    impl, text = hits[0]
    open(impl, "w").write(text.replace(old, new))
    return oracle.build(out_dir=src, source_dir=src)


def test_real_oracle_passes_quick_pins(oracle_mod):
    assert P.run_all(oracle_mod, quick=True) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    path = _build_mutant(str(tmp_path), old, new)
    fails = P.run_all(oracle, libpath=path, quick=True)
    assert fails, "mutant %s passed every pin" % name
