"""Plant plausible slips in a copy of the oracle (on the CPU) and check that the
pins in test_oracle.py catch every one of them.

The pin files (test_oracle.py for the Birkhoff functions, test_oracle_eot.py
for the general entropic OT, test_oracle_mix.py for the stream mixing) run
against every mutant.  Each mutant is oracle.c
with one textual edit (a flipped sign, a dropped term,
a transposed index, a lost gauge), compiled to a temporary library and loaded
by the oracle's Python wrapper through ORACLE_LIB in a child pytest run.
"""
import os
import pathlib
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
SRC = (ROOT / "oracle" / "oracle.c").read_text()

MUTANTS = {
    "control_unmutated": ("int oracle_nmax(void) { return ORACLE_NMAX; }", "int oracle_nmax(void) { return ORACLE_NMAX; }"),
    "bwd_sign": ("dH[i * n + j] = -Dij;", "dH[i * n + j] = Dij;"),
    "bwd_drop_Tdiagw": ("v[i] * T[i * n + j] + T[i * n + j] * w[j] - gam[i * n + j]",
                        "v[i] * T[i * n + j] - gam[i * n + j]"),
    "bwd_muc_transposed": ("muc += gam[i * n + j];", "muc += gam[j * n + i];"),
    "bwd_delta_sign": ("delta[j * m + k] = (j == k ? 1.0 : 0.0) - p;", "delta[j * m + k] = (j == k ? 1.0 : 0.0) + p;"),
    "bwd_rhs_sign": ("rhs[j] = muc - tmu;", "rhs[j] = muc + tmu;"),
    "bwd_v_transposed": ("s -= T[i * n + j] * w[j];", "s -= T[j * n + i] * w[j];"),
    "colupdate_transposed": ("for (int i = 0; i < n; ++i) u[i] = H[i * n + j] + alpha[i];",
                             "for (int i = 0; i < n; ++i) u[i] = H[j * n + i] + alpha[i];"),
    "alpha_sign": ("alpha[i] = -lse(u, n, 1);", "alpha[i] = lse(u, n, 1);"),
    "primal_beta_sign": ("exp(alpha[i] + beta[j] + H[i * n + j])", "exp(alpha[i] - beta[j] + H[i * n + j])"),
    "lost_gauge": ("beta_out[j] = beta[j] - beta[n - 1];", "beta_out[j] = beta[j];"),
    "hessian_sign": ("hess[j * m + k] = -p;", "hess[j * m + k] = p;"),
    "hessian_diag_self": ("if (l != j) o += T[i * n + l];", "if (l != j + 1) o += T[i * n + l];"),
    "hessian_diag_weight": ("p += T[i * n + j] * o;", "p += o;"),
    "gradient_sign": ("g[j] = c[j] - 1.0; gn2 += g[j] * g[j];", "g[j] = 1.0 - c[j]; gn2 += g[j] * g[j];"),
    "linesearch_df_sign": ("for (int j = 0; j < m; ++j) df -= gam * d[j];", "for (int j = 0; j < m; ++j) df += gam * d[j];"),
    "softmax_no_max_shift_wrong": ("double e = exp(H[i * n + j] + beta[j] - mu);", "double e = exp(H[i * n + j] - beta[j] - mu);"),
    # general entropic OT (cost M, marginals a and b, eta)
    "eot_alpha_drop_loga": ("alpha[i] = eta * log(a[i]) - eta * lse(u, m, 1);", "alpha[i] = -eta * lse(u, m, 1);"),
    "eot_beta_sign": ("beta[j] = eta * log(b[j]) - eta * lse(u, n, 1);", "beta[j] = eta * log(b[j]) + eta * lse(u, n, 1);"),
    "eot_alpha_drop_eta": ("for (int j = 0; j < m; ++j) u[j] = (beta[j] - M[i * m + j]) / eta;",
                           "for (int j = 0; j < m; ++j) u[j] = (beta[j] - M[i * m + j]);"),
    "eot_primal_beta_sign": ("exp((alpha[i] + beta[j] - M[i * m + j]) / eta)", "exp((alpha[i] - beta[j] - M[i * m + j]) / eta)"),
    "eot_sk_lost_gauge": ("for (int j = 0; j < m; ++j) beta_out[j] = beta[j] - beta[m - 1];",
                          "for (int j = 0; j < m; ++j) beta_out[j] = beta[j];"),
    "eot_plan_drop_a": ("for (int j = 0; j < m; ++j) T[i * m + j] *= a[i] / s;", "for (int j = 0; j < m; ++j) T[i * m + j] *= 1.0 / s;"),
    "eot_hessian_drop_inv_a": ("for (int i = 0; i < n; ++i) p += T[i * m + j] * T[i * m + k] / a[i];",
                               "for (int i = 0; i < n; ++i) p += T[i * m + j] * T[i * m + k];"),
    "eot_hessian_diag_drop_inv_a": ("p += T[i * m + j] / a[i] * o;", "p += T[i * m + j] * o;"),
    "eot_hessian_drop_eta": ("hess[j * k1 + k] = -p / eta;", "hess[j * k1 + k] = -p;"),
    "eot_hessian_diag_drop_eta": ("hess[j * k1 + k] = p / eta;", "hess[j * k1 + k] = p;"),
    "eot_gradient_marginal": ("for (int j = 0; j < k1; ++j) { g[j] = c[j] - b[j]; gn2 += g[j] * g[j]; }",
                              "for (int j = 0; j < k1; ++j) { g[j] = c[j] - 1.0 / m; gn2 += g[j] * g[j]; }"),
    "eot_df_drop_eta": ("df += eta * a[i] * log1p(acc);", "df += a[i] * log1p(acc);"),
    "eot_df_expm1_eta": ("acc += T[i * m + j] / a[i] * expm1(gam * d[j] / eta);", "acc += T[i * m + j] / a[i] * expm1(gam * d[j]);"),
    "eot_bwd_drop_inv_a": ("(v[i] / a[i] * T[i * m + j] + T[i * m + j] * w[j] - gam[i * m + j]) / eta",
                           "(v[i] * T[i * m + j] + T[i * m + j] * w[j] - gam[i * m + j]) / eta"),
    "eot_bwd_drop_eta": ("(v[i] / a[i] * T[i * m + j] + T[i * m + j] * w[j] - gam[i * m + j]) / eta",
                         "(v[i] / a[i] * T[i * m + j] + T[i * m + j] * w[j] - gam[i * m + j])"),
    "eot_bwd_delta_b": ("delta[j * k1 + k] = (j == k ? b[j] : 0.0) - p;", "delta[j * k1 + k] = (j == k ? 1.0 : 0.0) - p;"),
    "eot_bwd_rhs_drop_inv_a": ("tm += T[i * m + j] * mur[i] / a[i];", "tm += T[i * m + j] * mur[i];"),
    "eot_bwd_delta_drop_inv_a": ("for (int i = 0; i < n; ++i) p += T[i * m + j] / a[i] * T[i * m + k];",
                                 "for (int i = 0; i < n; ++i) p += T[i * m + j] * T[i * m + k];"),
    # mHC consumer mixing y = T x and its backward
    "mix_transposed": ("for (int j = 0; j < n; ++j) s += Tq[i * n + j] * xq[j * C + c];",
                       "for (int j = 0; j < n; ++j) s += Tq[j * n + i] * xq[j * C + c];"),
    "mix_bwd_dx_untransposed": ("for (int i = 0; i < n; ++i) s += Tq[i * n + j] * dyq[i * C + c];",
                                "for (int i = 0; i < n; ++i) s += Tq[j * n + i] * dyq[i * C + c];"),
    "mix_bwd_dT_transposed": ("for (int64_t c = 0; c < C; ++c) s += dyq[i * C + c] * xq[j * C + c];",
                              "for (int64_t c = 0; c < C; ++c) s += dyq[j * C + c] * xq[i * C + c];"),
}


def _run_mutant(name, tmp):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, "mutation anchor for %s not unique/found" % name
    src = tmp / ("%s.c" % name)
    lib = tmp / ("%s.so" % name)
    src.write_text(SRC.replace(old, new))
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", str(src), "-o", str(lib), "-lm"],
                   check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        str(ROOT / "tests" / "test_oracle.py"), str(ROOT / "tests" / "test_oracle_eot.py"),
                        str(ROOT / "tests" / "test_oracle_mix.py")],
                       cwd=str(ROOT), env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-400:]


def test_every_planted_slip_is_caught(tmp_path):
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda k: _run_mutant(k, tmp_path), sorted(MUTANTS)))
    by_name = {n: (rc, out) for n, rc, out in results}
    # the unmutated control must pass, otherwise a failure says nothing about the pins
    assert by_name.pop("control_unmutated")[0] == 0
    survived = [(n, out) for n, (rc, out) in by_name.items() if rc == 0]
    assert not survived, "mutants not caught by the oracle pins: %r" % survived
