"""The oracle's pins are sharp enough to catch plausible mistakes.

Each mutant below is a copy of ``oracle/oracle.cpp`` with one planted error
(a dropped term, a flipped sign, a transposed operand, a wrong index, a
mistyped tableau digit, a missing contraction, a wrong seed).  It is built on
the CPU into a temporary library and the pin battery of
``test_oracle_pins`` is run against it; at least one pin must fail.
"""
import concurrent.futures
import os
import subprocess
import tempfile

import numpy as np
import pytest

import workloads as W
import test_oracle_dense as dense
import test_oracle_pins as pins
import test_oracle_user_rhs as user

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "oracle.cpp")

MUTANTS = {
    "drop_first_stage_adjoint": (
        "rhs_vjp_p_acc<T, F>(kind, d, Y[i], p, kb, gp);\n    for (int c = 0; c < d; ++c) lacc[c] = lacc[c] + Wv[i][c];\n  }\n  for (int c = 0; c < d; ++c) lam[c] = lacc[c];\n}\n\n/* ------------------------------------------------------------------ */\n/* Fehlberg",
        "rhs_vjp_p_acc<T, F>(kind, d, Y[i], p, kb, gp);\n    for (int c = 0; c < d; ++c) if (i > 0) lacc[c] = lacc[c] + Wv[i][c];\n  }\n  for (int c = 0; c < d; ++c) lam[c] = lacc[c];\n}\n\n/* ------------------------------------------------------------------ */\n/* Fehlberg"),
    "lorenz_vjp_sign": ("w[2] = mac<F>(-b, v[2], (-y[0]) * v[1]);",
                        "w[2] = mac<F>(b, v[2], (-y[0]) * v[1]);"),
    "lorenz_vjp_index": ("w[1] = mac<F>(y[0], v[2], mac<F>(s, v[0], -v[1]));",
                         "w[1] = mac<F>(y[1], v[2], mac<F>(s, v[0], -v[1]));"),
    "lorenz_param_vjp": ("g[0] = mac<F>(y[1] - y[0], v[0], g[0]);",
                         "g[0] = mac<F>(y[0] - y[1], v[0], g[0]);"),
    "transposed_tableau_in_adjoint": ("if (tb.a[l][i] == 0.0) continue;\n        if (first) { acc = T(tb.a[l][i]) * Wv[l][c];",
                                      "if (tb.a[l][i] == 0.0) continue;\n        if (first) { acc = T(tb.a[i][l]) * Wv[l][c];"),
    "tsit5_digit": ("t.a[4][2] = 7.4955393428898365;", "t.a[4][2] = 7.4955393428988365;"),
    "dopri5_weight": ("t.a[6][3] = 125.0 / 192.0;", "t.a[6][3] = 125.0 / 191.0;"),
    "lu_transposed_solve": ("z[i] = mac<F>(-LU[j * d + i], z[j], z[i]);\n    z[i] = F ?",
                            "z[i] = mac<F>(-LU[i * d + j], z[j], z[i]);\n    z[i] = F ?"),
    "ros2_no_jac_contraction": (
        "for (int i = 0; i < d * d; ++i) Jb[i] = (-gh) * Wb[i];\n  rhs_jac_contract_acc<T, F>(kind, d, y, p, Jb, yb, gp);",
        "for (int i = 0; i < d * d; ++i) Jb[i] = (-gh) * Wb[i];"),
    "rodas3_no_jac_contraction": (
        "for (int q = 0; q < d * d; ++q) Jb[q] = (-gh) * Wb[q];\n  rhs_jac_contract_acc<T, F>(kind, d, y, p, Jb, yb, gp);",
        "for (int q = 0; q < d * d; ++q) Jb[q] = (-gh) * Wb[q];"),
    "ros2_wrong_weight": ("const T acc = mac<F>(T(0.5), s.k2[c], T(1.5) * s.k1[c]);",
                          "const T acc = mac<F>(T(0.5), s.k2[c], T(1.0) * s.k1[c]);"),
    "robertson_contraction_sign": ("gy[1] = mac<F>(-two_k2, Jb[4], gy[1]);",
                                   "gy[1] = mac<F>(two_k2, Jb[4], gy[1]);"),
    "lorenz96_vjp_index": ("const T vm1 = v[(j + d - 1) % d]", "const T vm1 = v[(j + d - 2) % d]"),
    "mse_seed_factor": ("lam[c] = mac<F>(T(2.0 * scale), y[c] - aux[c], lam[c]);",
                        "lam[c] = mac<F>(T(scale), y[c] - aux[c], lam[c]);"),
    "save_seed_off_by_one": ("for (; s_hi >= 0 && sidx[s_hi] == k; --s_hi)",
                             "for (; s_hi >= 0 && sidx[s_hi] == k + 1; --s_hi)"),
    "controller_growth_after_reject": ("if (after_reject) fac = std::min(fac, T(1.0));", ""),
    "error_norm_scale": ("sc[c] = mac<F>(rtol, std::max(absval(y[c]), absval(yn[c])), atol);",
                         "sc[c] = mac<F>(rtol, absval(y[c]), atol);"),
    "hermite_start_slope_sign": ("w[2] = th * u2;", "w[2] = -(th * u2);"),
    "hermite_end_weight": ("w[1] = t2 * mac<F>(S(-2.0), th, S(3.0));",
                           "w[1] = t2 * mac<F>(S(-2.0), th, S(2.0));"),
    "dense_seed_drops_end_slope": ("lam[c] = mac<F>(w[1], sb[c], lam[c]) + w1[c];",
                                   "lam[c] = mac<F>(w[1], sb[c], lam[c]);"),
    "dense_seed_vjp_at_wrong_state": ("rhs_vjp_y<T, F>(kind, d, yk1, p, v1, w1);",
                                      "rhs_vjp_y<T, F>(kind, d, yk, p, v1, w1);"),
    "dense_bypass_not_added": ("for (int c = 0; c < d; ++c) lam[c] = lam[c] + mu[c];", ""),
    "dense_fraction_origin": ("const double th = (ts - t) / h;",
                              "const double th = (t_end - ts) / h;"),
    "user_vjp_transposed": ("T acc = J[0][m] * v[0];\n      for (int i = 1; i < d; ++i) acc = mac<F>(J[i][m], v[i], acc);",
                            "T acc = J[m][0] * v[0];\n      for (int i = 1; i < d; ++i) acc = mac<F>(J[m][i], v[i], acc);"),
    "user_param_column": ("pd[q] = U(p[q], (wrt_p && q == m) ? T(1) : T(0));",
                          "pd[q] = U(p[q], (wrt_p && q == 0) ? T(1) : T(0));"),
    "dense_save_in_next_step": ("out.sidx[j] = nacc;\n            if (out.theta) out.theta[j] = th;",
                                "out.sidx[j] = nacc + 1;\n            if (out.theta) out.theta[j] = th;"),
    "rodas3_digit": ("t.c[3][2] = -8.0 / 3.0;", "t.c[3][2] = -7.0 / 3.0;"),
    "rodas3_weight": ("t.m[0] = 2.0; t.m[1] = 0.0;", "t.m[0] = 1.5; t.m[1] = 0.0;"),
    "rodas3_stage_sum_misses_c_term": (
        "        if (tb.gc[l][i] != 0.0) {\n          acc = first ? T(tb.gc[l][i]) * rb[l][c]",
        "        if (tb.gc[l][i] != 0.0 && l > i + 1) {\n          acc = first ? T(tb.gc[l][i]) * rb[l][c]"),
    "rodas3_wbar_from_wrong_stage": (
        "mac<F>(-rb[i][a], s.u[i][b], Wb[a * d + b]);",
        "mac<F>(-rb[i][a], s.u[tb.s - 1][b], Wb[a * d + b]);"),
    "rodas3_vjp_at_step_start": ("rhs_vjp_y<T, F>(kind, d, s.Y[i], p, fb, Yb[i]);",
                                 "rhs_vjp_y<T, F>(kind, d, y, p, fb, Yb[i]);"),
    "rkf78_digit": ("a[8][4] = 704.0 / 45.0;", "a[8][4] = 704.0 / 44.0;"),
    "rkf78_adjoint_drops_last_stage": ("      for (int l = i + 1; l <= 10; ++l) {\n        if (RK78.a[l][i] == 0.0) continue;",
                                       "      for (int l = i + 1; l <= 9; ++l) {\n        if (RK78.a[l][i] == 0.0) continue;"),
    "kinetics8_partial_of_wrong_reactant": ("cols[0] = r.a; vals[0] = k * y[r.b];",
                                            "cols[0] = r.a; vals[0] = k * y[r.a];"),
    "ros4_digit": ("t.c[3][0] = -112.0 / 125.0;", "t.c[3][0] = -111.0 / 125.0;"),
    "ros4_fourth_stage_at_wrong_point": ("t.a[3][0] = 48.0 / 25.0; t.a[3][1] = 6.0 / 25.0;",
                                         "t.a[3][0] = 48.0 / 25.0; t.a[3][2] = 6.0 / 25.0;"),
    "ros4_error_weight": ("t.e[0] = 17.0 / 54.0;", "t.e[0] = 19.0 / 54.0;"),
    "landing_next_step_from_unshortened_proposal": (
        "h = hs * fac;\n        after_reject = false;",
        "h = (land ? h : hs) * fac;\n        after_reject = false;"),
    "plain_controller_power_in_single_precision": (
        "  return std::pow(E, expo);", "  return T(std::exp2(float(expo) * std::log2(float(E))));"),
    "kinetics8_contraction_flipped": (
        "auto M = [&](int b) { return Jb[k.dst * 8 + b] - Jb[k.src * 8 + b]; };",
        "auto M = [&](int b) { return Jb[k.src * 8 + b] - Jb[k.dst * 8 + b]; };"),
}


def _battery():
    out = []
    for m in (W.TSIT5, W.DOPRI5):
        out.append((pins.test_tableau_order_conditions, dict(method=m)))
    out += [(pins.test_dopri5_rationals, {}), (pins.test_dopri5_stability_polynomial, {}),
            (pins.test_page5_enzyme_fixed_step_tsit5, {})]
    for m in (W.TSIT5, W.DOPRI5, W.ROS2, W.RODAS3):
        out.append((pins.test_linear_decay_closed_form, dict(method=m, fused=False)))
        out.append((pins.test_lorenz63_origin_linearisation, dict(method=m)))
    out.append((pins.test_rodas3_order_stability_and_estimator, {}))
    out.append((pins.test_ros4_order_stability_and_estimator, {}))
    out += [(pins.test_rkf78_tableau_is_fehlberg, {}),
            (pins.test_linear_decay_closed_form, dict(method=W.RKF78, fused=False))]
    for m in (W.TSIT5, W.DOPRI5):
        out.append((pins.test_lorenz96_fixed_point, dict(method=m)))
    out += [(pins.test_robertson_ros2_conservation, {"method": W.ROS2}),
            (pins.test_robertson_ros2_conservation, {"method": W.RODAS3}),
            (pins.test_kinetics8_conservation_and_reference, {"method": W.RODAS3}),
            (pins.test_dopri5_record_matches_scipy_rk45, {}),
            (pins.test_save_time_landing_matches_scipy_rk45, {}),
            (pins.test_loss_values_match_their_definitions, {}),
            (pins.test_rhs_vjp_against_dense_jacobian, {})]
    for case in pins.CASES:
        out.append((pins.test_adjoint_matches_dual_numbers, dict(case=case)))
    for case in pins.CASES:
        out.append((pins.test_adjoint_matches_finite_differences, dict(case=case)))
    out += [(dense.test_dense_hermite_remainder_on_linear_decay,
             dict(method=W.TSIT5, fused=False)),
            (dense.test_dense_fraction_one_is_the_clipped_save, dict(fused=False))]
    for case in dense.DCASES:
        out.append((dense.test_dense_record_mesh_bookkeeping, dict(case=case)))
        out.append((dense.test_dense_adjoint_matches_dual_numbers, dict(case=case, fused=False)))
    out += [(user.test_source_lorenz63_equals_builtin, {}),
            (user.test_source_rhs_products_match_finite_differences, {}),
            (user.test_source_adjoint_matches_duals_and_differences,
             dict(src=user.ALLFN, dim=3, P=3, name="allfn", fused=False))]
    return out


def _killed(orc):
    for fn, kw in _battery():
        try:
            fn(orc, **kw)
        except Exception:          # an assertion (or a numerical failure) kills it
            return fn.__name__
    return None


def _build_mutant(name: str, d: str) -> str:
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site of {name} not unique/found"
    mutated = os.path.join(d, f"oracle_{name}.cpp")
    with open(mutated, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(d, f"liboracle_{name}.so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", "-w", "-I", os.path.dirname(SRC), "-o", lib, mutated],
                   check=True)
    return lib


_BUILT = {}


def _mutant_lib(name: str, d: str) -> str:
    """The mutant's library.  In a single test process every mutant is built
    at the first request, several compilers at a time; under pytest-xdist
    each worker builds only the mutants it runs."""
    if os.environ.get("PYTEST_XDIST_WORKER"):
        return _build_mutant(name, d)
    if not _BUILT:
        with concurrent.futures.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
            names = sorted(MUTANTS)
            for n, lib in zip(names, ex.map(lambda m: _build_mutant(m, d), names)):
                _BUILT[n] = lib
    return _BUILT[name]


@pytest.fixture(scope="module")
def mutant_dir():
    with tempfile.TemporaryDirectory(prefix="oracle_mutants_") as d:
        yield d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(orc, mutant_dir, name):
    lib = _mutant_lib(name, mutant_dir)
    try:
        orc._swap_library(lib)
        killer = _killed(orc)
    finally:
        orc._swap_library(None)
    assert killer is not None, f"no pin catches mutant {name}"


def test_unmutated_oracle_passes_battery(orc):
    assert _killed(orc) is None
