"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: order conditions of the
published tableaux, closed forms of the replayed map on linear problems, the
gradient values printed on the DiffEqGPU page (Enzyme section), SciPy's RK45
(the same Dormand-Prince controller), dual-number forward mode, central finite
differences on the frozen mesh, and invariants of the Robertson and Lorenz-96
systems.  These run on the CPU only.
"""
import json
import math
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Tableaux
# ---------------------------------------------------------------------------

def _order_conditions(b, A, c, order):
    """Residuals of the Butcher order conditions up to ``order`` (<= 5)."""
    one = np.ones_like(c)
    r = [b @ one - 1, b @ c - 1 / 2]
    if order >= 3:
        r += [b @ c**2 - 1 / 3, b @ A @ c - 1 / 6]
    if order >= 4:
        r += [b @ c**3 - 1 / 4, b @ (c * (A @ c)) - 1 / 8, b @ A @ c**2 - 1 / 12,
              b @ A @ A @ c - 1 / 24]
    if order >= 5:
        r += [b @ c**4 - 1 / 5, b @ (c**2 * (A @ c)) - 1 / 10, b @ (c * (A @ c**2)) - 1 / 15,
              b @ (c * (A @ A @ c)) - 1 / 30, b @ ((A @ c) ** 2) - 1 / 20,
              b @ A @ c**3 - 1 / 20, b @ A @ (c * (A @ c)) - 1 / 40,
              b @ A @ A @ c**2 - 1 / 60, b @ A @ A @ A @ c - 1 / 120]
    return np.abs(np.array(r))


@pytest.mark.parametrize("method", [W.TSIT5, W.DOPRI5])
def test_tableau_order_conditions(orc, method):
    t = orc.tableau(method)
    A, b, c, e = t["a"], t["b"], t["c"], t["e"]
    assert np.allclose(A.sum(axis=1), c, rtol=0, atol=2e-15)      # row sums
    assert np.array_equal(A[6], b) and b[6] == 0.0                  # first same as last
    assert _order_conditions(b, A, c, 5).max() < 2e-15              # 5th order
    bh = b - e
    assert _order_conditions(bh, A, c, 4).max() < 3e-15             # embedded 4th order
    assert _order_conditions(bh, A, c, 5).max() > 1e-5              # ... and not 5th
    assert t["order"] == 5 and t["err_order"] == 4


def test_dopri5_rationals(orc):
    """Dormand-Prince coefficients are the published rationals, to the last bit."""
    t = orc.tableau(W.DOPRI5)
    exact = {
        (1, 0): Fr(1, 5), (2, 0): Fr(3, 40), (2, 1): Fr(9, 40), (3, 0): Fr(44, 45),
        (3, 1): Fr(-56, 15), (3, 2): Fr(32, 9), (4, 0): Fr(19372, 6561),
        (4, 1): Fr(-25360, 2187), (4, 2): Fr(64448, 6561), (4, 3): Fr(-212, 729),
        (5, 0): Fr(9017, 3168), (5, 1): Fr(-355, 33), (5, 2): Fr(46732, 5247),
        (5, 3): Fr(49, 176), (5, 4): Fr(-5103, 18656), (6, 0): Fr(35, 384),
        (6, 2): Fr(500, 1113), (6, 3): Fr(125, 192), (6, 4): Fr(-2187, 6784),
        (6, 5): Fr(11, 84)}
    for (i, j), v in exact.items():
        assert t["a"][i, j] == float(v), (i, j)
    bhat = [Fr(5179, 57600), 0, Fr(7571, 16695), Fr(393, 640), Fr(-92097, 339200),
            Fr(187, 2100), Fr(1, 40)]
    b = [exact.get((6, j), Fr(0)) for j in range(7)]
    for j in range(7):
        assert t["e"][j] == float(b[j] - bhat[j]), j
    # exact order conditions in rationals
    A = [[exact.get((i, j), Fr(0)) for j in range(7)] for i in range(7)]
    c = [sum(row) for row in A]
    assert sum(b) == 1 and sum(bi * ci for bi, ci in zip(b, c)) == Fr(1, 2)
    assert sum(bi * ci**4 for bi, ci in zip(b, c)) == Fr(1, 5)


def _stability_poly(t):
    """Coefficients of R(z) = 1 + z b^T (I - zA)^{-1} 1 = sum_j (b^T A^{j-1} 1) z^j."""
    A, b = t["a"], t["b"]
    s = len(b)
    one = np.ones(s)
    coef = [1.0]
    v = one.copy()
    for _ in range(s):
        coef.append(b @ v)
        v = A @ v
    return np.array(coef)


# Fehlberg 7(8), typed here from the published fractions independently of the
# oracle: rows of a (stage: {column: value}), the 7th- and 8th-order weights.
_F = Fr
_RK78_A = {
    1: {0: _F(2, 27)}, 2: {0: _F(1, 36), 1: _F(1, 12)}, 3: {0: _F(1, 24), 2: _F(1, 8)},
    4: {0: _F(5, 12), 2: _F(-25, 16), 3: _F(25, 16)}, 5: {0: _F(1, 20), 3: _F(1, 4), 4: _F(1, 5)},
    6: {0: _F(-25, 108), 3: _F(125, 108), 4: _F(-65, 27), 5: _F(125, 54)},
    7: {0: _F(31, 300), 4: _F(61, 225), 5: _F(-2, 9), 6: _F(13, 900)},
    8: {0: _F(2), 3: _F(-53, 6), 4: _F(704, 45), 5: _F(-107, 9), 6: _F(67, 90), 7: _F(3)},
    9: {0: _F(-91, 108), 3: _F(23, 108), 4: _F(-976, 135), 5: _F(311, 54), 6: _F(-19, 60),
        7: _F(17, 6), 8: _F(-1, 12)},
    10: {0: _F(2383, 4100), 3: _F(-341, 164), 4: _F(4496, 1025), 5: _F(-301, 82),
         6: _F(2133, 4100), 7: _F(45, 82), 8: _F(45, 164), 9: _F(18, 41)},
    11: {0: _F(3, 205), 5: _F(-6, 41), 6: _F(-3, 205), 7: _F(-3, 41), 8: _F(3, 41), 9: _F(6, 41)},
    12: {0: _F(-1777, 4100), 3: _F(-341, 164), 4: _F(4496, 1025), 5: _F(-289, 82),
         6: _F(2193, 4100), 7: _F(51, 82), 8: _F(33, 164), 9: _F(12, 41), 11: _F(1)},
}
_RK78_B7 = {0: _F(41, 840), 5: _F(34, 105), 6: _F(9, 35), 7: _F(9, 35), 8: _F(9, 280),
            9: _F(9, 280), 10: _F(41, 840)}
_RK78_B8 = {5: _F(34, 105), 6: _F(9, 35), 7: _F(9, 35), 8: _F(9, 280), 9: _F(9, 280),
            11: _F(41, 840), 12: _F(41, 840)}


def _rk78_float():
    A = np.zeros((13, 13))
    for i, row in _RK78_A.items():
        for j, v in row.items():
            A[i, j] = float(v)
    b = np.zeros(13)
    for j, v in _RK78_B7.items():
        b[j] = float(v)
    return {"a": A, "b": b}


def _rooted_trees(n, memo={}):
    """Rooted trees with n vertices, each a sorted tuple of its subtrees."""
    if n not in memo:
        if n == 1:
            memo[n] = [()]
        else:
            out = set()

            def forests(rem, maxsize, maxtree):
                if rem == 0:
                    yield ()
                    return
                for size in range(min(rem, maxsize), 0, -1):
                    for t in _rooted_trees(size):
                        if size == maxsize and maxtree is not None and t > maxtree:
                            continue
                        for rest in forests(rem - size, size, t):
                            yield (t,) + rest
            for f in forests(n - 1, n - 1, None):
                out.add(tuple(sorted(f)))
            memo[n] = sorted(out)
    return memo[n]


def _tree_density(t):
    """gamma(t): the order of t times the densities of its subtrees."""
    g = 1 + sum(_tree_order(c) for c in t)
    for c in t:
        g *= _tree_density(c)
    return g


def _tree_order(t):
    return 1 + sum(_tree_order(c) for c in t)


def _elementary_weight(t, A, s):
    """Per-stage vector of the elementary differential of t: the product over
    the subtrees u of (A Phi(u))."""
    v = [Fr(1)] * s
    for u in t:
        w = _elementary_weight(u, A, s)
        v = [v[i] * sum((A.get(i, {}).get(j, 0) * w[j] for j in range(s)), Fr(0))
             for i in range(s)]
    return v


def _order_defects(b, A, s, order):
    """Number of trees with up to ``order`` vertices whose condition
    b^T Phi(t) = 1/gamma(t) fails (exact rational arithmetic)."""
    bad = 0
    for n in range(1, order + 1):
        for t in _rooted_trees(n):
            phi = _elementary_weight(t, A, s)
            if sum((b.get(i, 0) * phi[i] for i in range(s)), Fr(0)) != Fr(1, _tree_density(t)):
                bad += 1
    return bad


def test_rkf78_tableau_is_fehlberg(orc):
    """The oracle holds Fehlberg's 7(8) coefficients: each equals the nearest
    double of the published fraction, and the fractions satisfy every order
    condition up to order 7 for the propagated weights (85 trees) and up to
    order 8 for the companion (200 trees), the propagated weights not order 8."""
    t = orc.rk78_tableau()
    assert t["order"] == 7 and t["err_order"] == 7
    A = np.zeros((13, 13))
    for i, row in _RK78_A.items():
        for j, v in row.items():
            A[i, j] = float(v)
    assert np.array_equal(t["a"], A)
    b7 = np.array([float(_RK78_B7.get(j, 0)) for j in range(13)])
    b8 = np.array([float(_RK78_B8.get(j, 0)) for j in range(13)])
    assert np.array_equal(t["b"], b7) and np.array_equal(t["e"], b7 - b8)
    assert sum(len(_rooted_trees(n)) for n in range(1, 9)) == 200
    assert _order_defects(_RK78_B7, _RK78_A, 13, 7) == 0
    assert _order_defects(_RK78_B8, _RK78_A, 13, 8) == 0
    assert _order_defects(_RK78_B7, _RK78_A, 13, 8) > 0


def test_rkf78_global_order_and_step_scaling(orc):
    """Global order 7 on Lorenz-63 with fixed steps, against SciPy's DOP853 at
    1e-14; recorded step counts grow as tol^(-1/8) (error estimate O(h^8))."""
    from scipy.integrate import solve_ivp
    u0 = np.array([[1.0, 1.0, 1.0]])
    pv = np.array([[10.0, 28.0, 8.0 / 3.0]])
    ref = solve_ivp(lambda t, y: [10 * (y[1] - y[0]), y[0] * (28 - y[2]) - y[1],
                                  y[0] * y[1] - 8 / 3 * y[2]], (0, 0.5), u0[0],
                    method="DOP853", rtol=1e-14, atol=1e-14).y[:, -1]
    errs = []
    for N in (10, 20, 40):
        pr = W.Problem(W.LORENZ63, 3, 3, W.RKF78, 0.0, 0.5, 1e-6, 1e-6, N)
        mesh = {"h": np.full((1, N), 0.5 / N), "n_steps": np.array([N]),
                "save_idx": np.array([[N]]), "status": np.zeros(1)}
        _, yN = orc.replay(pr, u0, pv, mesh)
        errs.append(np.abs(yN[0] - ref).max())
    orders = [math.log2(errs[i] / errs[i + 1]) for i in range(2)]
    assert all(6.5 < o < 7.6 for o in orders), (orders, errs)
    inp = W.make_inputs(1, 8)
    steps = []
    for tol in (1e-6, 1e-12):
        pr = W.Problem(W.LORENZ63, 3, 3, W.RKF78, 0.0, 1.0, tol, tol, 100000)
        m = orc.record(pr, inp["u0"], inp["p"])
        assert np.all(m["status"] == 0)
        steps.append(m["n_steps"].mean())
    assert 4.3 < steps[1] / steps[0] < 7.3, steps                  # 1e6^(1/8) = 5.6


def test_dopri5_stability_polynomial(orc):
    """Textbook: R(z) = sum_{j<=5} z^j/j! + z^6/600 for Dormand-Prince."""
    coef = _stability_poly(orc.tableau(W.DOPRI5))
    expect = [1 / math.factorial(j) for j in range(6)] + [1 / 600, 0.0]
    assert np.allclose(coef, expect, rtol=1e-14, atol=1e-17)


# ---------------------------------------------------------------------------
# Pages' printed values
# ---------------------------------------------------------------------------

def test_page5_enzyme_fixed_step_tsit5(orc):
    """Fixed-step Tsit5 gradient printed in the DiffEqGPU Enzyme example."""
    g = json.load(open(os.path.join(GOLDEN, "diffeqgpu_enzyme_tsit5.json")))
    pr = g["problem"]
    n = len(g["p"])
    N = pr["steps"]
    prob = W.Problem(W.LINEAR, 1, 1, W.TSIT5, pr["t0"], pr["t1"], 1e-6, 1e-6, N)
    mesh = {"h": np.full((n, N), pr["dt"]), "n_steps": np.full(n, N),
            "save_idx": np.full((n, 1), N), "status": np.zeros(n)}
    u0 = np.full((n, 1), pr["y0"])
    p = np.array(g["p"])[:, None]
    for fused in (False, True):
        loss, gu0, gp = orc.replay_grad(prob, u0, p, mesh, W.COTANGENT,
                                        aux=np.ones((n, 1, 1)), fused=fused)
        assert np.allclose(gp[:, 0], g["dloss_dp"], rtol=0, atol=5e-15), gp[:, 0]
        # the loss is the final state itself and its u0-gradient is R(z)^N
        assert np.allclose(gu0[:, 0], loss, rtol=1e-15)
    # the page's values fix the z^6 coefficient of Tsit5's stability polynomial
    coef = _stability_poly(orc.tableau(W.TSIT5))
    assert abs(coef[6] - 1.4328e-3) < 1e-6 and coef[7] == 0.0


# ---------------------------------------------------------------------------
# Closed forms on linear problems
# ---------------------------------------------------------------------------

def _R_erk(coef, z):
    return sum(cj * z**j for j, cj in enumerate(coef))


def _R_ros2(gamma, z):
    w = 1.0 / (1.0 - gamma * z)
    return 1 + 2 * z * w + 0.5 * z * z * w * w - z * w * w


def _rodas3_matrix(Z):
    """One Rodas3 step on y' = A y with Z = h A (any square matrix, complex
    allowed): the published stages with gamma = 1/2 applied to the identity,
    u_i = (I - Z/2)^-1 (Z/2 Y_i + sum_j c_ij/2 u_j)."""
    I = np.eye(Z.shape[0], dtype=complex if np.iscomplexobj(Z) else float)
    Wi = np.linalg.inv(I - 0.5 * Z)
    u0 = Wi @ (0.5 * Z @ I)
    u1 = Wi @ (0.5 * Z @ I + 2.0 * u0)
    Y2 = I + 2.0 * u0
    u2 = Wi @ (0.5 * Z @ Y2 + 0.5 * u0 - 0.5 * u1)
    Y3 = Y2 + u2
    u3 = Wi @ (0.5 * Z @ Y3 + 0.5 * u0 - 0.5 * u1 - (4.0 / 3.0) * u2)
    return I + 2.0 * u0 + u2 + u3


def _R_rodas3(z):
    return _rodas3_matrix(np.array([[z]]))[0, 0]


# Shampine's fourth-order Rosenbrock parameters (ACM TOMS 8, 1982), typed here
# from the publication as fractions, independently of the oracle's doubles:
# transformed form with gamma = 1/2, stage points a, stage couplings c,
# weights m and error weights e (fourth minus third order).
ROS4_A = {(1, 0): Fr(2), (2, 0): Fr(48, 25), (2, 1): Fr(6, 25),
          (3, 0): Fr(48, 25), (3, 1): Fr(6, 25)}
ROS4_C = {(1, 0): Fr(-8), (2, 0): Fr(372, 25), (2, 1): Fr(12, 5),
          (3, 0): Fr(-112, 125), (3, 1): Fr(-54, 125), (3, 2): Fr(-2, 5)}
ROS4_M = [Fr(19, 9), Fr(1, 2), Fr(25, 108), Fr(125, 108)]
ROS4_E = [Fr(17, 54), Fr(7, 36), Fr(0), Fr(125, 108)]


def _ros4_matrix(Z, weights=None):
    """One step of the four-stage scheme on y' = A y with Z = h A:
    u_i = (I - Z/2)^-1 (Z/2 Y_i + sum_j c_ij/2 u_j), Y_i = I + sum_j a_ij u_j,
    result I + sum_i w_i u_i (w = m by default)."""
    w = ROS4_M if weights is None else weights
    I = np.eye(Z.shape[0], dtype=complex if np.iscomplexobj(Z) else float)
    Wi = np.linalg.inv(I - 0.5 * Z)
    u = []
    for i in range(4):
        Y = I + sum(float(ROS4_A.get((i, j), 0)) * u[j] for j in range(i))
        u.append(Wi @ (0.5 * Z @ Y + sum(0.5 * float(ROS4_C.get((i, j), 0)) * u[j]
                                         for j in range(i))))
    return I + sum(float(w[i]) * u[i] for i in range(4))


def _R_ros4(z):
    return _ros4_matrix(np.array([[z]]))[0, 0]


def _complex_step(fn, z):
    eps = 1e-30
    return (fn(z + 1j * eps)).imag / eps


@pytest.mark.parametrize("method", [W.TSIT5, W.DOPRI5, W.ROS2, W.RODAS3, W.RKF78, W.ROS4])
@pytest.mark.parametrize("fused", [False, True])
def test_linear_decay_closed_form(orc, method, fused):
    """y' = -k y on an arbitrary mesh: y_N = y0 prod R(-k h_n); exact derivative
    d y_N / dk from R'(z) (complex step on the closed form)."""
    rng = np.random.default_rng(7)
    N = 37
    n = 4
    ks = np.array([0.5, 3.0, 11.0, 0.01])
    h = rng.uniform(0.01, 0.2, size=(n, N))
    y0 = np.array([1.7, -0.3, 2.0, 1.0])
    if method == W.ROS2:
        g = orc.ros2_gamma()
        assert g == 1.0 + 1.0 / math.sqrt(2.0)
        assert abs(_R_ros2(g, -1e12)) < 1e-11            # L-stable: R(-inf) = 0
        R = lambda z: _R_ros2(g, z)
    elif method == W.RODAS3:
        R = _R_rodas3
    elif method == W.ROS4:
        R = _R_ros4
    else:
        coef = _stability_poly(_rk78_float() if method == W.RKF78 else orc.tableau(method))
        R = lambda z: _R_erk(coef, z)
    prob = W.Problem(W.LINEAR, 1, 1, method, 0.0, 1.0, 1e-6, 1e-6, N)
    mesh = {"h": h, "n_steps": np.full(n, N), "save_idx": np.full((n, 1), N),
            "status": np.zeros(n)}
    p = -ks[:, None]
    _, yN = orc.replay(prob, y0[:, None], p, mesh, fused=fused)
    loss, gu0, gp = orc.replay_grad(prob, y0[:, None], p, mesh, W.COTANGENT,
                                    aux=np.ones((n, 1, 1)), fused=fused)
    for i in range(n):
        z = -ks[i] * h[i]
        Rz = np.array([R(zz) for zz in z])
        prod = np.prod(Rz)
        assert yN[i, 0] == pytest.approx(y0[i] * prod, rel=2e-14)
        assert gu0[i, 0] == pytest.approx(prod, rel=2e-14)
        dR = np.array([_complex_step(R, zz) for zz in z])
        # d/dp of prod R(p h_n) with p = -k
        dprod = prod * np.sum(h[i] * dR / Rz)
        assert gp[i, 0] == pytest.approx(y0[i] * dprod, rel=2e-13, abs=1e-300)


def test_rodas3_order_stability_and_estimator(orc):
    """What identifies a correct Rodas3, from the mathematics alone:
    - the oracle's one-step map of y' = z y is the closed form above;
    - R(z) - e^z = O(z^4), with a nonzero z^4 term (order exactly 3);
    - A-stable (|R| <= 1 on the imaginary axis and the negative real axis)
      and L-stable (R(-inf) = 0);
    - global order 3 on Lorenz-63 with fixed steps, against SciPy's DOP853 at
      a tolerance far below the errors measured;
    - a second-order embedded estimate: the recorded step count grows as
      tol^(-1/3) (local error estimate O(h^3))."""
    from scipy.integrate import solve_ivp
    prob = W.Problem(W.LINEAR, 1, 1, W.RODAS3, 0.0, 1.0, 1e-6, 1e-6, 1)
    one = {"h": np.ones((1, 1)), "n_steps": np.array([1]), "save_idx": np.array([[1]]),
           "status": np.zeros(1)}
    for z in (-50.0, -1.3, -0.01, 0.2, 1.5):
        _, y1 = orc.replay(prob, np.ones((1, 1)), np.array([[z]]), one)
        assert y1[0, 0] == pytest.approx(_R_rodas3(z), rel=1e-14)
    e1, e2 = _R_rodas3(0.02) - math.exp(0.02), _R_rodas3(0.01) - math.exp(0.01)
    assert 14.0 < e1 / e2 < 18.0 and abs(e2) > 1e-13            # C z^4, C != 0
    assert abs(_R_rodas3(-1e12)) < 1e-11
    assert max(abs(_R_rodas3(1j * y)) for y in np.logspace(-3, 6, 400)) <= 1.0 + 1e-12
    assert max(abs(_R_rodas3(-x)) for x in np.logspace(-3, 12, 400)) <= 1.0 + 1e-12
    # global order on Lorenz-63 over [0, 0.5]
    u0 = np.array([[1.0, 1.0, 1.0]])
    pv = np.array([[10.0, 28.0, 8.0 / 3.0]])
    ref = solve_ivp(lambda t, y: [10 * (y[1] - y[0]), y[0] * (28 - y[2]) - y[1],
                                  y[0] * y[1] - 8 / 3 * y[2]], (0, 0.5), u0[0],
                    method="DOP853", rtol=1e-13, atol=1e-13).y[:, -1]
    errs = []
    for N in (40, 80, 160, 320):
        pr = W.Problem(W.LORENZ63, 3, 3, W.RODAS3, 0.0, 0.5, 1e-6, 1e-6, N)
        mesh = {"h": np.full((1, N), 0.5 / N), "n_steps": np.array([N]),
                "save_idx": np.array([[N]]), "status": np.zeros(1)}
        _, yN = orc.replay(pr, u0, pv, mesh)
        errs.append(np.abs(yN[0] - ref).max())
    orders = [math.log2(errs[i] / errs[i + 1]) for i in range(3)]
    assert all(2.7 < o < 3.3 for o in orders[1:]), orders
    # step counts against the tolerance
    inp = W.make_inputs(1, 8)
    steps = []
    for tol in (1e-6, 1e-9):
        pr = W.Problem(W.LORENZ63, 3, 3, W.RODAS3, 0.0, 1.0, tol, tol, 100000)
        m = orc.record(pr, inp["u0"], inp["p"])
        assert np.all(m["status"] == 0)
        steps.append(m["n_steps"].mean())
    assert 7.0 < steps[1] / steps[0] < 14.0, steps                # 1000^(1/3) = 10


def test_ros4_order_stability_and_estimator(orc):
    """What identifies a correct fourth-order Rosenbrock step with a
    third-order companion, from the mathematics alone:
    - the oracle's one-step map of y' = z y is the closed form of the
      fractions above;
    - R(z) - e^z = O(z^5) with a nonzero z^5 term (order exactly 4), and the
      companion m - e gives O(z^4) (order 3);
    - A-stable (|R| <= 1 on the imaginary axis and the negative real axis)
      with R(-inf) = 1/3;
    - global order 4 on Lorenz-63 with fixed steps (nonlinear: every order
      condition, not only the linear ones), against SciPy's DOP853;
    - the recorded step count grows as tol^(-1/4) (a third-order estimate)."""
    from scipy.integrate import solve_ivp
    prob = W.Problem(W.LINEAR, 1, 1, W.ROS4, 0.0, 1.0, 1e-6, 1e-6, 1)
    one = {"h": np.ones((1, 1)), "n_steps": np.array([1]), "save_idx": np.array([[1]]),
           "status": np.zeros(1)}
    for z in (-50.0, -1.3, -0.01, 0.2, 1.5):
        _, y1 = orc.replay(prob, np.ones((1, 1)), np.array([[z]]), one)
        assert y1[0, 0] == pytest.approx(_R_ros4(z), rel=1e-14)
    e1, e2 = _R_ros4(0.04) - math.exp(0.04), _R_ros4(0.02) - math.exp(0.02)
    assert 28.0 < e1 / e2 < 36.0 and abs(e2) > 1e-13            # C z^5, C != 0
    emb = [mi - ei for mi, ei in zip(ROS4_M, ROS4_E)]
    Re = lambda z: _ros4_matrix(np.array([[z]]), emb)[0, 0]
    c1, c2 = Re(0.04) - math.exp(0.04), Re(0.02) - math.exp(0.02)
    assert 14.0 < c1 / c2 < 18.0                                 # companion: C z^4
    assert _R_ros4(-1e12) == pytest.approx(1.0 / 3.0, abs=1e-9)
    assert max(abs(_R_ros4(1j * y)) for y in np.logspace(-3, 6, 400)) <= 1.0 + 1e-12
    assert max(abs(_R_ros4(-x)) for x in np.logspace(-3, 12, 400)) <= 1.0 + 1e-12
    u0 = np.array([[1.0, 1.0, 1.0]])
    pv = np.array([[10.0, 28.0, 8.0 / 3.0]])
    ref = solve_ivp(lambda t, y: [10 * (y[1] - y[0]), y[0] * (28 - y[2]) - y[1],
                                  y[0] * y[1] - 8 / 3 * y[2]], (0, 0.5), u0[0],
                    method="DOP853", rtol=1e-13, atol=1e-13).y[:, -1]
    errs = []
    for N in (50, 100, 200, 400):
        pr = W.Problem(W.LORENZ63, 3, 3, W.ROS4, 0.0, 0.5, 1e-6, 1e-6, N)
        mesh = {"h": np.full((1, N), 0.5 / N), "n_steps": np.array([N]),
                "save_idx": np.array([[N]]), "status": np.zeros(1)}
        _, yN = orc.replay(pr, u0, pv, mesh)
        errs.append(np.abs(yN[0] - ref).max())
    orders = [math.log2(errs[i] / errs[i + 1]) for i in range(3)]
    assert all(3.8 < o < 4.3 for o in orders), orders
    inp = W.make_inputs(1, 8)
    steps = []
    for tol in (1e-6, 1e-9):
        pr = W.Problem(W.LORENZ63, 3, 3, W.ROS4, 0.0, 1.0, tol, tol, 100000)
        m = orc.record(pr, inp["u0"], inp["p"])
        assert np.all(m["status"] == 0)
        steps.append(m["n_steps"].mean())
    assert 4.2 < steps[1] / steps[0] < 7.5, steps               # 1000^(1/4) = 5.6


def _matrix_R(method, orc, Z):
    I = np.eye(Z.shape[0])
    if method == W.ROS2:
        g = orc.ros2_gamma()
        Wm = np.linalg.inv(I - g * Z)
        return I + 2 * Z @ Wm + 0.5 * Z @ Z @ Wm @ Wm - Z @ Wm @ Wm
    if method == W.RODAS3:
        return _rodas3_matrix(Z)
    if method == W.ROS4:
        return _ros4_matrix(Z)
    coef = _stability_poly(_rk78_float() if method == W.RKF78 else orc.tableau(method))
    out = np.zeros_like(Z)
    Zp = I.copy()
    for cj in coef:
        out = out + cj * Zp
        Zp = Zp @ Z
    return out


@pytest.mark.parametrize("method", [W.TSIT5, W.DOPRI5, W.ROS2, W.RODAS3, W.RKF78, W.ROS4])
def test_lorenz63_origin_linearisation(orc, method):
    """At the origin Lorenz-63 is a fixed point; the replay's Jacobian is the
    product of R(h_n A) with A = [[-s, s, 0], [r, -1, 0], [0, 0, -b]].  A
    cotangent w at the end must come back as (prod R)^T w."""
    rng = np.random.default_rng(11)
    N, n = 25, 3
    h = rng.uniform(0.005, 0.05, size=(n, N))
    p = np.array([[10.0, 28.0, 8 / 3], [6.0, 15.0, 1.5], [8.0, 22.0, 2.2]])
    w = rng.standard_normal((n, 1, 3))
    prob = W.Problem(W.LORENZ63, 3, 3, method, 0.0, 1.0, 1e-6, 1e-6, N)
    mesh = {"h": h, "n_steps": np.full(n, N), "save_idx": np.full((n, 1), N),
            "status": np.zeros(n)}
    u0 = np.zeros((n, 3))
    loss, gu0, gp = orc.replay_grad(prob, u0, p, mesh, W.COTANGENT, aux=w)
    for i in range(n):
        s, r, b = p[i]
        A = np.array([[-s, s, 0], [r, -1, 0], [0, 0, -b]])
        M = np.eye(3)
        for k in range(N):
            M = _matrix_R(method, orc, h[i, k] * A) @ M
        expect = M.T @ w[i, 0]
        assert np.allclose(gu0[i], expect, rtol=1e-12, atol=1e-12 * np.abs(expect).max())
        assert np.all(gp[i] == 0.0)


@pytest.mark.parametrize("method", [W.TSIT5, W.DOPRI5])
def test_lorenz96_fixed_point(orc, method):
    """x = F 1 is an exact fixed point of Lorenz-96 (f == 0 bitwise).  The
    replay's Jacobian is prod R(h_n A) with the circulant linearisation A, and
    d x_N / dF follows the linear inhomogeneous recursion
    e_{n+1} = R(h A) e_n + h Phi(h A) 1, Phi(Z) = (R(Z) - I) Z^{-1}."""
    d, N, n = 64, 20, 2
    rng = np.random.default_rng(5)
    F = np.array([8.0, 7.3])
    h = rng.uniform(0.01, 0.05, size=(n, N))
    u0 = F[:, None] * np.ones((n, d))
    w = rng.standard_normal((n, 1, d))
    prob = W.Problem(W.LORENZ96, d, 1, method, 0.0, 1.0, 1e-6, 1e-6, N)
    mesh = {"h": h, "n_steps": np.full(n, N), "save_idx": np.full((n, 1), N),
            "status": np.zeros(n)}
    _, yN = orc.replay(prob, u0, F[:, None], mesh)
    assert np.array_equal(yN, u0)
    loss, gu0, gp = orc.replay_grad(prob, u0, F[:, None], mesh, W.COTANGENT, aux=w)
    coef = _stability_poly(orc.tableau(method))
    I = np.eye(d)
    for i in range(n):
        A = np.zeros((d, d))
        for r in range(d):
            A[r, (r + 1) % d] += F[i]
            A[r, (r - 2) % d] -= F[i]
            A[r, (r - 1) % d] += 0.0     # x_{i+1} - x_{i-2} = 0 at the fixed point
            A[r, r] -= 1.0
        M = I.copy()
        e = np.zeros(d)
        for k in range(N):
            Z = h[i, k] * A
            Rm = np.zeros((d, d)); Phi = np.zeros((d, d)); Zp = I.copy()
            for j, cj in enumerate(coef):
                Rm += cj * Zp
                if j >= 1:
                    Phi += cj * (Zp @ np.linalg.inv(Z))
                Zp = Zp @ Z
            e = Rm @ e + h[i, k] * (Phi @ np.ones(d))
            M = Rm @ M
        assert np.allclose(gu0[i], M.T @ w[i, 0], rtol=1e-11, atol=1e-12)
        assert gp[i, 0] == pytest.approx(w[i, 0] @ e, rel=1e-11)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("method", [W.ROS2, W.RODAS3, W.ROS4])
def test_robertson_ros2_conservation(orc, method):
    """1^T f = 0 for Robertson, so 1^T J = 0 and a Rosenbrock step (ROS2,
    Rodas3: every stage is W^-1 of a combination of f values and earlier
    stages) keeps y1+y2+y3 fixed for any k and h; the adjoint of the linear
    functional 1^T y_N is 1 for u0 and 0 for k."""
    inp = W.make_inputs(4, 64)
    prob = W.WORKLOADS[4].problem(method=method)
    m = orc.record(prob, inp["u0"], inp["p"])
    assert np.all(m["status"] == 0)
    ys, yN = orc.replay(prob, inp["u0"], inp["p"], m)
    assert np.allclose(yN.sum(1), inp["u0"].sum(1), rtol=0, atol=1e-13)
    n = inp["u0"].shape[0]
    loss, gu0, gp = orc.replay_grad(prob, inp["u0"], inp["p"], m, W.COTANGENT,
                                    aux=np.ones((n, 1, 3)))
    assert np.allclose(gu0, 1.0, rtol=0, atol=1e-11)
    # scale of each k-gradient term: |dL/dk| would be O(y/k) for a generic functional
    assert np.all(np.abs(gp * inp["p"]) < 1e-9)


# the eight-species cycle written out from its reaction list, independently
# of the oracle: (source, target, parameter, coefficient, reactants)
_KIN8 = [(0, 1, 0, 1.0, (0,)), (1, 2, 1, 1.0, (1, 1)), (1, 0, 2, 1.0, (1, 2)),
         (2, 3, 3, 1.0, (2,)), (3, 4, 3, 10.0, (3,)), (4, 5, 1, 1e-3, (4, 4)),
         (5, 6, 0, 25.0, (5,)), (6, 7, 2, 0.1, (6, 2)), (7, 0, 3, 0.01, (7,))]


def _kin8_f(y, p):
    S = np.zeros((8, 9))
    w = np.zeros(9)
    for r, (src, dst, q, c, reac) in enumerate(_KIN8):
        S[src, r] -= 1.0
        S[dst, r] += 1.0
        w[r] = c * p[q] * np.prod([y[a] for a in reac])
    return S @ w


@pytest.mark.parametrize("method", [W.ROS2, W.RODAS3, W.ROS4])
def test_kinetics8_conservation_and_reference(orc, method):
    """The eight-species cycle: every reaction moves one unit, so both
    Rosenbrock methods keep sum y fixed and the gradient of sum y_N is 1 for
    u0 and 0 for the rates; the recorded solution agrees with SciPy's Radau
    on the system written out above from its reaction list."""
    from scipy.integrate import solve_ivp
    inp = W.make_inputs(6, 6)
    prob = W.WORKLOADS[6].problem(method=method, t1=30.0, max_steps=20000)
    m = orc.record(prob, inp["u0"], inp["p"])
    assert np.all(m["status"] == 0)
    ys, yN = orc.replay(prob, inp["u0"], inp["p"], m)
    assert np.allclose(yN.sum(1), 1.0, rtol=0, atol=1e-13)
    loss, gu0, gp = orc.replay_grad(prob, inp["u0"], inp["p"], m, W.COTANGENT,
                                    aux=np.ones((6, 1, 8)))
    assert np.allclose(gu0, 1.0, rtol=0, atol=1e-10)
    assert np.all(np.abs(gp * inp["p"]) < 1e-8)
    for i in range(2):
        ref = solve_ivp(lambda t, y: _kin8_f(y, inp["p"][i]), (0, 30.0), inp["u0"][i],
                        method="Radau", rtol=1e-11, atol=1e-15).y[:, -1]
        assert np.allclose(yN[i], ref, rtol=1e-4, atol=2e-9), (method, i)


def test_record_equals_replay_bitwise(orc):
    """The replay reproduces the recorded states bit for bit (both roundings)."""
    for wid, n in [(1, 64), (2, 32), (3, 32), (4, 8), (5, 8)]:
        w = W.WORKLOADS[wid]
        inp = W.make_inputs(wid, n)
        prob = w.problem()
        for fused in (False, True):
            m = orc.record(prob, inp["u0"], inp["p"], fused=fused)
            assert np.all(m["status"] == 0)
            ys, _ = orc.replay(prob, inp["u0"], inp["p"], m, fused=fused)
            assert np.array_equal(ys, m["y_save"]), (wid, fused)


def test_record_accepts_only_small_errors(orc):
    """Re-evaluating every recorded step gives E <= 1 (the accept test)."""
    for wid, n in [(1, 128), (3, 64), (4, 16)]:
        w = W.WORKLOADS[wid]
        inp = W.make_inputs(wid, n)
        prob = w.problem()
        m = orc.record(prob, inp["u0"], inp["p"])
        E = orc.mesh_max_err(prob, inp["u0"], inp["p"], m)
        assert np.all(E <= 1.0) and np.all(E > 0.01)


def test_save_times_are_mesh_points(orc):
    """Steps are clipped onto save times: the partial sums of h hit them."""
    w = W.WORKLOADS[3]
    inp = W.make_inputs(3, 64)
    prob = w.problem()
    u0 = inp["u0"].astype(np.float64); p = inp["p"].astype(np.float64)
    m = orc.record(prob, u0, p)
    for i in range(64):
        cs = np.concatenate([[0.0], np.cumsum(m["h"][i])])
        for s, ts in enumerate(prob.save_times):
            assert cs[m["save_idx"][i, s]] == pytest.approx(ts, rel=1e-13)
        assert m["save_idx"][i, -1] == m["n_steps"][i]


def test_global_error_tracks_tolerance(orc):
    """y' = -y on [0, 1]: the recorded solve's error at t=1 stays below the
    tolerance scale and shrinks as the tolerance does."""
    for method in (W.TSIT5, W.DOPRI5, W.ROS2, W.RODAS3, W.RKF78, W.ROS4):
        errs = []
        for tol in (1e-4, 1e-6, 1e-8):
            prob = W.Problem(W.LINEAR, 1, 1, method, 0.0, 1.0, tol, tol, 100000)
            m = orc.record(prob, np.ones((1, 1)), -np.ones((1, 1)))
            err = abs(m["y_save"][0, 0, 0] - math.exp(-1.0))
            errs.append(err)
            assert err < 20 * tol, (method, tol, err)
        assert errs[2] < errs[0]


def test_status_codes(orc):
    w = W.WORKLOADS[1]
    inp = W.make_inputs(1, 4)
    u0, p = inp["u0"], inp["p"].copy()
    m = orc.record(w.problem(max_steps=3), u0, p)
    assert np.all(m["status"] == orc.LANE_MAX_STEPS) and np.all(m["n_steps"] == 3)
    p[1, 0] = np.nan
    m = orc.record(w.problem(), u0, p)
    assert m["status"][1] == orc.LANE_NONFINITE and m["n_steps"][1] == 0
    assert np.all(m["status"][[0, 2, 3]] == 0)
    # an overflowing right-hand side makes every error estimate non-finite:
    # each attempt is rejected with the smallest factor until h underflows
    m = orc.record(w.problem(), np.full((4, 3), 1e200), inp["p"])
    assert np.all(m["status"] == orc.LANE_DT_UNDERFLOW) and np.all(m["n_steps"] == 0)
    # a tolerance far below rounding cannot reach t1 within max_steps
    m = orc.record(w.problem(rtol=1e-300, atol=1e-300), u0, inp["p"])
    assert np.all(m["status"] != 0)
    m = orc.record(w.problem(max_attempts=5), u0, inp["p"])
    assert np.all(m["status"] == orc.LANE_MAX_ATTEMPTS) and np.all(m["n_attempts"] == 5)
    # failed lanes give NaN gradients
    m = orc.record(w.problem(max_steps=3), u0, inp["p"])
    loss, gu0, gp = orc.replay_grad(w.problem(max_steps=3), u0, inp["p"], m)
    assert np.all(np.isnan(gp)) and np.all(np.isnan(loss))


# ---------------------------------------------------------------------------
# Textbook / library routines
# ---------------------------------------------------------------------------

def _lorenz(p):
    s, r, b = p
    return lambda t, u: np.array([s * (u[1] - u[0]), u[0] * (r - u[2]) - u[1],
                                  u[0] * u[1] - b * u[2]])


def test_dopri5_record_matches_scipy_rk45(orc):
    """SciPy's RK45 is Dormand-Prince with the same RMS error norm and
    I-controller (safety 0.9, factors in [0.2, 10], no growth right after a
    reject).  Given the same first step, the oracle's plain mode (the
    textbook controller, its power in double precision as in SciPy) accepts
    the same steps: the same number, and step sizes within 1e-8 relative.
    The fused mode takes the power in single precision, as the kernels do;
    its step counts still equal SciPy's."""
    from scipy.integrate import solve_ivp
    inp = W.make_inputs(2, 6)
    for i in range(6):
        prob = W.Problem(W.LORENZ63, 3, 3, W.DOPRI5, 0.0, 2.0, 1e-8, 1e-8, 4096, dt0=1e-3)
        m = orc.record(prob, inp["u0"][i:i + 1], inp["p"][i:i + 1])
        sol = solve_ivp(_lorenz(inp["p"][i]), (0.0, 2.0), inp["u0"][i], method="RK45",
                        rtol=1e-8, atol=1e-8, first_step=1e-3)
        hs = np.diff(sol.t)
        N = m["n_steps"][0]
        assert N == len(hs)
        assert np.allclose(m["h"][0, :N], hs, rtol=1e-8)
        assert np.allclose(m["y_save"][0, 0], sol.y[:, -1], rtol=1e-6, atol=1e-8)
        mf = orc.record(prob, inp["u0"][i:i + 1], inp["p"][i:i + 1], fused=True)
        assert mf["n_steps"][0] == N


def test_save_time_landing_matches_scipy_rk45(orc):
    """The landing rule for save times (reading R6): every save time is a mesh
    point, the step that would pass it is shortened to end on it, and the
    next trial step comes from that shortened step's error norm.  SciPy's
    RK45, started again at each save time with the step size it proposed at
    the end of the previous segment (its t_bound shortens the last step of a
    segment the same way, and its next proposal comes from that step), gives
    the same steps: the same count per segment and step sizes within 1e-6
    relative (the two sides' error norms differ in the last bits and the
    differences drift over about 150 chaotic steps; a next step taken from the
    unshortened proposal would differ at order one), and the same saved
    states."""
    from scipy.integrate import RK45
    inp = W.make_inputs(2, 6)
    saves = (0.3, 0.9, 1.5, 2.0)
    for i in range(6):
        prob = W.Problem(W.LORENZ63, 3, 3, W.DOPRI5, 0.0, 2.0, 1e-8, 1e-8, 4096,
                         save_times=saves, dt0=1e-3)
        m = orc.record(prob, inp["u0"][i:i + 1], inp["p"][i:i + 1])
        hs, idx, ys = [], [], []
        t, y, h0 = 0.0, inp["u0"][i].copy(), 1e-3
        for ts in saves:
            sol = RK45(_lorenz(inp["p"][i]), t, y, ts, rtol=1e-8, atol=1e-8, first_step=h0)
            while sol.status == "running":
                tp = sol.t
                sol.step()
                hs.append(sol.t - tp)
            assert sol.status == "finished" and sol.t == ts
            t, y, h0 = sol.t, sol.y.copy(), sol.h_abs
            idx.append(len(hs))
            ys.append(y)
        hs = np.array(hs)
        N = m["n_steps"][0]
        assert N == len(hs)
        assert np.array_equal(m["save_idx"][0], idx)
        assert np.allclose(m["h"][0, :N], hs, rtol=1e-6, atol=0)
        assert np.allclose(m["y_save"][0], np.array(ys), rtol=1e-10, atol=1e-12)


def test_initial_step_matches_textbook(orc):
    """Starting step of Hairer-Norsett-Wanner I.II.4 (SciPy's select_initial_step
    implements the same algorithm), with the method order 5."""
    from scipy.integrate._ivp.common import select_initial_step
    inp = W.make_inputs(2, 8)
    prob = W.WORKLOADS[2].problem()
    for i in range(8):
        f = _lorenz(inp["p"][i])
        y0 = inp["u0"][i]
        ref = select_initial_step(f, 0.0, y0, 10.0, np.inf, f(0.0, y0), 1, 5, 1e-8, 1e-8)
        assert orc.initial_step(prob, y0, inp["p"][i]) == pytest.approx(ref, rel=1e-12)


# ---------------------------------------------------------------------------
# Adjoint vs forward mode and finite differences
# ---------------------------------------------------------------------------

def _cases():
    # (problem, u0, p, loss, aux, scale)
    out = []
    inp = W.make_inputs(1, 6)
    out.append(("lorenz63_tsit5", W.WORKLOADS[1].problem(), inp["u0"], inp["p"],
                W.SUMSQ_FINAL, None))
    inp = W.make_inputs(2, 6)
    out.append(("lorenz63_dopri5_saves", W.WORKLOADS[2].problem(t1=1.5, save_times=(0.5, 1.0, 1.5)),
                inp["u0"], inp["p"], W.COTANGENT,
                np.random.default_rng(1).standard_normal((6, 3, 3))))
    inp = W.make_inputs(3, 6)
    out.append(("lorenz63_mse", W.WORKLOADS[3].problem(t1=2.0, save_times=(0.5, 1.0, 2.0)),
                inp["u0"].astype(np.float64), inp["p"].astype(np.float64), W.MSE_SAVE,
                np.random.default_rng(2).standard_normal((6, 3, 3))))
    inp = W.make_inputs(4, 4)
    out.append(("robertson_ros2", W.WORKLOADS[4].problem(t1=30.0), inp["u0"], inp["p"],
                W.SUMSQ_FINAL, None))
    out.append(("robertson_tsit5", W.WORKLOADS[4].problem(t1=0.5, method=W.TSIT5, max_steps=8192),
                inp["u0"], inp["p"], W.SUMSQ_FINAL, None))
    inp = W.make_inputs(5, 3)
    out.append(("lorenz96", W.WORKLOADS[5].problem(t1=0.5), inp["u0"], inp["p"],
                W.SUMSQ_FINAL, None))
    out.append(("lorenz96_dopri5", W.WORKLOADS[5].problem(t1=0.5, method=W.DOPRI5), inp["u0"],
                inp["p"], W.COTANGENT, np.random.default_rng(3).standard_normal((3, 1, 64))))
    out.append(("linear_ros2", W.Problem(W.LINEAR, 1, 1, W.ROS2, 0.0, 2.0, 1e-6, 1e-6, 20000),
                np.array([[1.0], [2.0]]), np.array([[-0.7], [0.4]]), W.SUMSQ_FINAL, None))
    inp = W.make_inputs(4, 4)
    out.append(("robertson_rodas3", W.WORKLOADS[4].problem(t1=300.0, method=W.RODAS3),
                inp["u0"], inp["p"], W.SUMSQ_FINAL, None))
    inp = W.make_inputs(1, 6)
    out.append(("lorenz63_rkf78_saves", W.WORKLOADS[1].problem(
        method=W.RKF78, rtol=1e-9, atol=1e-9, save_times=(0.3, 0.7, 1.0)), inp["u0"], inp["p"],
        W.MSE_SAVE, np.random.default_rng(6).standard_normal((6, 3, 3))))
    inp = W.make_inputs(4, 4)
    out.append(("robertson_rkf78", W.WORKLOADS[4].problem(t1=0.3, method=W.RKF78, max_steps=8192),
                inp["u0"], inp["p"], W.SUMSQ_FINAL, None))
    inp = W.make_inputs(6, 3)
    out.append(("kinetics8_rodas3_saves", W.WORKLOADS[6].problem(t1=20.0, save_times=(0.5, 20.0)),
                inp["u0"], inp["p"], W.COTANGENT,
                np.random.default_rng(5).standard_normal((3, 2, 8))))
    out.append(("kinetics8_ros2", W.WORKLOADS[6].problem(t1=0.5, method=W.ROS2, max_steps=8192),
                inp["u0"], inp["p"], W.SUMSQ_FINAL, None))
    inp = W.make_inputs(1, 6)
    out.append(("lorenz63_rodas3_saves", W.WORKLOADS[1].problem(
        method=W.RODAS3, max_steps=4096, save_times=(0.3, 0.7, 1.0)), inp["u0"], inp["p"],
        W.MSE_SAVE, np.random.default_rng(4).standard_normal((6, 3, 3))))
    inp = W.make_inputs(4, 4)
    out.append(("robertson_ros4", W.WORKLOADS[4].problem(t1=300.0, method=W.ROS4),
                inp["u0"], inp["p"], W.SUMSQ_FINAL, None))
    inp = W.make_inputs(1, 6)
    out.append(("lorenz63_ros4_saves", W.WORKLOADS[1].problem(
        method=W.ROS4, max_steps=4096, save_times=(0.3, 0.7, 1.0)), inp["u0"], inp["p"],
        W.MSE_SAVE, np.random.default_rng(8).standard_normal((6, 3, 3))))
    inp = W.make_inputs(6, 3)
    out.append(("kinetics8_ros4", W.WORKLOADS[6].problem(t1=5.0, method=W.ROS4),
                inp["u0"], inp["p"], W.SUMSQ_FINAL, None))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_adjoint_matches_dual_numbers(orc, case):
    """<grad, v> equals the forward-mode derivative along v (dot-product test)."""
    name, prob, u0, p, lk, aux = case
    m = orc.record(prob, u0, p)
    assert np.all(m["status"] == 0)
    loss, gu0, gp = orc.replay_grad(prob, u0, p, m, lk, aux=aux, scale=0.7)
    rng = np.random.default_rng(4)
    for _ in range(3):
        du0 = rng.standard_normal(u0.shape)
        dp = rng.standard_normal(p.shape) * p
        l2, dl, _, _ = orc.replay_jvp(prob, u0, p, du0, dp, m, lk, aux=aux, scale=0.7)
        assert np.allclose(l2, loss, rtol=1e-14)
        adj = (gu0 * du0).sum(1) + (gp * dp).sum(1)
        assert np.allclose(adj, dl, rtol=1e-11, atol=1e-11 * np.abs(dl).max()), name


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_adjoint_matches_dual_numbers(orc, case):
    """The fused-rounding mode (the kernels' arithmetic schedule, including the
    per-component accumulation of the Lorenz-96 F-gradient) passes the same
    dot-product test, and stays within rounding of the plain mode."""
    name, prob, u0, p, lk, aux = case
    m = orc.record(prob, u0, p, fused=True)
    assert np.all(m["status"] == 0)
    loss, gu0, gp = orc.replay_grad(prob, u0, p, m, lk, aux=aux, scale=0.7, fused=True)
    lp, gu0p, gpp = orc.replay_grad(prob, u0, p, m, lk, aux=aux, scale=0.7, fused=False)
    rng = np.random.default_rng(5)
    for _ in range(3):
        du0 = rng.standard_normal(u0.shape)
        dp = rng.standard_normal(p.shape) * p
        _, dl, _, _ = orc.replay_jvp(prob, u0, p, du0, dp, m, lk, aux=aux, scale=0.7)
        adj = (gu0 * du0).sum(1) + (gp * dp).sum(1)
        assert np.allclose(adj, dl, rtol=1e-11, atol=1e-11 * np.abs(dl).max()), name
    assert np.allclose(gp, gpp, rtol=1e-10, atol=1e-12 * np.abs(gpp).max()), name
    assert np.allclose(gu0, gu0p, rtol=1e-10, atol=1e-12 * np.abs(gu0p).max()), name


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_adjoint_matches_finite_differences(orc, case):
    """Central differences of the replayed loss on the frozen mesh."""
    name, prob, u0, p, lk, aux = case
    m = orc.record(prob, u0, p)
    loss, gu0, gp = orc.replay_grad(prob, u0, p, m, lk, aux=aux)
    for q in range(p.shape[1]):
        eps = 1e-6 * np.abs(p[:, q])
        pp = p.copy(); pp[:, q] += eps
        pm = p.copy(); pm[:, q] -= eps
        lp = orc.replay_grad(prob, u0, pp, m, lk, aux=aux)[0]
        lm = orc.replay_grad(prob, u0, pm, m, lk, aux=aux)[0]
        fd = (lp - lm) / (2 * eps)
        assert np.allclose(gp[:, q], fd, rtol=2e-5, atol=1e-6 * np.abs(fd).max()), (name, q)
    for c in range(min(u0.shape[1], 4)):
        eps = 1e-6
        up = u0.copy(); up[:, c] += eps
        um = u0.copy(); um[:, c] -= eps
        fd = (orc.replay_grad(prob, up, p, m, lk, aux=aux)[0] -
              orc.replay_grad(prob, um, p, m, lk, aux=aux)[0]) / (2 * eps)
        assert np.allclose(gu0[:, c], fd, rtol=2e-5, atol=1e-6 * np.abs(fd).max()), (name, c)


def test_loss_values_match_their_definitions(orc):
    """Loss kinds against their formulas evaluated on the replayed states."""
    prob = W.WORKLOADS[3].problem(t1=2.0, save_times=(0.5, 1.0, 2.0))
    inp = W.make_inputs(3, 8)
    u0 = inp["u0"].astype(np.float64); p = inp["p"].astype(np.float64)
    m = orc.record(prob, u0, p)
    ys, yN = orc.replay(prob, u0, p, m)
    tg = np.random.default_rng(0).standard_normal((8, 3, 3))
    L = orc.replay_grad(prob, u0, p, m, W.MSE_SAVE, aux=tg, scale=0.25)[0]
    assert np.allclose(L, 0.25 * ((ys - tg) ** 2).sum((1, 2)), rtol=1e-13)
    L = orc.replay_grad(prob, u0, p, m, W.COTANGENT, aux=tg, scale=2.0)[0]
    assert np.allclose(L, 2.0 * (ys * tg).sum((1, 2)), rtol=1e-12)
    L = orc.replay_grad(prob, u0, p, m, W.SUMSQ_FINAL, scale=3.0)[0]
    assert np.allclose(L, 3.0 * (yN**2).sum(1), rtol=1e-13)


def test_rhs_vjp_against_dense_jacobian(orc):
    """J^T v and J_p^T v of each system against finite-difference Jacobians."""
    rng = np.random.default_rng(9)
    for kind, d, P in [(W.LORENZ63, 3, 3), (W.ROBERTSON, 3, 3), (W.LORENZ96, 8, 1),
                       (W.LINEAR, 1, 1), (W.KINETICS8, 8, 4)]:
        y = rng.standard_normal(d)
        p = rng.uniform(0.5, 2.0, P)
        v = rng.standard_normal(d)
        f, wy, gp, J = orc.rhs(kind, y, p, v)
        Jfd = np.zeros((d, d)); Jpfd = np.zeros((d, P))
        for j in range(d):
            e = np.zeros(d); e[j] = 1e-6
            Jfd[:, j] = (orc.rhs(kind, y + e, p, v)[0] - orc.rhs(kind, y - e, p, v)[0]) / 2e-6
        for q in range(P):
            e = np.zeros(P); e[q] = 1e-6
            Jpfd[:, q] = (orc.rhs(kind, y, p + e, v)[0] - orc.rhs(kind, y, p - e, v)[0]) / 2e-6
        assert np.allclose(wy, Jfd.T @ v, rtol=1e-7, atol=1e-8)
        assert np.allclose(gp, Jpfd.T @ v, rtol=1e-7, atol=1e-8)
        if J is not None:
            assert np.allclose(J, Jfd, rtol=1e-7, atol=1e-8)


def test_fp32_oracle_tracks_fp64(orc):
    """The FP32 oracle stays close to the FP64 oracle on its own mesh."""
    w = W.WORKLOADS[3]
    inp = W.make_inputs(3, 32)
    prob = w.problem(t1=1.0, save_times=(0.5, 1.0))
    m32 = orc.record(prob, inp["u0"], inp["p"])
    m64 = {k: (v.astype(np.float64) if v is not None and v.dtype == np.float32 else v)
           for k, v in m32.items()}
    l32, g32, p32 = orc.replay_grad(prob, inp["u0"], inp["p"], m32)
    l64, g64, p64 = orc.replay_grad(prob, inp["u0"].astype(np.float64),
                                    inp["p"].astype(np.float64), m64)
    assert np.allclose(p32, p64, rtol=1e-3, atol=1e-3 * np.abs(p64).max())


# ---------------------------------------------------------------------------
# Forward-mode sensitivities (tangents carried through the replay)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("method", [W.TSIT5, W.DOPRI5, W.ROS2, W.RODAS3, W.RKF78, W.ROS4])
@pytest.mark.parametrize("fused", [False, True])
def test_sensitivities_linear_closed_form(orc, method, fused):
    """y' = p y on an arbitrary mesh: dy_N/dy0 = prod R(p h_n) and
    dy_N/dp = y_N sum h_n R'(p h_n) / R(p h_n), from the stability function."""
    rng = np.random.default_rng(11)
    N, n = 29, 3
    h = rng.uniform(0.01, 0.2, size=(n, N))
    y0 = np.array([1.3, -0.4, 2.0])
    pv = np.array([-0.6, -4.0, 0.35])
    if method == W.ROS2:
        g = orc.ros2_gamma()
        R = lambda z: _R_ros2(g, z)
    elif method == W.RODAS3:
        R = _R_rodas3
    elif method == W.ROS4:
        R = _R_ros4
    else:
        coef = _stability_poly(_rk78_float() if method == W.RKF78 else orc.tableau(method))
        R = lambda z: _R_erk(coef, z)
    prob = W.Problem(W.LINEAR, 1, 1, method, 0.0, 1.0, 1e-6, 1e-6, N)
    mesh = {"h": h, "n_steps": np.full(n, N), "save_idx": np.full((n, 1), N),
            "status": np.zeros(n)}
    sens, loss, gu0, gp = orc.replay_sens(prob, y0[:, None], pv[:, None], mesh, fused=fused)
    for i in range(n):
        z = pv[i] * h[i]
        Rz = np.array([R(zz) for zz in z])
        prod = np.prod(Rz)
        dR = np.array([_complex_step(R, zz) for zz in z])
        assert sens[i, 0, 0, 0] == pytest.approx(prod, rel=2e-14)
        assert sens[i, 0, 0, 1] == pytest.approx(y0[i] * prod * np.sum(h[i] * dR / Rz), rel=2e-13)
        # final-state loss y_N^2: gradient 2 y_N dy_N/dtheta
        yN = y0[i] * prod
        assert gu0[i, 0] == pytest.approx(2 * yN * prod, rel=2e-13)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("fused", [False, True])
def test_sensitivity_gradient_matches_adjoint(orc, case, fused):
    """The loss gradient through forward tangents equals the reverse sweep's
    (both are the exact derivative of the same discrete map); the tangents of
    the final state match central differences on the frozen mesh."""
    name, prob, u0, p, lk, aux = case
    m = orc.record(prob, u0, p, fused=fused)
    sens, loss, gu0, gp = orc.replay_sens(prob, u0, p, m, lk, aux=aux, scale=0.7, fused=fused)
    la, ga, pa = orc.replay_grad(prob, u0, p, m, lk, aux=aux, scale=0.7, fused=fused)
    assert np.allclose(loss, la, rtol=1e-13)
    assert np.allclose(gu0, ga, rtol=1e-10, atol=1e-11 * np.abs(ga).max()), name
    assert np.allclose(gp, pa, rtol=1e-10, atol=1e-11 * np.abs(pa).max()), name
    # tangents of the final state against central differences in the parameters
    d = prob.dim
    for q in range(p.shape[1]):
        eps = 1e-6 * np.abs(p[:, q])
        pp = p.copy(); pp[:, q] += eps
        pm = p.copy(); pm[:, q] -= eps
        yp = orc.replay(prob, u0, pp, m, fused=fused)[1]
        ym = orc.replay(prob, u0, pm, m, fused=fused)[1]
        fd = (yp - ym) / (2 * eps[:, None])
        last = m["save_idx"].argmax(axis=1)
        sq = sens[np.arange(len(u0)), last, :, d + q]
        if np.all(m["save_idx"].max(axis=1) == m["n_steps"]):
            assert np.allclose(sq, fd, rtol=3e-5, atol=1e-6 * np.abs(fd).max()), (name, q)


def test_fused_and_plain_sensitivities_agree(orc):
    """The two roundings of the tangent arithmetic agree to rounding level on a
    short horizon."""
    prob = W.WORKLOADS[1].problem()
    inp = W.make_inputs(1, 16)
    m = orc.record(prob, inp["u0"], inp["p"], fused=True)
    sf = orc.replay_sens(prob, inp["u0"], inp["p"], m, fused=True)[0]
    sp = orc.replay_sens(prob, inp["u0"], inp["p"], m, fused=False)[0]
    assert np.allclose(sf, sp, rtol=1e-12, atol=1e-13 * np.abs(sp).max())
    assert not np.array_equal(sf, sp)      # the schedules do differ
