"""Pins of the oracle's path for right-hand sides given as source (the body of
``template <class T> void f(const T *y, const T *p, T *dy)``, the form the
HIP library compiles at run time).

What fixes the expected values:
 - the built-in Lorenz-63 of the oracle, written independently by hand with
   its own vector-Jacobian products: the same system given as source must
   give the same mesh and, in plain rounding, the same gradient;
 - physics of a Kepler orbit (energy and angular momentum are conserved by
   the exact flow, so the recorded solution conserves them to the tolerance);
 - dual-number forward mode (the JVP check) and central finite differences
   on the frozen mesh, for a right-hand side that uses every function the
   source may call;
 - finite-difference Jacobians of f itself.
CPU only.
"""
import numpy as np
import pytest

import workloads as W

L63 = """
    dy[0] = p[0] * (y[1] - y[0]);
    dy[1] = y[0] * (p[1] - y[2]) - y[1];
    dy[2] = y[0] * y[1] - p[2] * y[2];
"""

# planar Kepler orbit, p = (GM)
KEPLER = """
    const T r2 = y[0] * y[0] + y[1] * y[1];
    const T r3 = r2 * sqrt(r2);
    dy[0] = y[2];
    dy[1] = y[3];
    dy[2] = -p[0] * y[0] / r3;
    dy[3] = -p[0] * y[1] / r3;
"""

# every function and mixed-constant form the source may use
ALLFN = """
    const T a = y[0] * y[0] + T(1);
    dy[0] = p[0] * sin(y[1]) - 0.5 * y[0] + exp(-a) / (T(2) + y[1] * y[1]);
    dy[1] = p[1] * cos(y[0]) - tanh(y[1]) + log(a) * 0.1 - 2.0 / (3.0 + a);
    dy[2] = -p[2] * y[2] + pow(a, 0.75) * 0.05 - sqrt(a) / 7 + (y[0] - 1.0) * 0.01;
"""

USER = 1024


def _kepler_inputs(n, seed=3):
    rng = np.random.default_rng(seed)
    ecc = 0.1 + 0.5 * rng.random(n)          # eccentricities
    r0 = 1.0 - ecc                            # start at pericentre, GM = 1
    v0 = np.sqrt((1 + ecc) / (1 - ecc))
    u0 = np.stack([r0, np.zeros(n), np.zeros(n), v0], axis=1)
    p = 1.0 + 0.05 * rng.standard_normal((n, 1))
    return u0, p


def test_source_lorenz63_equals_builtin(orc):
    """Lorenz-63 as source against the hand-written built-in: same mesh in
    both roundings; in plain rounding the same loss and gradient; in fused
    rounding (where the built-in fuses its multiply-adds and the source does
    not) gradients within 1e-12 on a shared mesh."""
    orc.set_user_rhs(L63, 3, 3)
    inp = W.make_inputs(1, 32)
    pb = W.WORKLOADS[1].problem(save_times=(0.3, 0.7, 1.0))
    pu = pb.replace(rhs=USER)
    aux = np.random.default_rng(1).standard_normal((32, 3, 3))
    mb = orc.record(pb, inp["u0"], inp["p"])
    mu = orc.record(pu, inp["u0"], inp["p"])
    assert np.array_equal(mb["h"], mu["h"]) and np.array_equal(mb["y_save"], mu["y_save"])
    for fused in (False, True):
        m = orc.record(pb, inp["u0"], inp["p"], fused=fused)
        for lk in (W.SUMSQ_FINAL, W.MSE_SAVE, W.COTANGENT):
            lb, gb, qb = orc.replay_grad(pb, inp["u0"], inp["p"], m, lk, aux=aux, fused=fused)
            lu, gu, qu = orc.replay_grad(pu, inp["u0"], inp["p"], m, lk, aux=aux, fused=fused)
            tol = 1e-15 if not fused else 1e-12
            assert np.allclose(lu, lb, rtol=tol, atol=0)
            assert np.allclose(gu, gb, rtol=tol, atol=tol * np.abs(gb).max())
            assert np.allclose(qu, qb, rtol=tol, atol=tol * np.abs(qb).max())


def test_source_rhs_products_match_finite_differences(orc):
    """J^T v and J_p^T v from the dual passes against central differences of
    f (through a one-step replay of tiny size, whose derivative is I + hJ)."""
    orc.set_user_rhs(ALLFN, 3, 3)
    prob = W.Problem(USER, 3, 3, W.TSIT5, 0.0, 1.0, 1e-6, 1e-6, 4)
    rng = np.random.default_rng(5)
    for _ in range(4):
        y = rng.standard_normal((1, 3))
        p = 1.0 + rng.random((1, 3))
        h = 1e-3
        mesh = {"h": np.array([[h, 0, 0, 0]]), "n_steps": np.array([1], np.int32),
                "save_idx": np.array([[1]], np.int32), "status": np.zeros(1, np.int32)}
        v = rng.standard_normal((1, 1, 3))
        _, gu, gp = orc.replay_grad(prob, y, p, mesh, W.COTANGENT, aux=v)
        eps = 1e-6
        for c in range(3):
            yp, ym = y.copy(), y.copy()
            yp[0, c] += eps
            ym[0, c] -= eps
            fd = (orc.replay(prob, yp, p, mesh)[1] - orc.replay(prob, ym, p, mesh)[1]) / (2 * eps)
            assert abs(gu[0, c] - (fd[0] * v[0, 0]).sum()) < 1e-8 * max(1, abs(gu[0, c]))
        for q in range(3):
            pp, pm = p.copy(), p.copy()
            pp[0, q] += eps
            pm[0, q] -= eps
            fd = (orc.replay(prob, y, pp, mesh)[1] - orc.replay(prob, y, pm, mesh)[1]) / (2 * eps)
            assert abs(gp[0, q] - (fd[0] * v[0, 0]).sum()) < 1e-9 * max(1, abs(gp[0, q]))


@pytest.mark.parametrize("method", [W.TSIT5, W.DOPRI5])
def test_source_kepler_conserves_energy_and_momentum(orc, method):
    """A Kepler orbit given as source: energy v^2/2 - GM/r and angular
    momentum x v_y - y v_x after one revolution stay within the tolerance."""
    orc.set_user_rhs(KEPLER, 4, 1)
    u0, p = _kepler_inputs(16)
    prob = W.Problem(USER, 4, 1, method, 0.0, 2 * np.pi, 1e-10, 1e-10, 20000)
    m = orc.record(prob, u0, p)
    assert np.all(m["status"] == 0)
    yN = m["y_save"][:, 0, :]

    def invariants(y, gm):
        r = np.hypot(y[:, 0], y[:, 1])
        return 0.5 * (y[:, 2] ** 2 + y[:, 3] ** 2) - gm / r, y[:, 0] * y[:, 3] - y[:, 1] * y[:, 2]

    e0, l0 = invariants(u0, p[:, 0])
    e1, l1 = invariants(yN, p[:, 0])
    assert np.all(np.abs(e1 - e0) < 1e-7 * np.abs(e0))
    assert np.all(np.abs(l1 - l0) < 1e-7 * np.abs(l0))


@pytest.mark.parametrize("src,dim,P,name", [(KEPLER, 4, 1, "kepler"), (ALLFN, 3, 3, "allfn")])
@pytest.mark.parametrize("fused", [False, True])
def test_source_adjoint_matches_duals_and_differences(orc, src, dim, P, name, fused):
    """Dot-product test against dual-number forward mode and central
    differences on the frozen mesh, with losses at save times."""
    orc.set_user_rhs(src, dim, P)
    n = 6
    rng = np.random.default_rng(7)
    if name == "kepler":
        u0, p = _kepler_inputs(n)
        prob = W.Problem(USER, 4, 1, W.DOPRI5, 0.0, 3.0, 1e-9, 1e-9, 4096,
                         save_times=(1.0, 2.0, 3.0))
    else:
        u0 = 0.5 * rng.standard_normal((n, 3))
        p = 1.0 + rng.random((n, 3))
        prob = W.Problem(USER, 3, 3, W.TSIT5, 0.0, 2.0, 1e-8, 1e-8, 4096,
                         save_times=(0.5, 1.3, 2.0))
    aux = rng.standard_normal((n, 3, dim))
    m = orc.record(prob, u0, p, fused=fused)
    assert np.all(m["status"] == 0)
    loss, gu0, gp = orc.replay_grad(prob, u0, p, m, W.MSE_SAVE, aux=aux, scale=0.5, fused=fused)
    for _ in range(3):
        du0 = rng.standard_normal(u0.shape)
        dp = rng.standard_normal(p.shape) * p
        _, dl, _, _ = orc.replay_jvp(prob, u0, p, du0, dp, m, W.MSE_SAVE, aux=aux, scale=0.5)
        adj = (gu0 * du0).sum(1) + (gp * dp).sum(1)
        assert np.allclose(adj, dl, rtol=1e-10, atol=1e-11 * np.abs(dl).max()), name
    for q in range(P):
        eps = 1e-6 * np.abs(p[:, q])
        pp, pm = p.copy(), p.copy()
        pp[:, q] += eps
        pm[:, q] -= eps
        fd = (orc.replay_grad(prob, u0, pp, m, W.MSE_SAVE, aux=aux, scale=0.5)[0] -
              orc.replay_grad(prob, u0, pm, m, W.MSE_SAVE, aux=aux, scale=0.5)[0]) / (2 * eps)
        assert np.allclose(gp[:, q], fd, rtol=1e-5, atol=1e-7 * np.abs(fd).max()), (name, q)


def test_source_fp32_tracks_fp64(orc):
    """The single-precision path of a source right-hand side follows the
    double-precision one to single-precision accuracy."""
    orc.set_user_rhs(ALLFN, 3, 3)
    rng = np.random.default_rng(9)
    u0 = 0.5 * rng.standard_normal((8, 3))
    p = 1.0 + rng.random((8, 3))
    prob = W.Problem(USER, 3, 3, W.TSIT5, 0.0, 1.0, 1e-5, 1e-5, 4096)
    m64 = orc.record(prob, u0, p)
    m32 = orc.record(prob, u0.astype(np.float32), p.astype(np.float32))
    assert np.all(m32["status"] == 0)
    l64, g64, q64 = orc.replay_grad(prob, u0, p, m64, W.SUMSQ_FINAL)
    l32, g32, q32 = orc.replay_grad(prob, u0.astype(np.float32), p.astype(np.float32), m32,
                                    W.SUMSQ_FINAL)
    assert np.allclose(l32, l64, rtol=1e-3)
    assert np.allclose(q32, q64, rtol=1e-2, atol=1e-3 * np.abs(q64).max())


def test_source_rhs_rejected_with_ros2_and_wrong_shape(orc):
    orc.set_user_rhs(L63, 3, 3)
    inp = W.make_inputs(1, 2)
    with pytest.raises(ValueError):
        orc.record(W.Problem(USER, 3, 3, W.ROS2, 0.0, 1.0, 1e-6, 1e-6, 100), inp["u0"], inp["p"])
    with pytest.raises(ValueError):
        orc.record(W.Problem(USER, 3, 2, W.TSIT5, 0.0, 1.0, 1e-6, 1e-6, 100), inp["u0"],
                   inp["p"][:, :2])


L96_STENCIL = "return (y(1) - y(-2)) * y(-1) - y(0) + p[0];"


@pytest.mark.parametrize("dim", [64, 17, 5])
def test_stencil_lorenz96_equals_builtin(orc, dim):
    """Lorenz-96 written as a cyclic stencil (component i from y(o) =
    y[(i + o) mod d]) against the hand-written built-in Lorenz-96: in plain
    rounding the same mesh, saves and loss, and the gradient within 1e-12 on
    a shared mesh (the source multiplies then subtracts where the built-in
    fuses; the derivatives come from the generic dual passes).  A mistake in
    the offsets or in the cyclic index (i - o for i + o, no wrap) changes the
    system and fails this."""
    orc.set_user_stencil(L96_STENCIL, dim, 1, (-2, -1, 0, 1))
    n = 12
    inp = W.make_inputs(5, n)
    u0 = np.ascontiguousarray(inp["u0"][:, :dim])
    pb = W.WORKLOADS[5].problem(dim=dim, t1=0.5, save_times=(0.2, 0.5))
    pu = pb.replace(rhs=USER)
    aux = np.random.default_rng(3).standard_normal((n, 2, dim))
    mb = orc.record(pb, u0, inp["p"])
    mu = orc.record(pu, u0, inp["p"])
    assert np.array_equal(mb["n_steps"], mu["n_steps"])
    assert np.allclose(mu["y_save"], mb["y_save"], rtol=1e-13, atol=1e-13)
    lb, gb, qb = orc.replay_grad(pb, u0, inp["p"], mb, W.MSE_SAVE, aux=aux)
    lu, gu, qu = orc.replay_grad(pu, u0, inp["p"], mb, W.MSE_SAVE, aux=aux)
    assert np.allclose(lu, lb, rtol=1e-12, atol=0)
    assert np.allclose(gu, gb, rtol=1e-12, atol=1e-12 * np.abs(gb).max())
    assert np.allclose(qu, qb, rtol=1e-12, atol=1e-12 * np.abs(qb).max())


def test_stencil_undeclared_offset_is_nan(orc):
    """y(o) for an offset that was not declared is NaN, so the record fails
    as non-finite instead of reading a value the GPU kernels would not
    provide."""
    orc.set_user_stencil("return y(1) - y(2);", 8, 1, (1,))
    prob = W.Problem(USER, 8, 1, W.TSIT5, 0.0, 1.0, 1e-6, 1e-6, 64)
    m = orc.record(prob, np.ones((2, 8)), np.ones((2, 1)))
    assert np.all(m["status"] != 0)
