"""Pins of the oracle's dense output: save times read from the cubic Hermite
interpolant of the accepted step that contains them, instead of steps
shortened to land on them ("Differentiable astrophysics at scale",
Methodology, dense output; the interpolant is this library's reading).

What fixes the expected values here, none of it the oracle itself:
 - the Hermite remainder theorem: for a smooth y, y(t) - H(t) =
   y''''(xi) / 4! (t - t_k)^2 (t - t_{k+1})^2, so on y' = p y with a fine
   fixed-step mesh the error of a save at fraction th is
   -h^4 th^2 (1 - th)^2 p^4 e^{p t} / 24 to leading order, and halving h
   divides it by 16 (the integrator's own error is of higher order);
 - the exact derivative t e^{p t} of the exact solution, approached at the
   same order by the gradient of the interpolated saves;
 - th = 1 reduces the interpolant to the step's end state, i.e. to the
   save of the clipping record on the same mesh;
 - dual-number forward mode, central finite differences on the frozen mesh
   (step sizes and fractions held fixed) and the forward sensitivities;
 - the mesh bookkeeping: each save lies in the step its index names, at the
   fraction its time gives.
CPU only.
"""
import math

import numpy as np
import pytest

import workloads as W


def _dense_cases():
    """(name, problem, u0, p, loss kind, aux) with dense output."""
    out = []
    inp = W.make_inputs(2, 6)
    out.append(("lorenz63_dopri5_cot",
                W.WORKLOADS[2].problem(t1=1.5, save_times=(0.31, 0.5, 0.77, 1.2, 1.5), dense=1),
                inp["u0"], inp["p"], W.COTANGENT,
                np.random.default_rng(11).standard_normal((6, 5, 3))))
    inp = W.make_inputs(3, 6)
    out.append(("lorenz63_tsit5_mse",
                W.WORKLOADS[3].problem(t1=2.0, save_times=tuple(0.25 * s for s in range(1, 9)),
                                       dense=1),
                inp["u0"].astype(np.float64), inp["p"].astype(np.float64), W.MSE_SAVE,
                np.random.default_rng(12).standard_normal((6, 8, 3))))
    inp = W.make_inputs(5, 3)
    out.append(("lorenz96_tsit5_cot",
                W.WORKLOADS[5].problem(t1=0.5, save_times=(0.1, 0.23, 0.4), dense=1),
                inp["u0"], inp["p"], W.COTANGENT,
                np.random.default_rng(13).standard_normal((3, 3, 64))))
    inp = W.make_inputs(4, 4)
    out.append(("robertson_dopri5_mse",
                W.WORKLOADS[4].problem(t1=0.5, method=W.DOPRI5, max_steps=8192,
                                       save_times=(0.05, 0.2, 0.45), dense=1),
                inp["u0"], inp["p"], W.MSE_SAVE,
                np.abs(np.random.default_rng(14).standard_normal((4, 3, 3)))))
    return out


DCASES = _dense_cases()


def _fixed_mesh(N, T1, js, th):
    """Fixed-step mesh of N steps over [0, T1] with saves in steps js at
    fractions th (save index = step + 1)."""
    h = T1 / N
    return {"h": np.full((1, N), h), "n_steps": np.array([N], np.int32),
            "save_idx": (np.asarray(js) + 1)[None].astype(np.int32),
            "save_theta": np.asarray(th, dtype=np.float64)[None],
            "status": np.zeros(1, np.int32)}


# ---------------------------------------------------------------------------
# The interpolant
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("method", [W.TSIT5, W.DOPRI5])
@pytest.mark.parametrize("fused", [False, True])
def test_dense_hermite_remainder_on_linear_decay(orc, method, fused):
    """y' = p y on fixed meshes: the save error follows the Hermite remainder
    (fourth order, leading constant th^2 (1 - th)^2 p^4 e^{p t} / 24)."""
    p, T1 = -1.3, 2.0
    u0 = np.array([[1.0]])
    pp = np.array([[p]])
    for thv in (0.3, 0.5, 0.85):
        errs = []
        for N in (16, 32, 64):
            h = T1 / N
            js = np.array([N // 4, N // 2, 3 * N // 4])
            th = np.full(3, thv)
            ts = (js + th) * h
            prob = W.Problem(W.LINEAR, 1, 1, method, 0.0, T1, 1e-6, 1e-6, N,
                             save_times=tuple(ts), dense=1)
            ys, _ = orc.replay(prob, u0, pp, _fixed_mesh(N, T1, js, th), fused=fused)
            err = ys[0, :, 0] - np.exp(p * ts)
            errs.append(np.abs(err).max())
            if N == 64:
                pred = -(h**4) * thv**2 * (1 - thv) ** 2 * p**4 * np.exp(p * ts) / 24
                assert np.allclose(err / pred, 1.0, atol=0.06), (thv, err / pred)
        r = np.array(errs[:-1]) / np.array(errs[1:])
        assert np.all((r > 13.0) & (r < 17.5)), (method, thv, r)


@pytest.mark.parametrize("method", [W.TSIT5, W.DOPRI5])
def test_dense_gradient_converges_to_exact_derivative(orc, method):
    """d/dp of the interpolated saves tends to d/dp e^{p t} = t e^{p t}, and
    d/dy0 to e^{p t}, at fourth order."""
    p, T1 = -1.3, 2.0
    u0 = np.array([[1.0]])
    pp = np.array([[p]])
    eg, eu = [], []
    for N in (16, 32, 64):
        h = T1 / N
        js = np.array([N // 4, N // 2, 3 * N // 4])
        th = np.array([0.3, 0.5, 0.85])
        ts = (js + th) * h
        prob = W.Problem(W.LINEAR, 1, 1, method, 0.0, T1, 1e-6, 1e-6, N,
                         save_times=tuple(ts), dense=1)
        aux = np.ones((1, 3, 1))
        _, gu0, gp = orc.replay_grad(prob, u0, pp, _fixed_mesh(N, T1, js, th), W.COTANGENT,
                                     aux=aux)
        eg.append(abs(gp[0, 0] - (ts * np.exp(p * ts)).sum()))
        eu.append(abs(gu0[0, 0] - np.exp(p * ts).sum()))
    for e in (eg, eu):
        r = np.array(e[:-1]) / np.array(e[1:])
        assert np.all((r > 12.0) & (r < 17.5)), (method, r)


@pytest.mark.parametrize("fused", [False, True])
def test_dense_fraction_one_is_the_clipped_save(orc, fused):
    """On a clipping record's mesh (every save a mesh point, fraction 1), the
    dense replay gives the same saves bit for bit, and the same gradient up to
    rounding."""
    inp = W.make_inputs(3, 8)
    u0 = inp["u0"].astype(np.float64)
    p = inp["p"].astype(np.float64)
    prob = W.WORKLOADS[3].problem(t1=2.0, save_times=(0.5, 0.75, 1.3, 2.0))
    m = orc.record(prob, u0, p, fused=fused)
    assert np.all(m["status"] == 0)
    assert np.all(m["save_theta"] == 1.0)
    ys_clip, yN_clip = orc.replay(prob, u0, p, m, fused=fused)
    dprob = prob.replace(dense=1)
    ys_dense, yN_dense = orc.replay(dprob, u0, p, m, fused=fused)
    assert np.array_equal(ys_clip, ys_dense)
    assert np.array_equal(yN_clip, yN_dense)
    tg = np.random.default_rng(7).standard_normal((8, 4, 3))
    for lk in (W.MSE_SAVE, W.COTANGENT):
        lc, gc, pc = orc.replay_grad(prob, u0, p, m, lk, aux=tg, scale=0.3, fused=fused)
        ld, gd, pd = orc.replay_grad(dprob, u0, p, m, lk, aux=tg, scale=0.3, fused=fused)
        assert np.array_equal(lc, ld)
        assert np.allclose(gd, gc, rtol=1e-12, atol=1e-13 * np.abs(gc).max())
        assert np.allclose(pd, pc, rtol=1e-12, atol=1e-13 * np.abs(pc).max())


# ---------------------------------------------------------------------------
# The dense record
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", DCASES, ids=[c[0] for c in DCASES])
def test_dense_record_mesh_bookkeeping(orc, case):
    """Steps end only at t1; each save sits in the step its index names, at
    the fraction its time gives (t accumulated in double as the record does,
    the last step ending exactly at t1); the record's saves equal the dense
    replay's bit for bit."""
    name, prob, u0, p, lk, aux = case
    for fused in (False, True):
        m = orc.record(prob, u0, p, fused=fused)
        assert np.all(m["status"] == 0), name
        ys, _ = orc.replay(prob, u0, p, m, fused=fused)
        assert np.array_equal(ys, m["y_save"]), name
        clip = orc.record(prob.replace(dense=0), u0, p, fused=fused)
        assert np.all(m["n_steps"] <= clip["n_steps"]), name
        dt = u0.dtype.type
        for i in range(u0.shape[0]):
            N = int(m["n_steps"][i])
            h = m["h"][i]
            t_start = [prob.t0]
            for k in range(N - 1):
                t_start.append(t_start[-1] + float(h[k]))
            t_end = t_start[1:] + [prob.t1]
            for s, ts in enumerate(prob.save_times):
                k = int(m["save_idx"][i, s]) - 1
                assert 0 <= k < N, name
                assert t_start[k] < ts <= t_end[k], (name, i, s)
                if ts >= t_end[k]:
                    want = dt(1.0)
                else:
                    want = dt(min(1.0, (ts - t_start[k]) / float(h[k])))
                assert m["save_theta"][i, s] == want, (name, i, s)


def test_dense_saves_track_a_tight_reference(orc):
    """Lorenz-63 saves read from the interpolant at rtol = atol = 1e-8 agree
    with a clipping record at 1e-12 to the interpolant's accuracy."""
    inp = W.make_inputs(2, 16)
    saves = (0.31, 0.5, 0.77, 1.2, 1.5)
    dprob = W.WORKLOADS[2].problem(t1=1.5, save_times=saves, dense=1)
    ref = W.WORKLOADS[2].problem(t1=1.5, save_times=saves, rtol=1e-12, atol=1e-12,
                                 max_steps=65536)
    md = orc.record(dprob, inp["u0"], inp["p"])
    mr = orc.record(ref, inp["u0"], inp["p"], with_h=False)
    scale = np.abs(mr["y_save"]).max(axis=2, keepdims=True)
    err = np.abs(md["y_save"] - mr["y_save"]) / scale
    assert err.max() < 1e-5, err.max()


# ---------------------------------------------------------------------------
# The dense adjoint
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", DCASES, ids=[c[0] for c in DCASES])
@pytest.mark.parametrize("fused", [False, True])
def test_dense_adjoint_matches_dual_numbers(orc, case, fused):
    """<grad, v> equals the forward-mode derivative along v through the dense
    replay (dual numbers, plain rounding)."""
    name, prob, u0, p, lk, aux = case
    m = orc.record(prob, u0, p, fused=fused)
    loss, gu0, gp = orc.replay_grad(prob, u0, p, m, lk, aux=aux, scale=0.7, fused=fused)
    rng = np.random.default_rng(21)
    for _ in range(3):
        du0 = rng.standard_normal(u0.shape)
        dp = rng.standard_normal(p.shape) * p
        l2, dl, _, _ = orc.replay_jvp(prob, u0, p, du0, dp, m, lk, aux=aux, scale=0.7)
        assert np.allclose(l2, loss, rtol=1e-12), name
        adj = (gu0 * du0).sum(1) + (gp * dp).sum(1)
        assert np.allclose(adj, dl, rtol=1e-11, atol=1e-11 * np.abs(dl).max()), name


@pytest.mark.parametrize("case", DCASES, ids=[c[0] for c in DCASES])
def test_dense_adjoint_matches_finite_differences(orc, case):
    """Central differences of the dense replay's loss, mesh and fractions
    frozen."""
    name, prob, u0, p, lk, aux = case
    m = orc.record(prob, u0, p)
    loss, gu0, gp = orc.replay_grad(prob, u0, p, m, lk, aux=aux)
    for q in range(p.shape[1]):
        eps = 1e-6 * np.abs(p[:, q])
        pp = p.copy(); pp[:, q] += eps
        pm = p.copy(); pm[:, q] -= eps
        fd = (orc.replay_grad(prob, u0, pp, m, lk, aux=aux)[0] -
              orc.replay_grad(prob, u0, pm, m, lk, aux=aux)[0]) / (2 * eps)
        assert np.allclose(gp[:, q], fd, rtol=2e-5, atol=1e-6 * np.abs(fd).max()), (name, q)
    for c in range(min(u0.shape[1], 4)):
        eps = 1e-6 * max(1.0, float(np.abs(u0[:, c]).max()))
        up = u0.copy(); up[:, c] += eps
        um = u0.copy(); um[:, c] -= eps
        fd = (orc.replay_grad(prob, up, p, m, lk, aux=aux)[0] -
              orc.replay_grad(prob, um, p, m, lk, aux=aux)[0]) / (2 * eps)
        assert np.allclose(gu0[:, c], fd, rtol=2e-5, atol=1e-6 * np.abs(fd).max()), (name, c)


@pytest.mark.parametrize("case", DCASES[:2] + DCASES[3:], ids=[c[0] for c in DCASES[:2] + DCASES[3:]])
@pytest.mark.parametrize("fused", [False, True])
def test_dense_sensitivities_match_adjoint(orc, case, fused):
    """Forward sensitivities of the interpolated saves give the adjoint's
    gradient, and their loss is the adjoint's loss."""
    name, prob, u0, p, lk, aux = case
    m = orc.record(prob, u0, p, fused=fused)
    loss, gu0, gp = orc.replay_grad(prob, u0, p, m, lk, aux=aux, scale=0.4, fused=fused)
    sens, ls, su0, sp = orc.replay_sens(prob, u0, p, m, lk, aux=aux, scale=0.4, fused=fused)
    assert np.allclose(ls, loss, rtol=1e-13), name
    assert np.allclose(su0, gu0, rtol=1e-11, atol=1e-12 * np.abs(gu0).max()), name
    assert np.allclose(sp, gp, rtol=1e-11, atol=1e-12 * np.abs(gp).max()), name
    ys, _ = orc.replay(prob, u0, p, m, fused=fused)
    assert sens.shape == (u0.shape[0], prob.n_save_eff, prob.dim, prob.dim + prob.n_params)
    assert np.all(np.isfinite(sens)) and np.all(np.isfinite(ys))


def test_dense_needs_explicit_method(orc):
    prob = W.WORKLOADS[4].problem(t1=1.0, save_times=(0.5,), dense=1)
    inp = W.make_inputs(4, 2)
    with pytest.raises(ValueError):
        orc.record(prob, inp["u0"], inp["p"])
