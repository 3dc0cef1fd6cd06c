"""Dense output on the GPU (saves read from the cubic Hermite interpolant of
the accepted step that contains them) against the oracle's dense mode.

Gates as for the landing saves: on a shared (oracle-recorded) mesh, losses,
gradients and saved states within 1e-12 relative per trajectory in FP64
(fused-rounding oracle) and 1e-4 in FP32; checkpoint intervals and the
sorted replay table give bitwise identical gradients; the GPU record's saves
equal its replay's bit for bit, and its save fractions follow from its own
step sizes."""
import numpy as np
import pytest

import workloads as W
from helpers import (aux_to_dev, elem_err, grad_elem_err, grad_rel_err, mesh_to_dev,
                     mesh_to_host, mse_targets, to_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {np.float64: 1e-12, np.float32: 1e-4}


@pytest.fixture(scope="module")
def da():
    import discrete_adjoint_amd as da
    assert torch.cuda.is_available()
    return da


def _print(*a):
    print(*a, flush=True)


# (name, workload, problem changes, loss, lanes)
CASES = [
    ("l63_dopri5_cot", 2, dict(t1=2.0, save_times=(0.31, 0.5, 0.77, 1.2, 1.9)), W.COTANGENT, 1000),
    ("l63_tsit5_mse_f64", 1, dict(save_times=tuple(0.1 * s for s in range(1, 11))), W.MSE_SAVE,
     1024),
    ("l63_tsit5_mse_f32", 3, dict(), W.MSE_SAVE, 1500),
    ("robertson_tsit5_mse", 4, dict(t1=0.3, method=W.TSIT5, max_steps=8192,
                                    save_times=(0.01, 0.1, 0.25)), W.MSE_SAVE, 300),
    ("linear_dopri5_cot", None, dict(), W.COTANGENT, 700),
    # many saves per step: 40 save times inside [0.5, 0.52] and one at t1
    ("l63_tsit5_crowded", 1, dict(save_times=tuple(np.linspace(0.5, 0.52, 40)) + (1.0,)),
     W.COTANGENT, 260),
    # Lorenz-96 on the wavefront kernels: d = 64 (DPP neighbours) and d = 40
    ("l96_tsit5_cot", 5, dict(t1=0.5, save_times=(0.1, 0.23, 0.4)), W.COTANGENT, 200),
    ("l96_d40_dopri5_mse", 5, dict(dim=40, method=W.DOPRI5, t1=0.5,
                                   save_times=(0.05, 0.3, 0.5)), W.MSE_SAVE, 150),
]


def _case(orc, wid, kw, lk, n):
    if wid is None:
        prob = W.Problem(W.LINEAR, 1, 1, W.DOPRI5, 0.0, 3.0, 1e-7, 1e-7, 512,
                         save_times=(0.2, 1.0, 2.5, 3.0), dense=1)
        rng = np.random.default_rng(8)
        u0 = 1.0 + rng.random((n, 1))
        p = -0.2 - rng.random((n, 1))
        dt = np.float64
    else:
        w = W.WORKLOADS[wid]
        prob = w.problem(dense=1, **kw)
        inp = W.make_inputs(wid, n)
        u0, p = np.ascontiguousarray(inp["u0"][:, :prob.dim]), inp["p"]
        dt = w.np_dtype
    S, d = prob.n_save_eff, prob.dim
    if lk == W.MSE_SAVE and wid == 3:
        aux, st = mse_targets(orc, 3, n, W.make_inputs(3, n))
        scale = 1.0 / (n * S * d)
    else:
        aux = np.random.default_rng(9).standard_normal((n, S, d)).astype(dt)
        scale = 0.5
    return prob, u0, p, aux, scale, dt


@pytest.mark.parametrize("name,wid,kw,lk,n", CASES, ids=[c[0] for c in CASES])
def test_dense_on_oracle_mesh(da, orc, name, wid, kw, lk, n):
    """Shared mesh: saves, loss and gradient of the GPU dense replay against
    the oracle's; every checkpoint interval and the sorted replay table give
    the same gradient bit for bit."""
    prob, u0n, pn, aux, scale, dt = _case(orc, wid, kw, lk, n)
    _print(f"case: dense on oracle mesh, {name}, n={n}")
    m = orc.record(prob, u0n, pn, fused=True)
    assert np.all(m["status"] == 0)
    yo, _ = orc.replay(prob, u0n, pn, m, fused=True)
    lo, go, po = orc.replay_grad(prob, u0n, pn, m, lk, aux=aux, scale=scale, fused=True)
    mesh = mesh_to_dev(m, prob.max_steps, torch)
    u0, p = to_dev(u0n, torch), to_dev(pn, torch)
    auxd = aux_to_dev(aux, torch)
    yg = da.replay_fwd(prob, u0, p, mesh)
    loss, gu0, gp = da.replay_grad(prob, u0, p, mesh, lk, aux=auxd, scale=scale)
    torch.cuda.synchronize()
    tol = TOL[dt]
    ygn = yg.cpu().numpy().transpose(2, 0, 1)             # [n, S, d]
    ey = elem_err(ygn.reshape(n, -1), yo.reshape(n, -1))
    eg = grad_elem_err(gu0.cpu().numpy().T, gp.cpu().numpy().T, go, po)
    el = np.abs(loss.cpu().numpy() - lo) / np.abs(lo)
    _print(f"  element-wise: saves max rel {ey.max():.3e} (bitwise lanes {np.mean(ey == 0):.3f}), "
           f"grad max rel {eg.max():.3e}, loss max rel {el.max():.3e}")
    assert ey.max() <= tol and eg.max() <= tol
    if prob.rhs == W.LORENZ96:
        # the wavefront adds the loss over components pairwise, the oracle in
        # sequence: both within 4 d eps of the sum of |terms|
        mag = scale * (np.abs(yo * aux).sum((1, 2)) if lk == W.COTANGENT
                       else ((yo - aux) ** 2).sum((1, 2)))
        assert np.all(np.abs(loss.cpu().numpy() - lo) <= 4 * prob.dim * 2.3e-16 * mag)
    else:
        assert el.max() <= tol
    ref = (gu0.clone(), gp.clone())
    for ck in (2, 4, 8):
        l2, g2, q2 = da.replay_grad(prob.replace(checkpoint=ck), u0, p, mesh, lk, aux=auxd,
                                    scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(g2, ref[0]) and torch.equal(q2, ref[1]), ck
    sm = da.mesh_sort(prob, mesh)
    l3, g3, q3 = da.replay_grad(prob, u0, p, sm, lk, aux=auxd, scale=scale)
    y3 = da.replay_fwd(prob, u0, p, sm)
    torch.cuda.synchronize()
    assert torch.equal(g3, ref[0]) and torch.equal(q3, ref[1])
    assert torch.equal(y3, yg)


@pytest.mark.parametrize("name,wid,kw,lk,n", CASES, ids=[c[0] for c in CASES])
def test_dense_gpu_record(da, orc, name, wid, kw, lk, n):
    """GPU dense record: steps end only at t1, the save fractions follow from
    the GPU's own step sizes (t accumulated in double, the last step ending at
    t1), the recorded saves equal the GPU replay's and the forward solve's bit
    for bit, every accepted step passes the oracle's error test, and the step
    counts agree with the oracle's dense record."""
    prob, u0n, pn, aux, scale, dt = _case(orc, wid, kw, lk, n)
    _print(f"case: dense GPU record, {name}, n={n}")
    u0, p = to_dev(u0n, torch), to_dev(pn, torch)
    mesh, ys = da.record(prob, u0, p)
    yr = da.replay_fwd(prob, u0, p, mesh)
    yf, nsf, stf = da.solve_fwd(prob, u0, p)
    torch.cuda.synchronize()
    assert torch.equal(ys, yr)
    assert torch.equal(ys, yf)
    mg = mesh_to_host(mesh, prob.max_steps)
    assert np.all(mg["status"] == 0)
    assert np.array_equal(nsf.cpu().numpy(), mg["n_steps"])
    mo = orc.record(prob, u0n, pn, fused=True)
    ng, no = mg["n_steps"], mo["n_steps"]
    _print(f"  max |dN| {np.abs(ng - no).max()}, mean steps {ng.mean():.1f}")
    assert np.all(np.abs(ng - no) <= np.maximum(8, 0.1 * no))
    E = orc.mesh_max_err(prob, u0n, pn, mg, fused=True)
    assert np.all(E <= 1 + 1e-6), E.max()
    for i in range(0, n, max(1, n // 40)):
        N = int(ng[i])
        h = mg["h"][i]
        t_start = [prob.t0]
        for k in range(N - 1):
            t_start.append(t_start[-1] + float(h[k]))
        t_end = t_start[1:] + [prob.t1]
        for s, ts in enumerate(prob.save_times):
            k = int(mg["save_idx"][i, s]) - 1
            assert 0 <= k < N and t_start[k] < ts <= t_end[k], (i, s)
            want = 1.0 if ts >= t_end[k] else min(1.0, (ts - t_start[k]) / float(h[k]))
            assert mg["save_theta"][i, s] == dt(want), (i, s)
    # lanes whose mesh equals the oracle's bit for bit also share the saves
    same = np.array([ng[i] == no[i] and np.array_equal(mg["h"][i, :ng[i]], mo["h"][i, :no[i]])
                     for i in range(n)])
    _print(f"  bitwise-equal meshes {same.mean():.3f}")
    if same.any():
        assert np.array_equal(mg["save_idx"][same], mo["save_idx"][same])
        assert np.array_equal(mg["save_theta"][same], mo["save_theta"][same])
        ysn = ys.cpu().numpy().transpose(2, 0, 1)
        e = elem_err(ysn[same].reshape(same.sum(), -1), mo["y_save"][same].reshape(same.sum(), -1))
        assert e.max() <= TOL[dt]


@pytest.mark.parametrize("fused_record", [True])
def test_dense_fraction_one_on_a_landing_mesh(da, orc, fused_record):
    """A landing record's mesh (fraction 1 at every save) replayed with dense
    output gives the landing saves bit for bit and the landing gradient to
    rounding."""
    w = W.WORKLOADS[1]
    prob = w.problem(save_times=(0.2, 0.45, 0.7, 1.0))
    n = 600
    inp = W.make_inputs(1, n)
    u0, p = to_dev(inp["u0"], torch), to_dev(inp["p"], torch)
    _print(f"case: dense fraction one, n={n}")
    mesh, ys = da.record(prob, u0, p)
    torch.cuda.synchronize()
    assert torch.all(mesh.save_theta == 1)
    dprob = prob.replace(dense=1)
    yd = da.replay_fwd(dprob, u0, p, mesh)
    aux = aux_to_dev(np.random.default_rng(2).standard_normal((n, 4, 3)), torch)
    lc, gc, pc = da.replay_grad(prob, u0, p, mesh, W.MSE_SAVE, aux=aux, scale=0.3)
    ld, gd, pd = da.replay_grad(dprob, u0, p, mesh, W.MSE_SAVE, aux=aux, scale=0.3)
    torch.cuda.synchronize()
    assert torch.equal(yd, ys)
    assert torch.equal(ld, lc)
    e = grad_rel_err(gd.cpu().numpy().T, pd.cpu().numpy().T, gc.cpu().numpy().T,
                     pc.cpu().numpy().T)
    _print(f"  dense vs landing gradient max rel {e.max():.3e}")
    assert e.max() <= 1e-12


SENS_CASES = [c for c in CASES if c[0] in ("l63_dopri5_cot", "l63_tsit5_mse_f64",
                                           "robertson_tsit5_mse", "l63_tsit5_crowded")]


@pytest.mark.parametrize("name,wid,kw,lk,n", SENS_CASES, ids=[c[0] for c in SENS_CASES])
def test_dense_sensitivities(da, orc, name, wid, kw, lk, n):
    """Forward sensitivities of the interpolated saves against the oracle's,
    and their gradient against the GPU reverse sweep."""
    prob, u0n, pn, aux, scale, dt = _case(orc, wid, kw, lk, n)
    n = min(n, 400)
    u0n, pn, aux = u0n[:n], pn[:n], aux[:n]
    _print(f"case: dense sensitivities, {name}, n={n}")
    m = orc.record(prob, u0n, pn, fused=True)
    so, lo, go, po = orc.replay_sens(prob, u0n, pn, m, lk, aux=aux, scale=scale, fused=True)
    mesh = mesh_to_dev(m, prob.max_steps, torch)
    u0, p = to_dev(u0n, torch), to_dev(pn, torch)
    auxd = aux_to_dev(aux, torch)
    sg, lg, gu0, gp = da.replay_sens(prob, u0, p, mesh, lk, aux=auxd, scale=scale)
    la, ga, pa = da.replay_grad(prob, u0, p, mesh, lk, aux=auxd, scale=scale)
    torch.cuda.synchronize()
    sgn = sg.cpu().numpy().transpose(3, 0, 1, 2)
    es = elem_err(sgn.reshape(n, -1), so.reshape(n, -1))
    eg = grad_elem_err(gu0.cpu().numpy().T, gp.cpu().numpy().T, go, po)
    ea = grad_rel_err(gu0.cpu().numpy().T, gp.cpu().numpy().T, ga.cpu().numpy().T,
                      pa.cpu().numpy().T)
    _print(f"  sens max rel {es.max():.3e}, grad {eg.max():.3e}, forward vs reverse {ea.max():.3e}")
    assert es.max() <= 1e-12 and eg.max() <= 1e-12
    assert ea.max() <= 1e-9


def test_dense_full_size_fp32_sampled(da, orc):
    """The calibration workload (2^16 trajectories, FP32, MSE at 10 save
    times) with dense output: GPU record and gradient at full size, sampled
    trajectories against the FP32 oracle on the GPU's own mesh."""
    w = W.WORKLOADS[3]
    prob = w.problem(dense=1)
    n = w.n
    inp = W.make_inputs(3, n)
    aux, st = mse_targets(orc, 3, n, inp)
    scale = 1.0 / (n * w.n_save_eff * w.dim)
    _print(f"case: dense full size FP32, n={n}")
    u0, p = to_dev(inp["u0"], torch), to_dev(inp["p"], torch)
    mesh, ys = da.record(prob, u0, p)
    sm = da.mesh_sort(prob, mesh)
    loss, gu0, gp = da.replay_grad(prob, u0, p, sm, W.MSE_SAVE, aux=aux_to_dev(aux, torch),
                                   scale=scale)
    torch.cuda.synchronize()
    mg = mesh_to_host(mesh, prob.max_steps)
    assert np.all(mg["status"] == 0)
    idx = np.random.default_rng(4).choice(n, 512, replace=False)
    sub = {k: v[idx] for k, v in mg.items()}
    lo, go, po = orc.replay_grad(prob, inp["u0"][idx], inp["p"][idx], sub, W.MSE_SAVE,
                                 aux=aux[idx], scale=scale, fused=True)
    eg = grad_elem_err(gu0.cpu().numpy().T[idx], gp.cpu().numpy().T[idx], go, po)
    el = np.abs(loss.cpu().numpy()[idx] - lo) / np.abs(lo)
    _print(f"  sampled grad element-wise max rel {eg.max():.3e}, loss {el.max():.3e}; "
           f"mean steps {mg['n_steps'].mean():.1f}")
    assert eg.max() <= 1e-4 and el.max() <= 1e-4
