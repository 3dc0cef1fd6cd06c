"""Right-hand sides compiled at run time (da_rhs_register) on the GPU, against
the oracle's source path (the same source built by g++ into a plugin and
differentiated by the oracle's own dual numbers).

Gates: on shared (oracle-recorded) meshes, losses, gradients, saved states
and sensitivities within 1e-12 relative per trajectory in FP64 (fused
oracle) and 1e-4 in FP32, norm-wise (the largest difference over the
vector's largest element): the device's and the host's exp, sin, pow and
the like differ in the last bits, and the derivatives come from tangent
passes on the GPU and Jacobian columns in the oracle, so the differences
scale with the vector rather than with each element; the same system written as source and built in
gives the same gradient to 1e-12; checkpoint intervals, the replay table and
dense output behave as for the built-in systems; the GPU record of a Kepler
orbit conserves its invariants."""
import numpy as np
import pytest

import workloads as W
from helpers import aux_to_dev, grad_rel_err, mesh_to_dev, mesh_to_host, rel_err, to_dev
from test_oracle_user_rhs import ALLFN, KEPLER, L63, _kepler_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def da():
    import discrete_adjoint_amd as da
    assert torch.cuda.is_available()
    return da


@pytest.fixture(scope="module")
def rhs(da):
    """Registered right-hand sides, by (name, dtype, method); released at the end."""
    ids = {}

    def get(name, dtype, method):
        key = (name, dtype, method)
        if key not in ids:
            src, dim, P = {"l63": (L63, 3, 3), "kepler": (KEPLER, 4, 1),
                           "allfn": (ALLFN, 3, 3)}[name]
            print(f"  registering {name} {dtype} method {method}", flush=True)
            ids[key] = da.register_rhs(src, dim, P, dtype, method)
        return ids[key]

    yield get
    for rid in ids.values():
        da.release_rhs(rid)


def _print(*a):
    print(*a, flush=True)


def _shared_mesh_case(da, orc, prob, src, dim, P, u0n, pn, lk, aux, scale, tol):
    orc.set_user_rhs(src, dim, P)
    m = orc.record(prob, u0n, pn, fused=True)
    assert np.all(m["status"] == 0)
    yo, _ = orc.replay(prob, u0n, pn, m, fused=True)
    lo, go, po = orc.replay_grad(prob, u0n, pn, m, lk, aux=aux, scale=scale, fused=True)
    mesh = mesh_to_dev(m, prob.max_steps, torch)
    u0, p = to_dev(u0n, torch), to_dev(pn, torch)
    auxd = None if aux is None else aux_to_dev(aux, torch)
    yg = da.replay_fwd(prob, u0, p, mesh)
    loss, gu0, gp = da.replay_grad(prob, u0, p, mesh, lk, aux=auxd, scale=scale)
    torch.cuda.synchronize()
    n = u0n.shape[0]
    ey = rel_err(yg.cpu().numpy().transpose(2, 0, 1).reshape(n, -1), yo.reshape(n, -1))
    eg = grad_rel_err(gu0.cpu().numpy().T, gp.cpu().numpy().T, go, po)
    el = np.abs(loss.cpu().numpy() - lo) / np.abs(lo)
    _print(f"  saves max rel {ey.max():.3e}, grad max rel {eg.max():.3e} "
           f"(bitwise lanes {np.mean(eg == 0):.3f}), loss {el.max():.3e}")
    assert ey.max() <= tol and eg.max() <= tol and el.max() <= tol
    return m, mesh, u0, p, auxd, (loss, gu0, gp)


@pytest.mark.parametrize("method", [W.TSIT5, W.DOPRI5])
def test_source_lorenz63_on_oracle_mesh(da, orc, rhs, method):
    """Lorenz-63 as source: GPU against the oracle's source path, and against
    the built-in Lorenz-63 of the GPU on the same mesh."""
    rid = rhs("l63", torch.float64, method)
    n = 1000
    inp = W.make_inputs(1, n)
    prob = W.WORKLOADS[1].problem(rhs=rid, method=method, save_times=(0.25, 0.6, 1.0))
    aux = np.random.default_rng(2).standard_normal((n, 3, 3))
    _print(f"case: source Lorenz-63, method {method}, n={n}")
    m, mesh, u0, p, auxd, (loss, gu0, gp) = _shared_mesh_case(
        da, orc, prob, L63, 3, 3, inp["u0"], inp["p"], W.MSE_SAVE, aux, 0.2, 1e-12)
    pb = prob.replace(rhs=W.LORENZ63)
    lb, gb, qb = da.replay_grad(pb, u0, p, mesh, W.MSE_SAVE, aux=auxd, scale=0.2)
    torch.cuda.synchronize()
    eb = grad_rel_err(gu0.cpu().numpy().T, gp.cpu().numpy().T, gb.cpu().numpy().T,
                      qb.cpu().numpy().T)
    _print(f"  source vs built-in gradient max rel {eb.max():.3e}")
    assert eb.max() <= 1e-12


def test_source_variants_checkpoints_table_dense_sens(da, orc, rhs):
    """A source right-hand side through every kernel variant: checkpoint
    intervals and the sorted replay table (bitwise equal gradients), dense
    output and forward sensitivities against the oracle."""
    rid = rhs("l63", torch.float64, W.DOPRI5)
    n = 700
    inp = W.make_inputs(2, n)
    prob = W.WORKLOADS[2].problem(rhs=rid, t1=1.5, save_times=(0.4, 0.9, 1.5))
    aux = np.random.default_rng(4).standard_normal((n, 3, 3))
    _print(f"case: source variants, n={n}")
    m, mesh, u0, p, auxd, (loss, gu0, gp) = _shared_mesh_case(
        da, orc, prob, L63, 3, 3, inp["u0"], inp["p"], W.COTANGENT, aux, 0.5, 1e-12)
    for ck in (2, 4, 8):
        _, g2, q2 = da.replay_grad(prob.replace(checkpoint=ck), u0, p, mesh, W.COTANGENT,
                                   aux=auxd, scale=0.5)
        torch.cuda.synchronize()
        assert torch.equal(g2, gu0) and torch.equal(q2, gp), ck
    sm = da.mesh_sort(prob, mesh)
    _, g3, q3 = da.replay_grad(prob, u0, p, sm, W.COTANGENT, aux=auxd, scale=0.5)
    torch.cuda.synchronize()
    assert torch.equal(g3, gu0) and torch.equal(q3, gp)
    # forward sensitivities
    so, lo, go, po = orc.replay_sens(prob, inp["u0"], inp["p"], m, W.COTANGENT, aux=aux,
                                     scale=0.5, fused=True)
    sg, lg, su0, sp = da.replay_sens(prob, u0, p, mesh, W.COTANGENT, aux=auxd, scale=0.5)
    torch.cuda.synchronize()
    es = rel_err(sg.cpu().numpy().transpose(3, 0, 1, 2).reshape(n, -1), so.reshape(n, -1))
    _print(f"  sensitivities max rel {es.max():.3e}")
    assert es.max() <= 1e-12
    # the parameter directions alone
    sq, lq, gq = da.replay_sens_dirs(prob, u0, p, mesh, 3, 3, W.COTANGENT, aux=auxd, scale=0.5)
    torch.cuda.synchronize()
    assert torch.equal(sq, sg[:, :, 3:]) and torch.equal(gq, sp) and torch.equal(lq, lg)
    # dense output
    dprob = prob.replace(dense=1, save_times=(0.33, 0.9, 1.21))
    md = orc.record(dprob, inp["u0"], inp["p"], fused=True)
    lo, go, po = orc.replay_grad(dprob, inp["u0"], inp["p"], md, W.COTANGENT, aux=aux, scale=0.5,
                                 fused=True)
    ld, gd, pd = da.replay_grad(dprob, u0, p, mesh_to_dev(md, prob.max_steps, torch),
                                W.COTANGENT, aux=auxd, scale=0.5)
    meshd, ysd = da.record(dprob, u0, p)
    yrd = da.replay_fwd(dprob, u0, p, meshd)
    torch.cuda.synchronize()
    ed = grad_rel_err(gd.cpu().numpy().T, pd.cpu().numpy().T, go, po)
    _print(f"  dense gradient max rel {ed.max():.3e}")
    assert ed.max() <= 1e-12
    assert torch.equal(ysd, yrd)


@pytest.mark.parametrize("method", [W.TSIT5, W.DOPRI5])
def test_source_kepler(da, orc, rhs, method):
    """Kepler orbits (sqrt and division in f): GPU gradient on the oracle's
    mesh, the GPU record against the oracle's, and the invariants of the GPU
    record after one revolution."""
    rid = rhs("kepler", torch.float64, method)
    n = 512
    u0n, pn = _kepler_inputs(n)
    prob = W.Problem(rid, 4, 1, method, 0.0, 2 * np.pi, 1e-10, 1e-10, 20000,
                     save_times=(1.0, 2.0, 2 * np.pi))
    aux = np.random.default_rng(6).standard_normal((n, 3, 4))
    _print(f"case: source Kepler, method {method}, n={n}")
    _shared_mesh_case(da, orc, prob, KEPLER, 4, 1, u0n, pn, W.MSE_SAVE, aux, 1.0 / n, 1e-12)
    u0, p = to_dev(u0n, torch), to_dev(pn, torch)
    mesh, ys = da.record(prob, u0, p)
    torch.cuda.synchronize()
    mg = mesh_to_host(mesh, prob.max_steps)
    mo = orc.record(prob, u0n, pn, fused=True)
    assert np.all(mg["status"] == 0)
    assert np.all(np.abs(mg["n_steps"] - mo["n_steps"]) <= np.maximum(2, 0.01 * mo["n_steps"]))
    yN = ys.cpu().numpy()[-1].T
    r0, r1 = np.hypot(u0n[:, 0], u0n[:, 1]), np.hypot(yN[:, 0], yN[:, 1])
    e0 = 0.5 * (u0n[:, 2] ** 2 + u0n[:, 3] ** 2) - pn[:, 0] / r0
    e1 = 0.5 * (yN[:, 2] ** 2 + yN[:, 3] ** 2) - pn[:, 0] / r1
    _print(f"  mean steps {mg['n_steps'].mean():.1f}, max |dE/E| {np.max(np.abs(e1 - e0) / np.abs(e0)):.2e}")
    assert np.all(np.abs(e1 - e0) < 1e-7 * np.abs(e0))


def test_source_every_function_fp64_and_fp32(da, orc, rhs):
    """The source that calls every allowed function, in both precisions."""
    n = 600
    rng = np.random.default_rng(10)
    u0n = 0.5 * rng.standard_normal((n, 3))
    pn = 1.0 + rng.random((n, 3))
    for dt, tol in ((np.float64, 1e-12), (np.float32, 1e-4)):
        tdt = torch.float64 if dt == np.float64 else torch.float32
        rid = rhs("allfn", tdt, W.TSIT5)
        prob = W.Problem(rid, 3, 3, W.TSIT5, 0.0, 2.0, 1e-6, 1e-6, 4096, save_times=(0.5, 2.0))
        aux = rng.standard_normal((n, 2, 3)).astype(dt)
        _print(f"case: source with every function, {dt.__name__}, n={n}")
        _shared_mesh_case(da, orc, prob, ALLFN, 3, 3, u0n.astype(dt), pn.astype(dt),
                          W.MSE_SAVE, aux, 0.1, tol)


def test_source_every_function_intervals_and_order(da, orc, rhs):
    """The source that calls every allowed function (a gradient kernel near the
    register limit) in FP64 at checkpoint intervals 1, 2, 4 and 8, on the
    oracle's mesh in trajectory order and in replay order, with the final-state
    loss and with losses at saves: every combination against the oracle."""
    n = 600
    rng = np.random.default_rng(10)
    u0n = 0.5 * rng.standard_normal((n, 3))
    pn = 1.0 + rng.random((n, 3))
    rid = rhs("allfn", torch.float64, W.TSIT5)
    orc.set_user_rhs(ALLFN, 3, 3)
    u0, p = to_dev(u0n, torch), to_dev(pn, torch)
    for lk, st in ((W.SUMSQ_FINAL, ()), (W.MSE_SAVE, (0.5, 2.0))):
        prob = W.Problem(rid, 3, 3, W.TSIT5, 0.0, 2.0, 1e-6, 1e-6, 4096, save_times=st)
        aux = rng.standard_normal((n, len(st), 3)) if st else None
        m = orc.record(prob, u0n, pn, fused=True)
        assert np.all(m["status"] == 0)
        lo, go, po = orc.replay_grad(prob, u0n, pn, m, lk, aux=aux, scale=0.1, fused=True)
        mesh = mesh_to_dev(m, prob.max_steps, torch)
        sm = da.mesh_sort(prob, mesh)
        auxd = None if aux is None else aux_to_dev(aux, torch)
        for ck in (1, 2, 4, 8):
            for order, me in (("trajectory", mesh), ("replay", sm)):
                _print(f"case: every function, loss {lk}, checkpoint {ck}, {order} order, n={n}")
                loss, gu0, gp = da.replay_grad(prob.replace(checkpoint=ck), u0, p, me, lk,
                                               aux=auxd, scale=0.1)
                torch.cuda.synchronize()
                eg = grad_rel_err(gu0.cpu().numpy().T, gp.cpu().numpy().T, go, po)
                el = np.abs(loss.cpu().numpy() - lo) / np.abs(lo)
                _print(f"  grad max rel {eg.max():.3e}, loss {el.max():.3e}")
                assert eg.max() <= 1e-12 and el.max() <= 1e-12


def test_registration_errors(da, rhs):
    """A source that does not compile reports the compiler's message; a
    problem that does not fit the registration is refused; a released
    identifier is unknown."""
    with pytest.raises(da.DadjError) as e:
        da.register_rhs("dy[0] = y[0] +;", 1, 1)
    assert e.value.code == -1 and "error" in str(e.value)
    rid = rhs("l63", torch.float64, W.TSIT5)
    u0 = torch.zeros(3, 4, dtype=torch.float64, device="cuda")
    p = torch.ones(3, 4, dtype=torch.float64, device="cuda")
    with pytest.raises(da.DadjError) as e:          # another method than registered
        da.record(W.Problem(rid, 3, 3, W.DOPRI5, 0.0, 1.0, 1e-6, 1e-6, 100), u0, p)
    assert e.value.code == -2
    tmp = da.register_rhs(L63, 3, 3, torch.float64, W.TSIT5)
    da.release_rhs(tmp)
    with pytest.raises(da.DadjError) as e:
        da.record(W.Problem(tmp, 3, 3, W.TSIT5, 0.0, 1.0, 1e-6, 1e-6, 100), u0, p)
    assert e.value.code == -1
    with pytest.raises(da.DadjError):
        da.release_rhs(tmp)
