"""Cyclic-stencil right-hand sides compiled at run time for the wavefront
kernels (da_rhs_register_stencil), against the oracle's source path for the
same stencil (the source built by g++ into a plugin whose f is the vector of
the components, differentiated by the oracle's own dual numbers).

Gates: on shared (oracle-recorded) meshes, saved states, losses, gradients
and sensitivities within 1e-12 relative per trajectory in FP64 (fused
oracle) and 1e-4 in FP32, norm-wise (the largest difference over the
vector's largest element): the two sides take the derivatives by different
routes (the GPU from one tangent per stencil offset, the oracle from its
Jacobian columns), so their rounding differences scale with the vector and
an element-wise gate would measure the route, not the kernel; Lorenz-96 written as a stencil gives the built-in
Lorenz-96's gradient to 1e-12 on the same mesh; a GPU-recorded mesh is
within the step-count gate of the oracle's; checkpoint intervals and the
replay table give bitwise equal gradients."""
import numpy as np
import pytest

import workloads as W
from helpers import aux_to_dev, grad_rel_err, mesh_to_dev, mesh_to_host, rel_err, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# Lorenz-96 as a stencil: x_i' = (x_{i+1} - x_{i-2}) x_{i-1} - x_i + F
L96S = "return (y(1) - y(-2)) * y(-1) - y(0) + p[0];"
L96S_OFF = (-2, -1, 0, 1)
# diffusion, centred advection and tanh damping, two parameters
DIFF = ("const T lap = y(1) - T(2) * y(0) + y(-1);\n"
        "return p[0] * lap - p[1] * tanh(y(0)) + T(0.5) * (y(2) - y(-2));")
DIFF_OFF = (-2, -1, 0, 1, 2)


@pytest.fixture(scope="module")
def da():
    import discrete_adjoint_amd as da
    assert torch.cuda.is_available()
    return da


@pytest.fixture(scope="module")
def stencil(da):
    """Registered stencils by (name, dim, dtype, method); released at the end."""
    ids = {}

    def get(name, dim, dtype, method):
        key = (name, dim, dtype, method)
        if key not in ids:
            src, P, off = {"l96": (L96S, 1, L96S_OFF), "diff": (DIFF, 2, DIFF_OFF)}[name]
            print(f"  registering stencil {name} d={dim} {dtype} method {method}", flush=True)
            ids[key] = da.register_rhs_stencil(src, dim, P, off, dtype, method)
        return ids[key]

    yield get
    for rid in ids.values():
        da.release_rhs(rid)


def _print(*a):
    print(*a, flush=True)


def _diff_inputs(n, dim, dt=np.float64, seed=3):
    rng = np.random.default_rng(seed)
    u0 = rng.standard_normal((n, dim)).astype(dt)
    p = np.stack([1.0 + rng.random(n), 0.5 + 0.5 * rng.random(n)], axis=1).astype(dt)
    return u0, p


def _shared_mesh(da, orc, prob, src, dim, P, off, u0n, pn, lk, aux, scale, tol, sens=False):
    orc.set_user_stencil(src, dim, P, off)
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
    _print(f"  saves max rel {ey.max():.3e} (bitwise lanes {np.mean(ey == 0):.3f}), "
           f"grad max rel {eg.max():.3e}, loss {el.max():.3e}")
    assert ey.max() <= tol and eg.max() <= tol and el.max() <= tol
    if sens:
        so, lso, gso, pso = orc.replay_sens(prob, u0n, pn, m, lk, aux=aux, scale=scale,
                                            fused=True)
        sg, lg, su0, sp = da.replay_sens(prob, u0, p, mesh, lk, aux=auxd, scale=scale)
        torch.cuda.synchronize()
        es = rel_err(sg.cpu().numpy().transpose(3, 0, 1, 2).reshape(n, -1), so.reshape(n, -1))
        esg = grad_rel_err(su0.cpu().numpy().T, sp.cpu().numpy().T, gso, pso)
        _print(f"  sensitivities max rel {es.max():.3e}, their gradient {esg.max():.3e}")
        assert es.max() <= tol and esg.max() <= tol
        sq, lq, gq = da.replay_sens_dirs(prob, u0, p, mesh, dim, P, lk, aux=auxd, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(sq, sg[:, :, dim:]) and torch.equal(gq, sp)
    return m, mesh, u0, p, auxd, (loss, gu0, gp)


@pytest.mark.parametrize("dim,n,method", [(64, 64, W.TSIT5), (17, 200, W.TSIT5),
                                          (64, 48, W.DOPRI5)])
def test_stencil_lorenz96(da, orc, stencil, dim, n, method):
    """Lorenz-96 as a stencil: GPU against the oracle's stencil path (saves,
    loss, gradient, sensitivities), against the GPU's built-in Lorenz-96 on
    the same mesh, and the GPU record against the oracle's."""
    rid = stencil("l96", dim, torch.float64, method)
    inp = W.make_inputs(5, n)
    u0n = np.ascontiguousarray(inp["u0"][:, :dim])
    pn = inp["p"]
    prob = W.WORKLOADS[5].problem(rhs=rid, dim=dim, method=method, t1=1.0)
    _print(f"case: stencil Lorenz-96, d={dim}, n={n}, method {method}")
    m, mesh, u0, p, auxd, (loss, gu0, gp) = _shared_mesh(
        da, orc, prob, L96S, dim, 1, L96S_OFF, u0n, pn, W.SUMSQ_FINAL, None, 1.0, 1e-12,
        sens=dim != 64 or method == W.TSIT5)
    pb = prob.replace(rhs=W.LORENZ96)
    lb, gb, qb = da.replay_grad(pb, u0, p, mesh, W.SUMSQ_FINAL)
    torch.cuda.synchronize()
    eb = grad_rel_err(gu0.cpu().numpy().T, gp.cpu().numpy().T, gb.cpu().numpy().T,
                      qb.cpu().numpy().T)
    _print(f"  stencil vs built-in gradient max rel {eb.max():.3e}")
    assert eb.max() <= 1e-12
    mg, ys = da.record(prob, u0, p)
    yr = da.replay_fwd(prob, u0, p, mg)
    torch.cuda.synchronize()
    mh = mesh_to_host(mg, prob.max_steps)
    assert np.all(mh["status"] == 0)
    assert np.all(np.abs(mh["n_steps"] - m["n_steps"]) <= np.maximum(2, 0.01 * m["n_steps"]))
    assert torch.equal(ys, yr)


def test_stencil_two_parameters_fp64_fp32_dense(da, orc, stencil):
    """A two-parameter stencil with five offsets and tanh, d = 40: MSE loss at
    save times in FP64 and FP32, then with dense output (FP64)."""
    n, dim = 300, 40
    rng = np.random.default_rng(12)
    for dt, tol in ((np.float64, 1e-12), (np.float32, 1e-4)):
        tdt = torch.float64 if dt == np.float64 else torch.float32
        rid = stencil("diff", dim, tdt, W.TSIT5)
        u0n, pn = _diff_inputs(n, dim, dt)
        prob = W.Problem(rid, dim, 2, W.TSIT5, 0.0, 1.0, 1e-6, 1e-6, 4096,
                         save_times=(0.3, 0.7, 1.0))
        aux = rng.standard_normal((n, 3, dim)).astype(dt)
        _print(f"case: two-parameter stencil, {dt.__name__}, n={n}")
        _shared_mesh(da, orc, prob, DIFF, dim, 2, DIFF_OFF, u0n, pn, W.MSE_SAVE, aux,
                     1.0 / (n * 3 * dim), tol, sens=True)
    rid = stencil("diff", dim, torch.float64, W.TSIT5)
    u0n, pn = _diff_inputs(n, dim)
    dprob = W.Problem(rid, dim, 2, W.TSIT5, 0.0, 1.0, 1e-6, 1e-6, 4096,
                      save_times=(0.33, 0.71, 0.9), dense=1)
    aux = rng.standard_normal((n, 3, dim))
    _print(f"case: two-parameter stencil, dense output, n={n}")
    _shared_mesh(da, orc, dprob, DIFF, dim, 2, DIFF_OFF, u0n, pn, W.MSE_SAVE, aux,
                 1.0 / (n * 3 * dim), 1e-12, sens=True)


def test_stencil_checkpoints_and_table(da, orc, stencil):
    """Checkpoint intervals and the sorted replay table give bitwise equal
    gradients for a registered stencil."""
    n, dim = 500, 64
    rid = stencil("diff", dim, torch.float64, W.TSIT5)
    u0n, pn = _diff_inputs(n, dim, seed=5)
    prob = W.Problem(rid, dim, 2, W.TSIT5, 0.0, 0.8, 1e-7, 1e-7, 4096)
    u0, p = to_dev(u0n, torch), to_dev(pn, torch)
    _print(f"case: stencil checkpoints and table, n={n}")
    mesh, _ = da.record(prob, u0, p)
    l1, g1, q1 = da.replay_grad(prob, u0, p, mesh, W.SUMSQ_FINAL)
    torch.cuda.synchronize()
    assert torch.isfinite(g1).all() and torch.isfinite(q1).all()
    for ck in (2, 4, 8):
        _, g2, q2 = da.replay_grad(prob.replace(checkpoint=ck), u0, p, mesh, W.SUMSQ_FINAL)
        torch.cuda.synchronize()
        assert torch.equal(g2, g1) and torch.equal(q2, q1), ck
    sm = da.mesh_sort(prob, mesh)
    _, g3, q3 = da.replay_grad(prob, u0, p, sm, W.SUMSQ_FINAL)
    torch.cuda.synchronize()
    assert torch.equal(g3, g1) and torch.equal(q3, q1)


def test_stencil_registration_checks(da, stencil):
    """Offsets outside [-3, 3] or repeated, and a dimension above 64, are
    refused before compiling; a source that does not compile reports the
    compiler's message; a problem of another shape is refused."""
    for off, dim in (((-4, 0), 32), ((1, 1), 32), ((0,), 65), ((), 32)):
        with pytest.raises(da.DadjError) as e:
            da.register_rhs_stencil(L96S, dim, 1, off)
        assert e.value.code == -1
    with pytest.raises(da.DadjError) as e:
        da.register_rhs_stencil("return y(0) +;", 32, 1, (0,))
    assert e.value.code == -1 and "error" in str(e.value)
    rid = stencil("l96", 17, torch.float64, W.TSIT5)
    u0 = torch.zeros(18, 4, dtype=torch.float64, device="cuda")
    p = torch.ones(1, 4, dtype=torch.float64, device="cuda")
    with pytest.raises(da.DadjError) as e:
        da.record(W.Problem(rid, 18, 1, W.TSIT5, 0.0, 1.0, 1e-6, 1e-6, 100), u0, p)
    assert e.value.code == -1
