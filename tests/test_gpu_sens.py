"""Forward-mode sensitivities on the GPU (da_replay_sens) against the oracle.

The oracle's fused mode evaluates the tangents with the same written fma
schedule; gates: sensitivities, loss and gradients within 1e-12 relative per
trajectory (FP64) on shared meshes; the forward-mode gradient agrees with the
reverse sweep's (a different evaluation of the same derivative) to 1e-10 on
short horizons."""
import numpy as np
import pytest

import workloads as W
from helpers import aux_to_dev, elem_err, grad_elem_err, grad_rel_err, mesh_to_dev, rel_err, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def da():
    import discrete_adjoint_amd as da
    assert torch.cuda.is_available()
    return da


def _print(*a):
    print(*a, flush=True)


def _sens_err(sg, so):
    """Per-trajectory max |difference| / max |reference| over all entries
    (norm-wise; used against the FP64 oracle in FP32)."""
    n = so.shape[0]
    a = sg.reshape(n, -1)
    b = so.reshape(n, -1)
    ok = np.isfinite(b)
    num = np.max(np.where(ok, np.abs(a - b), 0), axis=1)
    den = np.maximum(np.max(np.where(ok, np.abs(b), 0), axis=1), 1e-300)
    return num / den


def _sens_elem_err(sg, so):
    """Per-trajectory max over the entries of |difference| / |reference|,
    entry by entry (an exactly zero reference entry must be exactly zero);
    entries where the reference is not finite are skipped."""
    n = so.shape[0]
    a = sg.reshape(n, -1).astype(np.float64)
    b = so.reshape(n, -1).astype(np.float64)
    ok = np.isfinite(b)
    return elem_err(np.where(ok, a, 0.0), np.where(ok, b, 0.0))


CASES = [
    ("lorenz63_tsit5", 1, dict(), W.SUMSQ_FINAL, 700),
    ("lorenz63_dopri5_short", 2, dict(t1=1.5), W.SUMSQ_FINAL, 500),
    ("lorenz63_dopri5_saves_cot", 2, dict(t1=2.0, save_times=(0.4, 1.1, 2.0)), W.COTANGENT, 400),
    ("lorenz63_tsit5_saves_mse", 1, dict(save_times=(0.25, 0.5, 0.75)), W.MSE_SAVE, 300),
    ("robertson_tsit5", 4, dict(t1=0.3, method=W.TSIT5, max_steps=8192), W.SUMSQ_FINAL, 130),
    ("robertson_ros2", 4, dict(t1=100.0), W.SUMSQ_FINAL, 300),
    ("robertson_ros2_saves_mse", 4, dict(t1=1e3, save_times=(1.0, 10.0, 1e3)), W.MSE_SAVE, 200),
    ("lorenz63_ros2_saves_cot", 1, dict(method=W.ROS2, rtol=1e-4, atol=1e-4, max_steps=2048,
                                        save_times=(0.3, 0.7, 1.0)), W.COTANGENT, 300),
]


@pytest.mark.parametrize("name,wid,kw,lk,n", CASES, ids=[c[0] for c in CASES])
def test_sensitivities_on_oracle_mesh(da, orc, name, wid, kw, lk, n):
    w = W.WORKLOADS[wid]
    prob = w.problem(**kw)
    inp = W.make_inputs(wid, n)
    u0n = inp["u0"].astype(np.float64)
    pn = inp["p"].astype(np.float64)
    _print(f"case: sensitivities {name}, n={n}")
    m = orc.record(prob, u0n, pn, fused=True)
    assert np.all(m["status"] == 0)
    S = prob.n_save_eff
    aux = None if lk == W.SUMSQ_FINAL else np.random.default_rng(3).standard_normal((n, S, 3))
    so, lo, go, po = orc.replay_sens(prob, u0n, pn, m, lk, aux=aux, scale=0.7, fused=True)
    mesh = mesh_to_dev(m, prob.max_steps, torch)
    u0, p = to_dev(u0n, torch), to_dev(pn, torch)
    sg, lg, gu0, gp = da.replay_sens(prob, u0, p, mesh, lk,
                                     aux=None if aux is None else aux_to_dev(aux, torch),
                                     scale=0.7)
    torch.cuda.synchronize()
    sgn = sg.cpu().numpy().transpose(3, 0, 1, 2)          # [n, S, d, Q]
    es = _sens_elem_err(sgn, so)
    eg = grad_elem_err(gu0.cpu().numpy().T, gp.cpu().numpy().T, go, po)
    el = np.abs(lg.cpu().numpy() - lo) / np.abs(lo)
    _print(f"  sens max rel {es.max():.3e}, grad max rel {eg.max():.3e}, "
           f"bitwise sens lanes {np.mean(es == 0):.3f}")
    assert es.max() <= 1e-12 and eg.max() <= 1e-12 and el.max() <= 1e-12
    # forward and reverse mode give the same gradient
    la, ga, pa = da.replay_grad(prob, u0, p, mesh, lk,
                                aux=None if aux is None else aux_to_dev(aux, torch), scale=0.7)
    torch.cuda.synchronize()
    ea = grad_rel_err(gu0.cpu().numpy().T, gp.cpu().numpy().T, ga.cpu().numpy().T,
                      pa.cpu().numpy().T)
    _print(f"  forward vs reverse mode: max rel {ea.max():.3e}")
    assert ea.max() <= 1e-10


def test_sensitivity_options_and_errors(da, orc):
    """Sensitivities alone (no loss), a replay order with its table, and
    failed trajectories."""
    w = W.WORKLOADS[1]
    prob = w.problem(max_steps=45)
    n = 300
    inp = W.make_inputs(1, n)
    inp["p"][7, 1] = np.nan
    _print("case: sensitivity options, n=300")
    u0, p = to_dev(inp["u0"], torch), to_dev(inp["p"], torch)
    mesh, _ = da.record(prob, u0, p)
    sm = da.mesh_sort(prob, mesh)
    s1, l1, g1, q1 = da.replay_sens(prob, u0, p, mesh)
    s2, l2, g2, q2 = da.replay_sens(prob, u0, p, sm)
    s3, _, _, _ = da.replay_sens(prob, u0, p, sm, loss_kind=None)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(s1), torch.nan_to_num(s2))
    assert torch.equal(torch.nan_to_num(s1), torch.nan_to_num(s3))
    assert torch.equal(torch.nan_to_num(g1), torch.nan_to_num(g2))
    st = mesh.status.cpu().numpy()
    bad = st != 0
    assert bad[7] and bad.sum() >= 1
    assert np.all(np.isnan(q1.cpu().numpy()[:, bad]))
    assert np.all(np.isnan(s1.cpu().numpy()[..., bad]))
    assert not np.any(np.isnan(q1.cpu().numpy()[:, ~bad]))


L96_CASES = [
    # d = 64: neighbours by DPP rotations; 17 direction groups, the last one
    # holding only the F direction
    ("d64_tsit5_final", 64, W.TSIT5, W.SUMSQ_FINAL, dict(), 48),
    ("d64_tsit5_cot_dense", 64, W.TSIT5, W.COTANGENT,
     dict(dense=1, save_times=(0.13, 0.5, 0.77)), 32),
    # d < 64: neighbours by cross-lane reads; d = 17 leaves a partly used group
    ("d40_dopri5_mse", 40, W.DOPRI5, W.MSE_SAVE, dict(save_times=(0.25, 0.5, 1.0)), 40),
    ("d17_tsit5_cot", 17, W.TSIT5, W.COTANGENT, dict(save_times=(0.1, 0.6, 1.0)), 64),
]


@pytest.mark.parametrize("name,dim,method,lk,kw,n", L96_CASES, ids=[c[0] for c in L96_CASES])
def test_l96_sensitivities_on_oracle_mesh(da, orc, name, dim, method, lk, kw, n):
    """Lorenz-96 on the wavefront kernel (one trajectory per wavefront, four
    directions per lane): sensitivities, loss and gradient against the
    oracle's fused mode on its mesh, and the gradient against the reverse
    sweep."""
    inp = W.make_inputs(5, n)
    u0n = np.ascontiguousarray(inp["u0"][:, :dim])
    pn = inp["p"]
    prob = W.Problem(W.LORENZ96, dim, 1, method, 0.0, 1.0, 1e-7, 1e-7, 4096)
    prob = prob.replace(**kw)
    _print(f"case: Lorenz-96 sensitivities {name}, n={n}")
    m = orc.record(prob, u0n, pn, fused=True)
    assert np.all(m["status"] == 0)
    S = prob.n_save_eff
    aux = None if lk == W.SUMSQ_FINAL else np.random.default_rng(dim).standard_normal((n, S, dim))
    so, lo, go, po = orc.replay_sens(prob, u0n, pn, m, lk, aux=aux, scale=0.4, fused=True)
    mesh = mesh_to_dev(m, prob.max_steps, torch)
    u0, p = to_dev(u0n, torch), to_dev(pn, torch)
    auxd = None if aux is None else aux_to_dev(aux, torch)
    sg, lg, gu0, gp = da.replay_sens(prob, u0, p, mesh, lk, aux=auxd, scale=0.4)
    la, ga, pa = da.replay_grad(prob, u0, p, mesh, lk, aux=auxd, scale=0.4)
    torch.cuda.synchronize()
    es = _sens_elem_err(sg.cpu().numpy().transpose(3, 0, 1, 2), so)
    eg = grad_elem_err(gu0.cpu().numpy().T, gp.cpu().numpy().T, go, po)
    el = np.abs(lg.cpu().numpy() - lo) / np.abs(lo)
    ea = grad_rel_err(gu0.cpu().numpy().T, gp.cpu().numpy().T, ga.cpu().numpy().T,
                      pa.cpu().numpy().T)
    _print(f"  sens max rel {es.max():.3e} (bitwise lanes {np.mean(es == 0):.3f}), "
           f"grad {eg.max():.3e}, loss {el.max():.3e}, forward vs reverse {ea.max():.3e}")
    assert es.max() <= 1e-12 and eg.max() <= 1e-12 and el.max() <= 1e-12
    assert ea.max() <= 1e-10


RANGE_CASES = [
    ("lorenz63_dopri5", W.Problem(W.LORENZ63, 3, 3, W.DOPRI5, 0.0, 1.5, 1e-8, 1e-8, 4096,
                                  save_times=(0.4, 1.1, 1.5)), 1, 500,
     [(3, 3), (0, 1), (5, 1), (1, 4)]),
    ("robertson_ros2", W.WORKLOADS[4].problem(t1=100.0), 4, 300, [(3, 3), (2, 1)]),
    ("l96_d64_tsit5", W.Problem(W.LORENZ96, 64, 1, W.TSIT5, 0.0, 1.0, 1e-7, 1e-7, 4096,
                                save_times=(0.3, 1.0)), 5, 96, [(64, 1), (30, 7), (0, 65)]),
    ("l96_d40_dopri5_dense", W.Problem(W.LORENZ96, 40, 1, W.DOPRI5, 0.0, 1.0, 1e-7, 1e-7, 4096,
                                       save_times=(0.37, 0.81), dense=1), 5, 80,
     [(40, 1), (38, 3)]),
]


@pytest.mark.parametrize("name,prob,wid,n,ranges", RANGE_CASES, ids=[c[0] for c in RANGE_CASES])
def test_direction_ranges_equal_full_call(da, name, prob, wid, n, ranges):
    """da_replay_sens_dirs over a range of directions gives, bit for bit, that
    range of da_replay_sens's sensitivities and gradient, and the same loss
    (the directions do not interact; a single Lorenz-96 direction runs one
    per lane)."""
    inp = W.make_inputs(wid, n)
    u0n = np.ascontiguousarray(inp["u0"][:, :prob.dim])
    u0, p = to_dev(u0n, torch), to_dev(inp["p"], torch)
    S = prob.n_save_eff
    auxd = aux_to_dev(np.random.default_rng(11).standard_normal((n, S, prob.dim)), torch)
    _print(f"case: direction ranges {name}, n={n}")
    mesh, _ = da.record(prob, u0, p)
    sf, lf, gu0, gp = da.replay_sens(prob, u0, p, mesh, W.COTANGENT, aux=auxd, scale=0.25)
    torch.cuda.synchronize()
    assert torch.all(mesh.status == 0)
    gall = torch.cat([gu0, gp])
    for qb, qc in ranges:
        sr, lr, gr = da.replay_sens_dirs(prob, u0, p, mesh, qb, qc, W.COTANGENT, aux=auxd,
                                         scale=0.25)
        torch.cuda.synchronize()
        assert sr.shape == (S, prob.dim, qc, n) and gr.shape == (qc, n)
        assert torch.equal(sr, sf[:, :, qb:qb + qc]), (qb, qc)
        assert torch.equal(gr, gall[qb:qb + qc]), (qb, qc)
        assert torch.equal(lr, lf), (qb, qc)
    _print(f"  {len(ranges)} ranges equal to the full call")


def test_l96_sensitivity_options(da):
    """Lorenz-96 forward mode with an ensemble that does not fill its last
    workgroup, a failed trajectory (NaN everywhere, the others finite), the
    replay order with its table (bit-for-bit the same as the record order),
    and sensitivities without a loss."""
    n, dim = 97, 64
    inp = W.make_inputs(5, n)
    inp["p"][5, 0] = np.nan
    prob = W.Problem(W.LORENZ96, dim, 1, W.TSIT5, 0.0, 0.6, 1e-7, 1e-7, 4096,
                     save_times=(0.2, 0.6))
    _print(f"case: Lorenz-96 sensitivity options, n={n}")
    u0, p = to_dev(inp["u0"], torch), to_dev(inp["p"], torch)
    mesh, _ = da.record(prob, u0, p)
    sm = da.mesh_sort(prob, mesh)
    auxd = aux_to_dev(np.random.default_rng(2).standard_normal((n, 2, dim)), torch)
    s1, l1, g1, q1 = da.replay_sens(prob, u0, p, mesh, W.MSE_SAVE, aux=auxd, scale=0.5)
    s2, l2, g2, q2 = da.replay_sens(prob, u0, p, sm, W.MSE_SAVE, aux=auxd, scale=0.5)
    s3, _, _, _ = da.replay_sens(prob, u0, p, sm, loss_kind=None)
    torch.cuda.synchronize()
    bad = mesh.status.cpu().numpy() != 0
    assert bad[5] and bad.sum() == 1
    for a, b in ((s1, s2), (s1, s3), (l1, l2), (g1, g2), (q1, q2)):
        assert torch.equal(torch.nan_to_num(a), torch.nan_to_num(b))
    s1n = s1.cpu().numpy()
    assert np.all(np.isnan(s1n[..., bad])) and np.all(np.isfinite(s1n[..., ~bad]))
    for t in (l1, g1, q1):
        tn = t.cpu().numpy()
        assert np.all(np.isnan(tn[..., bad])) and np.all(np.isfinite(tn[..., ~bad]))


def test_ros2_sensitivities_with_row_exchanges(da, orc):
    """ROS2 on Lorenz-63 over a coarse hand-made mesh (per-trajectory step
    sizes 0.02..0.2), where the LU of W = I - gamma h J exchanges rows in some
    lanes of every wavefront and not in others: tangents through the pivoted
    factors and both solves against the oracle, and against the reverse sweep."""
    n, N = 256, 10
    inp = W.make_inputs(1, n)
    u0n, pn = inp["u0"], inp["p"]
    hl = 0.02 + 0.18 * np.random.default_rng(8).random(n)
    g = orc.ros2_gamma()
    col0 = np.abs(np.stack([1 + g * hl * pn[:, 0], -g * hl * (pn[:, 1] - u0n[:, 2]),
                            -g * hl * u0n[:, 1]]))
    piv = np.argmax(col0, axis=0)          # pivot row of the first column, first step
    for w0 in range(0, n, 64):
        assert 0 < np.count_nonzero(piv[w0:w0 + 64]) < 64
    m = {"h": np.repeat(hl[:, None], N, 1), "n_steps": np.full(n, N, np.int32),
         "save_idx": np.tile(np.array([3, 7, 10], np.int32), (n, 1)),
         "status": np.zeros(n, np.int32)}
    prob = W.Problem(W.LORENZ63, 3, 3, W.ROS2, 0.0, 2.0, 1e-6, 1e-6, N,
                     save_times=(0.6, 1.4, 2.0))
    aux = np.random.default_rng(5).standard_normal((n, 3, 3))
    _print(f"case: ROS2 sensitivities with row exchanges, n={n}")
    so, lo, go, po = orc.replay_sens(prob, u0n, pn, m, W.MSE_SAVE, aux=aux, scale=0.3, fused=True)
    mesh = mesh_to_dev(m, N, torch)
    u0, p = to_dev(u0n, torch), to_dev(pn, torch)
    sg, lg, gu0, gp = da.replay_sens(prob, u0, p, mesh, W.MSE_SAVE, aux=aux_to_dev(aux, torch),
                                     scale=0.3)
    la, ga, pa = da.replay_grad(prob, u0, p, mesh, W.MSE_SAVE, aux=aux_to_dev(aux, torch),
                                scale=0.3)
    torch.cuda.synchronize()
    es = _sens_elem_err(sg.cpu().numpy().transpose(3, 0, 1, 2), so)
    eg = grad_elem_err(gu0.cpu().numpy().T, gp.cpu().numpy().T, go, po)
    ea = grad_rel_err(gu0.cpu().numpy().T, gp.cpu().numpy().T, ga.cpu().numpy().T,
                      pa.cpu().numpy().T)
    _print(f"  sens max rel {es.max():.3e} (bitwise lanes {np.mean(es == 0):.3f}), "
           f"grad {eg.max():.3e}, forward vs reverse {ea.max():.3e}")
    assert es.max() <= 1e-12 and eg.max() <= 1e-12 and ea.max() <= 1e-10


@pytest.mark.parametrize("wid", [2, 4, 5])
def test_full_size_sensitivities_sampled(da, orc, wid):
    """Lorenz-63 with Dopri5 (2^20 trajectories), Robertson with ROS2 (65536)
    and Lorenz-96 at d = 64 (16384) at full size: record, replay order with
    table, forward-mode gradient; sampled trajectories against the oracle on
    the GPU's mesh."""
    w = W.WORKLOADS[wid]
    prob = w.problem()
    inp = W.make_inputs(wid)
    n = w.n
    _print(f"case: full-size sensitivities, {w.name}, n={n}")
    u0, p = to_dev(inp["u0"], torch), to_dev(inp["p"], torch)
    mesh, _ = da.record(prob, u0, p, save=False)
    sm = da.mesh_sort(prob, mesh)
    _, loss, gu0, gp = da.replay_sens(prob, u0, p, sm, with_sens=False)
    torch.cuda.synchronize()
    perm = sm.perm.cpu().numpy()
    rng = np.random.default_rng(31)
    k = 64 if wid == 2 else 24
    tr = perm[np.unique(np.concatenate([rng.choice(n, k, replace=False), [0, n - 1]]))]
    N = int(sm.n_steps.max().item())
    idx = torch.from_numpy(tr.astype(np.int64)).cuda()
    h = sm.h.index_select(1, idx).permute(1, 0, 2).reshape(len(tr), -1)[:, :N].cpu().numpy()
    sub = {"h": np.ascontiguousarray(h), "n_steps": sm.n_steps.cpu().numpy()[tr],
           "save_idx": sm.save_idx.cpu().numpy()[:, tr].T.copy(),
           "status": sm.status.cpu().numpy()[tr]}
    pn = prob.replace(max_steps=N)
    so, lo, go, po = orc.replay_sens(pn, inp["u0"][tr], inp["p"][tr], sub, fused=True)
    eg = grad_elem_err(gu0.cpu().numpy()[:, tr].T, gp.cpu().numpy()[:, tr].T, go, po)
    _print(f"  sampled {len(tr)}: element-wise max rel {eg.max():.3e}")
    assert eg.max() <= 1e-12


@pytest.mark.parametrize("wid,kw", [(3, dict(t1=1.0, save_times=(0.5, 1.0))),
                                    (4, dict(t1=10.0, rtol=1e-4, atol=1e-8)),
                                    (5, dict(t1=0.5, rtol=1e-5, atol=1e-5))],
                         ids=["lorenz63_tsit5", "robertson_ros2", "lorenz96_tsit5"])
def test_sensitivities_fp32(da, orc, wid, kw):
    """FP32 tangents against the FP64 oracle on the FP32 mesh (the tangent
    arithmetic in single precision; the oracle's forward mode runs in double
    only), norm-wise: single-precision rounding is measured against the
    vector's scale, since entries far below it carry FP32 errors far above
    1e-4 of themselves."""
    w = W.WORKLOADS[wid]
    prob = w.problem(**kw)
    n = 200
    inp = {k: v.astype(np.float32) for k, v in W.make_inputs(wid, n).items()}
    _print(f"case: FP32 sensitivities, {w.name}, n=200")
    m = orc.record(prob, inp["u0"], inp["p"], fused=True)
    assert np.all(m["status"] == 0)
    m64 = dict(m)
    m64["h"] = m["h"].astype(np.float64)
    so, lo, go, po = orc.replay_sens(prob, inp["u0"].astype(np.float64),
                                     inp["p"].astype(np.float64), m64, fused=True)
    sg, lg, gu0, gp = da.replay_sens(prob, to_dev(inp["u0"], torch), to_dev(inp["p"], torch),
                                     mesh_to_dev(m, prob.max_steps, torch))
    torch.cuda.synchronize()
    es = _sens_err(sg.cpu().numpy().transpose(3, 0, 1, 2).astype(np.float64), so)
    eg = grad_rel_err(gu0.cpu().numpy().T.astype(np.float64), gp.cpu().numpy().T.astype(np.float64),
                      go, po)
    _print(f"  FP32 against the FP64 oracle: sens max rel {es.max():.3e}, grad {eg.max():.3e}")
    assert es.max() <= 1e-4 and eg.max() <= 1e-4
