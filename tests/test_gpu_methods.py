"""The higher-order methods on the GPU against the oracle: Rodas3 (the
third-order Rosenbrock method, also on the eight-species kinetics system with
ROS2), the fourth-order Rosenbrock method with its third-order companion
(Shampine's four-stage parameters) and Fehlberg 7(8) (the seventh-order
explicit pair).

Gates: on oracle-recorded meshes, saves, losses and gradients element by
element within 1e-12 relative of the oracle's fused-rounding mode in FP64
(the kernels' arithmetic schedule), and within PLAIN_TOL of its
plain-rounding mode (four times the largest gap between the oracle's two
modes on the same inputs, measured by the oracle alone); in FP32 within
1e-4 of the FP32 oracle's fused mode and within twice the oracle's own FP32
rounding spread of the FP64 oracle; the GPU's records agree with the
oracle's (step counts, error norms, states); checkpoint intervals and the
replay table give bit-for-bit the same gradients; forward-mode
sensitivities against the oracle (element-wise) and against the reverse
sweep (norm-wise: two different arithmetic routes); the
Robertson workload and the eight-species cycle with Rodas3 (65536
trajectories; Robertson also with the fourth-order method) and Lorenz-63
with Fehlberg 7(8) (2^20) at full size, sampled."""
import numpy as np
import pytest

import workloads as W
from helpers import (aux_to_dev, elem_err, fp32_against_fp64, grad_elem_err, grad_rel_err,
                     mesh_to_dev, mesh_to_host, plain_gap_gate, smallest_component,
                     step_count_gate, to_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def da():
    import discrete_adjoint_amd as da
    assert torch.cuda.is_available()
    return da


def _print(*a):
    print(*a, flush=True)


def _linear_inputs(n):
    rng = np.random.default_rng(5)
    return {"u0": 1.0 + rng.random((n, 1)), "p": -3.0 * rng.random((n, 1)) + 0.2}


CASES = [
    ("robertson_full", W.WORKLOADS[4].problem(method=W.RODAS3), 4, W.SUMSQ_FINAL, 300),
    ("robertson_saves_mse", W.WORKLOADS[4].problem(method=W.RODAS3, t1=1e3,
                                                   save_times=(1.0, 10.0, 1e3)),
     4, W.MSE_SAVE, 200),
    ("lorenz63_saves_cot", W.WORKLOADS[1].problem(method=W.RODAS3, max_steps=4096,
                                                  save_times=(0.3, 0.7, 1.0)),
     1, W.COTANGENT, 400),
    ("linear", W.Problem(W.LINEAR, 1, 1, W.RODAS3, 0.0, 4.0, 1e-8, 1e-8, 4096,
                         save_times=(1.0, 4.0)), None, W.COTANGENT, 300),
    # the eight-species cycle (8 x 8 factors per lane)
    ("kinetics8", W.WORKLOADS[6].problem(t1=20.0), 6, W.SUMSQ_FINAL, 256),
    ("kinetics8_ros2_saves", W.WORKLOADS[6].problem(method=W.ROS2, t1=0.5, max_steps=8192,
                                                    save_times=(0.1, 0.5)),
     6, W.COTANGENT, 128),
    # the fourth-order Rosenbrock method
    ("ros4_robertson_full", W.WORKLOADS[4].problem(method=W.ROS4), 4, W.SUMSQ_FINAL, 300),
    ("ros4_robertson_saves_mse", W.WORKLOADS[4].problem(method=W.ROS4, t1=1e3,
                                                        save_times=(1.0, 10.0, 1e3)),
     4, W.MSE_SAVE, 200),
    ("ros4_lorenz63_saves_cot", W.WORKLOADS[1].problem(method=W.ROS4, max_steps=4096,
                                                       save_times=(0.3, 0.7, 1.0)),
     1, W.COTANGENT, 400),
    ("ros4_linear", W.Problem(W.LINEAR, 1, 1, W.ROS4, 0.0, 4.0, 1e-8, 1e-8, 4096,
                              save_times=(1.0, 4.0)), None, W.COTANGENT, 300),
    ("ros4_kinetics8", W.WORKLOADS[6].problem(method=W.ROS4, t1=20.0), 6, W.SUMSQ_FINAL, 256),
    # Fehlberg 7(8)
    ("rkf78_lorenz63_saves_mse", W.WORKLOADS[1].problem(method=W.RKF78, rtol=1e-9, atol=1e-9,
                                                        save_times=(0.3, 0.7, 1.0)),
     1, W.MSE_SAVE, 400),
    ("rkf78_lorenz63_tight", W.WORKLOADS[2].problem(method=W.RKF78, t1=2.0, rtol=1e-12,
                                                    atol=1e-12),
     2, W.SUMSQ_FINAL, 300),
    ("rkf78_robertson", W.WORKLOADS[4].problem(method=W.RKF78, t1=0.3, max_steps=8192),
     4, W.SUMSQ_FINAL, 200),
    ("rkf78_linear", W.Problem(W.LINEAR, 1, 1, W.RKF78, 0.0, 4.0, 1e-10, 1e-10, 4096,
                               save_times=(1.0, 4.0)), None, W.COTANGENT, 300),
]


# Element-wise gate against the plain-rounding oracle on each case's inputs:
# four times the largest element-wise gap between the oracle's plain and fused
# modes on the oracle's mesh (measured, in order: 4.7e-13, 1.5e-13, 1.7e-12,
# 2.8e-14, 2.8e-13, 7.0e-14, 3.2e-13, 8.6e-14, 1.6e-12, 1.6e-14, 4.7e-13,
# 2.2e-12, 1.4e-12, 3.1e-11, 1.4e-14).
PLAIN_TOL = {"robertson_full": 2e-12, "robertson_saves_mse": 6e-13, "lorenz63_saves_cot": 7e-12,
             "linear": 2e-13, "kinetics8": 2e-12, "kinetics8_ros2_saves": 3e-13,
             "ros4_robertson_full": 2e-12, "ros4_robertson_saves_mse": 4e-13,
             "ros4_lorenz63_saves_cot": 7e-12, "ros4_linear": 7e-14, "ros4_kinetics8": 2e-12,
             "rkf78_lorenz63_saves_mse": 9e-12, "rkf78_lorenz63_tight": 6e-12,
             "rkf78_robertson": 2e-10, "rkf78_linear": 6e-14}


@pytest.mark.parametrize("name,prob,wid,lk,n", CASES, ids=[c[0] for c in CASES])
def test_method_against_oracle(da, orc, name, prob, wid, lk, n):
    inp = _linear_inputs(n) if wid is None else W.make_inputs(wid, n)
    u0n, pn = inp["u0"].astype(np.float64), inp["p"].astype(np.float64)
    d = prob.dim
    S = prob.n_save_eff
    aux = None if lk == W.SUMSQ_FINAL else np.random.default_rng(9).standard_normal((n, S, d))
    _print(f"case: {W.METHOD_NAMES[prob.method]} {name}, n={n}")
    m = orc.record(prob, u0n, pn, fused=True)
    assert np.all(m["status"] == 0)
    yo, _ = orc.replay(prob, u0n, pn, m, fused=True)
    lo, go, po = orc.replay_grad(prob, u0n, pn, m, lk, aux=aux, scale=0.3, fused=True)
    mesh = mesh_to_dev(m, prob.max_steps, torch)
    u0, p = to_dev(u0n, torch), to_dev(pn, torch)
    auxd = None if aux is None else aux_to_dev(aux, torch)
    yg = da.replay_fwd(prob, u0, p, mesh)
    loss, gu0, gp = da.replay_grad(prob, u0, p, mesh, lk, aux=auxd, scale=0.3)
    torch.cuda.synchronize()
    ey = elem_err(yg.cpu().numpy().transpose(2, 0, 1).reshape(n, -1), yo.reshape(n, -1))
    g1, g2 = gu0.cpu().numpy().T, gp.cpu().numpy().T
    eg = grad_elem_err(g1, g2, go, po)
    el = np.abs(loss.cpu().numpy() - lo) / np.abs(lo)
    _, gop, pop = orc.replay_grad(prob, u0n, pn, m, lk, aux=aux, scale=0.3, fused=False)
    ep = grad_elem_err(g1, g2, gop, pop)
    _print(f"  mean steps {m['n_steps'].mean():.1f}; element-wise: saves max rel {ey.max():.3e}, "
           f"grad max rel {eg.max():.3e} (bitwise lanes {np.mean(eg == 0):.3f}), loss "
           f"{el.max():.3e}; smallest component / lane's largest {smallest_component(go, po):.2e}; "
           f"vs plain-rounding oracle {ep.max():.3e} (gate {PLAIN_TOL[name]:.0e})")
    assert ey.max() <= 1e-12 and eg.max() <= 1e-12 and el.max() <= 1e-12
    assert ep.max() <= PLAIN_TOL[name]
    # the GPU's record: the oracle's mesh, and the replay's states
    mg_dev, ys = da.record(prob, u0, p)
    yr = da.replay_fwd(prob, u0, p, mg_dev)
    torch.cuda.synchronize()
    assert torch.equal(ys, yr)
    mg = mesh_to_host(mg_dev, prob.max_steps)
    assert np.all(mg["status"] == 0)
    # the controller's single-precision power rounds differently in the last
    # bit on the two sides, so the meshes are held to the same record, not to
    # the same bits: step counts within max(2, 1%) or the oracle's own spread
    # under that rounding difference, every GPU step accepted by the oracle's
    # error norm, and the GPU's states those of the oracle's replay of the
    # GPU mesh
    E = orc.mesh_max_err(prob, u0n, pn, mg, fused=True)
    yo2, _ = orc.replay(prob, u0n, pn, mg, fused=True)
    er = elem_err(ys.cpu().numpy().transpose(2, 0, 1).reshape(n, -1), yo2.reshape(n, -1))
    gate, spread = step_count_gate(orc, prob, u0n, pn, m["n_steps"])
    dN = np.abs(mg["n_steps"] - m["n_steps"])
    _print(f"  GPU record: mean steps {mg['n_steps'].mean():.1f} (oracle {m['n_steps'].mean():.1f}),"
           f" max |dN| {dN.max()} (oracle's own spread {spread}), max error norm {E.max():.4f},"
           f" states vs oracle replay {er.max():.3e}")
    assert np.all(dN <= gate)
    assert np.all(E <= 1 + 1e-6) and er.max() <= 1e-12
    # checkpoint intervals and the replay table
    for ck in (2, 4, 8):
        _, g2, q2 = da.replay_grad(prob.replace(checkpoint=ck), u0, p, mesh, lk, aux=auxd,
                                   scale=0.3)
        torch.cuda.synchronize()
        assert torch.equal(g2, gu0) and torch.equal(q2, gp), ck
    sm = da.mesh_sort(prob, mesh)
    _, g3, q3 = da.replay_grad(prob, u0, p, sm, lk, aux=auxd, scale=0.3)
    torch.cuda.synchronize()
    assert torch.equal(g3, gu0) and torch.equal(q3, gp)
    # forward-mode sensitivities
    so, _, gso, pso = orc.replay_sens(prob, u0n, pn, m, lk, aux=aux, scale=0.3, fused=True)
    sg, _, gs, ps = da.replay_sens(prob, u0, p, mesh, lk, aux=auxd, scale=0.3)
    torch.cuda.synchronize()
    sgn = sg.cpu().numpy().transpose(3, 0, 1, 2).reshape(n, -1)
    es = elem_err(sgn, so.reshape(n, -1))
    ef = grad_elem_err(gs.cpu().numpy().T, ps.cpu().numpy().T, gso, pso)
    ea = grad_rel_err(gs.cpu().numpy().T, ps.cpu().numpy().T, gu0.cpu().numpy().T,
                      gp.cpu().numpy().T)
    _print(f"  sensitivities max rel {es.max():.3e}, forward-mode grad {ef.max():.3e}, "
           f"forward vs reverse {ea.max():.3e}")
    assert es.max() <= 1e-12 and ef.max() <= 1e-12 and ea.max() <= 1e-10


@pytest.mark.parametrize("method", [W.ROS2, W.RODAS3, W.ROS4], ids=["ros2", "rodas3", "ros4"])
def test_rosenbrock4_fp32(da, orc, method):
    """FP32 Rosenbrock methods (ROS2 and the four-stage ones) on Robertson
    against the FP32 oracle and the FP64 oracle on the FP32 mesh."""
    prob = W.WORKLOADS[4].problem(method=method, t1=100.0, rtol=1e-4, atol=1e-8)
    n = 256
    inp = {k: v.astype(np.float32) for k, v in W.make_inputs(4, n).items()}
    _print(f"case: {W.METHOD_NAMES[method]} FP32, n={n}")
    m = orc.record(prob, inp["u0"], inp["p"], fused=True)
    assert np.all(m["status"] == 0)
    m64 = dict(m)
    m64["h"] = m["h"].astype(np.float64)
    lo, go, po = orc.replay_grad(prob, inp["u0"].astype(np.float64),
                                 inp["p"].astype(np.float64), m64, W.SUMSQ_FINAL)
    _, gf, pf = orc.replay_grad(prob, inp["u0"], inp["p"], m, W.SUMSQ_FINAL, fused=True)
    _, gq, pq = orc.replay_grad(prob, inp["u0"], inp["p"], m, W.SUMSQ_FINAL, fused=False)
    u0, p = to_dev(inp["u0"], torch), to_dev(inp["p"], torch)
    loss, gu0, gp = da.replay_grad(prob, u0, p, mesh_to_dev(m, prob.max_steps, torch))
    mg, _ = da.record(prob, u0, p)
    torch.cuda.synchronize()
    g1, g2 = gu0.cpu().numpy().T, gp.cpu().numpy().T
    et = grad_elem_err(g1, g2, gf, pf)
    e64 = grad_elem_err(g1, g2, go, po)
    eb = np.maximum(fp32_against_fp64(g1, go, gq, gf), fp32_against_fp64(g2, po, pq, pf))
    ns = mg.n_steps.cpu().numpy()
    gate, spread = step_count_gate(orc, prob, inp["u0"], inp["p"], m["n_steps"])
    _print(f"  element-wise: vs the FP32 oracle {et.max():.3e}, vs the FP64 oracle {e64.max():.3e} "
           f"(gate ratio {eb.max():.3f}); steps GPU {ns.mean():.1f} oracle "
           f"{m['n_steps'].mean():.1f}, max |dN| {np.abs(ns - m['n_steps']).max()} (spread {spread})")
    assert et.max() <= 1e-4 and eb.max() <= 1.0
    assert np.all(mg.status.cpu().numpy() == 0)
    assert np.all(np.abs(ns - m["n_steps"]) <= gate)


@pytest.mark.parametrize("wid,method", [(4, W.ROS2), (4, W.RODAS3), (4, W.ROS4), (6, W.RODAS3)],
                         ids=["robertson-ros2", "robertson-rodas3", "robertson-ros4",
                              "kinetics8-rodas3"])
def test_total_concentration_full_size(da, wid, method):
    """The Robertson system and the eight-species reaction cycle conserve the
    sum of their concentrations, and a Rosenbrock step with the exact
    Jacobian keeps that linear invariant of the discrete map.  So for the
    loss L = sum of the final state (cotangent of ones) the exact discrete
    adjoint is dL/du0 = (1, ..., 1) and dL/dk = 0.  Checked on every one of
    the 65536 trajectories in the benchmark's launch configuration (record,
    lane ordering with the replay table, the library's interval), at 1e-12:
    the oracle's own deviations on the Robertson workload are below 1e-14
    (dL/dk scaled by k; a single component's dy1/dk * k is about 0.05)."""
    w = W.WORKLOADS[wid]
    prob = w.problem(method=method)
    inp = W.make_inputs(wid)
    n = w.n
    _print(f"case: total concentration, workload {wid}, {W.METHOD_NAMES[method]}, n={n}")
    u0, p = to_dev(inp["u0"], torch), to_dev(inp["p"], torch)
    mesh, _ = da.record(prob, u0, p, save=False)
    sm = da.mesh_sort(prob, mesh)
    ones = torch.ones((1, w.dim, n), dtype=torch.float64, device="cuda")
    loss, gu0, gp = da.ReplayGrad(prob, u0, p, sm, W.COTANGENT, aux=ones)()
    torch.cuda.synchronize()
    assert int(sm.status.abs().max()) == 0
    dl = (loss - 1).abs().max().item()
    du = (gu0 - 1).abs().max().item()
    dk = (gp * p).abs().max().item()
    _print(f"  max |L - 1| {dl:.2e}, max |dL/du0 - 1| {du:.2e}, max |dL/dk * k| {dk:.2e}")
    assert dl <= 1e-12 and du <= 1e-12 and dk <= 1e-12


@pytest.mark.parametrize("method", [W.RODAS3, W.ROS4], ids=["rodas3", "ros4"])
def test_rosenbrock4_robertson_full_size_sampled(da, orc, method):
    """Robertson with a four-stage Rosenbrock method at the workload's full
    size and tolerances (65536 trajectories, t in [0, 1e5], rtol 1e-6, atol
    1e-10): record, replay order with table, one gradient pass; sampled
    trajectories against the oracle on the GPU's mesh and against the
    oracle's record."""
    w = W.WORKLOADS[4]
    prob = w.problem(method=method)
    inp = W.make_inputs(4)
    n = w.n
    _print(f"case: {W.METHOD_NAMES[method]} Robertson at full size, n={n}")
    u0, p = to_dev(inp["u0"], torch), to_dev(inp["p"], torch)
    mesh, _ = da.record(prob, u0, p, save=False)
    sm = da.mesh_sort(prob, mesh)
    loss, gu0, gp = da.ReplayGrad(prob, u0, p, sm, W.SUMSQ_FINAL)()
    torch.cuda.synchronize()
    st = sm.status.cpu().numpy()
    assert np.all(st == 0)
    perm = sm.perm.cpu().numpy()
    ns_all = sm.n_steps.cpu().numpy()
    rng = np.random.default_rng(41)
    slots = np.unique(np.concatenate([rng.choice(n, 48, replace=False), [0, n - 1]]))
    tr = perm[slots]
    N = int(ns_all.max())
    idx = torch.from_numpy(tr.astype(np.int64)).cuda()
    h = sm.h.index_select(1, idx).permute(1, 0, 2).reshape(len(tr), -1)[:, :N].cpu().numpy()
    sub = {"h": np.ascontiguousarray(h), "n_steps": ns_all[tr],
           "save_idx": sm.save_idx.cpu().numpy()[:, tr].T.copy(), "status": st[tr]}
    pn = prob.replace(max_steps=N)
    lo, go, po = orc.replay_grad(pn, inp["u0"][tr], inp["p"][tr], sub, W.SUMSQ_FINAL, fused=True)
    g1, g2 = gu0.cpu().numpy()[:, tr].T, gp.cpu().numpy()[:, tr].T
    err = grad_elem_err(g1, g2, go, po)
    ep, tp = plain_gap_gate(orc, pn, inp["u0"][tr], inp["p"][tr], sub, W.SUMSQ_FINAL, None, 1.0,
                            g1, g2, go, po)
    mo = orc.record(prob, inp["u0"][tr], inp["p"][tr], fused=True, with_h=False)
    gate, spread = step_count_gate(orc, prob, inp["u0"][tr], inp["p"][tr], mo["n_steps"])
    dN = np.abs(sub["n_steps"] - mo["n_steps"])
    _print(f"  sampled {len(tr)}: element-wise max rel {err.max():.3e}, vs plain {ep.max():.3e} "
           f"(gate {tp:.2e}); mean steps {ns_all.mean():.1f} "
           f"(max {N}); oracle record of the sample {mo['n_steps'].mean():.1f}, max |dN| "
           f"{dN.max()} (oracle's own spread {spread})")
    assert err.max() <= 1e-12 and ep <= tp
    assert np.all(dN <= gate)


def test_kinetics8_full_size_sampled(da, orc):
    """The eight-species cycle at full size (65536 trajectories, Rodas3, t in
    [0, 100]): record, replay order with table, one gradient pass; sampled
    trajectories against the oracle on the GPU's mesh and its record; sum y
    conserved by the GPU's record."""
    w = W.WORKLOADS[6]
    prob = w.problem()
    inp = W.make_inputs(6)
    n = w.n
    _print(f"case: kinetics8 at full size, n={n}")
    u0, p = to_dev(inp["u0"], torch), to_dev(inp["p"], torch)
    mesh, ys = da.record(prob, u0, p)
    sm = da.mesh_sort(prob, mesh)
    loss, gu0, gp = da.ReplayGrad(prob, u0, p, sm, W.SUMSQ_FINAL)()
    torch.cuda.synchronize()
    st = sm.status.cpu().numpy()
    assert np.all(st == 0)
    yN = ys.cpu().numpy()[-1]
    assert np.max(np.abs(yN.sum(0) - 1.0)) < 1e-12
    perm = sm.perm.cpu().numpy()
    ns_all = sm.n_steps.cpu().numpy()
    rng = np.random.default_rng(43)
    slots = np.unique(np.concatenate([rng.choice(n, 32, replace=False), [0, n - 1]]))
    tr = perm[slots]
    N = int(ns_all.max())
    idx = torch.from_numpy(tr.astype(np.int64)).cuda()
    h = sm.h.index_select(1, idx).permute(1, 0, 2).reshape(len(tr), -1)[:, :N].cpu().numpy()
    sub = {"h": np.ascontiguousarray(h), "n_steps": ns_all[tr],
           "save_idx": sm.save_idx.cpu().numpy()[:, tr].T.copy(), "status": st[tr]}
    pn = prob.replace(max_steps=N)
    lo, go, po = orc.replay_grad(pn, inp["u0"][tr], inp["p"][tr], sub, W.SUMSQ_FINAL, fused=True)
    g1, g2 = gu0.cpu().numpy()[:, tr].T, gp.cpu().numpy()[:, tr].T
    err = grad_elem_err(g1, g2, go, po)
    ep, tp = plain_gap_gate(orc, pn, inp["u0"][tr], inp["p"][tr], sub, W.SUMSQ_FINAL, None, 1.0,
                            g1, g2, go, po)
    mo = orc.record(prob, inp["u0"][tr], inp["p"][tr], fused=True, with_h=False)
    _print(f"  sampled {len(tr)}: element-wise max rel {err.max():.3e}, vs plain {ep.max():.3e} "
           f"(gate {tp:.2e}); smallest component / lane's largest "
           f"{smallest_component(go, po):.2e}; mean steps {ns_all.mean():.1f} "
           f"(max {N}); oracle record of the sample {mo['n_steps'].mean():.1f}")
    assert err.max() <= 1e-12 and ep <= tp
    assert np.all(np.abs(sub["n_steps"] - mo["n_steps"]) <= np.maximum(2, 0.01 * mo["n_steps"]))


def test_rkf78_lorenz63_full_size_sampled(da, orc):
    """Lorenz-63 with Fehlberg 7(8) at the headline workload's size and
    tolerances (2^20 trajectories, t in [0, 10], 1e-8): record, replay order
    with table, one gradient pass; sampled trajectories against the oracle on
    the GPU's mesh and against the oracle's record."""
    w = W.WORKLOADS[2]
    prob = w.problem(method=W.RKF78)
    inp = W.make_inputs(2)
    n = w.n
    _print(f"case: Fehlberg 7(8) Lorenz-63 at full size, n={n}")
    u0, p = to_dev(inp["u0"], torch), to_dev(inp["p"], torch)
    mesh, _ = da.record(prob, u0, p, save=False)
    sm = da.mesh_sort(prob, mesh)
    loss, gu0, gp = da.ReplayGrad(prob, u0, p, sm, W.SUMSQ_FINAL)()
    torch.cuda.synchronize()
    st = sm.status.cpu().numpy()
    assert np.all(st == 0)
    perm = sm.perm.cpu().numpy()
    ns_all = sm.n_steps.cpu().numpy()
    rng = np.random.default_rng(47)
    slots = np.unique(np.concatenate([rng.choice(n, 40, replace=False), [0, n - 1]]))
    tr = perm[slots]
    N = int(ns_all.max())
    idx = torch.from_numpy(tr.astype(np.int64)).cuda()
    h = sm.h.index_select(1, idx).permute(1, 0, 2).reshape(len(tr), -1)[:, :N].cpu().numpy()
    sub = {"h": np.ascontiguousarray(h), "n_steps": ns_all[tr],
           "save_idx": sm.save_idx.cpu().numpy()[:, tr].T.copy(), "status": st[tr]}
    pn = prob.replace(max_steps=N)
    lo, go, po = orc.replay_grad(pn, inp["u0"][tr], inp["p"][tr], sub, W.SUMSQ_FINAL, fused=True)
    g1, g2 = gu0.cpu().numpy()[:, tr].T, gp.cpu().numpy()[:, tr].T
    err = grad_elem_err(g1, g2, go, po)
    ep, tp = plain_gap_gate(orc, pn, inp["u0"][tr], inp["p"][tr], sub, W.SUMSQ_FINAL, None, 1.0,
                            g1, g2, go, po)
    mo = orc.record(prob, inp["u0"][tr], inp["p"][tr], fused=True, with_h=False)
    _print(f"  sampled {len(tr)}: element-wise max rel {err.max():.3e}, vs plain {ep.max():.3e} "
           f"(gate {tp:.2e}); smallest component / lane's largest "
           f"{smallest_component(go, po):.2e}; mean steps {ns_all.mean():.1f} "
           f"(max {N}); oracle record of the sample {mo['n_steps'].mean():.1f}")
    assert err.max() <= 1e-12 and ep <= tp
    assert np.all(np.abs(sub["n_steps"] - mo["n_steps"]) <= np.maximum(2, 0.01 * mo["n_steps"]))


@pytest.mark.parametrize("method", [W.ROS2, W.RODAS3, W.ROS4], ids=["ros2", "rodas3", "ros4"])
def test_rosenbrock_failed_lanes_and_edge_sizes(da, orc, method):
    """Robertson to t = 1000 with a NaN rate (lane 5), an overflowing start
    (lane 7), an infinite rate (lane 9) and a step limit at the median step
    count, so about half the trajectories stop at it.  On the oracle's mesh:
    NaN loss and gradients exactly where the oracle's record failed, the
    oracle's values elsewhere.  The GPU's own record: the oracle's status for
    the three broken lanes, and for every lane whose unconstrained step
    count is clear of the limit by more than the step-count gate.  n = 1 and
    n = 0 run."""
    n = 130
    inp = W.make_inputs(4, n)
    inp["p"][5, 0] = np.nan
    inp["u0"][7, :] = 1e200
    inp["p"][9, 1] = np.inf
    base = W.WORKLOADS[4].problem(method=method, t1=1e3, max_steps=16384)
    free = orc.record(base, inp["u0"], inp["p"], fused=True, with_h=False)
    ok_free = free["status"] == 0
    limit = int(np.median(free["n_steps"][ok_free]))
    prob = base.replace(max_steps=limit)
    _print(f"case: {W.METHOD_NAMES[method]} failed lanes, n={n}, max_steps={limit}")
    m = orc.record(prob, inp["u0"], inp["p"], fused=True)
    bad = m["status"] != 0
    assert bad.sum() > 10 and (~bad).sum() > 10
    lo, go, po = orc.replay_grad(prob, inp["u0"], inp["p"], m, fused=True)
    u0, p = to_dev(inp["u0"], torch), to_dev(inp["p"], torch)
    loss, gu0, gp = da.replay_grad(prob, u0, p, mesh_to_dev(m, prob.max_steps, torch))
    torch.cuda.synchronize()
    gu0n, gpn, ln = gu0.cpu().numpy().T, gp.cpu().numpy().T, loss.cpu().numpy()
    assert np.all(np.isnan(gpn[bad])) and np.all(np.isnan(gu0n[bad])) and np.all(np.isnan(ln[bad]))
    assert np.all(np.isfinite(gpn[~bad])) and np.all(np.isfinite(gu0n[~bad]))
    assert grad_elem_err(gu0n[~bad], gpn[~bad], go[~bad], po[~bad]).max() <= 1e-12
    mesh, _ = da.record(prob, u0, p)
    torch.cuda.synchronize()
    st = mesh.status.cpu().numpy()
    assert np.array_equal(st[[5, 7, 9]], m["status"][[5, 7, 9]])
    assert st[5] == da.LANE_NONFINITE and st[7] == da.LANE_DT_UNDERFLOW
    gate, spread = step_count_gate(orc, base, inp["u0"], inp["p"], free["n_steps"])
    clear = ok_free & (np.abs(free["n_steps"] - limit) > gate)
    _print(f"  oracle failed {bad.sum()}, GPU failed {(st != 0).sum()}; {clear.sum()} lanes clear "
           f"of the limit (spread {spread})")
    assert clear.sum() > 10 and np.array_equal(st[clear], m["status"][clear])
    # n = 1 and n = 0
    m1, _ = da.record(base, u0[:, :1].contiguous(), p[:, :1].contiguous())
    l1, g1, q1 = da.replay_grad(base, u0[:, :1].contiguous(), p[:, :1].contiguous(), m1)
    torch.cuda.synchronize()
    assert m1.status.item() == 0 and np.isfinite(q1.cpu().numpy()).all()
    e = torch.empty((3, 0), dtype=torch.float64, device="cuda")
    m0, _ = da.record(base, e, e)
    r0 = da.replay_grad(base, e, e, m0, max_n_steps=0)
    assert r0[0].numel() == 0
