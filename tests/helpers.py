"""Shared helpers of the tests: layout conversion and error measures."""
import numpy as np

import workloads as W


def to_dev(x, torch, dev="cuda"):
    """Lane-major numpy [n, C] -> component-major device tensor [C, n]."""
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x).T)).to(dev)


def aux_to_dev(a, torch, dev="cuda"):
    """[n, S, d] -> [S, d, n]."""
    return torch.from_numpy(np.ascontiguousarray(np.transpose(a, (1, 2, 0)))).to(dev)


def mesh_to_host(mesh, N):
    """Device mesh (tiled log, trajectory order) -> oracle dict (lane-major)
    with the first N steps of every trajectory (the oracle's row length is its
    problem's max_steps); the replay order, if any, is not part of it."""
    ns = mesh.n_steps.cpu().numpy()
    h = mesh.steps(N).cpu().numpy()
    out = {"h": h, "n_steps": ns, "save_idx": mesh.save_idx.cpu().numpy().T.copy(),
           "status": mesh.status.cpu().numpy()}
    if mesh.save_theta is not None:
        out["save_theta"] = mesh.save_theta.cpu().numpy().T.copy()
    return out


def tile_steps(h_rows, max_steps, B):
    """[n, N] step sizes -> tiled [T, n, B] log with zero padding."""
    n, N = h_rows.shape
    T = (max_steps + B - 1) // B
    full = np.zeros((n, T * B), dtype=h_rows.dtype)
    full[:, :N] = h_rows
    return np.ascontiguousarray(full.reshape(n, T, B).transpose(1, 0, 2))


def mesh_to_dev(m, max_steps, torch, dev="cuda"):
    import discrete_adjoint_amd as da
    B = 16 if m["h"].dtype == np.float64 else 32
    h = tile_steps(m["h"], max_steps, B)
    th = None
    if "save_theta" in m:
        th = torch.from_numpy(np.ascontiguousarray(m["save_theta"].T)).to(dev)
    return da.Mesh(torch.from_numpy(h).to(dev),
                   torch.from_numpy(np.ascontiguousarray(m["n_steps"].astype(np.int32))).to(dev),
                   torch.from_numpy(np.ascontiguousarray(m["save_idx"].T.astype(np.int32))).to(dev),
                   torch.from_numpy(np.ascontiguousarray(m["status"].astype(np.int32))).to(dev),
                   save_theta=th)


def rel_err(g, ref):
    """Per-lane ||g - ref||_inf / max(||ref||_inf, 1e-300) over the last axis:
    the norm-wise measure, used where two different arithmetic routes are
    compared (forward mode against the reverse sweep, a registered right-hand
    side against a built-in one), whose rounding differences on a component
    scale with the vector, not with the component."""
    num = np.max(np.abs(g - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-300)
    return num / den


def grad_rel_err(gu0, gp, gu0_ref, gp_ref):
    """Per-lane max of the norm-wise relative errors of the two gradient
    vectors."""
    return np.maximum(rel_err(gu0, gu0_ref), rel_err(gp, gp_ref))


def elem_err(g, ref):
    """Per-lane max over the last axis of |g - ref| / |ref|, element by
    element, with no absolute floor: an element whose reference is exactly
    zero must be exactly zero (else the error is infinite), and NaN counts as
    equal only to NaN at the same place."""
    g = np.asarray(g, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    a = np.abs(ref)
    d = np.abs(g - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.where(a > 0, d / np.where(a > 0, a, 1.0), np.where(d == 0, 0.0, np.inf))
    e = np.where(np.isnan(g) & np.isnan(ref), 0.0, e)
    e = np.where(np.isnan(e), np.inf, e)
    return e.max(axis=-1)


def grad_elem_err(gu0, gp, gu0_ref, gp_ref):
    """Per-lane max of the element-wise relative errors of the two gradient
    vectors (every component, the smallest included, held to the tolerance
    on its own)."""
    return np.maximum(elem_err(gu0, gu0_ref), elem_err(gp, gp_ref))


def smallest_component(gu0_ref, gp_ref):
    """Smallest |component| relative to its lane's largest, over both
    gradient vectors: how far below the vector's scale the element-wise gate
    reaches."""
    r = []
    for g in (gu0_ref, gp_ref):
        a = np.abs(np.asarray(g, dtype=np.float64))
        r.append((a.min(axis=-1) / np.maximum(a.max(axis=-1), 1e-300)).min())
    return min(r)


def fp32_against_fp64(g32, ref64, plain32, fused32, tol=1e-4):
    """Per-lane max over elements of |g - r64| / (2 s + tol |r64|), where r64
    is the FP64 oracle's gradient of the same FP32 mesh and inputs, and s the
    larger distance of the oracle's two FP32 roundings (plain and fused) from
    it: the GPU's FP32 result must be within twice the oracle's own FP32
    rounding spread of the FP64 value, plus tol relative.  <= 1 passes.  It
    needs neither side's arithmetic order: chaotic lanes, where two correct
    FP32 roundings differ by far more than 1e-4, get the bar their own
    rounding sensitivity sets."""
    g32, r, p32, f32 = (np.asarray(x, dtype=np.float64) for x in (g32, ref64, plain32, fused32))
    s = np.maximum(np.abs(p32 - r), np.abs(f32 - r))
    bar = 2.0 * s + tol * np.abs(r)
    d = np.abs(g32 - r)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.where(bar > 0, d / np.where(bar > 0, bar, 1.0), np.where(d == 0, 0.0, np.inf))
    e = np.where(np.isnan(e), np.inf, e)
    return e.max(axis=-1)


def mse_targets(orc, wid, n, inp):
    """Targets of the calibration workload: FP64 oracle record with the perturbed
    parameters at the save times, cast to the workload dtype; [n, S, d]."""
    w = W.WORKLOADS[wid]
    prob = w.problem()
    m = orc.record(prob, inp["u0"].astype(np.float64), inp["p_true"], with_h=False)
    return m["y_save"].astype(w.np_dtype), m["status"]


def step_count_gate(orc, prob, u0, p, n_ref, eps=1e-7, fused=True):
    """Per-lane bound on |N_gpu - N_oracle| for a GPU record against the
    oracle's record n_ref (taken in the given rounding mode): max(2, 1% of
    the oracle's count), widened to the largest change the oracle's own
    record (same mode) shows on any lane when its step factor is scaled by
    1 +- eps.  The two sides' single-precision controller powers differ in
    the last bit (relative 6e-8), and the textbook controller of the plain
    mode differs from both by more, so a method or precision whose step
    sequence such a perturbation moves cannot be held closer than this.
    Returns the bound and that spread."""
    spread = 0
    for s in (1.0 + eps, 1.0 - eps):
        pr = prob.replace(safety=(prob.safety or 0.9) * s)
        m = orc.record(pr, u0, p, fused=fused, with_h=False)
        spread = max(spread, int(np.max(np.abs(m["n_steps"] - n_ref))))
    return np.maximum(np.maximum(2, 0.01 * n_ref), spread), spread


def plain_gap_gate(orc, prob, u0, p, mesh, lk, aux, scale, g1, g2, go, po, factor=4.0):
    """FP64 gradients g1 (u0) and g2 (p) against the oracle's plain-rounding
    mode on the same mesh, element by element, with the tolerance measured by
    the oracle alone on the same trajectories: `factor` times the largest
    element-wise gap between its plain mode and its fused mode (go, po).
    Returns (error, tolerance); the caller asserts error <= tolerance."""
    _, gop, pop = orc.replay_grad(prob, u0, p, mesh, lk, aux=aux, scale=scale, fused=False)
    gap = grad_elem_err(go, po, gop, pop).max()
    return grad_elem_err(g1, g2, gop, pop).max(), factor * gap


def attempt_count_gate(orc, prob, u0, p, natt_ref, eps=1e-7, fused=True):
    """As step_count_gate, for the record's trial steps (accepted plus
    rejected): max(2, 1% of the oracle's count), widened to the largest
    change of any trajectory's count under the same perturbation of the
    step factor.  Returns the bound and that spread."""
    spread = 0
    for s in (1.0 + eps, 1.0 - eps):
        pr = prob.replace(safety=(prob.safety or 0.9) * s)
        m = orc.record(pr, u0, p, fused=fused, with_h=False)
        spread = max(spread, int(np.max(np.abs(m["n_attempts"] - natt_ref))))
    return np.maximum(np.maximum(2, 0.01 * natt_ref), spread), spread
