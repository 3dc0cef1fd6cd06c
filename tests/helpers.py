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
    B = 8 if m["h"].dtype == np.float64 else 16
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
    """Per-lane ||g - ref||_inf / max(||ref||_inf, 1e-300) over the last axis."""
    num = np.max(np.abs(g - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-300)
    return num / den


def grad_rel_err(gu0, gp, gu0_ref, gp_ref):
    """Per-lane max of the relative errors of the two gradient vectors."""
    return np.maximum(rel_err(gu0, gu0_ref), rel_err(gp, gp_ref))


def mse_targets(orc, wid, n, inp):
    """Targets of the calibration workload: FP64 oracle record with the perturbed
    parameters at the save times, cast to the workload dtype; [n, S, d]."""
    w = W.WORKLOADS[wid]
    prob = w.problem()
    m = orc.record(prob, inp["u0"].astype(np.float64), inp["p_true"], with_h=False)
    return m["y_save"].astype(w.np_dtype), m["status"]


def step_count_gate(orc, prob, u0, p, n_ref, eps=1e-7):
    """Per-lane bound on |N_gpu - N_oracle| for a GPU record against the
    oracle's: max(2, 1% of the oracle's count), widened to the largest change
    the oracle's own record shows when its step factor is scaled by 1 +- eps.
    The two sides round the controller's single-precision power differently
    in the last bit (relative 6e-8), so a method whose step sequence that
    perturbation moves cannot be held closer than this.  Returns the bound
    and that spread."""
    spread = 0
    for s in (1.0 + eps, 1.0 - eps):
        pr = prob.replace(safety=(prob.safety or 0.9) * s)
        m = orc.record(pr, u0, p, fused=True, with_h=False)
        spread = max(spread, int(np.max(np.abs(m["n_steps"] - n_ref))))
    return np.maximum(np.maximum(2, 0.01 * n_ref), spread), spread
