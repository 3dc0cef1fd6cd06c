"""da_replay_grad_noalloc, the replay gradient with the library's static
device scratch as its workspace (for callers that cannot allocate), against
da_replay_grad with a caller workspace: the same outputs bit for bit, on
calls in a row with the later ones on a smaller ensemble (a replay order with
the replay table, none, and the replay order alone), with the scratch
holding the whole ensemble or only part of it (consecutive chunks), on the
lane kernels and the wavefront kernels; sizes beyond the scratch are
rejected before any launch."""
import numpy as np
import pytest

import workloads as W
from helpers import aux_to_dev, mse_targets, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def da():
    import discrete_adjoint_amd as da
    assert torch.cuda.is_available()
    return da


def _print(*a):
    print(*a, flush=True)


def _inputs(orc, wid, n):
    w = W.WORKLOADS[wid]
    inp = W.make_inputs(wid, n)
    aux, scale = None, 1.0
    if w.loss == W.MSE_SAVE:
        aux, st = mse_targets(orc, wid, n, inp)
        assert np.all(st == 0)
        scale = 1.0 / (n * w.n_save_eff * w.dim)
    return w, inp, aux, scale


def _chunk_lanes(da, prob, n, N, dt):
    per = da.replay_grad_workspace(prob, 1, N, dt)
    fit = da.NOALLOC_SCRATCH_BYTES // per
    return n if fit >= n else (fit // 256) * 256


# (workload, first n, second n): the first ensemble needs more than the
# scratch on workloads 2, 4 and 5 (chunks), the second less
CASES = [(2, 4000, 700), (3, 2500, 900), (4, 600, 300), (5, 1500, 200)]


@pytest.mark.parametrize("wid,n1,n2", CASES)
def test_noalloc_equals_replay_grad(da, orc, wid, n1, n2):
    for n, sort in ((n1, "table"), (n2, "none"), (n2, "order")):
        w, inp, aux, scale = _inputs(orc, wid, n)
        prob = w.problem()
        dt = torch.float64 if w.dtype == "f64" else torch.float32
        _print(f"case: noalloc replay gradient, workload {wid}, n={n}, sorted={sort}")
        u0, p = to_dev(inp["u0"], torch), to_dev(inp["p"], torch)
        auxd = None if aux is None else aux_to_dev(aux, torch)
        mesh, _ = da.record(prob, u0, p, save=False)
        if sort != "none":
            mesh = da.mesh_sort(prob, mesh, table=sort == "table")
        N = da.mesh_max_steps(mesh)
        ref = da.replay_grad(prob, u0, p, mesh, w.loss, aux=auxd, scale=scale, max_n_steps=N)
        ref = [t.clone() for t in ref]
        out = tuple(torch.full_like(t, float("nan")) for t in ref)
        got = da.replay_grad_noalloc(prob, u0, p, mesh, N, w.loss, aux=auxd, scale=scale, out=out)
        torch.cuda.synchronize()
        C = _chunk_lanes(da, prob, n, N, dt)
        _print(f"  max steps {N}, trajectories per chunk {C} ({-(-n // C)} chunks)")
        assert got[0].data_ptr() == out[0].data_ptr()
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
        st = mesh.status.cpu().numpy()
        assert np.all(st == 0) and torch.isfinite(ref[2]).all()


def test_noalloc_rejects_sizes_beyond_the_scratch(da, orc):
    """Lorenz-96 at d = 64 with 4096 steps needs 2 MiB per trajectory at
    checkpoint interval 1, so the scratch holds fewer than 256: the call
    returns DA_EWORKSPACE and leaves the outputs untouched."""
    w, inp, aux, scale = _inputs(orc, 5, 300)
    prob = w.problem()
    u0, p = to_dev(inp["u0"], torch), to_dev(inp["p"], torch)
    mesh, _ = da.record(prob, u0, p, save=False)
    N = da.mesh_max_steps(mesh)
    out = (torch.zeros(300, dtype=torch.float64, device="cuda"),
           torch.zeros((64, 300), dtype=torch.float64, device="cuda"),
           torch.zeros((1, 300), dtype=torch.float64, device="cuda"))
    with pytest.raises(da.DadjError) as ei:
        da.replay_grad_noalloc(prob, u0, p, mesh, 4096, out=out)
    assert ei.value.code == da.DA_EWORKSPACE and "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert all(torch.count_nonzero(t).item() == 0 for t in out)
    # the same mesh at its own largest step count fits, in chunks
    got = da.replay_grad_noalloc(prob, u0, p, mesh, N, out=out)
    ref = da.replay_grad(prob, u0, p, mesh, max_n_steps=N)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
