"""Mesh files (save_mesh / load_mesh): a record written and read back on the
host gives the same arrays; a file is refused for another problem, another
dtype's shapes or a foreign archive.  (The GPU test replays a loaded mesh
and compares bit for bit.)"""
import numpy as np
import pytest

import workloads as W

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def da():
    import discrete_adjoint_amd as da
    return da


def _host_mesh(da, prob, n, dt, rng):
    T, _, B = da.mesh_h_shape(prob, n, dt)
    S = max(1, len(prob.save_times))
    ns = rng.integers(1, prob.max_steps, n).astype(np.int32)
    h = np.zeros((n, T * B))
    for i in range(n):
        h[i, :ns[i]] = rng.random(ns[i]) + 1e-3
    h = torch.from_numpy(np.ascontiguousarray(h.reshape(n, T, B).transpose(1, 0, 2))).to(dt)
    return da.Mesh(h, torch.from_numpy(ns),
                   torch.from_numpy(rng.integers(0, 50, (S, n)).astype(np.int32)),
                   torch.from_numpy(rng.integers(0, 3, n).astype(np.int32)),
                   torch.from_numpy(rng.permutation(n).astype(np.int32)), None,
                   torch.from_numpy(rng.random((S, n))).to(dt),
                   torch.from_numpy((ns + rng.integers(0, 9, n)).astype(np.int32)))


@pytest.mark.parametrize("dt", [torch.float64, torch.float32])
def test_mesh_round_trip_on_the_host(da, tmp_path, dt):
    prob = W.WORKLOADS[3].problem(max_steps=37)
    m = _host_mesh(da, prob, 50, dt, np.random.default_rng(1))
    path = tmp_path / "mesh.npz"
    da.save_mesh(path, prob, m)
    r = da.load_mesh(path, prob, device="cpu")
    for k in ("h", "n_steps", "save_idx", "status", "perm", "save_theta", "n_attempts"):
        assert torch.equal(getattr(m, k), getattr(r, k)), k
    assert r.h_rows is None and r.h.dtype == dt
    # without the optional arrays
    m2 = da.Mesh(m.h, m.n_steps, m.save_idx, m.status)
    da.save_mesh(path, prob, m2)
    r2 = da.load_mesh(path, prob, device="cpu")
    assert r2.perm is None and r2.save_theta is None and r2.n_attempts is None
    assert torch.equal(r2.h, m.h)


def test_mesh_file_refused_for_another_problem(da, tmp_path):
    prob = W.WORKLOADS[3].problem(max_steps=37)
    m = _host_mesh(da, prob, 20, torch.float32, np.random.default_rng(2))
    path = tmp_path / "mesh.npz"
    da.save_mesh(path, prob, m)
    for other in (prob.replace(max_steps=38), prob.replace(t1=4.0), prob.replace(method=W.DOPRI5),
                  prob.replace(save_times=(1.0, 5.0)), prob.replace(dense=1)):
        with pytest.raises(ValueError):
            da.load_mesh(path, other, device="cpu")
    np.savez(tmp_path / "other.npz", h=np.zeros(3))
    with pytest.raises(ValueError):
        da.load_mesh(tmp_path / "other.npz", prob, device="cpu")
