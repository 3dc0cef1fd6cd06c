"""The C ABI library: it loads without a GPU, exports every entry point that
include/dadj.h declares, and rejects invalid arguments before any launch."""
import ctypes
import os
import re

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dadj.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(da_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def da():
    import discrete_adjoint_amd as da
    return da


def test_library_exports_every_declared_symbol(da):
    names = _declared()
    assert "da_record" in names and "da_replay_grad" in names and "da_solve_fwd" in names
    lib = ctypes.CDLL(da.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(da.EXPORTS)
    assert da.version() >= 100


def _call_record(da, prob, n=4, dtype_code=0, **kw):
    P, keep = da.cproblem(prob, __import__("torch").float64)
    P.dtype = dtype_code
    m = da._Mesh(1, 1, 1, 1, None)
    return da.library().da_record(ctypes.byref(P), n, ctypes.c_void_p(8), ctypes.c_void_p(8),
                                  ctypes.byref(m), None, None)


@pytest.mark.parametrize("change,code", [
    (dict(t1=0.0), -1), (dict(rtol=0.0, atol=0.0), -1), (dict(max_steps=0), -1),
    (dict(dim=4), -1), (dict(method=7), -1), (dict(method=5), -1), (dict(rhs=9), -1),
    (dict(save_times=(0.5, 0.4)), -1), (dict(save_times=(0.5, 2.0)), -1),
    (dict(rtol=-1.0), -1), (dict(safety=-0.5), -1),
])
def test_invalid_problems_rejected(da, change, code):
    prob = W.WORKLOADS[1].problem(**change)
    assert _call_record(da, prob) == code
    assert da.last_error() != ""


def test_unsupported_combinations(da):
    for method in (W.ROS2, W.RODAS3, W.ROS4):
        prob = W.Problem(W.LORENZ96, 64, 1, method, 0.0, 1.0, 1e-6, 1e-6, 100)
        assert _call_record(da, prob) == -2
        assert "Rosenbrock" in da.last_error()
        assert _call_record(da, W.WORKLOADS[4].problem(method=method, dense=1)) == -2
        assert "dense" in da.last_error()
    for method in (W.TSIT5, W.DOPRI5):          # the kinetics system is stiff
        assert _call_record(da, W.WORKLOADS[6].problem(method=method)) == -2
        assert "Rosenbrock" in da.last_error()
    assert _call_record(da, W.WORKLOADS[6].problem(dim=7)) == -1
    assert _call_record(da, W.WORKLOADS[6].problem(method=W.RKF78)) == -2
    assert _call_record(da, W.WORKLOADS[1].problem(method=W.RKF78, dense=1)) == -2
    assert "dense" in da.last_error()
    assert _call_record(da, W.WORKLOADS[5].problem(method=W.RKF78)) == -2
    assert "Lorenz-96" in da.last_error()
    for dim in (3, 65):
        prob = W.Problem(W.LORENZ96, dim, 1, W.TSIT5, 0.0, 1.0, 1e-6, 1e-6, 100)
        assert _call_record(da, prob) == -1


def test_lorenz96_workspace_rows(da):
    """The wavefront kernels keep a whole 64-value row per checkpoint."""
    prob = W.Problem(W.LORENZ96, 40, 1, W.TSIT5, 0.0, 1.0, 1e-6, 1e-6, 100, checkpoint=1)
    assert da.replay_grad_workspace(prob, 100, 50) == 100 * 50 * 64 * 8


def test_bad_dtype_and_sizes(da):
    prob = W.WORKLOADS[1].problem()
    assert _call_record(da, prob, dtype_code=5) == -1
    assert _call_record(da, prob, n=-1) == -1
    assert _call_record(da, prob, n=2**33) == -1


def test_null_pointers_rejected(da):
    prob = W.WORKLOADS[1].problem()
    P, keep = da.cproblem(prob, __import__("torch").float64)
    lib = da.library()
    assert lib.da_record(ctypes.byref(P), 4, None, None, None, None, None) == -1
    m = da._Mesh(1, 1, 1, 1, None)
    assert lib.da_record(ctypes.byref(P), 4, None, ctypes.c_void_p(8), ctypes.byref(m), None,
                         None) == -1
    loss = da._Loss(1, None, 1.0)   # MSE without targets
    assert lib.da_replay_grad(ctypes.byref(P), 4, ctypes.c_void_p(8), ctypes.c_void_p(8),
                              ctypes.byref(m), ctypes.byref(loss), None, None, None, 10,
                              ctypes.c_void_p(8), 1 << 20, None) == -1
    loss = da._Loss(0, None, 1.0)
    m = da._Mesh(128, 8, 8, 8, None)   # plausible (aligned) addresses; nothing is launched
    # workspace for fewer than 256 trajectories
    assert lib.da_replay_grad(ctypes.byref(P), 4096, ctypes.c_void_p(8), ctypes.c_void_p(8),
                              ctypes.byref(m), ctypes.byref(loss), None, None, None, 10,
                              ctypes.c_void_p(8), 100, None) == -4
    assert lib.da_replay_grad(ctypes.byref(P), 4, ctypes.c_void_p(8), ctypes.c_void_p(8),
                              ctypes.byref(m), ctypes.byref(loss), None, None, None, 10**6,
                              ctypes.c_void_p(8), 1 << 30, None) == -1
    # sorting needs a permutation array and workspace
    mo = da._Mesh(128, 8, 8, 8, None)
    assert lib.da_mesh_sort(ctypes.byref(P), 4, ctypes.byref(mo), ctypes.c_void_p(8), 1 << 20,
                            None) == -1
    mo = da._Mesh(128, 8, 8, 8, 8)
    assert lib.da_mesh_sort(ctypes.byref(P), 4, ctypes.byref(mo), ctypes.c_void_p(8), 4,
                            None) == -4
    # a replay table needs 1 <= rows <= max_steps
    mr = da._Mesh(128, 8, 8, 8, 8, 64, 0)
    assert lib.da_replay_fwd(ctypes.byref(P), 4, ctypes.c_void_p(8), ctypes.c_void_p(8),
                             ctypes.byref(mr), ctypes.c_void_p(8), None) == -1
    mr = da._Mesh(128, 8, 8, 8, 8, 64, prob.max_steps + 1)
    assert lib.da_replay_fwd(ctypes.byref(P), 4, ctypes.c_void_p(8), ctypes.c_void_p(8),
                             ctypes.byref(mr), ctypes.c_void_p(8), None) == -1
    assert "rows" in da.last_error()
    # the record writes 128-byte chunks: a step log aligned to 64 bytes only is refused
    mu = da._Mesh(192, 8, 8, 8, None)
    assert lib.da_record(ctypes.byref(P), 4, ctypes.c_void_p(8), ctypes.c_void_p(8),
                         ctypes.byref(mu), None, None) == -1
    assert "aligned" in da.last_error()


def test_dense_output_checks(da):
    """Dense output: flag 0/1, explicit methods only, and the mesh must carry
    save_theta wherever a save is read."""
    lib = da.library()
    assert _call_record(da, W.WORKLOADS[1].problem(dense=2)) == -1
    assert "dense" in da.last_error()
    assert _call_record(da, W.WORKLOADS[4].problem(dense=1)) == -2
    prob = W.WORKLOADS[3].problem(dense=1)
    P, keep = da.cproblem(prob, __import__("torch").float32)
    m = da._Mesh(128, 8, 8, 8, None)          # aligned fake addresses, no save_theta
    args = (ctypes.c_void_p(8), ctypes.c_void_p(8), ctypes.byref(m))
    assert lib.da_record(ctypes.byref(P), 4, *args, None, None) == -1
    assert "save_theta" in da.last_error()
    assert lib.da_replay_fwd(ctypes.byref(P), 4, *args, ctypes.c_void_p(8), None) == -1
    assert "save_theta" in da.last_error()
    loss = da._Loss(1, ctypes.c_void_p(8), 1.0)
    assert lib.da_replay_grad(ctypes.byref(P), 4, *args, ctypes.byref(loss), None, None, None,
                              10, ctypes.c_void_p(8), 1 << 20, None) == -1
    assert "save_theta" in da.last_error()
    assert lib.da_replay_sens(ctypes.byref(P), 4, *args, None, None, None, None,
                              ctypes.c_void_p(8), None) == -1
    assert "save_theta" in da.last_error()


def test_sensitivity_direction_range_checks(da):
    """da_replay_sens_dirs refuses an empty range and one outside the d + P
    directions before it touches any buffer."""
    lib = da.library()
    for prob, Q in ((W.WORKLOADS[1].problem(), 6), (W.WORKLOADS[5].problem(), 65)):
        P, keep = da.cproblem(prob, __import__("torch").float64)
        m = da._Mesh(128, 8, 8, 8, None)          # aligned fake addresses
        args = (ctypes.c_void_p(8), ctypes.c_void_p(8), ctypes.byref(m))
        for qb, qc in ((0, 0), (-1, 2), (0, Q + 1), (Q - 1, 2), (Q, 1), (2, -3)):
            rc = lib.da_replay_sens_dirs(ctypes.byref(P), 4, *args, qb, qc, None, None, None,
                                         None, None)
            assert rc == -1, (qb, qc)
            assert "q_count" in da.last_error() or "direction range" in da.last_error()
        # an empty ensemble with a valid range is a no-op
        assert lib.da_replay_sens_dirs(ctypes.byref(P), 0, *args, Q - 1, 1, None, None, None,
                                       None, None) == 0


def test_rhs_registration_checks(da):
    """Argument checks of da_rhs_register, and compilation, which needs no
    GPU: a source with an error is refused with the compiler's message; a
    correct one compiles and then loads (or, without a device, says so)."""
    import torch
    lib = da.library()
    rid = ctypes.c_int32(-1)
    assert lib.da_rhs_register(None, ctypes.byref(rid)) == -1
    good = "dy[0] = -p[0] * y[0];"
    for dim, npar, dt, meth, body, code in [(0, 1, 0, 0, good, -1), (17, 1, 0, 0, good, -1),
                                            (1, 0, 0, 0, good, -1), (1, 17, 0, 0, good, -1),
                                            (1, 1, 5, 0, good, -1), (1, 1, 0, 2, good, -2),
                                            (1, 1, 0, 0, None, -1)]:
        d = da._RhsDef(dim, npar, dt, meth, None if body is None else body.encode())
        assert lib.da_rhs_register(ctypes.byref(d), ctypes.byref(rid)) == code, (dim, npar, dt,
                                                                                 meth)
    with pytest.raises(da.DadjError) as e:
        da.register_rhs("dy[0] = y[0] +;", 1, 1)
    assert e.value.code == -1 and "expected expression" in str(e.value)
    try:
        got = da.register_rhs(good, 1, 1, torch.float64, 1)
        da.release_rhs(got)
    except da.DadjError as err:
        assert err.code == -3 and "no current HIP device" in str(err)
    assert lib.da_rhs_release(5) == -1


def test_stencil_registration_checks(da):
    """Argument checks of da_rhs_register_stencil (dimension 2..64, 1..16
    parameters, 1..7 distinct offsets in [-3, 3], an explicit method), and a
    source with an error refused with the compiler's message; no GPU needed."""
    lib = da.library()
    rid = ctypes.c_int32(-1)
    assert lib.da_rhs_register_stencil(None, ctypes.byref(rid)) == -1
    good = "return p[0] * (y(1) - y(-1));"
    for dim, npar, dt, meth, offs, body, code in [
            (1, 1, 0, 0, (-1, 1), good, -1), (65, 1, 0, 0, (-1, 1), good, -1),
            (8, 0, 0, 0, (-1, 1), good, -1), (8, 17, 0, 0, (-1, 1), good, -1),
            (8, 1, 2, 0, (-1, 1), good, -1), (8, 1, 0, 2, (-1, 1), good, -2),
            (8, 1, 0, 0, (), good, -1), (8, 1, 0, 0, (-4, 1), good, -1),
            (8, 1, 0, 0, (-1, 4), good, -1), (8, 1, 0, 0, (1, -1, 1), good, -1),
            (8, 1, 0, 0, tuple(range(-3, 4)) + (0,), good, -1),
            (8, 1, 0, 0, (-1, 1), None, -1)]:
        arr = (ctypes.c_int32 * max(1, len(offs)))(*offs)
        d = da._RhsStencilDef(dim, npar, dt, meth, len(offs),
                              ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)),
                              None if body is None else body.encode())
        assert lib.da_rhs_register_stencil(ctypes.byref(d), ctypes.byref(rid)) == code, (
            dim, npar, dt, meth, offs)
    with pytest.raises(da.DadjError) as e:
        da.register_rhs_stencil("return y(0) +;", 8, 1, (0,))
    assert e.value.code == -1 and "expected expression" in str(e.value)


@pytest.mark.parametrize("ck", [3, 5, 16, -1])
def test_bad_checkpoint_rejected(da, ck):
    prob = W.WORKLOADS[1].problem(checkpoint=ck)
    assert _call_record(da, prob) == -1
    assert "checkpoint" in da.last_error()


def test_workspace_sizes(da):
    import torch
    prob = W.WORKLOADS[2].problem(checkpoint=1)
    assert da.replay_grad_workspace(prob, 1000, 700) == 1000 * 700 * 3 * 8
    assert da.replay_grad_workspace(prob, 1000, 700, torch.float32) == 1000 * 700 * 3 * 4
    for ck in (2, 4, 8):
        assert da.replay_grad_workspace(prob.replace(checkpoint=ck), 1000, 700) == \
            1000 * ((700 + ck - 1) // ck) * 3 * 8
    assert da.replay_grad_workspace(prob.replace(checkpoint=0), 1000, 700) > 0
    assert da.mesh_sort_workspace(prob, 1 << 20) >= 3 * 4 * (1 << 20)


def test_default_checkpoint_interval(da):
    """The library's checkpoint interval (checkpoint = 0), read from the
    workspace it asks for: on built-in systems of up to four components other
    than Lorenz-96, without dense output and with no save times, 4 for ROS2
    and 2 for Tsit5, Dopri5, Rodas3 and the fourth-order Rosenbrock method in
    FP64, 4 for all five in FP32; 2 for ROS2 in FP64 with save times; 1 for
    every other method, dimension, save times and right-hand side."""
    import torch

    def interval(prob, dt=torch.float64, n=1000, N=700):
        row = 64 if prob.rhs == W.LORENZ96 else prob.dim
        size = dt.itemsize
        ws = da.replay_grad_workspace(prob.replace(checkpoint=0), n, N, dt)
        for ck in (1, 2, 4, 8):
            if ws == n * ((N + ck - 1) // ck) * row * size:
                return ck
        raise AssertionError(ws)

    rob = W.WORKLOADS[4].problem()                                      # ROS2, Robertson
    assert rob.save_times == ()
    assert interval(rob) == 4
    assert interval(rob.replace(save_times=(1.0, 1e5))) == 2
    assert interval(rob, torch.float32) == 4
    assert interval(rob.replace(save_times=(1.0, 1e5)), torch.float32) == 1
    assert interval(W.WORKLOADS[1].problem(method=W.ROS2)) == 4        # ROS2, Lorenz-63
    assert interval(W.WORKLOADS[6].problem(method=W.ROS2)) == 1        # ROS2, d = 8
    for m in (W.RODAS3, W.ROS4):
        assert interval(W.WORKLOADS[4].problem(method=m)) == 2
        assert interval(W.WORKLOADS[4].problem(method=m), torch.float32) == 4
        assert interval(W.WORKLOADS[4].problem(method=m, save_times=(1.0, 1e5))) == 1
        assert interval(W.WORKLOADS[6].problem(method=m)) == 1          # d = 8
    for wid in (1, 2):                                                  # Tsit5, Dopri5
        prob = W.WORKLOADS[wid].problem()
        assert prob.save_times == ()
        assert interval(prob) == 2
        assert interval(prob, torch.float32) == 4
        assert interval(prob.replace(save_times=(0.5, 1.0))) == 1
        assert interval(prob.replace(save_times=(0.5, 1.0), dense=1)) == 1
    for wid in (3, 5, 6):          # FP32 with saves, Lorenz-96, the kinetics system
        assert interval(W.WORKLOADS[wid].problem()) == 1
    assert interval(W.WORKLOADS[5].problem(dim=4)) == 1                 # Lorenz-96 at d = 4
    assert interval(W.WORKLOADS[2].problem(method=W.RKF78)) == 1
    # the entry point that reports it
    assert da.checkpoint_interval(W.WORKLOADS[4].problem()) == 4
    assert da.checkpoint_interval(W.WORKLOADS[4].problem(), torch.float32) == 4
    assert da.checkpoint_interval(W.WORKLOADS[2].problem()) == 2
    assert da.checkpoint_interval(W.WORKLOADS[3].problem()) == 1
    assert da.checkpoint_interval(W.WORKLOADS[2].problem(checkpoint=4)) == 4
    assert da.checkpoint_interval(W.WORKLOADS[4].problem(checkpoint=3)) == 0


def test_step_log_length(da):
    import torch
    lib = da.library()
    for wid, dt, B in ((2, torch.float64, 16), (3, torch.float32, 32)):
        prob = W.WORKLOADS[wid].problem(max_steps=1001)
        P, keep = da.cproblem(prob, dt)
        assert lib.da_mesh_h_elems(ctypes.byref(P), 300) == ((1001 + B - 1) // B) * 300 * B
        assert da.mesh_h_shape(prob, 300, dt) == ((1001 + B - 1) // B, 300, B)
        assert lib.da_mesh_h_elems(ctypes.byref(P), 0) == 0
