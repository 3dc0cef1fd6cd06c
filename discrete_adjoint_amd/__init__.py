"""MI355X record-and-replay discrete adjoint for ODE ensembles.

Thin Python binding of ``libdadj.so`` (declared in ``include/dadj.h``): it
checks and marshals torch tensors (device pointers, the current HIP stream)
and calls the C ABI.  Every step of the computation runs in the library's HIP
kernels; there is no fallback.  Importing fails loudly if the library has not
been built (``python discrete_adjoint_amd/_build.py`` or
``__graft_entry__.build()``).

Layout: per-trajectory tensors are component-major, shape [C, n] (trajectory
index last and contiguous): u0 [d, n], p [P, n], y_save [S, d, n], grad_u0
[d, n], grad_p [P, n], with S = max(1, len(problem.save_times)).  The mesh is
h [T, n, B] (tiled step log: B = 16 steps per 128-byte chunk in float64, 32 in
float32, T = ceil(max_steps / B); ``Mesh.steps()`` gives the [n, max_steps]
view), n_steps [n], save_idx [S, n], status [n], perm [n] or None (a
replay order), h_rows [rows, n] or None (the replay table: step k of the
trajectory of lane j at [k, j]; ``mesh_sort`` fills these two) and
save_theta [S, n] (the step fraction of each save: 1 where steps land on the
save times, the interpolation point with ``problem.dense = 1``).

The problem description is ``workloads.Problem`` (or any object with the same
fields) plus a dtype taken from the tensors.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# DADJ_LIBRARY may name another build of the same sources (e.g. one made
# with different build options); the default is the in-tree libdadj.so.
LIB_PATH = os.environ.get("DADJ_LIBRARY") or os.path.join(_HERE, "libdadj.so")

DA_F64, DA_F32 = 0, 1
TSIT5, DOPRI5, ROS2, RODAS3, RKF78, ROS4 = 0, 1, 2, 3, 4, 5
LINEAR, LORENZ63, ROBERTSON, LORENZ96 = 0, 1, 2, 3
SUMSQ_FINAL, MSE_SAVE, COTANGENT = 0, 1, 2
LANE_OK, LANE_MAX_STEPS, LANE_DT_UNDERFLOW, LANE_NONFINITE, LANE_MAX_ATTEMPTS = range(5)
DA_OK, DA_EINVAL, DA_EUNSUPPORTED, DA_EHIP, DA_EWORKSPACE = 0, -1, -2, -3, -4
MAX_SAVES = 128

EXPORTS = ("da_record", "da_solve_fwd", "da_mesh_h_elems", "da_mesh_sort_workspace", "da_mesh_sort",
           "da_mesh_pad",
           "da_mesh_max_steps", "da_replay_fwd", "da_replay_grad_workspace", "da_replay_grad",
           "da_replay_grad_noalloc", "da_checkpoint_interval",
           "da_replay_sens", "da_replay_sens_dirs", "da_rhs_register", "da_rhs_register_stencil",
           "da_rhs_release", "da_last_error", "da_version")


class DadjError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dadj error {code}: {msg}")
        self.code = code


class _Problem(ctypes.Structure):
    _fields_ = [
        ("rhs", ctypes.c_int32), ("dim", ctypes.c_int32), ("n_params", ctypes.c_int32),
        ("method", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("t0", ctypes.c_double), ("t1", ctypes.c_double),
        ("rtol", ctypes.c_double), ("atol", ctypes.c_double), ("dt0", ctypes.c_double),
        ("max_steps", ctypes.c_int32), ("max_attempts", ctypes.c_int32),
        ("n_save", ctypes.c_int32), ("save_times", ctypes.POINTER(ctypes.c_double)),
        ("safety", ctypes.c_double), ("fac_min", ctypes.c_double), ("fac_max", ctypes.c_double),
        ("checkpoint", ctypes.c_int32), ("dense", ctypes.c_int32),
    ]


class _Mesh(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("n_steps", ctypes.c_void_p),
                ("save_idx", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("perm", ctypes.c_void_p), ("h_rows", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("save_theta", ctypes.c_void_p),
                ("defer_pad", ctypes.c_int32), ("n_attempts", ctypes.c_void_p)]


class _RhsDef(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int32), ("n_params", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("method", ctypes.c_int32), ("f_body", ctypes.c_char_p)]


class _RhsStencilDef(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int32), ("n_params", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("method", ctypes.c_int32), ("n_offsets", ctypes.c_int32),
                ("offsets", ctypes.POINTER(ctypes.c_int32)), ("f_body", ctypes.c_char_p)]


class _Loss(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("aux", ctypes.c_void_p), ("scale", ctypes.c_double)]


def _load_library() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                          "(python discrete_adjoint_amd/_build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    P = ctypes.POINTER(_Problem)
    M = ctypes.POINTER(_Mesh)
    lib.da_record.argtypes = [P, i64, vp, vp, M, vp, vp]
    lib.da_solve_fwd.argtypes = [P, i64, vp, vp, vp, vp, vp, vp]
    lib.da_mesh_h_elems.argtypes = [P, i64]
    lib.da_mesh_h_elems.restype = ctypes.c_int64
    lib.da_mesh_sort_workspace.argtypes = [P, i64]
    lib.da_mesh_sort_workspace.restype = ctypes.c_size_t
    lib.da_mesh_sort.argtypes = [P, i64, M, vp, ctypes.c_size_t, vp]
    lib.da_mesh_max_steps.argtypes = [i64, M, ctypes.POINTER(ctypes.c_int32), vp]
    lib.da_mesh_pad.argtypes = [P, i64, M, vp]
    lib.da_replay_fwd.argtypes = [P, i64, vp, vp, M, vp, vp]
    lib.da_replay_grad_workspace.argtypes = [P, i64, i32]
    lib.da_replay_grad_workspace.restype = ctypes.c_size_t
    lib.da_checkpoint_interval.argtypes = [P]
    lib.da_checkpoint_interval.restype = ctypes.c_int32
    lib.da_replay_grad.argtypes = [P, i64, vp, vp, M, ctypes.POINTER(_Loss), vp, vp, vp, i32, vp,
                                   ctypes.c_size_t, vp]
    lib.da_replay_grad_noalloc.argtypes = [P, i64, vp, vp, M, ctypes.POINTER(_Loss), vp, vp, vp,
                                           i32, vp]
    lib.da_replay_sens.argtypes = [P, i64, vp, vp, M, ctypes.POINTER(_Loss), vp, vp, vp, vp, vp]
    lib.da_replay_sens_dirs.argtypes = [P, i64, vp, vp, M, i32, i32, ctypes.POINTER(_Loss), vp,
                                        vp, vp, vp]
    lib.da_rhs_register.argtypes = [ctypes.POINTER(_RhsDef), ctypes.POINTER(ctypes.c_int32)]
    lib.da_rhs_register_stencil.argtypes = [ctypes.POINTER(_RhsStencilDef),
                                            ctypes.POINTER(ctypes.c_int32)]
    lib.da_rhs_release.argtypes = [i32]
    lib.da_last_error.restype = ctypes.c_char_p
    for name in ("da_record", "da_solve_fwd", "da_mesh_sort", "da_mesh_max_steps", "da_mesh_pad",
                 "da_replay_fwd", "da_replay_grad", "da_replay_grad_noalloc", "da_replay_sens",
                 "da_replay_sens_dirs",
                 "da_rhs_register", "da_rhs_register_stencil",
                 "da_rhs_release", "da_version"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


_lib = _load_library()


def library() -> ctypes.CDLL:
    return _lib


def version() -> int:
    return _lib.da_version()


def last_error() -> str:
    return _lib.da_last_error().decode()


def _check(rc: int):
    if rc != DA_OK:
        raise DadjError(rc, last_error())


def register_rhs(f_body: str, dim: int, n_params: int, dtype=torch.float64,
                 method: int = 0) -> int:
    """Compile the kernels for a right-hand side given as the C++ body of
    ``template <class T> void f(const T *y, const T *p, T *dy)`` (see
    da_rhs_register in include/dadj.h) for one dtype and explicit method
    (0 = Tsit5, 1 = Dopri5).  Returns the rhs identifier for the problem."""
    rid = ctypes.c_int32(0)
    d = _RhsDef(dim, n_params, _dtype_code(dtype), method, f_body.encode())
    _check(_lib.da_rhs_register(ctypes.byref(d), ctypes.byref(rid)))
    return int(rid.value)


def register_rhs_stencil(f_body: str, dim: int, n_params: int, offsets, dtype=torch.float64,
                         method: int = 0) -> int:
    """Compile the wavefront kernels for a cyclic-stencil right-hand side of
    dimension up to 64: component i of f is the C++ body of
    ``template <class T, class Y> T f(const Y &y, const T *p)`` with y(o) the
    component i + o (mod dim) for each o in `offsets` (see
    da_rhs_register_stencil in include/dadj.h).  Returns the rhs identifier."""
    offs = (ctypes.c_int32 * len(offsets))(*[int(o) for o in offsets])
    rid = ctypes.c_int32(0)
    d = _RhsStencilDef(dim, n_params, _dtype_code(dtype), method, len(offsets),
                       ctypes.cast(offs, ctypes.POINTER(ctypes.c_int32)), f_body.encode())
    _check(_lib.da_rhs_register_stencil(ctypes.byref(d), ctypes.byref(rid)))
    return int(rid.value)


def release_rhs(rhs_id: int) -> None:
    """Unload the kernels of a registered right-hand side."""
    _check(_lib.da_rhs_release(rhs_id))


def _dtype_code(dt) -> int:
    if dt == torch.float64:
        return DA_F64
    if dt == torch.float32:
        return DA_F32
    raise TypeError(f"unsupported dtype {dt}")


def cproblem(prob, dtype) -> tuple:
    """ctypes problem struct (and the array that backs save_times, which the
    caller keeps alive).  The pointer is made from the array's address: a
    cast of the array itself ties the two in a reference cycle, and freeing
    those by the cycle collector made each call about ten times slower."""
    st = (ctypes.c_double * max(1, len(prob.save_times)))(*prob.save_times)
    P = _Problem(prob.rhs, prob.dim, prob.n_params, prob.method, _dtype_code(dtype),
                 prob.t0, prob.t1, prob.rtol, prob.atol, prob.dt0, prob.max_steps,
                 prob.max_attempts, len(prob.save_times),
                 ctypes.cast(ctypes.addressof(st), ctypes.POINTER(ctypes.c_double))
                 if len(prob.save_times) else None,
                 prob.safety, prob.fac_min, prob.fac_max, getattr(prob, "checkpoint", 0),
                 getattr(prob, "dense", 0))
    return P, st


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, shape, dtype, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def chunk_steps(dtype) -> int:
    """Steps per 128-byte chunk of the step log."""
    return 16 if dtype == torch.float64 else 32


@dataclasses.dataclass
class Mesh:
    """The record: tiled step log h [T, n, B], n_steps [n], save_idx [S, n],
    status [n]; an optional replay order perm [n] (None = identity) and
    replay table h_rows [rows, n]; save fractions save_theta [S, n] (needed
    with dense output); the record's trial steps n_attempts [n] (accepted
    plus rejected; written by the record when present)."""
    h: torch.Tensor
    n_steps: torch.Tensor
    save_idx: torch.Tensor
    status: torch.Tensor
    perm: Optional[torch.Tensor] = None
    h_rows: Optional[torch.Tensor] = None
    save_theta: Optional[torch.Tensor] = None
    n_attempts: Optional[torch.Tensor] = None

    @property
    def n(self) -> int:
        return self.n_steps.shape[0]

    def steps(self, max_steps: Optional[int] = None) -> torch.Tensor:
        """Step sizes as an [n, K] tensor (a copy), K = max_steps or T * B."""
        T, n, B = self.h.shape
        out = self.h.permute(1, 0, 2).reshape(n, T * B)
        return (out if max_steps is None else out[:, :max_steps]).contiguous()

    def c(self) -> _Mesh:
        return _Mesh(self.h.data_ptr(), self.n_steps.data_ptr(), self.save_idx.data_ptr(),
                     self.status.data_ptr(), None if self.perm is None else self.perm.data_ptr(),
                     None if self.h_rows is None else self.h_rows.data_ptr(),
                     0 if self.h_rows is None else self.h_rows.shape[0],
                     None if self.save_theta is None else self.save_theta.data_ptr(), 0,
                     None if self.n_attempts is None else self.n_attempts.data_ptr())


def mesh_h_shape(prob, n: int, dtype) -> tuple:
    B = chunk_steps(dtype)
    return ((prob.max_steps + B - 1) // B, n, B)


def empty_mesh(prob, n: int, dtype, device="cuda", with_perm: bool = False) -> Mesh:
    S = max(1, len(prob.save_times))
    h = torch.empty(mesh_h_shape(prob, n, dtype), dtype=dtype, device=device)
    P, keep = cproblem(prob, dtype)
    assert h.numel() == _lib.da_mesh_h_elems(ctypes.byref(P), n) or n == 0
    return Mesh(h,
                torch.empty(n, dtype=torch.int32, device=device),
                torch.empty((S, n), dtype=torch.int32, device=device),
                torch.empty(n, dtype=torch.int32, device=device),
                torch.empty(n, dtype=torch.int32, device=device) if with_perm else None,
                None,
                torch.empty((S, n), dtype=dtype, device=device),
                torch.empty(n, dtype=torch.int32, device=device))


def _inputs(prob, u0: torch.Tensor, p: torch.Tensor):
    n = u0.shape[-1]
    _need(u0, (prob.dim, n), u0.dtype, "u0")
    _need(p, (prob.n_params, n), u0.dtype, "p")
    return n, u0.dtype


def record(prob, u0, p, mesh: Optional[Mesh] = None, save: bool = True, stream=None,
           defer_pad: bool = False):
    """Adaptive solve per trajectory; returns (mesh, y_save or None).  With
    ``defer_pad`` the chunks after each trajectory's last step are left for
    ``mesh_pad`` (which nothing on the replay path waits for)."""
    n, dt = _inputs(prob, u0, p)
    S = max(1, len(prob.save_times))
    if mesh is None:
        mesh = empty_mesh(prob, n, dt, u0.device)
    ys = torch.empty((S, prob.dim, n), dtype=dt, device=u0.device) if save else None
    P, keep = cproblem(prob, dt)
    cm = mesh.c()
    cm.defer_pad = int(defer_pad)
    _check(_lib.da_record(ctypes.byref(P), n, _ptr(u0), _ptr(p), ctypes.byref(cm), _ptr(ys),
                          _stream(stream)))
    return mesh, ys


def solve_fwd(prob, u0, p, stream=None):
    """Forward-only adaptive solve: (y_save [S, d, n], n_steps [n], status [n])."""
    n, dt = _inputs(prob, u0, p)
    S = max(1, len(prob.save_times))
    ys = torch.empty((S, prob.dim, n), dtype=dt, device=u0.device)
    ns = torch.empty(n, dtype=torch.int32, device=u0.device)
    st = torch.empty(n, dtype=torch.int32, device=u0.device)
    P, keep = cproblem(prob, dt)
    _check(_lib.da_solve_fwd(ctypes.byref(P), n, _ptr(u0), _ptr(p), _ptr(ys), _ptr(ns), _ptr(st),
                             _stream(stream)))
    return ys, ns, st


def mesh_sort_workspace(prob, n: int, dtype=torch.float64) -> int:
    P, keep = cproblem(prob, dtype)
    return int(_lib.da_mesh_sort_workspace(ctypes.byref(P), n))


def mesh_sort(prob, mesh: Mesh, perm: Optional[torch.Tensor] = None, table: bool = True,
              rows: Optional[int] = None, h_rows: Optional[torch.Tensor] = None,
              workspace=None, stream=None) -> Mesh:
    """The same record with a replay order by decreasing step count and, with
    ``table``, the replay table of ``rows`` rows (default: the largest step
    count, read back from the GPU).  Returns a new Mesh that shares the
    record's arrays; ``perm`` and ``h_rows`` may be given to reuse storage."""
    n = mesh.n
    dt = mesh.h.dtype
    dev = mesh.h.device
    if perm is None:
        perm = torch.empty(n, dtype=torch.int32, device=dev)
    if table and h_rows is None:
        if rows is None:
            rows = max(1, mesh_max_steps(mesh, stream))
        h_rows = torch.empty((rows, n), dtype=dt, device=dev)
    if not table:
        h_rows = None
    need = mesh_sort_workspace(prob, n, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    out = Mesh(mesh.h, mesh.n_steps, mesh.save_idx, mesh.status, perm, h_rows, mesh.save_theta,
               mesh.n_attempts)
    P, keep = cproblem(prob, dt)
    co = out.c()
    _check(_lib.da_mesh_sort(ctypes.byref(P), n, ctypes.byref(co), _ptr(workspace),
                             workspace.numel(), _stream(stream)))
    return out


# Mesh files: a numpy .npz archive of plain arrays (no pickled objects).
MESH_FORMAT = 2  # 2: 128-byte chunks in the step log (1: 64-byte)
# problem fields a record depends on: a mesh is replayed only under these
_MESH_KEYS = ("rhs", "dim", "n_params", "method", "t0", "t1", "max_steps", "dense")


def save_mesh(path, prob, mesh: Mesh) -> None:
    """Write the record to `path` (.npz): the tiled step log, n_steps,
    save_idx, status, save_theta, n_attempts and the replay order when set
    (the replay table is rebuilt on load), with the problem fields it
    depends on (right-hand side, dimensions, method, interval, save times,
    max_steps, dense output) and the dtype.  The record is the artefact that
    is replayed for many gradient passes until a re-record, so it can be kept
    across processes."""
    import numpy as np
    arrays = {"format": np.int64(MESH_FORMAT),
              "dtype": np.array(str(mesh.h.dtype).replace("torch.", "")),
              "save_times": np.asarray(prob.save_times, dtype=np.float64),
              "h": mesh.h.cpu().numpy(), "n_steps": mesh.n_steps.cpu().numpy(),
              "save_idx": mesh.save_idx.cpu().numpy(), "status": mesh.status.cpu().numpy()}
    for k in _MESH_KEYS:
        arrays["prob_" + k] = np.asarray(getattr(prob, k))
    for k in ("save_theta", "n_attempts", "perm"):
        t = getattr(mesh, k)
        if t is not None:
            arrays[k] = t.cpu().numpy()
    with open(path, "wb") as f:
        np.savez(f, **arrays)


def load_mesh(path, prob, device="cuda", table: bool = True) -> Mesh:
    """Read a record written by save_mesh and check it against `prob` (the
    fields it depends on, the save times and the array shapes).  With a
    stored replay order and `table`, the replay table is rebuilt on a GPU
    device (da_mesh_sort, which recomputes the order; it must equal the
    stored one).  Raises ValueError on any mismatch."""
    import numpy as np
    with np.load(path, allow_pickle=False) as z:
        d = {k: z[k] for k in z.files}
    if int(d.get("format", -1)) != MESH_FORMAT:
        raise ValueError(f"{path}: not a mesh file of format {MESH_FORMAT}")
    for k in _MESH_KEYS:
        want, got = getattr(prob, k), d["prob_" + k].item()
        if want != got:
            raise ValueError(f"{path}: recorded with {k} = {got}, the problem has {want}")
    if not np.array_equal(d["save_times"], np.asarray(prob.save_times, dtype=np.float64)):
        raise ValueError(f"{path}: recorded with other save times")
    dt = {"float64": torch.float64, "float32": torch.float32}[str(d["dtype"])]
    n = d["n_steps"].shape[0]
    S = max(1, len(prob.save_times))
    shapes = {"h": mesh_h_shape(prob, n, dt), "save_idx": (S, n), "status": (n,),
              "save_theta": (S, n), "n_attempts": (n,), "perm": (n,)}
    for k, shp in shapes.items():
        if k in d and tuple(d[k].shape) != tuple(shp):
            raise ValueError(f"{path}: {k} has shape {d[k].shape}, expected {shp}")

    def dev(k):
        return None if k not in d else torch.from_numpy(np.ascontiguousarray(d[k])).to(device)
    mesh = Mesh(dev("h"), dev("n_steps"), dev("save_idx"), dev("status"), dev("perm"), None,
                dev("save_theta"), dev("n_attempts"))
    if mesh.perm is not None and table and torch.device(device).type == "cuda":
        sm = mesh_sort(prob, Mesh(mesh.h, mesh.n_steps, mesh.save_idx, mesh.status, None, None,
                                  mesh.save_theta, mesh.n_attempts))
        if not torch.equal(sm.perm, mesh.perm):
            raise ValueError(f"{path}: the stored replay order is not the record's")
        mesh = sm
    return mesh


def mesh_pad(prob, mesh: Mesh, stream=None) -> None:
    """Zero padding of a record taken with ``defer_pad`` (on ``stream``,
    which must be ordered after the record)."""
    P, keep = cproblem(prob, mesh.h.dtype)
    cm = mesh.c()
    _check(_lib.da_mesh_pad(ctypes.byref(P), mesh.n, ctypes.byref(cm), _stream(stream)))


def mesh_max_steps(mesh: Mesh, stream=None) -> int:
    out = ctypes.c_int32(0)
    cm = mesh.c()
    _check(_lib.da_mesh_max_steps(mesh.n, ctypes.byref(cm), ctypes.byref(out), _stream(stream)))
    return int(out.value)


def replay_fwd(prob, u0, p, mesh: Mesh, stream=None) -> torch.Tensor:
    """Fixed-step replay; returns y_save [S, d, n] (trajectory order)."""
    n, dt = _inputs(prob, u0, p)
    S = max(1, len(prob.save_times))
    ys = torch.empty((S, prob.dim, n), dtype=dt, device=u0.device)
    P, keep = cproblem(prob, dt)
    cm = mesh.c()
    _check(_lib.da_replay_fwd(ctypes.byref(P), n, _ptr(u0), _ptr(p), ctypes.byref(cm), _ptr(ys),
                              _stream(stream)))
    return ys


def replay_grad_workspace(prob, n: int, max_n_steps: int, dtype=torch.float64) -> int:
    P, keep = cproblem(prob, dtype)
    return int(_lib.da_replay_grad_workspace(ctypes.byref(P), n, max_n_steps))


def checkpoint_interval(prob, dtype=torch.float64) -> int:
    """The reverse sweep's checkpoint interval for prob (its own, or the
    library's choice when prob.checkpoint is 0)."""
    P, keep = cproblem(prob, dtype)
    return int(_lib.da_checkpoint_interval(ctypes.byref(P)))


class ReplayGrad:
    """Reusable replay-gradient call: holds outputs and workspace so that
    repeated passes against one record allocate nothing."""

    def __init__(self, prob, u0, p, mesh: Mesh, loss_kind: int = SUMSQ_FINAL, aux=None,
                 scale: float = 1.0, max_n_steps: Optional[int] = None,
                 ws_bytes: Optional[int] = None):
        n, dt = _inputs(prob, u0, p)
        S = max(1, len(prob.save_times))
        if aux is not None:
            _need(aux, (S, prob.dim, n), dt, "aux")
        self.prob, self.u0, self.p, self.mesh, self.aux = prob, u0, p, mesh, aux
        self.n = n
        self.max_n_steps = mesh_max_steps(mesh) if max_n_steps is None else int(max_n_steps)
        need = replay_grad_workspace(prob, n, self.max_n_steps, dt)
        nb = need if ws_bytes is None else int(ws_bytes)
        self.ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=u0.device)
        self.loss = torch.empty(n, dtype=dt, device=u0.device)
        self.grad_u0 = torch.empty((prob.dim, n), dtype=dt, device=u0.device)
        self.grad_p = torch.empty((prob.n_params, n), dtype=dt, device=u0.device)
        self._P, self._keep = cproblem(prob, dt)
        self._cm = mesh.c()
        self._loss = _Loss(loss_kind, None if aux is None else aux.data_ptr(), scale)

    def __call__(self, stream=None):
        _check(_lib.da_replay_grad(ctypes.byref(self._P), self.n, _ptr(self.u0), _ptr(self.p),
                                   ctypes.byref(self._cm), ctypes.byref(self._loss),
                                   _ptr(self.loss), _ptr(self.grad_u0), _ptr(self.grad_p),
                                   self.max_n_steps, _ptr(self.ws), self.ws.numel(),
                                   _stream(stream)))
        return self.loss, self.grad_u0, self.grad_p


def replay_grad(prob, u0, p, mesh: Mesh, loss_kind: int = SUMSQ_FINAL, aux=None,
                scale: float = 1.0, max_n_steps: Optional[int] = None,
                ws_bytes: Optional[int] = None, stream=None):
    """Replay + reverse sweep: (loss [n], grad_u0 [d, n], grad_p [P, n])."""
    call = ReplayGrad(prob, u0, p, mesh, loss_kind, aux, scale, max_n_steps, ws_bytes)
    return call(stream)


def replay_grad_noalloc(prob, u0, p, mesh: Mesh, max_n_steps: int, loss_kind: int = SUMSQ_FINAL,
                        aux=None, scale: float = 1.0, out=None, stream=None):
    """da_replay_grad_noalloc: the replay gradient with the library's static
    device scratch as workspace (no allocation in the call).  out = (loss
    [n], grad_u0 [d, n], grad_p [P, n]) are written when given, else
    allocated here; returns them."""
    n, dt = _inputs(prob, u0, p)
    S = max(1, len(prob.save_times))
    if aux is not None:
        _need(aux, (S, prob.dim, n), dt, "aux")
    if out is None:
        out = (torch.empty(n, dtype=dt, device=u0.device),
               torch.empty((prob.dim, n), dtype=dt, device=u0.device),
               torch.empty((prob.n_params, n), dtype=dt, device=u0.device))
    loss, gu0, gp = out
    _need(loss, (n,), dt, "loss")
    _need(gu0, (prob.dim, n), dt, "grad_u0")
    _need(gp, (prob.n_params, n), dt, "grad_p")
    P, keep = cproblem(prob, dt)
    cm = mesh.c()
    lobj = _Loss(loss_kind, None if aux is None else aux.data_ptr(), scale)
    _check(_lib.da_replay_grad_noalloc(ctypes.byref(P), n, _ptr(u0), _ptr(p), ctypes.byref(cm),
                                       ctypes.byref(lobj), _ptr(loss), _ptr(gu0), _ptr(gp),
                                       int(max_n_steps), _stream(stream)))
    return loss, gu0, gp


NOALLOC_SCRATCH_BYTES = 64 << 20


def replay_sens(prob, u0, p, mesh: Mesh, loss_kind: Optional[int] = SUMSQ_FINAL, aux=None,
                scale: float = 1.0, with_sens: bool = True, stream=None):
    """Forward-mode sensitivities: (sens [S, d, d+P, n] or None, loss [n],
    grad_u0 [d, n], grad_p [P, n]); loss_kind None computes only sens."""
    n, dt = _inputs(prob, u0, p)
    S = max(1, len(prob.save_times))
    Q = prob.dim + prob.n_params
    dev = u0.device
    if aux is not None:
        _need(aux, (S, prob.dim, n), dt, "aux")
    sens = torch.empty((S, prob.dim, Q, n), dtype=dt, device=dev) if with_sens else None
    loss = torch.empty(n, dtype=dt, device=dev)
    gu0 = torch.empty((prob.dim, n), dtype=dt, device=dev)
    gp = torch.empty((prob.n_params, n), dtype=dt, device=dev)
    P, keep = cproblem(prob, dt)
    cm = mesh.c()
    lp = None
    if loss_kind is not None:
        lobj = _Loss(loss_kind, None if aux is None else aux.data_ptr(), scale)
        lp = ctypes.byref(lobj)
    _check(_lib.da_replay_sens(ctypes.byref(P), n, _ptr(u0), _ptr(p), ctypes.byref(cm), lp,
                               _ptr(loss), _ptr(gu0), _ptr(gp), _ptr(sens), _stream(stream)))
    return sens, loss, gu0, gp


def replay_sens_dirs(prob, u0, p, mesh: Mesh, q_begin: int, q_count: int,
                     loss_kind: Optional[int] = SUMSQ_FINAL, aux=None, scale: float = 1.0,
                     with_sens: bool = True, stream=None):
    """Forward-mode sensitivities along the unit directions q_begin ..
    q_begin + q_count - 1 of the d + P (u0 components, then parameters):
    (sens [S, d, q_count, n] or None, loss [n], grad [q_count, n])."""
    n, dt = _inputs(prob, u0, p)
    S = max(1, len(prob.save_times))
    dev = u0.device
    if aux is not None:
        _need(aux, (S, prob.dim, n), dt, "aux")
    sens = torch.empty((S, prob.dim, q_count, n), dtype=dt, device=dev) if with_sens else None
    loss = torch.empty(n, dtype=dt, device=dev)
    grad = torch.empty((max(q_count, 0), n), dtype=dt, device=dev)
    P, keep = cproblem(prob, dt)
    cm = mesh.c()
    lp = None
    if loss_kind is not None:
        lobj = _Loss(loss_kind, None if aux is None else aux.data_ptr(), scale)
        lp = ctypes.byref(lobj)
    _check(_lib.da_replay_sens_dirs(ctypes.byref(P), n, _ptr(u0), _ptr(p), ctypes.byref(cm),
                                    int(q_begin), int(q_count), lp, _ptr(loss), _ptr(grad),
                                    _ptr(sens), _stream(stream)))
    return sens, loss, grad
