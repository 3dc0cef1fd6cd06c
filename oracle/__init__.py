"""Python access to the plain CPU oracle (``oracle.cpp``).

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library
never calls it, and it never calls the HIP library.

Arrays here are numpy, lane-major: u0 [n, d], p [n, P], h [n, max_steps],
save_idx [n, S], save_theta [n, S], y_save [n, S, d] with
S = max(1, len(save_times)).  With ``prob.dense`` the saves are read from the
cubic Hermite interpolant of the step that contains them, and ``save_theta``
(the step fraction of each save, part of the mesh) is required by the
replays.  The
dtype of ``u0`` (float64 or float32) selects the precision.  ``fused=True``
evaluates every multiply-add as one correctly rounded fma; ``fused=False``
rounds each multiply and add separately.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess
import tempfile
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

# status codes of a lane
LANE_OK, LANE_MAX_STEPS, LANE_DT_UNDERFLOW, LANE_NONFINITE, LANE_MAX_ATTEMPTS = range(5)


# A library to load instead of liboracle.so (the sanitizer build, in a
# process that preloads the sanitizer runtime).
_ENV_LIB = "ORACLE_LIBRARY"
_SAN_LIB = os.path.join(_HERE, "liboracle_san.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile oracle.cpp into liboracle.so (g++, -O2, no fp contraction,
    OpenMP).  With `sanitize`, into liboracle_san.so with AddressSanitizer
    and UndefinedBehaviorSanitizer (every report fatal); a process loads it
    through ORACLE_LIBRARY with the ASan runtime preloaded."""
    out = _SAN_LIB if sanitize else _LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-Wall", *(SANITIZE_FLAGS if sanitize else []), "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


class _Problem(ctypes.Structure):
    _fields_ = [
        ("rhs", ctypes.c_int32), ("dim", ctypes.c_int32), ("n_params", ctypes.c_int32),
        ("method", ctypes.c_int32),
        ("t0", ctypes.c_double), ("t1", ctypes.c_double), ("rtol", ctypes.c_double),
        ("atol", ctypes.c_double), ("dt0", ctypes.c_double),
        ("max_steps", ctypes.c_int32), ("max_attempts", ctypes.c_int32),
        ("n_save", ctypes.c_int32), ("save_times", ctypes.POINTER(ctypes.c_double)),
        ("safety", ctypes.c_double), ("fac_min", ctypes.c_double), ("fac_max", ctypes.c_double),
        ("dense", ctypes.c_int32),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get(_ENV_LIB)
        if not path:
            path = _LIB
            if not os.path.exists(_LIB):
                build(force=True)
        _lib = ctypes.CDLL(path)
        _lib.orc_ros2_gamma.restype = ctypes.c_double
    return _lib


def _swap_library(path: Optional[str]):
    """Point this module at another build of oracle.cpp (None restores the
    default).  Used by the test that plants mistakes in copies of the source."""
    global _lib
    _lib = None
    if path is not None:
        _lib = ctypes.CDLL(path)
        _lib.orc_ros2_gamma.restype = ctypes.c_double


def _cprob(prob):
    st = np.ascontiguousarray(np.asarray(prob.save_times, dtype=np.float64))
    P = _Problem(prob.rhs, prob.dim, prob.n_params, prob.method, prob.t0, prob.t1, prob.rtol,
                 prob.atol, prob.dt0, prob.max_steps, prob.max_attempts, len(prob.save_times),
                 st.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if len(st) else None,
                 prob.safety, prob.fac_min, prob.fac_max, int(getattr(prob, "dense", 0)))
    return P, st  # keep st alive


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def _sfx(dt):
    if dt == np.float64:
        return "f64"
    if dt == np.float32:
        return "f32"
    raise TypeError(f"unsupported dtype {dt}")


_PLUGIN = r'''
#include "user_types.h"
namespace user {
struct Src {
  template <class T> static void f(const T *y, const T *p, T *dy) {
#line 1 "rhs"
%s
  }
};
}  // namespace user
typedef user::UDual<double, false> DP64;
typedef user::UDual<double, true> DF64;
typedef user::UDual<float, false> DP32;
typedef user::UDual<float, true> DF32;
extern "C" {
#define ORC_USER_F(NAME, TYPE) \
  void NAME(const TYPE *y, const TYPE *p, TYPE *o) { user::Src::f(y, p, o); }
ORC_USER_F(orc_user_f64, double)
ORC_USER_F(orc_user_f32, float)
ORC_USER_F(orc_user_dp64, DP64)
ORC_USER_F(orc_user_df64, DF64)
ORC_USER_F(orc_user_dp32, DP32)
ORC_USER_F(orc_user_df32, DF32)
}
'''
# A cyclic stencil (the form of the wavefront kernels' registered right-hand
# sides): component i of f from the components i + o (mod d) of the declared
# offsets o; the whole vector is those components in order.
_STENCIL_PLUGIN = r'''
#include <limits>
#include "user_types.h"
namespace user {
constexpr int SD = %d, NOFF = %d;
constexpr int OFF[NOFF] = {%s};
template <class V> struct SY {
  const V *yv;
  int i, d;
  V operator()(int o) const {
    for (int s = 0; s < NOFF; ++s)
      if (OFF[s] == o) return yv[((i + o) %% d + d) %% d];
    return V(std::numeric_limits<double>::quiet_NaN());
  }
};
struct Stencil {
  template <class T, class Y> static T g(const Y &y, const T *p) {
#line 1 "rhs"
%s
  }
};
struct Src {
  template <class T> static void f(const T *y, const T *p, T *dy) {
    for (int i = 0; i < SD; ++i) {
      SY<T> acc;
      acc.yv = y;
      acc.i = i;
      acc.d = SD;
      dy[i] = Stencil::g<T>(acc, p);
    }
  }
};
}  // namespace user
''' + _PLUGIN[_PLUGIN.index("typedef user::UDual<double, false> DP64;"):]
_plugins = {}


def set_user_rhs(f_body: str, dim: int, n_params: int) -> None:
    """Make the caller's right-hand side (the body of
    ``template <class T> void f(const T *y, const T *p, T *dy)``, the same
    source the HIP library compiles) the oracle's right-hand side for every
    problem whose rhs code is >= 1024.  It is built with g++ into a plugin
    (cached by source) and evaluated on reals and dual numbers."""
    _set_plugin(_PLUGIN % f_body, dim, n_params)


def set_user_stencil(f_body: str, dim: int, n_params: int, offsets) -> None:
    """As set_user_rhs for a cyclic stencil (the source of
    da_rhs_register_stencil): the body of
    ``template <class T, class Y> T f(const Y &y, const T *p)`` gives
    component i from y(o) = y[(i + o) mod dim] for the declared offsets o
    (NaN for others); the oracle's f is the vector of those components, and
    its derivatives are the generic ones of any registered right-hand side."""
    offs = [int(o) for o in offsets]
    src = _STENCIL_PLUGIN % (dim, len(offs), ", ".join(map(str, offs)), f_body)
    _set_plugin(src, dim, n_params)


def _set_plugin(source: str, dim: int, n_params: int) -> None:
    key = hashlib.sha256(f"{dim} {n_params}\n{source}".encode()).hexdigest()[:16]
    if key not in _plugins:
        d = os.path.join(tempfile.gettempdir(), "dadj_oracle_rhs")
        os.makedirs(d, exist_ok=True)
        src = os.path.join(d, f"rhs_{key}.cpp")
        lib = os.path.join(d, f"rhs_{key}.so")
        if not os.path.exists(lib):
            with open(src, "w") as f:
                f.write(source)
            tmp = lib + f".{os.getpid()}.tmp"
            subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
                            "-fPIC", "-shared", "-I", _HERE, "-o", tmp, src], check=True)
            os.replace(tmp, lib)
        _plugins[key] = ctypes.CDLL(lib)
    pl = _plugins[key]
    ptrs = [ctypes.cast(getattr(pl, n), ctypes.c_void_p)
            for n in ("orc_user_f64", "orc_user_f32", "orc_user_dp64", "orc_user_df64",
                      "orc_user_dp32", "orc_user_df32")]
    _check(_load().orc_set_user_rhs(ctypes.c_int32(dim), ctypes.c_int32(n_params), *ptrs),
           "set_user_rhs")


def max_threads(nthreads: int = 0) -> int:
    return _load().orc_max_threads(ctypes.c_int(nthreads))


def ros2_gamma() -> float:
    return _load().orc_ros2_gamma()


def tableau(method: int) -> dict:
    """Tableau of Tsit5 (0) or Dopri5 (1): c[7], a[7,7], b[7], e = b - bhat."""
    c = np.zeros(7); a = np.zeros((7, 7)); b = np.zeros(7); e = np.zeros(7)
    info = np.zeros(2, dtype=np.int32)
    _check(_load().orc_tableau(method, _ptr(c), _ptr(a), _ptr(b), _ptr(e), _ptr(info)),
           "tableau")
    return {"c": c, "a": a, "b": b, "e": e, "order": int(info[0]), "err_order": int(info[1])}


def rk78_tableau() -> dict:
    """The Fehlberg 7(8) coefficients as the oracle holds them: a[13, 13],
    b (7th-order weights), e = b7 - b8."""
    a = np.zeros((13, 13)); b = np.zeros(13); e = np.zeros(13)
    info = np.zeros(2, dtype=np.int32)
    _check(_load().orc_rk78_tableau(_ptr(a), _ptr(b), _ptr(e), _ptr(info)), "rk78_tableau")
    return {"a": a, "b": b, "e": e, "order": int(info[0]), "err_order": int(info[1])}


def record(prob, u0, p, fused: bool = False, nthreads: int = 0, with_h: bool = True) -> dict:
    """Adaptive solve per lane; returns the mesh and saved states."""
    u0 = np.ascontiguousarray(u0)
    dt = u0.dtype.type
    p = np.ascontiguousarray(p, dtype=dt)
    n = u0.shape[0]
    S = prob.n_save_eff
    h = np.zeros((n, prob.max_steps), dtype=dt) if with_h else None
    ns = np.zeros(n, dtype=np.int32)
    sidx = np.zeros((n, S), dtype=np.int32)
    status = np.zeros(n, dtype=np.int32)
    theta = np.zeros((n, S), dtype=dt)
    ysave = np.zeros((n, S, prob.dim), dtype=dt)
    natt = np.zeros(n, dtype=np.int32)
    P, keep = _cprob(prob)
    fn = getattr(_load(), "orc_record_" + _sfx(dt))
    _check(fn(ctypes.byref(P), ctypes.c_int64(n), _ptr(u0), _ptr(p), ctypes.c_int32(int(fused)),
              _ptr(h), _ptr(ns), _ptr(sidx), _ptr(theta), _ptr(status), _ptr(ysave), _ptr(natt),
              ctypes.c_int32(nthreads)), "record")
    return {"h": h, "n_steps": ns, "save_idx": sidx, "save_theta": theta, "status": status,
            "y_save": ysave, "n_attempts": natt}


def _theta(prob, mesh, dt):
    if not getattr(prob, "dense", 0):
        return None
    return np.ascontiguousarray(mesh["save_theta"], dtype=dt)


def replay(prob, u0, p, mesh, fused: bool = False, nthreads: int = 0):
    """Fixed-step replay of ``mesh``; returns (y_save [n,S,d], y_final [n,d])."""
    u0 = np.ascontiguousarray(u0)
    dt = u0.dtype.type
    p = np.ascontiguousarray(p, dtype=dt)
    n = u0.shape[0]
    S = prob.n_save_eff
    h = np.ascontiguousarray(mesh["h"], dtype=dt)
    ns = np.ascontiguousarray(mesh["n_steps"], dtype=np.int32)
    sidx = np.ascontiguousarray(mesh["save_idx"], dtype=np.int32)
    th = _theta(prob, mesh, dt)
    ysave = np.zeros((n, S, prob.dim), dtype=dt)
    yfin = np.zeros((n, prob.dim), dtype=dt)
    P, keep = _cprob(prob)
    fn = getattr(_load(), "orc_replay_" + _sfx(dt))
    _check(fn(ctypes.byref(P), ctypes.c_int64(n), _ptr(u0), _ptr(p), ctypes.c_int32(int(fused)),
              _ptr(h), _ptr(ns), _ptr(sidx), _ptr(th), _ptr(ysave), _ptr(yfin),
              ctypes.c_int32(nthreads)), "replay")
    return ysave, yfin


def replay_grad(prob, u0, p, mesh, loss_kind: int = 0, aux: Optional[np.ndarray] = None,
                scale: float = 1.0, fused: bool = False, nthreads: int = 0):
    """Replay + exact discrete adjoint; returns (loss [n], grad_u0 [n,d], grad_p [n,P]).

    ``aux`` is [n, S, d]: targets (MSE_SAVE) or cotangents (COTANGENT)."""
    u0 = np.ascontiguousarray(u0)
    dt = u0.dtype.type
    p = np.ascontiguousarray(p, dtype=dt)
    n = u0.shape[0]
    h = np.ascontiguousarray(mesh["h"], dtype=dt)
    ns = np.ascontiguousarray(mesh["n_steps"], dtype=np.int32)
    sidx = np.ascontiguousarray(mesh["save_idx"], dtype=np.int32)
    status = np.ascontiguousarray(mesh["status"], dtype=np.int32)
    th = _theta(prob, mesh, dt)
    ax = None if aux is None else np.ascontiguousarray(aux, dtype=dt)
    loss = np.zeros(n, dtype=dt)
    gu0 = np.zeros((n, prob.dim), dtype=dt)
    gp = np.zeros((n, prob.n_params), dtype=dt)
    P, keep = _cprob(prob)
    fn = getattr(_load(), "orc_replay_grad_" + _sfx(dt))
    _check(fn(ctypes.byref(P), ctypes.c_int64(n), _ptr(u0), _ptr(p), ctypes.c_int32(int(fused)),
              _ptr(h), _ptr(ns), _ptr(sidx), _ptr(th), _ptr(status), ctypes.c_int32(loss_kind),
              _ptr(ax), ctypes.c_double(scale), _ptr(loss), _ptr(gu0), _ptr(gp),
              ctypes.c_int32(nthreads)), "replay_grad")
    return loss, gu0, gp


def replay_jvp(prob, u0, p, du0, dp, mesh, loss_kind: int = 0,
               aux: Optional[np.ndarray] = None, scale: float = 1.0):
    """Forward-mode (dual number) derivative of the replayed loss along (du0, dp).

    Returns (loss [n], dloss [n], y_save [n,S,d], dy_save [n,S,d]); float64 only."""
    u0 = np.ascontiguousarray(u0, dtype=np.float64)
    p = np.ascontiguousarray(p, dtype=np.float64)
    du0 = np.ascontiguousarray(du0, dtype=np.float64)
    dp = np.ascontiguousarray(dp, dtype=np.float64)
    n = u0.shape[0]
    S = prob.n_save_eff
    h = np.ascontiguousarray(mesh["h"], dtype=np.float64)
    ns = np.ascontiguousarray(mesh["n_steps"], dtype=np.int32)
    sidx = np.ascontiguousarray(mesh["save_idx"], dtype=np.int32)
    th = _theta(prob, mesh, np.float64)
    ax = None if aux is None else np.ascontiguousarray(aux, dtype=np.float64)
    loss = np.zeros(n); dloss = np.zeros(n)
    ys = np.zeros((n, S, prob.dim)); dys = np.zeros((n, S, prob.dim))
    P, keep = _cprob(prob)
    _check(_load().orc_replay_jvp_f64(ctypes.byref(P), ctypes.c_int64(n), _ptr(u0), _ptr(p),
                                      _ptr(du0), _ptr(dp), _ptr(h), _ptr(ns), _ptr(sidx),
                                      _ptr(th), ctypes.c_int32(loss_kind), _ptr(ax),
                                      ctypes.c_double(scale), _ptr(loss), _ptr(dloss), _ptr(ys),
                                      _ptr(dys)), "replay_jvp")
    return loss, dloss, ys, dys


def replay_sens(prob, u0, p, mesh, loss_kind: int = 0, aux: Optional[np.ndarray] = None,
                scale: float = 1.0, fused: bool = False):
    """Forward-mode sensitivities of the replay along the d + P unit directions
    (u0 components, then parameters), float64.

    Returns (sens [n, S, d, d+P], loss [n], grad_u0 [n, d], grad_p [n, P]); the
    gradient is the loss gradient by the chain rule through the tangents."""
    u0 = np.ascontiguousarray(u0, dtype=np.float64)
    p = np.ascontiguousarray(p, dtype=np.float64)
    n = u0.shape[0]
    S = prob.n_save_eff
    Q = prob.dim + prob.n_params
    h = np.ascontiguousarray(mesh["h"], dtype=np.float64)
    ns = np.ascontiguousarray(mesh["n_steps"], dtype=np.int32)
    sidx = np.ascontiguousarray(mesh["save_idx"], dtype=np.int32)
    status = np.ascontiguousarray(mesh["status"], dtype=np.int32)
    th = _theta(prob, mesh, np.float64)
    ax = None if aux is None else np.ascontiguousarray(aux, dtype=np.float64)
    sens = np.zeros((n, S, prob.dim, Q))
    loss = np.zeros(n)
    gu0 = np.zeros((n, prob.dim))
    gp = np.zeros((n, prob.n_params))
    P, keep = _cprob(prob)
    _check(_load().orc_replay_sens_f64(ctypes.byref(P), ctypes.c_int64(n), _ptr(u0), _ptr(p),
                                       ctypes.c_int32(int(fused)), _ptr(h), _ptr(ns), _ptr(sidx),
                                       _ptr(th), _ptr(status), ctypes.c_int32(loss_kind), _ptr(ax),
                                       ctypes.c_double(scale), _ptr(sens), _ptr(loss), _ptr(gu0),
                                       _ptr(gp)), "replay_sens")
    return sens, loss, gu0, gp


def mesh_max_err(prob, u0, p, mesh, fused: bool = False, nthreads: int = 0):
    """Largest embedded error norm E over the steps of ``mesh``, per lane."""
    u0 = np.ascontiguousarray(u0)
    dt = u0.dtype.type
    p = np.ascontiguousarray(p, dtype=dt)
    n = u0.shape[0]
    h = np.ascontiguousarray(mesh["h"], dtype=dt)
    ns = np.ascontiguousarray(mesh["n_steps"], dtype=np.int32)
    out = np.zeros(n, dtype=dt)
    P, keep = _cprob(prob)
    fn = getattr(_load(), "orc_mesh_max_err_" + _sfx(dt))
    _check(fn(ctypes.byref(P), ctypes.c_int64(n), _ptr(u0), _ptr(p), ctypes.c_int32(int(fused)),
              _ptr(h), _ptr(ns), _ptr(out), ctypes.c_int32(nthreads)), "mesh_max_err")
    return out


def initial_step(prob, y0, p) -> float:
    y0 = np.ascontiguousarray(y0, dtype=np.float64)
    p = np.ascontiguousarray(p, dtype=np.float64)
    h0 = np.zeros(1)
    P, keep = _cprob(prob)
    _check(_load().orc_initial_step_f64(ctypes.byref(P), _ptr(y0), _ptr(p), _ptr(h0)),
           "initial_step")
    return float(h0[0])


def rhs(kind: int, y, p, v):
    """f(y), J(y)^T v, J_p(y)^T v and the Jacobian of the systems the
    Rosenbrock methods take (None for Lorenz-96), float64."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    p = np.ascontiguousarray(p, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    d = y.shape[0]
    jac = d <= 8 and kind != 3
    f = np.zeros(d); wy = np.zeros(d); gp = np.zeros(p.shape[0]); J = np.zeros(d * d)
    _check(_load().orc_rhs_f64(ctypes.c_int32(kind), ctypes.c_int32(d), _ptr(y), _ptr(p),
                               _ptr(v), _ptr(f), _ptr(wy), _ptr(gp),
                               _ptr(J) if jac else None), "rhs")
    return f, wy, gp, J.reshape(d, d) if jac else None
