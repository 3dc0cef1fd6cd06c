"""Seeded synthetic workloads for the ODE-ensemble record/replay/adjoint path.

This module only defines problem sizes and draws random inputs.  It holds none
of the method's arithmetic, so both the CPU oracle and the HIP library can be
fed from it without sharing any numerical code.

Five workloads, all synthetic (the pages name the systems, not data files):

1. Lorenz-63, n=1024, FP64, u0=(1,0,0), (sigma, rho, beta) = (10, 28, 8/3)
   scaled per component by U[0.5, 1.0]; t in [0, 1]; Tsit5; rtol=atol=1e-6;
   at most 512 accepted steps; loss = sum of squared final states.
2. Lorenz-63, n=2**20, FP64, same parameter law, u0 = (1,0,0) + N(0, 0.1^2)
   per component; t in [0, 10]; Dopri5; rtol=atol=1e-8; at most 4096 steps;
   one record then 10 gradient passes.  Loss: sum of squared final states.
3. Lorenz-63, n=65536, FP32, u0=(1,0,0), same parameter law; t in [0, 5];
   Tsit5; rtol=atol=1e-5; loss = mean squared error at the 10 save times
   0.5, 1.0, ..., 5.0 against targets from perturbed parameters
   p * (1 + 0.05 N(0,1)).  The targets are produced by the oracle, so this
   module only draws the perturbation.
4. Robertson, n=65536, FP64, k = (0.04, 3e7, 1e4) * exp(0.1 N(0,1)) per
   component, y0 = (1,0,0), t in [0, 1e5], ROS2, rtol=1e-6, atol=1e-10,
   at most 16384 steps; loss = sum of squared final states.
5. Lorenz-96 with N=64, n=16384, FP64, F = 8 U[0.9, 1.1],
   x0 = F + N(0, 0.01^2) per component, t in [0, 2], Tsit5, rtol=atol=1e-7,
   at most 4096 steps; loss = sum of squared final states.

A sixth workload stands in for the HIRES test problem that the pages pair
with higher-order stiff methods (its equations are not on the pages):
6. The eight-species mass-action reaction cycle (d = 8, P = 4), n=65536, FP64,
   rates p = (0.04, 3e7, 1e4, 1) * exp(0.1 N(0,1)) per component,
   y0 = (1, 0, ..., 0), t in [0, 100], Rodas3, rtol=1e-6, atol=1e-10, at most
   2048 steps; loss = sum of squared final states.

Random draws use ``numpy.random.default_rng(seed)`` with seed = workload
number, in this order: parameter multipliers [n, P], then initial-state noise
[n, d] (workloads 2 and 5), then target perturbations [n, P] (workload 3).
Arrays are lane-major: shape [n, d] and [n, P].
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Integer codes shared by convention (not by code) with both implementations.
TSIT5, DOPRI5, ROS2, RODAS3, RKF78, ROS4 = 0, 1, 2, 3, 4, 5
LINEAR, LORENZ63, ROBERTSON, LORENZ96, KINETICS8 = 0, 1, 2, 3, 4
SUMSQ_FINAL, MSE_SAVE, COTANGENT = 0, 1, 2

METHOD_NAMES = {TSIT5: "tsit5", DOPRI5: "dopri5", ROS2: "ros2", RODAS3: "rodas3",
                RKF78: "rkf78", ROS4: "ros4"}
RHS_NAMES = {LINEAR: "linear", LORENZ63: "lorenz63", ROBERTSON: "robertson",
             LORENZ96: "lorenz96", KINETICS8: "kinetics8"}


@dataclasses.dataclass(frozen=True)
class Problem:
    """One ensemble IVP family: right-hand side, method and solver options.

    Zero for ``dt0``, ``max_attempts``, ``safety``, ``fac_min`` and ``fac_max``
    selects the default (automatic starting step, 4 * max_steps attempts,
    0.9, 0.2, 10).  ``checkpoint`` only schedules the GPU reverse sweep.
    ``save_times`` must be strictly increasing in (t0, t1]; empty means the
    final state is the only save.  ``dense = 1`` reads the save times from an
    interpolant of the accepted step that contains them instead of shortening
    steps to land on them.
    """
    rhs: int
    dim: int
    n_params: int
    method: int
    t0: float
    t1: float
    rtol: float
    atol: float
    max_steps: int
    save_times: tuple = ()
    dt0: float = 0.0
    max_attempts: int = 0
    safety: float = 0.0
    fac_min: float = 0.0
    fac_max: float = 0.0
    checkpoint: int = 0     # reverse-sweep checkpoint interval (0 = automatic)
    dense: int = 0          # 1: saves read from the step interpolant, not landed on

    @property
    def n_save_eff(self) -> int:
        return max(1, len(self.save_times))

    def replace(self, **kw) -> "Problem":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Problem definition of one ensemble workload (sizes and tolerances)."""
    wid: int
    name: str
    rhs: int
    dim: int
    n_params: int
    method: int
    dtype: str              # "f64" or "f32"
    n: int
    t0: float
    t1: float
    rtol: float
    atol: float
    max_steps: int
    loss: int
    save_times: tuple = ()
    passes: int = 1

    @property
    def np_dtype(self):
        return np.float64 if self.dtype == "f64" else np.float32

    @property
    def n_save_eff(self) -> int:
        return max(1, len(self.save_times))

    def problem(self, **kw) -> Problem:
        base = Problem(self.rhs, self.dim, self.n_params, self.method, self.t0, self.t1,
                       self.rtol, self.atol, self.max_steps, tuple(self.save_times))
        return dataclasses.replace(base, **kw) if kw else base


WORKLOADS = {
    1: Workload(1, "lorenz63_tsit5_f64_n1024", LORENZ63, 3, 3, TSIT5, "f64",
                1024, 0.0, 1.0, 1e-6, 1e-6, 512, SUMSQ_FINAL),
    2: Workload(2, "lorenz63_dopri5_f64_n1048576", LORENZ63, 3, 3, DOPRI5, "f64",
                1 << 20, 0.0, 10.0, 1e-8, 1e-8, 4096, SUMSQ_FINAL, passes=10),
    3: Workload(3, "lorenz63_tsit5_f32_n65536_mse10", LORENZ63, 3, 3, TSIT5, "f32",
                65536, 0.0, 5.0, 1e-5, 1e-5, 4096, MSE_SAVE,
                save_times=tuple(0.5 * s for s in range(1, 11))),
    4: Workload(4, "robertson_ros2_f64_n65536", ROBERTSON, 3, 3, ROS2, "f64",
                65536, 0.0, 1e5, 1e-6, 1e-10, 16384, SUMSQ_FINAL),
    5: Workload(5, "lorenz96_n64_tsit5_f64_n16384", LORENZ96, 64, 1, TSIT5, "f64",
                16384, 0.0, 2.0, 1e-7, 1e-7, 4096, SUMSQ_FINAL),
    6: Workload(6, "kinetics8_rodas3_f64_n65536", KINETICS8, 8, 4, RODAS3, "f64",
                65536, 0.0, 100.0, 1e-6, 1e-10, 2048, SUMSQ_FINAL),
}

LORENZ_P0 = (10.0, 28.0, 8.0 / 3.0)
ROBERTSON_K0 = (0.04, 3e7, 1e4)
KINETICS8_K0 = (0.04, 3e7, 1e4, 1.0)


def make_inputs(wid: int, n: Optional[int] = None) -> dict:
    """Draw the seeded inputs of workload ``wid`` for ``n`` lanes (default: full size).

    Returns a dict with ``u0`` [n, d] and ``p`` [n, P] in the workload's dtype,
    plus ``p_true`` [n, P] (float64) for workload 3.
    """
    w = WORKLOADS[wid]
    n = w.n if n is None else int(n)
    rng = np.random.default_rng(wid)
    out = {}
    if w.rhs == LORENZ63:
        mult = rng.uniform(0.5, 1.0, size=(n, 3))
        p = np.asarray(LORENZ_P0)[None, :] * mult
        u0 = np.zeros((n, 3))
        u0[:, 0] = 1.0
        if wid == 2:
            u0 = u0 + 0.1 * rng.standard_normal((n, 3))
        if wid == 3:
            out["p_true"] = p * (1.0 + 0.05 * rng.standard_normal((n, 3)))
    elif w.rhs == ROBERTSON:
        mult = np.exp(0.1 * rng.standard_normal((n, 3)))
        p = np.asarray(ROBERTSON_K0)[None, :] * mult
        u0 = np.zeros((n, 3))
        u0[:, 0] = 1.0
    elif w.rhs == KINETICS8:
        mult = np.exp(0.1 * rng.standard_normal((n, 4)))
        p = np.asarray(KINETICS8_K0)[None, :] * mult
        u0 = np.zeros((n, 8))
        u0[:, 0] = 1.0
    elif w.rhs == LORENZ96:
        F = 8.0 * rng.uniform(0.9, 1.1, size=(n, 1))
        p = F
        u0 = F + 0.01 * rng.standard_normal((n, w.dim))
    else:  # pragma: no cover - no workload uses LINEAR
        raise ValueError(wid)
    dt = w.np_dtype
    out["u0"] = np.ascontiguousarray(u0.astype(dt))
    out["p"] = np.ascontiguousarray(p.astype(dt))
    return out
