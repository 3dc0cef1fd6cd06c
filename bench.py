"""Benchmark of the record-and-replay discrete adjoint on one MI355X.

Default workload: Lorenz-63 ensemble of 2^20 trajectories in FP64, Dopri5,
rtol = atol = 1e-8, t in [0, 10], at most 4096 steps, loss = sum of squared
final states; one record then 10 replay-gradient passes against it.  Inputs
are synthetic (seeded, see workloads/) and resident on the GPU before the
timed region.  --workload selects one of the other ensembles.

One timed step is that whole job: record, lane ordering (the replay order by
decreasing step count), and the gradient passes, which read the tiled step log
through the replay order.  --replay-table also builds the replay table in the
job (one contiguous row of step sizes per replay step) for the passes to read
instead; at 10 passes it no longer pays for itself.
value = trajectories * passes / step time (trajectory-gradients/s).

Printed on one JSON line, besides the standard fields (metric, value, unit, steps, config):
  roofline      the gradient kernel (k_replay_grad) against the vector ALU
                peak of its dtype: algorithmic FLOPs per launch (the exact
                operation count of the replay step and its adjoint per
                populated step, stage recomputation excluded, times the
                populated steps of the record) / mean launch time from HIP
                events on the launch stream; traffic = HBM bytes per launch
                from rocprofv3 FETCH_SIZE and WRITE_SIZE counters, each scaled
                by what the counter reads for a copy of known size, when the
                kernel sources match the ones the counters were taken with,
                else null;
  clock_adjusted  the same achieved rate against the vector peak at the
                shader clock the counters measured while the gradient kernel
                ran (GRBM_GUI_ACTIVE per XCD over the launch time), and the
                executed rate (SQ_INSTS_VALU_*_F64, or _F32 in single precision: stage recomputation and
                padded steps included) over the live launch time; from the
                committed counter summary of the workload when the kernel
                sources match it, else null;
  record_log    bytes of the zero-padded step log the record writes, and the
                rate over the record time;
  replay_fwd    the fused fixed-step replay alone (saved states, no
                gradient) on the job's replay order and a replay table (built
                outside the timed job when the job has none), with its
                algorithmic FLOP rate (the forward part of flop_per_step);
  ordering_ms   the lane ordering inside the job (and the replay table when
                the job builds one);
  cpu_baseline  the CPU oracle (plain C++, OpenMP) on a bounded sample of the
                same workload, as trajectory-gradients/s of the same job;
  record_stats  accepted and rejected trial steps per trajectory and the
                trajectories per lane status of the record;
  other_workloads  (default run only) one job of each other gradient
                workload at its full size, timed after the headline: job and
                gradient-pass times, and the pass's algorithmic rate against
                its dtype's vector peak.

--gpus N with N > 1 is not supported (the library runs on one GPU).
"""
import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Vector ALU peaks of MI355X (256 CUs x 2.4 GHz): FP64 128 flop/clock/CU;
# FP32 256 flop/clock/CU (packed; unpacked FP32 runs at the FP64 rate).
PEAK_TFLOPS = {"f64": 78.6, "f32": 157.3}

# Algorithmic FLOPs per populated step (FMA = 2, add/sub/mul/div = 1,
# negation = 0) of the replay step plus its adjoint, stage recomputation
# excluded, counted from the arithmetic schedule of the kernels:
#  Dopri5 / Lorenz-63: forward 6 right-hand sides x 8 + stage sums 46 per
#    component x 3 = 186; adjoint stage cotangent sums 40 x 3 = 120 + 6 stages
#    x (J^T v 13 + J_p^T v 7 + accumulate 3) = 138; total 444.
#  Tsit5 / Lorenz-63: forward 48 + 48 x 3 = 192; adjoint 42 x 3 + 138 = 264.
#  ROS2 / Robertson: forward (Jacobian 9, W 13, LU 13, two right-hand sides
#    26, two solves 30, stage and solution combinations 27) = 118; adjoint
#    (two transposed solves 30, J^T v and J_p^T v at both stages 66, Wbar 27,
#    cotangent combinations 36, dJ contraction 29) = 188; total 306.
#  Rodas3 / Robertson: forward (Jacobian 9, W 13, LU 13, four right-hand
#    sides 52, four solves 60, stage sums Y_i 18 and stage right-hand sides
#    48, solution 18 and error 3) = 234; adjoint (stage cotangents 60, four
#    transposed solves 60, Wbar 63, fbar 12, J^T v and J_p^T v at four stages
#    132, ybar sums 12, Jbar 9 and dJ contraction 29) = 377; total 611.
#  Fourth-order Rosenbrock (Shampine's parameters) / Robertson: its fourth
#    stage sits at the third stage's point (a_4j = a_3j), so three stage
#    points: forward as Rodas3 but three right-hand sides (39), three
#    nonzero a_ij of distinct points (stage sums Y_i 18), four nonzero m_i
#    (solution 24) and three nonzero e_i (error 15) = 239; adjoint as Rodas3
#    but three vector-Jacobian products (99) of the summed cotangents of the
#    shared point (3) and stage cotangents over nine nonzero a_li and gamma
#    c_li terms with four m_i (66) = 353; total 592.  (The kernel evaluates
#    the fourth stage's point and right-hand side as written; the compiler
#    merges them with the third's, being the same operations on the same
#    values, and runs two products at that point in reverse.)
#  Fehlberg 7(8) / Lorenz-63: forward (11 right-hand sides of 8 flop = 88,
#    stage sums over the nonzero a_ij and the solution over the 7 nonzero
#    b_j: 3 x 105 = 315) = 403; adjoint (stage cotangents 3 x 94 = 282, J^T v
#    and J_p^T v at 11 stages 220, lam sums 33) = 535; total 938.
#  Rodas3 / eight-species kinetics (dense 8 x 8 factors, as implemented):
#    forward (rate partials and Jacobian 14, W 73, LU 316, four right-hand
#    sides 112, four solves 480, stage sums Y_i 48 and stage right-hand sides
#    128, solution 48 and error 8) = 1227; adjoint (stage cotangents 160,
#    four transposed solves 480, Wbar 448, fbar 32, J^T v and J_p^T v at four
#    stages 288, ybar sums 32, Jbar 64 and dJ contraction 53) = 1557; total
#    2784.
#  Tsit5 / Lorenz-96 (d components): forward 6 x 4d + 48d = 72d; adjoint
#    42d + 6 x (J^T v 7d + J_p^T v d + accumulate d) = 96d; total 168d.
# Forward-mode sensitivities (all d + P unit directions as dual numbers, the
# state counted once): per direction the tangent of every right-hand side
# (Lorenz-63: 4 + 5 + 7 = 16 flop) and of the stage sums (same count as the
# state's), so Dopri5 / Lorenz-63: 186 + 6 x (6 x 16 + 138) = 1590 and
# Tsit5 / Lorenz-63: 192 + 6 x (6 x 16 + 144) = 1632.  Tsit5 / Lorenz-96:
# the state 72d, and per direction the tangents of six right-hand sides
# (6d each: difference, tangent multiply-add, sum) and of the stage sums
# (48d), so 72d + (d + 1) x 84d.  Not counted for ROS2 (None).
def sens_flop_per_step(method: str, rhs: str, dim: int):
    if (method, rhs) == ("tsit5", "lorenz96"):
        return 72 * dim + (dim + 1) * 84 * dim
    return {("dopri5", "lorenz63"): 1590, ("tsit5", "lorenz63"): 1632}.get((method, rhs))


def fwd_flop_per_step(method: str, rhs: str, dim: int):
    """The forward part of flop_per_step: one replay step (the da_replay_fwd
    kernel), from the same counts."""
    if rhs == "lorenz96" and method == "tsit5":
        return 72 * dim
    return {("dopri5", "lorenz63"): 186, ("tsit5", "lorenz63"): 192,
            ("ros2", "robertson"): 118, ("rodas3", "robertson"): 234,
            ("rodas3", "kinetics8"): 1227, ("rkf78", "lorenz63"): 403,
            ("ros4", "robertson"): 239}.get((method, rhs))


def flop_per_step(method: str, rhs: str, dim: int) -> int:
    table = {("dopri5", "lorenz63"): 444, ("tsit5", "lorenz63"): 456,
             ("ros2", "robertson"): 306, ("rodas3", "robertson"): 611,
             ("rodas3", "kinetics8"): 2784, ("rkf78", "lorenz63"): 938,
             ("ros4", "robertson"): 592}
    if rhs == "lorenz96" and method == "tsit5":
        return 168 * dim
    return table[(method, rhs)]


COUNTERS_DIR = os.path.join(ROOT, "profiles")

# Lorenz-63 written as the source of a run-time compiled right-hand side
# (--rhs-source): the same system as the built-in one, with the
# vector-Jacobian products taken by forward-mode tangents.
LORENZ63_SOURCE = """
    dy[0] = p[0] * (y[1] - y[0]);
    dy[1] = y[0] * (p[1] - y[2]) - y[1];
    dy[2] = y[0] * y[1] - p[2] * y[2];
"""
# Lorenz-96 written as a cyclic stencil for the wavefront kernels
# (--rhs-source on workload 5): component i from y(o) = y[(i + o) mod d].
LORENZ96_STENCIL = "return (y(1) - y(-2)) * y(-1) - y(0) + p[0];"
LORENZ96_OFFSETS = (-2, -1, 0, 1)
# Sources of the gradient kernel of each method family.
KERNEL_SOURCES = {
    "erk": ["lane_kernels.hpp", "erk_method.hpp", "erk.hip", "erk_grad_f64_dopri5.hip",
            "erk_grad_f64_tsit5.hip", "erk_grad_f32_dopri5.hip", "erk_grad_f32_tsit5.hip",
            "dadj_device.hpp", "dadj_internal.hpp"],
    "ros2": ["lane_kernels.hpp", "rosenbrock.hpp", "ros2.hip", "dadj_device.hpp",
             "dadj_internal.hpp"],
    "rodas3": ["lane_kernels.hpp", "rosenbrock.hpp", "rosenbrock4.hpp", "rodas3.hip",
               "dadj_device.hpp", "dadj_internal.hpp"],
    "ros4": ["lane_kernels.hpp", "rosenbrock.hpp", "rosenbrock4.hpp", "ros4.hip",
             "dadj_device.hpp", "dadj_internal.hpp"],
    "rkf78": ["lane_kernels.hpp", "rkf78.hip", "dadj_device.hpp", "dadj_internal.hpp"],
    "wave": ["wave_kernels.hpp", "l96.hip", "dadj_device.hpp", "dadj_internal.hpp"],
}


def kernel_family(method: str, rhs: str) -> str:
    if rhs == "lorenz96":
        return "wave"
    return method if method in ("ros2", "rodas3", "ros4", "rkf78") else "erk"


# The host-side part of the internal header (launcher declarations and the
# like) does not change any kernel: only the text before this marker counts.
HOST_SECTION = b"#ifndef __HIPCC_RTC__  // host side"


def kernel_source_hash(family: str = "erk") -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        path = os.path.join(ROOT, "discrete_adjoint_amd", "csrc", f)
        if os.path.exists(path):
            with open(path, "rb") as fh:
                text = fh.read()
            if f == "dadj_internal.hpp" and HOST_SECTION in text:
                text = text[:text.index(HOST_SECTION)]
            h.update(text)
    return h.hexdigest()[:16]


def _summary_interval(path: str) -> int:
    """Checkpoint interval a counter summary was taken at (1 when it does not
    say: every summary without the line was taken at interval 1)."""
    for line in open(path):
        if line.startswith("checkpoint_interval:"):
            return int(line.split(":", 1)[1].strip())
    return 1


def read_traffic(workload_name: str, family: str, dense: bool = False, interval: int = 1):
    """HBM bytes per gradient launch from the committed counter summary of the
    workload (its dense-output variant with `dense`), if it was taken with the
    current kernel sources at the same checkpoint interval."""
    sfx = "_dense" if dense else ""
    path = os.path.join(COUNTERS_DIR, f"replay_grad_{workload_name}{sfx}_counters.md")
    if not os.path.exists(path) or _summary_interval(path) != interval:
        return None
    src_hash, traffic = None, None
    for line in open(path):
        if line.startswith("kernel_source_hash:"):
            src_hash = line.split(":", 1)[1].strip()
        if line.startswith("hbm_bytes_per_launch:"):
            traffic = float(line.split(":", 1)[1].strip())
    return traffic if src_hash == kernel_source_hash(family) else None


def read_valu_clock(workload_name: str, family: str, interval: int = 1):
    """Shader clock and executed FP64 work of the gradient kernel from the
    committed counter summary of the workload (GRBM_GUI_ACTIVE per XCD over
    the launch time; SQ_INSTS_VALU_{FMA,MUL,ADD,TRANS}_F64), if it was taken
    with the current kernel sources at the same checkpoint interval."""
    path = os.path.join(COUNTERS_DIR, f"replay_grad_{workload_name}_valu_clock.md")
    if not os.path.exists(path) or _summary_interval(path) != interval:
        return None
    vals = {}
    for line in open(path):
        for key in ("kernel_source_hash", "clock_ghz", "valu_busy", "fp64_flop_executed_per_launch",
                    "fp32_flop_executed_per_launch"):
            if line.startswith(key + ":"):
                vals[key.replace("fp64_", "").replace("fp32_", "")] = line.split(":", 1)[1].strip()
    if vals.get("kernel_source_hash") != kernel_source_hash(family) or len(vals) < 4:
        return None
    return {"clock_ghz": float(vals["clock_ghz"]), "valu_busy": float(vals["valu_busy"]),
            "flop_executed_per_launch": float(vals["flop_executed_per_launch"]),
            "source": os.path.relpath(path, ROOT)}


def record_stats(mesh) -> dict:
    """Statistics of one record (the review's Strengths quote Table 5's step
    counts across the ensemble): accepted and rejected trial steps per
    trajectory (mean, max) and the trajectories per lane status."""
    import numpy as np
    ns = mesh.n_steps.cpu().numpy().astype(np.int64)
    na = mesh.n_attempts.cpu().numpy().astype(np.int64)
    st = mesh.status.cpu().numpy()
    rej = na - ns
    names = ("ok", "max_steps", "dt_underflow", "nonfinite", "max_attempts")
    hist = {nm: int((st == k).sum()) for k, nm in enumerate(names)}
    return {"accepted_mean": float(ns.mean()), "accepted_max": int(ns.max()),
            "accepted_max_over_mean": float(ns.max() / max(ns.mean(), 1e-300)),
            "rejected_total": int(rej.sum()), "rejected_mean": float(rej.mean()),
            "rejected_max": int(rej.max()), "reject_rate": float(rej.sum() / max(na.sum(), 1)),
            "status": hist}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wid: int, lanes: int, passes: int, max_seconds: float = 25.0,
                 dense: int = 0, method=None):
    """Oracle as it stands, plain rounding, all OpenMP threads: record + passes
    on the first `lanes` trajectories of the workload (with `method` in place
    of the workload's integrator, when given)."""
    import numpy as np
    import oracle
    import workloads as W
    w = W.WORKLOADS[wid]
    lanes = min(lanes, w.n)
    inp = W.make_inputs(wid, lanes)
    prob = w.problem(dense=dense)
    if method is not None:
        prob = prob.replace(method=method)
    cores = oracle.max_threads()
    aux, scale = None, 1.0
    if w.loss == W.MSE_SAVE:
        t = oracle.record(prob, inp["u0"].astype(np.float64), inp["p_true"], with_h=False)
        aux = t["y_save"].astype(w.np_dtype)
        scale = 1.0 / (lanes * w.n_save_eff * w.dim)
    t0 = time.perf_counter()
    m = oracle.record(prob, inp["u0"], inp["p"])
    t_rec = time.perf_counter() - t0
    N = int(m["n_steps"].max())
    m["h"] = np.ascontiguousarray(m["h"][:, :N])
    pn = prob.replace(max_steps=N)
    t_pass = []
    while len(t_pass) < 1 or (sum(t_pass) + t_rec < max_seconds and len(t_pass) < passes):
        t0 = time.perf_counter()
        oracle.replay_grad(pn, inp["u0"], inp["p"], m, w.loss, aux=aux, scale=scale)
        t_pass.append(time.perf_counter() - t0)
    t_job = t_rec + passes * float(np.mean(t_pass))
    return {"value": lanes * passes / t_job, "unit": "trajectory-gradients/s", "cores": cores,
            "kind": "oracle", "per_core": lanes * passes / t_job / cores,
            "cpu_model": cpu_model(),
            "sample": f"first {lanes} of {w.n} trajectories of the workload: record "
                      f"{t_rec:.2f} s + {len(t_pass)} timed gradient passes (mean "
                      f"{np.mean(t_pass):.3f} s); job time = record + {passes} passes"}


def copy_probe(gib: float = 1.0):
    """A plain device-to-device copy of known size, for counter calibration."""
    import torch
    n = int(gib * (1 << 30)) // 8
    a = torch.ones(n, dtype=torch.float64, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": n * 8, "launches": 3}))


# The other gradient workloads, timed after the headline in the default run so
# that its JSON line holds them too: (workload, method or None).
OTHER_WORKLOADS = ((1, None), (3, None), (4, None), (4, "rodas3"), (4, "ros4"), (5, None),
                   (6, None), (2, "rkf78"))


def other_workloads(da, W, torch, np, steps: int = 2, warmup: int = 1, table: bool = False) -> list:
    """One job each (record, lane ordering, one gradient pass; the replay
    table too with `table`) of the other workloads at their full sizes, `warmup` + `steps`
    times: job time and gradient-pass time from HIP events on the launch
    stream, and the pass's algorithmic rate against its dtype's vector peak."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    out = []
    for wid, method in OTHER_WORKLOADS:
        w = W.WORKLOADS[wid]
        if method is not None:
            code = {"rodas3": W.RODAS3, "ros4": W.ROS4, "rkf78": W.RKF78}[method]
            old = W.METHOD_NAMES[w.method]
            w = dataclasses.replace(w, method=code, name=w.name.replace(old, method))
        prob = w.problem()
        inp = W.make_inputs(wid)
        u0 = torch.from_numpy(np.ascontiguousarray(inp["u0"].T)).to(dev)
        p = torch.from_numpy(np.ascontiguousarray(inp["p"].T)).to(dev)
        n, dt = w.n, u0.dtype
        aux, scale = None, 1.0
        if w.loss == W.MSE_SAVE:
            pt = torch.from_numpy(np.ascontiguousarray(inp["p_true"].T.astype(inp["p"].dtype)))
            aux = torch.nan_to_num(da.solve_fwd(prob, u0, pt.to(dev))[0])
            scale = 1.0 / (n * w.n_save_eff * w.dim)
        mesh = da.empty_mesh(prob, n, dt, dev, with_perm=True)
        job_ms, pass_ms = [], []
        for r in range(warmup + steps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            da.record(prob, u0, p, mesh=mesh, save=False)
            N = da.mesh_max_steps(mesh)   # sizes the gradient workspace (host sync)
            sm = da.mesh_sort(prob, mesh, perm=mesh.perm, table=table)
            call = da.ReplayGrad(prob, u0, p, sm, w.loss, aux=aux, scale=scale, max_n_steps=N)
            e[1].record(stream)
            call()
            e[2].record(stream)
            torch.cuda.synchronize()
            if r >= warmup:
                job_ms.append(e[0].elapsed_time(e[2]))
                pass_ms.append(e[1].elapsed_time(e[2]))
        ns = mesh.n_steps.double()
        ok = torch.from_numpy(mesh.status.cpu().numpy() == 0).to(dev)
        total_steps = float(ns[ok].sum().item())
        mname, rname = W.METHOD_NAMES[w.method], W.RHS_NAMES[w.rhs]
        fps = flop_per_step(mname, rname, w.dim)
        pm = sum(pass_ms) / len(pass_ms)
        achieved = fps * total_steps / (pm * 1e-3) / 1e12
        out.append({"workload": w.name, "dtype": w.dtype, "n": n,
                    "checkpoint": da.checkpoint_interval(prob, dt),
                    "job_ms": sum(job_ms) / len(job_ms), "pass_ms": pm,
                    "trajectory_gradients_per_s": n / (pm * 1e-3),
                    "achieved_tflops": achieved, "peak": PEAK_TFLOPS[w.dtype],
                    "frac": achieved / PEAK_TFLOPS[w.dtype], "flop_per_step": fps,
                    "mean_steps": float(ns.mean().item())})
        del mesh, sm, call, u0, p, aux
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--checkpoint", type=int, default=0,
                    help="reverse-sweep checkpoint interval (0 = library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-lanes", type=int, default=262144)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--rhs-source", action="store_true",
                    help="Lorenz-63 and Lorenz-96 workloads: run the system as a right-hand "
                         "side compiled at run time from source (Lorenz-96: as a cyclic "
                         "stencil) instead of the built-in one")
    ap.add_argument("--method", choices=["rodas3", "ros4", "rkf78"], default=None,
                    help="rodas3 / ros4: workload 4 (Robertson) with the third- / "
                         "fourth-order Rosenbrock method instead of ROS2; rkf78: workload 2 "
                         "(Lorenz-63) with Fehlberg 7(8) instead of Dopri5; same tolerances")
    ap.add_argument("--dense", action="store_true",
                    help="read the save times from the step interpolant (dense output) "
                         "instead of landing steps on them")
    ap.add_argument("--replay-table", action="store_true",
                    help="build the replay table in each job and let the gradient passes read "
                         "it instead of the tiled log (always on with --rhs-source)")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other workloads that the default run times after the "
                         "headline")
    args = ap.parse_args()
    # right-hand sides compiled at run time keep the guarded replay, which reads
    # one step size at a time: for them the table is faster at any pass count
    args.replay_table = args.replay_table or args.rhs_source
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU mode (trajectories "
              "are independent, so shards of the ensemble would run on separate GPUs).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return

    import numpy as np
    import torch
    import discrete_adjoint_amd as da
    import workloads as W

    w = W.WORKLOADS[args.workload]
    if args.method in ("rodas3", "ros4"):
        if args.workload != 4:
            sys.exit(f"--method {args.method} is available for workload 4 (Robertson)")
        code = W.RODAS3 if args.method == "rodas3" else W.ROS4
        w = dataclasses.replace(w, method=code, name=w.name.replace("ros2", args.method))
    elif args.method == "rkf78":
        if args.workload != 2:
            sys.exit("--method rkf78 is available for workload 2 (Lorenz-63)")
        w = dataclasses.replace(w, method=W.RKF78, name=w.name.replace("dopri5", "rkf78"))
    prob = w.problem(checkpoint=args.checkpoint, dense=int(args.dense))
    if args.rhs_source:
        tdt = torch.float64 if w.dtype == "f64" else torch.float32
        t_reg = time.perf_counter()
        if w.rhs == W.LORENZ63:
            rid = da.register_rhs(LORENZ63_SOURCE, 3, 3, tdt, w.method)
        elif w.rhs == W.LORENZ96:
            rid = da.register_rhs_stencil(LORENZ96_STENCIL, w.dim, 1, LORENZ96_OFFSETS, tdt,
                                          w.method)
        else:
            sys.exit("--rhs-source is available for the Lorenz-63 and Lorenz-96 workloads")
        t_reg = time.perf_counter() - t_reg
        prob = prob.replace(rhs=rid)
    n = w.n
    passes = w.passes
    dev = torch.device("cuda:0")
    inp = W.make_inputs(args.workload)
    u0 = torch.from_numpy(np.ascontiguousarray(inp["u0"].T)).to(dev)
    p = torch.from_numpy(np.ascontiguousarray(inp["p"].T)).to(dev)
    dt = u0.dtype
    aux, scale = None, 1.0
    if w.loss == W.MSE_SAVE:
        # targets: the same solver on perturbed parameters (computed on the GPU,
        # outside the timed region; only their shape and scale matter here)
        pt = torch.from_numpy(np.ascontiguousarray(inp["p_true"].T.astype(inp["p"].dtype)))
        aux, _, _ = da.solve_fwd(prob, u0, pt.to(dev))
        aux = torch.nan_to_num(aux)
        scale = 1.0 / (n * w.n_save_eff * w.dim)
    mesh = da.empty_mesh(prob, n, dt, dev, with_perm=True)
    sort_ws = torch.empty(da.mesh_sort_workspace(prob, n, dt), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    state = {"call": None, "N": -1, "rows": None}

    def job(events=None):
        e = events
        if e: e["rec0"].record(stream)
        da.record(prob, u0, p, mesh=mesh, save=False)
        if e: e["rec1"].record(stream)
        N = da.mesh_max_steps(mesh)           # sizes the workspace (and the table) (host sync)
        if args.replay_table and N != state["N"]:
            state["rows"] = torch.empty((max(N, 1), n), dtype=dt, device=dev)
        sm = da.mesh_sort(prob, mesh, perm=mesh.perm, table=args.replay_table,
                          h_rows=state["rows"], workspace=sort_ws)
        if e: e["sort1"].record(stream)
        if N != state["N"]:
            state["call"] = da.ReplayGrad(prob, u0, p, sm, w.loss, aux=aux, scale=scale,
                                          max_n_steps=N)
            state["N"] = N
        for k in range(passes):
            if e: e["p0"][k].record(stream)
            state["call"]()
            if e: e["p1"][k].record(stream)

    for _ in range(args.warmup):
        job()
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ev = {"rec0": torch.cuda.Event(enable_timing=True),
              "rec1": torch.cuda.Event(enable_timing=True),
              "sort1": torch.cuda.Event(enable_timing=True),
              "p0": [torch.cuda.Event(enable_timing=True) for _ in range(passes)],
              "p1": [torch.cuda.Event(enable_timing=True) for _ in range(passes)]}
        job(ev)
        evs.append(ev)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    rec_ms = float(np.mean([e["rec0"].elapsed_time(e["rec1"]) for e in evs]))
    sort_ms = float(np.mean([e["rec1"].elapsed_time(e["sort1"]) for e in evs]))
    pass_all = [e["p0"][k].elapsed_time(e["p1"][k]) for e in evs for k in range(passes)]
    pass_ms = float(np.mean(pass_all))
    pass_med = float(np.median(pass_all))
    pass_total = float(np.mean([sum(e["p0"][k].elapsed_time(e["p1"][k]) for k in range(passes))
                                for e in evs]))
    # the forward legs below read a replay table (built here, outside the
    # timed job, when the job has none)
    leg_mesh = state["call"].mesh if args.replay_table else \
        da.mesh_sort(prob, mesh, perm=mesh.perm)
    # forward-mode gradient of the same loss on the same replay order and
    # table: all d + P directions, and the P parameter directions alone
    def timed(fn):
        out = []
        for r in range(3):
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            fn()
            a1.record(stream)
            torch.cuda.synchronize()
            if r > 0:
                out.append(a0.elapsed_time(a1))
        return out
    sens_ms = timed(lambda: da.replay_sens(prob, u0, p, leg_mesh, w.loss, aux=aux,
                                           scale=scale, with_sens=False))
    sens_p_ms = timed(lambda: da.replay_sens_dirs(prob, u0, p, leg_mesh, prob.dim,
                                                  prob.n_params, w.loss, aux=aux, scale=scale,
                                                  with_sens=False))
    # the fused fixed-step replay alone (da_replay_fwd: saved states, no
    # gradient) on the same replay order and table
    fwd_ms = timed(lambda: da.replay_fwd(prob, u0, p, leg_mesh))
    # forward-only adaptive solve of the same ensemble (outside the job)
    solve_ms = []
    for r in range(3):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        da.solve_fwd(prob, u0, p)
        a1.record(stream)
        torch.cuda.synchronize()
        if r > 0:
            solve_ms.append(a0.elapsed_time(a1))
    st = mesh.status.cpu().numpy()
    ns = mesh.n_steps.double()
    ok = torch.from_numpy(st == 0).to(dev)
    total_steps = float(ns[ok].sum().item())
    mean_steps = float(ns.mean().item())
    mname, rname = W.METHOD_NAMES[w.method], W.RHS_NAMES[w.rhs]
    flop_step = flop_per_step(mname, rname, w.dim)
    sens_flop = sens_flop_per_step(mname, rname, w.dim)
    fwd_flop = fwd_flop_per_step(mname, rname, w.dim)
    achieved = flop_step * total_steps / (pass_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    ck_used = da.checkpoint_interval(prob, dt)
    traffic = None if args.rhs_source else read_traffic(w.name, kernel_family(mname, rname),
                                                          args.dense, ck_used)
    clk = None if (args.rhs_source or args.dense) else \
        read_valu_clock(w.name, kernel_family(mname, rname), ck_used)
    log_bytes = (mesh.h.numel() * mesh.h.element_size() + mesh.n_steps.numel() * 4
                 + mesh.save_idx.numel() * 4 + mesh.status.numel() * 4)
    out = {
        "metric": "trajectory-gradients/s (Lorenz FP64, 1M traj) + % of FP64 vector peak",
        "value": n * passes / (ms_per_step * 1e-3),
        "unit": "trajectory-gradients/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "n": n, "method": mname, "rhs": rname, "dim": w.dim,
                   "t1": w.t1, "rtol": w.rtol, "atol": w.atol, "max_steps": w.max_steps,
                   "passes_per_record": passes, "checkpoint": ck_used,
                   "saves": "dense output" if args.dense else "steps land on save times",
                   "rhs_source": "compiled at run time from source, vector-Jacobian products by "
                                 "forward-mode tangents" if args.rhs_source else "built in",
                   "replay_table": bool(args.replay_table),
                   "step": f"record + lane ordering{' and replay table' if args.replay_table else ''}"
                           f" + {passes} gradient pass{'es' if passes > 1 else ''}"},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": traffic, "kernel": "k_replay_grad",
                     "flop_per_step": flop_step, "populated_steps_per_launch": total_steps},
        "clock_adjusted": None if clk is None else {
            "clock_ghz": clk["clock_ghz"],
            "peak_at_clock": 256 * 128 * clk["clock_ghz"] / 1e3 * (1 if w.dtype == "f64" else 2),
            "frac_at_clock": achieved / (256 * 128 * clk["clock_ghz"] / 1e3
                                         * (1 if w.dtype == "f64" else 2)),
            "valu_busy": clk["valu_busy"],
            "executed_tflops": clk["flop_executed_per_launch"] / (pass_ms * 1e-3) / 1e12,
            "source": clk["source"]},
        "per_pass": {"ms": pass_ms, "median_ms": pass_med,
                     f"total_ms_{passes}_passes": pass_total,
                     "trajectory_gradients_per_s": n / (pass_ms * 1e-3)},
        "record_ms": rec_ms, "ordering_ms": sort_ms,
        "record_log": {"bytes": log_bytes, "GB_per_s": log_bytes / (rec_ms * 1e-3) / 1e9,
                       "what": "zero-padded step log written by the record kernel "
                               "(step sizes, step counts, save indices, status)"},
        "forward_mode_grad": {
            "ms": float(np.mean(sens_ms)),
            "trajectory_gradients_per_s": n / (float(np.mean(sens_ms)) * 1e-3),
            "flop_per_step": sens_flop,
            "achieved_tflops": None if sens_flop is None
            else sens_flop * total_steps / (float(np.mean(sens_ms)) * 1e-3) / 1e12},
        "forward_mode_param_grad": {
            "ms": float(np.mean(sens_p_ms)),
            "directions": prob.n_params,
            "trajectory_gradients_per_s": n / (float(np.mean(sens_p_ms)) * 1e-3)},
        "replay_fwd": {
            "ms": float(np.mean(fwd_ms)),
            "trajectory_replays_per_s": n / (float(np.mean(fwd_ms)) * 1e-3),
            "flop_per_step": fwd_flop,
            "achieved_tflops": None if fwd_flop is None
            else fwd_flop * total_steps / (float(np.mean(fwd_ms)) * 1e-3) / 1e12,
            "frac": None if fwd_flop is None
            else fwd_flop * total_steps / (float(np.mean(fwd_ms)) * 1e-3) / 1e12 / peak},
        "solve_fwd": {"ms": float(np.mean(solve_ms)),
                      "trajectory_solves_per_s": n / (float(np.mean(solve_ms)) * 1e-3)},
        "mesh": {"mean_steps": mean_steps, "max_steps": state["N"],
                 "max_over_mean": state["N"] / mean_steps, "failed_lanes": int((st != 0).sum())},
        "record_stats": record_stats(mesh),
    }
    if args.rhs_source:
        out["rhs_registration_s"] = t_reg
    default_run = (args.workload == 2 and args.method is None and not args.rhs_source
                   and not args.dense and not args.checkpoint)
    if default_run and not args.no_others:
        out["other_workloads"] = other_workloads(da, W, torch, np, table=args.replay_table)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_lanes, passes,
                                           dense=int(args.dense), method=w.method)
        out["cpu_baseline"]["gpu_over_cpu"] = out["value"] / out["cpu_baseline"]["value"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
