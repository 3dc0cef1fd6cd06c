"""Benchmark of the record-and-replay discrete adjoint on one MI355X.

Workload: Lorenz-63 ensemble of 2^20 trajectories in FP64, Dopri5,
rtol = atol = 1e-8, t in [0, 10], at most 4096 steps, loss = sum of squared
final states; one record then 10 replay-gradient passes against it.  Inputs
are synthetic (seeded, see workloads/) and resident on the GPU before the
timed region.

One timed step is that whole job: record, lane ordering, 10 gradient passes.
value = trajectories * passes / step time (trajectory-gradients/s).

Printed on one JSON line, besides the driver's fields:
  roofline      the gradient kernel (k_replay_grad) against the FP64 vector
                ALU peak: algorithmic FLOPs per launch (exact count of the
                replay step and its adjoint per populated step, times the
                populated steps of the record) / mean launch time from HIP
                events on the launch stream; traffic = HBM bytes per launch
                from rocprofv3 FETCH_SIZE + WRITE_SIZE counters (scaled by a
                copy-kernel calibration), when the kernel sources match the
                ones the counters were taken with, else null;
  cpu_baseline  the CPU oracle (plain C++, OpenMP) on a bounded sample of the
                same workload, as trajectory-gradients/s of the same job.

--gpus N with N > 1 is not supported (this build runs on one GPU).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# FP64 vector peak of MI355X: 256 CUs x 128 FP64 flop/clock (64 FMA lanes) x 2.4 GHz
PEAK_FP64_TFLOPS = 78.6
# Algorithmic FLOPs per populated step (FMA = 2, add/sub/mul = 1, negation = 0)
# of the replay step plus its adjoint (stage recomputation excluded), counted
# from the arithmetic schedule of the kernel:
#   forward: 6 right-hand sides x 8 + stage sums 46 per component x 3 = 186
#   adjoint: stage cotangent sums 40 per component x 3 = 120
#            + 6 stages x (J^T v 13 + J_p^T v 7 + accumulate 3) = 138
FLOP_PER_STEP = {("dopri5", "lorenz63"): 186 + 258, ("tsit5", "lorenz63"): 192 + 264}
COUNTERS_FILE = os.path.join(ROOT, "profiles", "replay_grad_lorenz63_dopri5_n1048576_counters.md")
KERNEL_SOURCES = ["lane_kernels.hpp", "erk.hip", "dadj_device.hpp", "dadj_internal.hpp"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "discrete_adjoint_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch from the committed counter summary, if it was taken
    with the current kernel sources."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    src_hash, traffic = None, None
    for line in open(COUNTERS_FILE):
        if line.startswith("kernel_source_hash:"):
            src_hash = line.split(":", 1)[1].strip()
        if line.startswith("hbm_bytes_per_launch:"):
            traffic = float(line.split(":", 1)[1].strip())
    return traffic if src_hash == kernel_source_hash() else None


def cpu_baseline(wid: int, lanes: int, passes: int, max_seconds: float = 20.0):
    """Oracle as it stands, plain rounding, all OpenMP threads: record + passes
    on the first `lanes` trajectories of the workload."""
    import numpy as np
    import oracle
    import workloads as W
    w = W.WORKLOADS[wid]
    inp = W.make_inputs(wid, lanes)
    prob = w.problem()
    cores = oracle.max_threads()
    t0 = time.perf_counter()
    m = oracle.record(prob, inp["u0"], inp["p"])
    t_rec = time.perf_counter() - t0
    N = int(m["n_steps"].max())
    m["h"] = np.ascontiguousarray(m["h"][:, :N])
    pn = prob.replace(max_steps=N)
    t_pass = []
    while len(t_pass) < 2 or (sum(t_pass) + t_rec < max_seconds and len(t_pass) < passes):
        t0 = time.perf_counter()
        oracle.replay_grad(pn, inp["u0"], inp["p"], m)
        t_pass.append(time.perf_counter() - t0)
    t_job = t_rec + passes * float(np.mean(t_pass))
    return {"value": lanes * passes / t_job, "unit": "trajectory-gradients/s", "cores": cores,
            "kind": "oracle",
            "sample": f"first {lanes} trajectories of the workload: record {t_rec:.2f} s + "
                      f"{len(t_pass)} timed gradient passes (mean {np.mean(t_pass):.3f} s), "
                      f"job time = record + {passes} passes"}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-lanes", type=int, default=65536)
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU mode (trajectories "
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
    prob = w.problem()
    n = w.n
    passes = w.passes
    dev = torch.device("cuda:0")
    inp = W.make_inputs(args.workload)
    u0 = torch.from_numpy(np.ascontiguousarray(inp["u0"].T)).to(dev)
    p = torch.from_numpy(np.ascontiguousarray(inp["p"].T)).to(dev)
    dt = u0.dtype
    mesh = da.empty_mesh(prob, n, dt, dev, with_perm=True)
    sort_ws = torch.empty(da.mesh_sort_workspace(prob, n, dt), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    state = {"call": None, "N": -1}

    def job(events=None):
        e = events
        if e: e["rec0"].record(stream)
        da.record(prob, u0, p, mesh=mesh, save=False)
        if e: e["rec1"].record(stream)
        da.mesh_sort(prob, mesh, perm=mesh.perm, workspace=sort_ws)
        if e: e["sort1"].record(stream)
        N = da.mesh_max_steps(mesh)           # sizes the workspace (host sync)
        if N != state["N"]:
            state["call"] = da.ReplayGrad(prob, u0, p, mesh, W.SUMSQ_FINAL, max_n_steps=N)
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
    pass_ms = float(np.mean([e["p0"][k].elapsed_time(e["p1"][k]) for e in evs
                             for k in range(passes)]))
    ns = mesh.n_steps.double()
    total_steps = float(ns.sum().item())
    mean_steps = total_steps / n
    flop_step = FLOP_PER_STEP[(W.METHOD_NAMES[w.method], W.RHS_NAMES[w.rhs])]
    achieved = flop_step * total_steps / (pass_ms * 1e-3) / 1e12
    traffic = read_traffic()
    out = {
        "metric": "trajectory-gradients/s (Lorenz FP64, 1M traj) + % of FP64 vector peak",
        "value": n * passes / (ms_per_step * 1e-3),
        "unit": "trajectory-gradients/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": w.name, "n": n, "method": W.METHOD_NAMES[w.method],
                   "rhs": W.RHS_NAMES[w.rhs], "t1": w.t1, "rtol": w.rtol, "atol": w.atol,
                   "max_steps": w.max_steps, "passes_per_record": passes,
                   "step": "record + lane ordering + 10 gradient passes"},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP64_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_FP64_TFLOPS,
                     "traffic": traffic, "kernel": "k_replay_grad",
                     "flop_per_step": flop_step, "populated_steps_per_launch": total_steps},
        "per_pass": {"ms": pass_ms, "trajectory_gradients_per_s": n / (pass_ms * 1e-3)},
        "record_ms": rec_ms, "sort_ms": sort_ms,
        "mesh": {"mean_steps": mean_steps, "max_steps": state["N"],
                 "max_over_mean": state["N"] / mean_steps},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_lanes, passes)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
