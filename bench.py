#!/usr/bin/env python3
"""Achieved HBM bandwidth of the row RMSNorm forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--mode graph|eager]

A step is one pass of the forward (one kernel launch) over one batch: x [M, N]
read once, y [M, N] and rstd [M] written once, w [N] read once.  Batches
rotate over enough distinct (x, y, rstd) buffer sets (512 MiB or more in total)
that a step never finds its batch in the 256 MB Infinity Cache left by the
previous ones, so the bytes come from HBM.  All batches are resident in HBM
before the timed region.

GB/s = (2*M*N*s + N*s + 4*M) / seconds / 1e9, the read-plus-write formula of
"Rmsnorm Kernel Optimization" (Verification), with s = 2 bytes per element.
The timed region is bracketed by torch.cuda.synchronize() and HIP events on
the stream the kernels run on; in graph mode the K launches are captured once
into a HIP graph and the timed region replays it.

Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s and % of MI355X peak, RMSNorm fwd 16384x512 bf16"
PEAK_GBPS = 8000.0           # MI355X HBM3E, published
MALL_BYTES = 256 * 2 ** 20   # Infinity Cache
ROTATION_BYTES = 512 * 2 ** 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha256() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "memory_bound_row_rmsnorm_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_sha256():
        log(f"traffic: {path} was taken on other kernel sources; reporting null")
        return None
    return t.get("traffic_bytes_per_launch")


def cpu_baseline(wl, x_cpu, w_cpu, seconds: float):
    import oracle
    from memory_bound_row_rmsnorm_amd import workloads

    o = oracle.default()
    xb, wb = workloads.to_bits(x_cpu), workloads.to_bits(w_cpu)
    o.rmsnorm_fwd(xb[:8], wb, wl.eps, wl.offset, wl.dtype)      # load, touch
    reps, t0 = 0, time.perf_counter()
    while True:
        o.rmsnorm_fwd(xb, wb, wl.eps, wl.offset, wl.dtype)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    gbps = reps * wl.algorithmic_bytes() / dt / 1e9
    return {
        "value": round(gbps, 3),
        "unit": "GB/s",
        "cores": o.max_threads(),
        "kind": "oracle",
        "sample": f"{reps} full passes of the fp64 oracle over one {wl.M}x{wl.N} {wl.dtype} batch "
                  f"({dt:.1f} s wall), same algorithmic bytes per pass as a GPU step",
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--sets", type=int, default=0, help="rotation buffer sets (0 = auto)")
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph")
    ap.add_argument("--plan", default=None, help="JSON object overriding plan fields")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        log(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported. The row "
            "RMSNorm forward shards over rows with no communication; run one process per GPU.")
        return 2

    import torch

    from memory_bound_row_rmsnorm_amd import binding, workloads

    name = args.workload or workloads.HEADLINE
    wl = workloads.WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    per_set = 2 * wl.M * wl.N * 2 + 4 * wl.M
    sets = args.sets or max(2, min(64, math.ceil(ROTATION_BYTES / per_set)))

    log(f"workload {name}: M={wl.M} N={wl.N} {wl.dtype}, {sets} rotation sets "
        f"({sets * per_set / 2**20:.0f} MiB), mode {args.mode}")
    xs, ys, rs = [], [], []
    x0 = w0 = None
    for k in range(sets):
        x, w = workloads.make_inputs(wl, seed=k)
        if k == 0:
            x0, w0 = x, w
        xs.append(x.to(dev))
        ys.append(torch.empty_like(xs[-1]))
        rs.append(torch.empty(wl.M, dtype=torch.float32, device=dev))
    w_dev = w0.to(dev)

    plan = binding.plan_query(wl.M, wl.N, wl.dtype, xs[0].data_ptr(), w_dev.data_ptr(),
                              ys[0].data_ptr())
    if args.plan:
        plan = plan.copy(**json.loads(args.plan))
    res = binding.plan_resources(plan, wl.dtype)
    log("plan", plan.as_dict(), "resources", res)

    lib = binding.lib
    pplan = binding.ctypes.byref(plan)
    code = binding.DTYPE_NAMES[wl.dtype]
    argv = [(xs[k].data_ptr(), w_dev.data_ptr(), ys[k].data_ptr(), rs[k].data_ptr()) for k in range(sets)]

    def launch(i: int, stream_handle):
        xp, wp, yp, rp = argv[i % sets]
        st = lib.rmsnorm_fwd_with_plan(xp, wp, yp, rp, wl.M, wl.N, wl.eps, wl.offset, code, pplan,
                                       stream_handle)
        if st != 0:
            raise binding.RmsnormError(st, lib.rmsnorm_last_error().decode())

    stream = torch.cuda.current_stream()
    h = stream.cuda_stream or None
    for i in range(args.warmup):
        launch(i, h)
    torch.cuda.synchronize()

    graph = None
    if args.mode == "graph":
        # capture the K timed launches once; the timed region replays them
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.graph(graph, stream=cap):
            hc = torch.cuda.current_stream().cuda_stream
            for i in range(args.steps):
                launch(i, hc)
        torch.cuda.synchronize()
        graph.replay()          # untimed replay: first-replay setup stays out of the timing
        torch.cuda.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    if graph is not None:
        start.record()
        graph.replay()
        end.record()
    else:
        start.record()
        for i in range(args.steps):
            launch(i, h)
        end.record()
    end.synchronize()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / args.steps
    nbytes = wl.algorithmic_bytes()
    gbps = nbytes / (ms_per_step * 1e-3) / 1e9

    traffic = measured_traffic(name)
    out = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": name,
            "M": wl.M,
            "N": wl.N,
            "eps": wl.eps,
            "offset": wl.offset,
            "algorithmic_bytes_per_step": nbytes,
            "rotation_sets": sets,
            "launch": args.mode,
            "plan": {k: v for k, v in plan.as_dict().items()},
            "kernel_resources": res,
            "pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
            "wall_s_timed_region": round(wall_s, 4),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbps, 2),
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gbps / PEAK_GBPS, 4),
            "traffic": traffic,
        },
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle for about {args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(wl, x0, w0, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
