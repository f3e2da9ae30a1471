#!/usr/bin/env python3
"""Achieved HBM bandwidth of the row RMSNorm forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--mode graph|eager]

A step is one pass of the forward (one kernel launch) over one batch: x [M, N]
read once, y [M, N] and rstd [M] written once, w [N] read once.  Batches
rotate over S buffer sets held in one allocation (S copies of x, then S y
buffers), with S - 1 sets holding at least 1 GiB of x (four times the 256 MB
Infinity Cache; y is written with non-temporal stores and does not displace x
there).  Right before the timed launches one untimed walk touches every set in
order, and the timed launches continue the rotation, so whatever K is, every
timed launch reads an x that was last touched S - 1 sets earlier: its bytes
come from HBM (measured, the time per step stops changing once the rotation
passes about 400 MB of x).  All batches are resident in HBM before the timed
region.

GB/s = (2*M*N*s + N*s + 4*M) / seconds / 1e9, the read-plus-write formula of
"Rmsnorm Kernel Optimization" (Verification), with s = 2 bytes per element.
The timed region is bracketed by torch.cuda.synchronize(); HIP events on the
stream the kernels run on time it.  In graph mode (the default) the walk and
the K launches behind it are captured into one HIP graph, and the walk alone
into another; the time of the K launches is the first replay's time minus the
second's, so a graph launch's fixed cost, the same in both, cancels, and the K
launches run back to back behind the walk as in a long stream of launches.
The figure is the median of five such pairs of replays.

The default run (the 16384 x 512 bf16 headline) also times the 32768 x 8192
bf16 workload at four placements of y relative to x and reports it as a nested
record ("large_workload").

Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

def metric_name(direction: str, M: int, N: int, dtype: str) -> str:
    """The metric line's name; on the default workload (16384 x 512 bf16 forward) it reads
    "achieved HBM GB/s and % of MI355X peak, RMSNorm fwd 16384x512 bf16"."""
    return f"achieved HBM GB/s and % of MI355X peak, RMSNorm {direction} {M}x{N} {dtype}"
PEAK_GBPS = 8000.0           # MI355X HBM3E, published
MALL_BYTES = 256 * 2 ** 20   # Infinity Cache
ROTATION_X_BYTES = 4 * MALL_BYTES


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the forward kernels' own sources: a change to their code voids stored counters
FORWARD_SOURCES = ("rmsnorm_kernels.hip", "rmsnorm_device.hpp", "rmsnorm_internal.hpp")
# comments, string and character literals of C++ source (literals are kept, comments dropped)
_CXX_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^\\"\n])*"|\'(?:\\.|[^\\\'\n])*\'', re.S)


def code_of(source: str) -> str:
    """The source without comments, whitespace runs collapsed: edits to comments or layout leave
    it unchanged."""
    kept = _CXX_TOKENS.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", source)
    return " ".join(kept.split())


def kernel_source_sha256() -> str:
    h = hashlib.sha256()
    for name in FORWARD_SOURCES:
        with open(os.path.join(ROOT, "memory_bound_row_rmsnorm_amd", "csrc", name)) as f:
            h.update(name.encode() + b"\0" + code_of(f.read()).encode())
    return h.hexdigest()


def plan_key(plan_dict: dict) -> dict:
    """The launch a plan makes (kernel instance, shape, grid), without the
    device-dependent resident_grid."""
    return {k: v for k, v in plan_dict.items() if k != "resident_grid"}


def measured_traffic(workload: str, plan_dict: dict):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current forward kernel sources and the same launch plan; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_sha256():
        log(f"traffic: {path} was taken on other kernel sources; reporting null")
        return None
    if t.get("plan") != plan_key(plan_dict):
        log(f"traffic: {path} was taken with another launch plan; reporting null")
        return None
    return t.get("traffic_bytes_per_launch")


def counter_median_kib(path: str, kernel_substr: str, counter: str) -> float:
    import csv
    import statistics

    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {kernel_substr!r} in {path}")
    return statistics.median(vals)


def traffic_from_counters(wl, name: str, directory: str) -> dict:
    """HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs.

    Expects <dir>/<workload>_<kernel>_<COUNTER>_counter_collection.csv for
    kernel in (rmsnorm, copy): the runs of this script with --kernel rmsnorm
    and --kernel copy under `rocprofv3 --pmc FETCH_SIZE` and, separately,
    `--pmc WRITE_SIZE`.  Each counter is scaled by what it reads for the copy
    kernel, whose true bytes are known (M*N*2 read, M*N*2 written).
    """
    def f(kernel, counter, match):
        return counter_median_kib(
            os.path.join(directory, f"{name}_{kernel}_{counter}_counter_collection.csv"), match, counter)

    copy_bytes = wl.M * wl.N * wl.elem_bytes
    copy_fetch = f("copy", "FETCH_SIZE", "copyBuffer")
    copy_write = f("copy", "WRITE_SIZE", "copyBuffer")
    fetch_scale = copy_bytes / (copy_fetch * 1024)
    write_scale = copy_bytes / (copy_write * 1024)
    rms_fetch = f("rmsnorm", "FETCH_SIZE", "rmsnorm_")
    rms_write = f("rmsnorm", "WRITE_SIZE", "rmsnorm_")
    fetch_b = rms_fetch * 1024 * fetch_scale
    write_b = rms_write * 1024 * write_scale
    alg_read = wl.M * wl.N * wl.elem_bytes + wl.N * wl.elem_bytes
    alg_write = wl.M * wl.N * wl.elem_bytes + 4 * wl.M
    from memory_bound_row_rmsnorm_amd import binding

    # the plan the counted run used (default pointers align; the grid does not depend on the unit
    # count, which only sets resident_grid, left out of the key): host-only query
    plan = binding.plan_query(wl.M, wl.N, wl.dtype, cu_count=256)
    return {
        "workload": name,
        "kernel_source_sha256": kernel_source_sha256(),
        "plan": plan_key(plan.as_dict()),
        "counters_kib_per_dispatch": {"rmsnorm_FETCH_SIZE": rms_fetch, "rmsnorm_WRITE_SIZE": rms_write,
                                      "copy_FETCH_SIZE": copy_fetch, "copy_WRITE_SIZE": copy_write},
        "copy_bytes_each_way": copy_bytes,
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "fetch_bytes_per_launch": round(fetch_b),
        "write_bytes_per_launch": round(write_b),
        "traffic_bytes_per_launch": round(fetch_b + write_b),
        "algorithmic_read_bytes": alg_read,
        "algorithmic_write_bytes": alg_write,
        "traffic_over_algorithmic": (fetch_b + write_b) / (alg_read + alg_write),
    }


def load_copy_ceiling():
    """libcopy_ceiling.so (built with the package): the streaming copy the forward is measured
    against.  Raises when it has not been built."""
    import ctypes

    path = os.path.join(ROOT, "memory_bound_row_rmsnorm_amd", "libcopy_ceiling.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is not built: run python -m memory_bound_row_rmsnorm_amd.build")
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.copy_ceiling.argtypes = [vp, vp, i64, i32, i32, i64, vp]
    lib.copy_ceiling.restype = ctypes.c_int
    lib.copy_ceiling_sched.argtypes = [vp, vp, i64, i32, i32, i64, i32, vp]
    lib.copy_ceiling_sched.restype = ctypes.c_int
    lib.stream_part.argtypes = [vp, vp, i64, i32, i32, vp]
    lib.stream_part.restype = ctypes.c_int
    return lib


# the reference kernels of libcopy_ceiling.so: (name in a kernel trace, mode of stream_part, bytes per
# x byte moved); hip_copy is copy_ceiling itself
REFERENCE_KERNELS = {"hip_copy": ("copy_runs", 0, 2), "hip_read": ("read_runs", 1, 1),
                     "hip_write": ("write_runs", 2, 1), "hip_empty": ("empty_runs", 3, 0)}


def step_bytes(wl, kernel: str) -> int:
    """Bytes one launch of `kernel` moves on workload wl: the forward's algorithmic bytes, or a
    reference kernel's share of the M*N*s bytes of x (a copy moves them twice)."""
    if kernel == "rmsnorm":
        return wl.algorithmic_bytes()
    x_bytes = wl.M * wl.N * wl.elem_bytes
    return 2 * x_bytes if kernel == "copy" else REFERENCE_KERNELS[kernel][2] * x_bytes


def host_cpu_model() -> str:
    """The host processor's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, x_cpu, w_cpu, seconds: float, threads: int = 0):
    import oracle
    from memory_bound_row_rmsnorm_amd import workloads

    o = oracle.default()
    if threads > 0:
        o.set_threads(threads)
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
        "host_cpu": host_cpu_model(),
        "kind": "oracle",
        "sample": f"{reps} full passes of the fp64 oracle over one {wl.M}x{wl.N} {wl.dtype} batch "
                  f"({dt:.1f} s wall), same algorithmic bytes per pass as a GPU step",
    }


def bwd_algorithmic_bytes(wl) -> int:
    """x and dy read once, dx written once, w read once, rstd read once, fp32 dw written once."""
    s = wl.elem_bytes
    return 3 * wl.M * wl.N * s + wl.N * s + 4 * wl.M + 4 * wl.N


def bench_backward(args, wl, name, dev) -> int:
    import torch

    from memory_bound_row_rmsnorm_amd import binding, workloads

    read_bytes = 2 * wl.M * wl.N * wl.elem_bytes
    sets = args.sets or rotation_sets(read_bytes)
    log(f"backward {name}: M={wl.M} N={wl.N} {wl.dtype}, {sets} rotation sets")
    x0, w0 = workloads.make_inputs(wl, seed=0)
    dy0 = workloads.make_grad(wl, seed=0)
    x_d, dy_d, w_dev = x0.to(dev), dy0.to(dev), w0.to(dev)
    _, r_d = binding.rmsnorm_fwd(x_d, w_dev, wl.eps, wl.offset)     # rstd from the forward (input data only)
    # every set holds the same rows (the kernels' time does not depend on the values)
    xs = [x_d.clone() for _ in range(sets)]
    dys = [dy_d.clone() for _ in range(sets)]
    rs = [r_d.clone() for _ in range(sets)]
    dxs = [torch.empty_like(x_d) for _ in range(sets)]
    del x_d, dy_d, r_d
    dw = torch.empty(wl.N, dtype=torch.float32, device=dev)
    plan = binding.bwd_plan_query(wl.M, wl.N, wl.dtype, xs[0].data_ptr(), dys[0].data_ptr(), dxs[0].data_ptr())
    if args.plan:
        plan = plan.copy(**json.loads(args.plan))
        # the derived fields (rows per trip, trips, resident grid) of the plan as overridden
        done = binding.bwd_plan_validate(wl.M, wl.N, wl.dtype, plan, xs[0].data_ptr(), dys[0].data_ptr(),
                                         dxs[0].data_ptr())
        if done is not None:
            plan = done
    ws_bytes = plan.grid * wl.N * 4
    ws = torch.empty(ws_bytes // 4 + 4, dtype=torch.float32, device=dev)
    log("bwd plan", plan.as_dict(), f"workspace {ws_bytes} bytes")
    lib = binding.lib
    pplan = binding.ctypes.byref(plan)
    code = binding.DTYPE_NAMES[wl.dtype]

    def launch(k, h):
        st = lib.rmsnorm_bwd_with_plan(xs[k].data_ptr(), w_dev.data_ptr(), dys[k].data_ptr(), rs[k].data_ptr(),
                                       dxs[k].data_ptr(), dw.data_ptr(), wl.M, wl.N, wl.offset, code, pplan,
                                       ws.data_ptr(), ws.numel() * 4, h)
        if st != 0:
            raise binding.RmsnormError(st, lib.rmsnorm_last_error().decode())

    ms_per_step, _ = time_launches(launch, sets, args.steps, args.warmup, args.mode)
    nbytes = bwd_algorithmic_bytes(wl)
    gbps = nbytes / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": metric_name("bwd", wl.M, wl.N, wl.dtype),
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
            "pass": "bwd",
            "M": wl.M,
            "N": wl.N,
            "offset": wl.offset,
            "algorithmic_bytes_per_step": nbytes,
            "workspace_bytes": ws_bytes,
            "workspace_traffic_bytes_per_step": 2 * ws_bytes,
            "rotation_sets": sets,
            "inputs_sha256": {"x": workloads.sha256_of(x0), "w": workloads.sha256_of(w0),
                              "dy": workloads.sha256_of(dy0)},
            "inputs": inputs_label(sets, read_bytes),
            "launch": args.mode,
            "plan": plan.as_dict(),
            "pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
        },
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_GBPS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        import oracle

        o = oracle.default()
        xb, wb, db = (workloads.to_bits(t) for t in (x0, w0, dy0))
        _, r64 = o.rmsnorm_fwd(xb, wb, wl.eps, wl.offset, wl.dtype)
        reps, t0 = 0, time.perf_counter()
        while True:
            o.rmsnorm_bwd(xb, wb, db, r64, wl.offset, wl.dtype)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= args.cpu_seconds:
                break
        out["cpu_baseline"] = {"value": round(reps * nbytes / dt / 1e9, 3), "unit": "GB/s",
                               "cores": o.max_threads(), "host_cpu": host_cpu_model(), "kind": "oracle",
                               "sample": f"{reps} full passes of the fp64 oracle backward over one batch ({dt:.1f} s)"}
    print(json.dumps(out), flush=True)
    return 0


def rotation_sets(x_bytes: int, cap: int = 4096) -> int:
    """Buffer sets for a rotation in which, between two launches on one set, the other sets stream
    at least ROTATION_X_BYTES of x: ceil(ROTATION_X_BYTES / x_bytes) + 1 (at least 2, at most cap,
    which only binds below 256 KiB of x per launch)."""
    return max(2, min(cap, math.ceil(ROTATION_X_BYTES / x_bytes) + 1))


def inputs_label(sets: int, x_bytes: int) -> str:
    """How cold a launch's x is.  Every set is walked once, in order, right before the timed
    launches, and they rotate over all sets, so between two touches of one x the other sets'
    x streams (sets - 1) * x_bytes."""
    between = (sets - 1) * x_bytes
    if between >= ROTATION_X_BYTES:
        return f"cold in HBM ({between / 2**20:.0f} MiB of other x between two touches of one x)"
    return (f"warm: only {between / 2**20:.0f} MiB of other x between two touches of one x; rows may be "
            "cache-resident (Infinity Cache), not an HBM figure")


REGIONS = 5       # timed regions per measurement (median), at least
REGION_LAUNCHES = 500   # short runs take more regions, until they time about this many launches in all


def regions_for(steps: int) -> int:
    """Timed regions for `steps` launches each: 5, or more for short runs (25 at 20 steps), so the
    median is not left to a handful of noisy differences."""
    return max(REGIONS, min(41, -(-REGION_LAUNCHES // max(steps, 1))))


def time_launches(launch, sets: int, steps: int, warmup: int, mode: str):
    """Milliseconds per launch of `launch(k, stream_handle)` (set k) and the wall seconds of the
    bracketed region.

    W eager warm-up launches first.  Graph mode: two HIP graphs are captured, the walk (one launch
    on every set in order, k = 0 .. sets-1) and the walk followed, in the same graph, by exactly
    `steps` launches on sets i % sets.  Between torch.cuda.synchronize() calls, HIP events on the
    launch stream time one replay of the second graph and then one of the walk alone; their
    difference is the time of the `steps` launches running back to back behind the walk, as in a
    long stream of launches.  A graph launch and its event pair cost about 5-10 us once (the same
    in both replays, so it cancels; left in, it would add 0.3 us per step at 20 steps).  The
    result is the median over `regions_for(steps)` such pairs.  Eager mode: the walk, the start
    event, `steps` launches, the end event."""
    import statistics

    import torch

    stream = torch.cuda.current_stream()
    h = stream.cuda_stream or None
    for i in range(warmup):
        launch(i % sets, h)
    torch.cuda.synchronize()

    def timed(fn):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        fn()
        end.record()
        end.synchronize()
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    if mode == "graph":
        walk, walk_steps = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.graph(walk, stream=cap):
            hc = torch.cuda.current_stream().cuda_stream
            for k in range(sets):
                launch(k, hc)
        with torch.cuda.graph(walk_steps, stream=cap):
            hc = torch.cuda.current_stream().cuda_stream
            for k in range(sets):
                launch(k, hc)
            for i in range(steps):
                launch(i % sets, hc)
        torch.cuda.synchronize()
        walk_steps.replay()         # first replays: set-up stays out
        walk.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        diffs = [timed(walk_steps.replay) - timed(walk.replay) for _ in range(regions_for(steps))]
        wall = time.perf_counter() - t0
        time_launches.regions = [round(d / steps, 6) for d in diffs]
        return statistics.median(diffs) / steps, wall

    def eager():
        for k in range(sets):
            launch(k, h)

    torch.cuda.synchronize()
    eager()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        launch(i % sets, h)
    end.record()
    end.synchronize()
    torch.cuda.synchronize()
    time_launches.regions = [round(start.elapsed_time(end) / steps, 6)]
    return start.elapsed_time(end) / steps, time.perf_counter() - t0


class Rotation:
    """`sets` copies of one batch's x in one allocation, followed by `sets` y buffers placed
    `gap` bytes after the last x (y - x = sets * x_bytes + gap for every set), and rstd [sets, M].
    Every x holds the same rows (workloads.make_inputs, seed 0): the kernels' time does not depend
    on the values.  `place(gap)` moves the y buffers to another gap within the allocation."""

    @staticmethod
    def elems(wl, sets: int, max_gap: int = 0) -> int:
        """Elements of the allocation a rotation of `sets` sets of wl needs."""
        return 2 * sets * wl.M * wl.N + max_gap // wl.elem_bytes

    def __init__(self, wl, sets: int, dev, max_gap: int = 0, buf=None):
        import torch

        from memory_bound_row_rmsnorm_amd import workloads

        self.wl, self.sets = wl, sets
        es = wl.elem_bytes
        self.x_elems = wl.M * wl.N
        self.x_bytes = self.x_elems * es
        if max_gap % 256:
            raise ValueError("gaps must be multiples of 256 bytes")
        self.x_cpu, self.w_cpu = workloads.make_inputs(wl, seed=0)
        td = workloads.TORCH_DTYPES[wl.dtype]
        need = Rotation.elems(wl, sets, max_gap)
        if buf is None:
            self.buf = torch.empty(need, dtype=td, device=dev)
        else:                  # a slice of a caller's allocation (one allocation serves a whole sweep)
            if buf.numel() < need or buf.dtype != td:
                raise ValueError("the allocation is too small for this rotation")
            self.buf = buf[:need]
        self.buf[: sets * self.x_elems].view(sets, wl.M, wl.N).copy_(
            self.x_cpu.to(dev).unsqueeze(0).expand(sets, wl.M, wl.N))
        self.w = self.w_cpu.to(dev)
        self.rstd = torch.empty(sets * wl.M, dtype=torch.float32, device=dev)
        self.max_gap = max_gap
        self.place(0)

    def place(self, gap: int) -> None:
        if gap % 256 or gap > self.max_gap:
            raise ValueError("gap must be a multiple of 256 bytes within the allocation")
        self.gap = gap
        self.y_off = self.sets * self.x_elems + gap // self.wl.elem_bytes

    def x(self, k):
        return self.buf[k * self.x_elems:(k + 1) * self.x_elems].view(self.wl.M, self.wl.N)

    def y(self, k):
        o = self.y_off + k * self.x_elems
        return self.buf[o:o + self.x_elems].view(self.wl.M, self.wl.N)

    def pointers(self, k):
        es = self.wl.elem_bytes
        base = self.buf.data_ptr()
        return (base + k * self.x_bytes, self.w.data_ptr(), base + (self.y_off + k * self.x_elems) * es,
                self.rstd.data_ptr() + k * self.wl.M * 4)

    def y_minus_x(self) -> int:
        return (self.y_off) * self.wl.elem_bytes


def forward_launcher(rot: Rotation, plan, kernel: str = "rmsnorm", copy_vpl: int = 4, copy_threads: int = 256,
                     copy_stores: str = "serial"):
    """launch(k, stream_handle) for set k of the rotation: the forward with `plan`, torch's device
    copy of x into y, or the streaming copy of libcopy_ceiling.so."""
    from memory_bound_row_rmsnorm_amd import binding

    wl = rot.wl
    lib = binding.lib
    pplan = binding.ctypes.byref(plan)
    code = binding.DTYPE_NAMES[wl.dtype]
    copy_lib = load_copy_ceiling() if kernel in REFERENCE_KERNELS else None
    serial = {"serial": 1, "pipelined": 0}[copy_stores]

    def launch(k: int, h):
        if kernel == "copy":
            rot.y(k).copy_(rot.x(k))
            return
        xp, wp, yp, rp = rot.pointers(k)
        if kernel == "hip_copy":
            st = copy_lib.copy_ceiling_sched(xp, yp, rot.x_bytes, copy_vpl, copy_threads, 0, serial, h)
            if st != 0:
                raise RuntimeError(f"copy_ceiling returned {st}")
            return
        if kernel in REFERENCE_KERNELS:
            st = copy_lib.stream_part(xp, yp, rot.x_bytes, REFERENCE_KERNELS[kernel][1], copy_threads, h)
            if st != 0:
                raise RuntimeError(f"stream_part returned {st}")
            return
        st = lib.rmsnorm_fwd_with_plan(xp, wp, yp, rp, wl.M, wl.N, wl.eps, wl.offset, code, pplan, h)
        if st != 0:
            raise binding.RmsnormError(st, lib.rmsnorm_last_error().decode())

    return launch


def forward_plan(rot: Rotation, args):
    from memory_bound_row_rmsnorm_amd import binding

    wl = rot.wl
    xp, wp, yp, _ = rot.pointers(0)
    plan = binding.plan_query(wl.M, wl.N, wl.dtype, xp, wp, yp)
    if args.plan:
        plan = plan.copy(**json.loads(args.plan))
        # the derived fields (trips, rows per trip, resident grid) of the plan as overridden
        done = binding.plan_validate(wl.M, wl.N, wl.dtype, plan, xp, wp, yp)
        if done is not None:
            plan = done
    # the instance this call launches (the plan's, or its exact-width form) and its resources
    res = binding.kernel_query(wl.M, wl.N, wl.dtype, xp, wp, yp, plan=plan)
    return plan, res


def copy_grid_items(nbytes: int, vpl: int, threads: int) -> int:
    """Work-items of one libcopy_ceiling.so launch (one run of vpl KiB per wave)."""
    per_block = threads // 64 * 64 * vpl
    return -(-(nbytes // 16) // per_block) * threads


def gbps_of(nbytes: int, ms: float) -> float:
    return nbytes / (ms * 1e-3) / 1e9 if ms > 0 else 0.0


LARGE = "rmsnorm_32768x8192_bf16_outliers"
# y offsets past the last x at which the large workload is timed, in one allocation: its HBM rate
# depends on where y lies relative to x
LARGE_GAPS = (0, 16 << 10, 256 << 10, 16 << 20)


def large_rotation(dev):
    """The rotation of the 32768 x 8192 workload, with room for every gap of LARGE_GAPS."""
    from memory_bound_row_rmsnorm_amd import workloads

    wl = workloads.WORKLOADS[LARGE]
    return Rotation(wl, rotation_sets(wl.M * wl.N * wl.elem_bytes), dev, max_gap=max(LARGE_GAPS))


def bench_placements(args, rot, gaps, plan_json=None) -> dict:
    """The forward on rotation `rot` with y placed at each of `gaps` bytes after the last x (same
    protocol each time); the median over the placements is the record's value."""
    import statistics

    wl, sets = rot.wl, rot.sets
    plan, res = forward_plan(rot, argparse.Namespace(plan=plan_json))
    nbytes = wl.algorithmic_bytes()
    placements = []
    for gap in gaps:
        rot.place(gap)
        launch = forward_launcher(rot, plan)
        ms, _ = time_launches(launch, sets, args.steps, args.warmup, args.mode)
        placements.append({"y_minus_x_bytes": rot.y_minus_x(), "ms_per_step": round(ms, 6),
                           "value": round(gbps_of(nbytes, ms), 2),
                           "ms_per_step_regions": time_launches.regions})
        log(f"{wl.name} {wl.M}x{wl.N}: y - x = {rot.y_minus_x()} bytes: {ms * 1e3:.2f} us per step")
    ms_med = statistics.median(p["ms_per_step"] for p in placements)
    gbps = gbps_of(nbytes, ms_med)
    traffic = measured_traffic(wl.name, plan.as_dict())
    return {
        "workload": wl.name, "M": wl.M, "N": wl.N, "dtype": wl.dtype, "eps": wl.eps, "offset": wl.offset,
        "value": round(gbps, 2), "unit": "GB/s", "ms_per_step": round(ms_med, 6),
        "statistic": f"median over {len(placements)} placements of y relative to x",
        "min_ms_per_step": min(p["ms_per_step"] for p in placements),
        "max_ms_per_step": max(p["ms_per_step"] for p in placements),
        "pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
        "algorithmic_bytes_per_step": nbytes, "rotation_sets": sets, "inputs": inputs_label(sets, wl.M * wl.N * 2),
        "placements": placements, "plan": plan.as_dict(), "kernel_resources": res,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_GBPS, 4), "traffic": traffic},
    }


def trace_fit(path: str, wl, rows: list, steps: int, kernel: str, copy_vpl: int, copy_threads: int,
              fit_from: int) -> dict:
    """Per-launch kernel durations of a row-count sweep from a rocprofv3 kernel_trace.csv, and the
    least-squares line t = intercept + bytes / rate over the sweep points with M >= fit_from.

    A sweep point is identified by its dispatch size (work-items), which the rows determine; its
    timed launches are the last `steps` dispatches of that kernel and size in the trace."""
    import csv
    import statistics

    from memory_bound_row_rmsnorm_amd import binding

    if kernel != "rmsnorm" and kernel not in REFERENCE_KERNELS:
        raise SystemExit("--trace-fit takes --kernel rmsnorm or a libcopy_ceiling.so kernel")
    marker = "rmsnorm" if kernel == "rmsnorm" else REFERENCE_KERNELS[kernel][0]
    by_size = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if marker not in name:
                continue
            items = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"])
            by_size.setdefault(items, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), name))
    points = []
    for M in rows:
        w = wl.with_rows(M)
        if kernel == "rmsnorm":
            p = binding.plan_query(M, w.N, w.dtype, cu_count=256)
            items = p.grid * p.block_threads
            nbytes = w.algorithmic_bytes()
        else:
            items = copy_grid_items(M * w.N * w.elem_bytes, copy_vpl if kernel == "hip_copy" else 4, copy_threads)
            nbytes = step_bytes(w, kernel)
        rec = sorted(by_size.get(items, []))
        if len(rec) < steps:
            raise SystemExit(f"{path}: {len(rec)} dispatches of {kernel} with {items} work-items, need {steps}")
        timed = rec[-steps:]
        d = sorted((e - s) / 1e3 for s, e, _ in timed)
        span = (timed[-1][0] - timed[0][0]) / 1e3 / (steps - 1) if steps > 1 else None
        points.append({"M": M, "bytes": nbytes, "kernel": timed[-1][2], "mean_us": round(statistics.mean(d), 4),
                       "median_us": round(statistics.median(d), 4), "p10_us": round(d[len(d) // 10], 4),
                       "p90_us": round(d[(9 * len(d)) // 10], 4),
                       "start_to_start_us": round(span, 4) if span else None,
                       "gbps_mean": round(gbps_of(nbytes, statistics.mean(d) * 1e-3), 1) if nbytes else None})
    fit = [q for q in points if q["M"] >= fit_from]
    n = len(fit)
    if n >= 2 and any(q["bytes"] for q in fit):
        xs = [q["bytes"] for q in fit]
        ts = [q["mean_us"] for q in fit]
        mx, mt = sum(xs) / n, sum(ts) / n
        sxx = sum((a - mx) ** 2 for a in xs)
        slope = sum((a - mx) * (b - mt) for a, b in zip(xs, ts)) / sxx     # us per byte
        icpt = mt - slope * mx
        resid = max(abs(b - (icpt + slope * a)) for a, b in zip(xs, ts))
        line = {"intercept_us": round(icpt, 4), "rate_tb_per_s": round(1e-6 / slope, 4),
                "max_residual_us": round(resid, 4), "points": n, "from_rows": fit_from}
    else:
        line = None
    return {"trace": path, "kernel": kernel, "N": wl.N, "dtype": wl.dtype, "steps": steps, "points": points,
            "fit": line}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--rows", type=int, default=0, help="run the workload's recipe with this many rows")
    ap.add_argument("--cols", type=int, default=0, help="run the workload's recipe with rows of this many columns")
    ap.add_argument("--sweep-rows", default=None, metavar="M1,M2,...",
                    help="time the forward (or --kernel) at each row count in turn, one JSON line each, and exit")
    ap.add_argument("--sets", type=int, default=0, help="rotation buffer sets (0 = auto)")
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph")
    ap.add_argument("--plan", default=None, help="JSON object overriding plan fields")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-large", action="store_true",
                    help="skip the nested 32768x8192 record of the default (headline) run")
    ap.add_argument("--y-gaps", default=None, metavar="B1,B2,...",
                    help="time the forward with y placed at each of these byte gaps after the last x (one "
                         "allocation; --plan applies), print one JSON record of the placements, and exit")
    ap.add_argument("--traffic-from", default=None, metavar="DIR",
                    help="write profiles/traffic_<workload>.json from rocprofv3 counter CSVs in DIR "
                         "and exit (no GPU needed)")
    ap.add_argument("--trace-fit", default=None, metavar="CSV",
                    help="kernel durations and the intercept/rate line of a --sweep-rows run traced by "
                         "rocprofv3 --kernel-trace, from its kernel_trace.csv (no GPU needed)")
    ap.add_argument("--fit-from", type=int, default=1024, help="--trace-fit: fit rows from this M on")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the CPU oracle baseline (0 = the OpenMP default: all host cores)")
    ap.add_argument("--tuned", default=None, metavar="JSON",
                    help="register the tuned plans of this file (python -m memory_bound_row_rmsnorm_amd.tune "
                         "--save) before planning")
    ap.add_argument("--pass", dest="direction", choices=["fwd", "bwd"], default="fwd",
                    help="bwd: time the backward (row pass + dw column pass) instead")
    ap.add_argument("--kernel", choices=["rmsnorm", "copy", *REFERENCE_KERNELS], default="rmsnorm",
                    help="copy: time torch's device copy of x into y instead (the runtime's copy "
                         "kernel; same rotation, 2*M*N*s bytes per step), the counter calibration "
                         "reference; hip_copy: the streaming copy of libcopy_ceiling.so (16-byte "
                         "non-temporal accesses, --copy-vpl KiB per wave), the practical ceiling; "
                         "hip_read / hip_write: its read half (x only) and write half (y only); "
                         "hip_empty: an empty kernel over the copy's grid (launch and completion)")
    ap.add_argument("--copy-vpl", type=int, default=4, choices=[1, 2, 4, 8],
                    help="hip_copy: contiguous KiB each wave moves per run")
    ap.add_argument("--copy-threads", type=int, default=256, help="hip_copy: workgroup size")
    ap.add_argument("--copy-stores", choices=["serial", "pipelined"], default="serial",
                    help="hip_copy: one store in flight per wave (each waits for the wave's earlier "
                         "memory operations), or stores back to back")
    args = ap.parse_args()

    if args.traffic_from:
        from memory_bound_row_rmsnorm_amd import workloads

        name = args.workload or workloads.HEADLINE
        t = traffic_from_counters(workloads.WORKLOADS[name], name, args.traffic_from)
        out = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
        with open(out, "w") as f:
            json.dump(t, f, indent=1)
            f.write("\n")
        print(json.dumps(t))
        return 0

    if args.trace_fit:
        from memory_bound_row_rmsnorm_amd import workloads

        if not args.sweep_rows:
            raise SystemExit("--trace-fit needs the --sweep-rows list of the traced run")
        wl = workloads.WORKLOADS[args.workload or workloads.HEADLINE]
        rows = [int(v) for v in args.sweep_rows.split(",")]
        print(json.dumps(trace_fit(args.trace_fit, wl, rows, args.steps, args.kernel, args.copy_vpl,
                                   args.copy_threads, args.fit_from)))
        return 0

    if args.gpus != 1:
        log(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported. The row "
            "RMSNorm forward shards over rows with no communication; run one process per GPU.")
        return 2

    import torch

    from memory_bound_row_rmsnorm_amd import binding, workloads

    name = args.workload or workloads.HEADLINE
    wl = workloads.WORKLOADS[name]
    if args.rows:
        wl = wl.with_rows(args.rows)
    if args.cols:
        wl = dataclasses.replace(wl, N=args.cols)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.direction == "bwd":
        return bench_backward(args, wl, name, dev)
    if args.tuned:
        log("tuned plans registered:", binding.load_tuned(args.tuned))

    if args.y_gaps:
        gaps = [int(v) for v in args.y_gaps.split(",")]
        rot = Rotation(wl, args.sets or rotation_sets(wl.M * wl.N * wl.elem_bytes), dev, max_gap=max(gaps))
        rec = bench_placements(args, rot, gaps, args.plan)
        rec["metric"] = metric_name("fwd", wl.M, wl.N, wl.dtype)
        print(json.dumps(rec), flush=True)
        return 0

    if args.sweep_rows:
        rows = [int(v) for v in args.sweep_rows.split(",")]
        # one allocation for every row count, as large as the largest rotation needs (allocations
        # made after others were freed measured up to 7% slower on 16384 x 512)
        cap = max(Rotation.elems(wl.with_rows(M), rotation_sets(M * wl.N * wl.elem_bytes)) for M in rows)
        pool = torch.empty(cap, dtype=workloads.TORCH_DTYPES[wl.dtype], device=dev)
        for M in rows:
            w = wl.with_rows(M)
            x_bytes = M * w.N * w.elem_bytes
            sets = rotation_sets(x_bytes)
            rot = Rotation(w, sets, dev, buf=pool)
            plan, res = forward_plan(rot, args)
            launch = forward_launcher(rot, plan, args.kernel, args.copy_vpl, args.copy_threads, args.copy_stores)
            ms, _ = time_launches(launch, sets, args.steps, args.warmup, args.mode)
            nbytes = step_bytes(w, args.kernel)
            print(json.dumps({"M": M, "N": w.N, "dtype": w.dtype, "kernel": args.kernel,
                              "instance": res["kernel"] if args.kernel == "rmsnorm" else args.kernel,
                              "sets": sets, "steps": args.steps, "ms_per_step": round(ms, 6),
                              "gbps": round(gbps_of(nbytes, ms), 1), "inputs": inputs_label(sets, x_bytes)}),
                  flush=True)
            del rot
        return 0

    x_bytes = wl.M * wl.N * wl.elem_bytes
    sets = args.sets or rotation_sets(x_bytes)
    log(f"workload {name}: M={wl.M} N={wl.N} {wl.dtype}, {sets} rotation sets "
        f"({sets * (2 * x_bytes + 4 * wl.M) / 2**20:.0f} MiB), mode {args.mode}")
    default_run = (name == workloads.HEADLINE and not args.rows and not args.cols and args.kernel == "rmsnorm"
                   and not args.plan and not args.sets and not args.tuned)
    # both rotations are allocated before either is timed (an allocation made after a large one was
    # freed measured up to 7% slower)
    large_rot = large_rotation(dev) if default_run and not args.no_large else None
    rot = Rotation(wl, sets, dev)
    plan, res = forward_plan(rot, args)
    log("plan", plan.as_dict(), "resources", res)
    launch = forward_launcher(rot, plan, args.kernel, args.copy_vpl, args.copy_threads, args.copy_stores)
    ms_per_step, wall_s = time_launches(launch, sets, args.steps, args.warmup, args.mode)
    nbytes = step_bytes(wl, args.kernel)
    gbps = gbps_of(nbytes, ms_per_step)
    log(f"{name}: {ms_per_step * 1e3:.3f} us per step, {gbps:.0f} GB/s")
    y_minus_x = rot.y_minus_x()
    x0, w0 = rot.x_cpu, rot.w_cpu

    reshaped = bool(args.rows or args.cols)
    traffic = measured_traffic(name, plan.as_dict()) if (args.kernel == "rmsnorm" and not reshaped) else None
    out = {
        "metric": metric_name("fwd", wl.M, wl.N, wl.dtype),
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
            "workload": name if not reshaped else f"{name} recipe at {wl.M} x {wl.N}",
            "M": wl.M,
            "N": wl.N,
            "eps": wl.eps,
            "offset": wl.offset,
            "algorithmic_bytes_per_step": nbytes,
            "rotation_sets": sets,
            # where y lies relative to x (every set): on wide rows the HBM rate depends on it
            "y_minus_x_bytes": y_minus_x,
            # the inputs every rotation set holds (seed 0), as drawn by workloads.make_inputs
            "inputs_sha256": {"x": workloads.sha256_of(x0), "w": workloads.sha256_of(w0)},
            "inputs": inputs_label(sets, x_bytes),
            "launch": args.mode,
            "kernel": args.kernel,
            **({"copy": {"kib_per_wave_run": args.copy_vpl, "threads": args.copy_threads,
                         "stores": args.copy_stores}}
               if args.kernel == "hip_copy" else {}),
            "plan": {k: v for k, v in plan.as_dict().items()},
            "kernel_resources": res,
            "pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
            "wall_s_timed_region": round(wall_s, 4),
            # the per-step time of each timed region (the value is their median)
            "ms_per_step_regions": time_launches.regions,
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
    if large_rot is not None:
        out["large_workload"] = bench_placements(args, large_rot, LARGE_GAPS)
    del rot, large_rot
    if not args.no_cpu_baseline and args.kernel == "rmsnorm":
        log(f"cpu baseline: oracle for about {args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(wl, x0, w0, args.cpu_seconds, args.cpu_threads)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
