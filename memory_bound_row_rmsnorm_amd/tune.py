"""Measured plan selection for the row RMSNorm forward on MI355X.

For each (M, N, dtype) shape this times every launch plan of a search space
on the current GPU, with inputs cold in HBM, and reports each plan's kernel
resources (VGPRs, LDS) and occupancy (resident workgroups per compute unit,
waves per SIMD) next to its bandwidth.  The best plan per shape can be saved
and registered for rmsnorm_fwd (``binding.load_tuned``), which then uses it
instead of its built-in rule for exactly that shape.

The search covers what decides a memory-bound row kernel's speed on gfx950:
rows per wave and loads in flight (row slots), workgroup size, vectors per
lane, the register budget and occupancy (the trade-off the cuTile report in
"Why cutile's rmsnorm required full register" tunes by hand, opening report
and replies), the XCD row grouping and an occupancy cap.

    python -m memory_bound_row_rmsnorm_amd.tune --shape 16384x512:bf16 --shape 32768x8192:bf16 \\
        --save tuned.json --table table.md

Timing: every plan's launches are captured in a HIP graph that rotates over
enough input sets (at least 1 GiB of x, four times the 256 MB Infinity Cache)
that no launch finds its rows in a cache; time per launch is the replay's
event time over the launch count, median of three replays.
"""
from __future__ import annotations

import argparse
import ctypes
import itertools
import json
import sys

import torch

from . import binding

PEAK_GBPS = 8000.0
ROTATION_X_BYTES = 1 << 30
TORCH_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
ELEM_BYTES = {"bf16": 2, "fp16": 2, "fp32": 4}


def algorithmic_bytes(M: int, N: int, dtype: str = "bf16") -> int:
    """x read and y written once, w read once, fp32 rstd written once."""
    es = ELEM_BYTES[dtype]
    return 2 * M * N * es + N * es + 4 * M


def candidates(M: int, N: int, dtype: str, quick: bool = False) -> list:
    """Every valid plan of the search space for this shape (16-byte aligned pointers)."""
    base = binding.plan_query(M, N, dtype, cu_count=256)
    raw = []
    epv = 16 // ELEM_BYTES[dtype]
    if N % epv == 0:
        nvec = N // epv
        threads_set = (64, 128, 256, 512, 1024)
        for lanes, slots, threads in itertools.product((4, 8, 16, 32, 64), (1, 2, 4, 8), threads_set):
            vpl = -(-nvec // lanes)
            rows_per_trip = (threads // 64) * (64 // lanes) * slots
            raw.append(base.copy(variant=1, lanes_per_row=lanes, vectors_per_lane=vpl, row_slots=slots,
                                 block_threads=threads, prefetch=0, xcd_group=1, max_blocks_per_cu=0,
                                 grid=-(-M // rows_per_trip)))
        groups = (1, 8, 16, 64) if quick else (1, 4, 8, 16, 32, 64, 128)
        caps = (0, 4) if quick else (0, 2, 3, 4, 6, 8)
        for threads in threads_set:
            if threads > max(64, nvec):
                continue
            vpt = -(-nvec // threads)
            for g, cap in itertools.product(groups, caps):
                raw.append(base.copy(variant=2, lanes_per_row=threads, vectors_per_lane=vpt, row_slots=1,
                                     block_threads=threads, prefetch=0, xcd_group=g, max_blocks_per_cu=cap,
                                     grid=M))
        if nvec > 1024:
            # rows too wide for a few vectors per thread: the two-pass tiled kernel
            for threads, vpt, g in itertools.product((256, 512, 1024), (2, 4), groups):
                raw.append(base.copy(variant=6, lanes_per_row=threads, vectors_per_lane=vpt, row_slots=1,
                                     block_threads=threads, prefetch=0, xcd_group=g, max_blocks_per_cu=0,
                                     grid=M))
    else:
        # rows that start unaligned: the shifted kernels (aligned chunks, per-row shifted weights)
        nch = -(-(N + epv - 1) // epv)
        if nch <= 128:
            for lanes, slots, threads, pf in itertools.product((8, 16, 32, 64), (1, 2, 4), (64, 128, 256, 512), (0, 1)):
                vpl = -(-nch // lanes)
                if vpl > 2:
                    continue
                rows_per_trip = (threads // 64) * (64 // lanes) * slots
                raw.append(base.copy(variant=5, lanes_per_row=lanes, vectors_per_lane=vpl, row_slots=slots,
                                     block_threads=threads, prefetch=pf, xcd_group=1, max_blocks_per_cu=0,
                                     grid=-(-M // rows_per_trip)))
        groups = (1, 8, 16) if quick else (1, 4, 8, 16)
        for threads in (64, 128, 256, 512, 1024):
            vpt = -(-nch // threads)
            if threads > max(64, nch) or vpt > 4:
                continue
            for g, wpre in itertools.product(groups, (0, 1)):   # weights after the reduction / with the row
                raw.append(base.copy(variant=4, lanes_per_row=threads, vectors_per_lane=vpt, row_slots=1,
                                     block_threads=threads, prefetch=wpre, xcd_group=g, max_blocks_per_cu=0,
                                     grid=M))
    for threads in (64, 256, 1024):
        raw.append(base.copy(variant=3, block_threads=threads, prefetch=0, xcd_group=1, max_blocks_per_cu=0,
                             grid=M))
    out, seen = [], set()
    for p in raw:
        v = binding.plan_validate(M, N, dtype, p, cu_count=256)
        if v is None:
            continue
        key = tuple(getattr(v, f) for f in binding.PLAN_FIELDS)
        if key not in seen:
            seen.add(key)
            out.append(v)
    return out


class Buffers:
    """Rotation sets of x, y and rstd on the GPU (values: N(0, 1))."""

    def __init__(self, M: int, N: int, dtype: str, device="cuda:0"):
        xbytes = M * N * ELEM_BYTES[dtype]
        self.sets = max(2, -(-ROTATION_X_BYTES // xbytes))
        g = torch.Generator(device=device).manual_seed(0)
        td = TORCH_DTYPES[dtype]
        self.x = [torch.randn(M, N, device=device, generator=g).to(td) for _ in range(self.sets)]
        self.y = [torch.empty_like(t) for t in self.x]
        self.r = [torch.empty(M, device=device, dtype=torch.float32) for _ in range(self.sets)]
        self.w = (1.0 + 0.1 * torch.randn(N, device=device, generator=g)).to(td)


def time_plan(plan, bufs: Buffers, M: int, N: int, dtype: str, steps: int, reps: int = 3) -> float:
    """Median microseconds per launch over `reps` graph replays of `steps` launches."""
    code = binding.DTYPE_NAMES[dtype]
    pp = ctypes.byref(plan)
    fwd = binding.lib.rmsnorm_fwd_with_plan

    def launch(i, stream):
        k = i % bufs.sets
        st = fwd(bufs.x[k].data_ptr(), bufs.w.data_ptr(), bufs.y[k].data_ptr(), bufs.r[k].data_ptr(), M, N,
                 1e-6, 0.0, code, pp, stream)
        if st:
            raise binding.RmsnormError(st, binding.lib.rmsnorm_last_error().decode())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(min(steps, 2 * bufs.sets)):
            launch(i, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(steps):
            launch(i, side.cuda_stream)
    # replay() enqueues on the current stream: the events go there too
    replay_stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps + 1):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(replay_stream)
        graph.replay()
        end.record(replay_stream)
        end.synchronize()
        times.append(start.elapsed_time(end) * 1e3 / steps)
    del graph
    return sorted(times[1:])[len(times[1:]) // 2]


def describe(p) -> str:
    name = binding.VARIANT_NAMES.get(p.variant, str(p.variant))
    if p.variant in (1, 5):
        s = f"{name} {p.lanes_per_row}x{p.vectors_per_lane} lanes x vectors, {p.row_slots} slots, {p.block_threads} thr"
    elif p.variant in (2, 4, 6):
        s = f"{name} {p.block_threads} thr x {p.vectors_per_lane} vectors"
    else:
        s = f"{name} {p.block_threads} thr"
    if p.xcd_group > 1:
        s += f", xcd_group {p.xcd_group}"
    if p.max_blocks_per_cu:
        s += f", <= {p.max_blocks_per_cu} WG/CU"
    if p.prefetch:
        s += ", weights with the row" if p.variant == 4 else ", prefetch"
    return s


def tune_shape(M: int, N: int, dtype: str, quick: bool = False, log=print) -> list:
    """Time every candidate; returns result dicts sorted fastest first."""
    cands = candidates(M, N, dtype, quick)
    bufs = Buffers(M, N, dtype)
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = algorithmic_bytes(M, N, dtype)
    est_us = nbytes / 5.0e6 + 2.0      # at 5 TB/s (5e6 bytes per microsecond), plus the launch floor
    steps = int(min(2000, max(20, 10000.0 / est_us)))   # about 10 ms of launches per replay
    results = []
    for i, p in enumerate(cands):
        dev_plan = binding.plan_validate(M, N, dtype, p, bufs.x[0].data_ptr(), bufs.w.data_ptr(),
                                         bufs.y[0].data_ptr(), cu_count=0)
        res = binding.kernel_query(M, N, dtype, bufs.x[0].data_ptr(), bufs.w.data_ptr(), bufs.y[0].data_ptr(),
                                   plan=dev_plan)
        us = time_plan(dev_plan, bufs, M, N, dtype, steps)
        wg_per_cu = dev_plan.resident_grid / cu
        r = {
            "plan": {f: getattr(dev_plan, f) for f in binding.PLAN_FIELDS},
            "describe": describe(dev_plan),
            "kernel": res["kernel"],
            "vgprs": res["vgprs"], "lds_bytes": res["lds_bytes"], "scratch_bytes": res["scratch_bytes"],
            "wg_per_cu": wg_per_cu,
            "waves_per_simd": wg_per_cu * (dev_plan.block_threads // 64) / 4.0,
            "us": us, "gbps": nbytes / (us * 1e-6) / 1e9,
        }
        r["frac_of_peak"] = r["gbps"] / PEAK_GBPS
        results.append(r)
        log(f"  [{i + 1}/{len(cands)}] {r['describe']:70s} {us:9.3f} us {r['gbps']:7.0f} GB/s", flush=True)
    del bufs
    torch.cuda.empty_cache()
    results.sort(key=lambda r: r["us"])
    return results


def markdown_table(M: int, N: int, dtype: str, results: list, top: int = 0) -> str:
    default = binding.plan_query(M, N, dtype, cu_count=256)
    dkey = tuple(getattr(default, f) for f in binding.PLAN_FIELDS if f != "grid")
    lines = [f"### {M} x {N} {dtype} ({algorithmic_bytes(M, N, dtype):,} algorithmic bytes per launch)", "",
             "| plan | VGPRs | LDS B | WG/CU | waves/SIMD | us | GB/s | % of 8 TB/s |",
             "|---|---|---|---|---|---|---|---|"]
    rows = results if not top else results[:top]
    for r in rows:
        key = tuple(r["plan"][f] for f in binding.PLAN_FIELDS if f != "grid")
        mark = " (library rule)" if key == dkey else ""
        lines.append(f"| {r['describe']}{mark} | {r['vgprs']} | {r['lds_bytes']} | {r['wg_per_cu']:.0f} | "
                     f"{r['waves_per_simd']:.1f} | {r['us']:.3f} | {r['gbps']:.0f} | {100 * r['frac_of_peak']:.1f} |")
    return "\n".join(lines) + "\n"


def parse_shape(s: str):
    dims, _, dtype = s.partition(":")
    M, N = (int(v) for v in dims.lower().split("x"))
    dtype = dtype or "bf16"
    if dtype not in TORCH_DTYPES:
        raise argparse.ArgumentTypeError(f"dtype must be one of {sorted(TORCH_DTYPES)}")
    return M, N, dtype


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--shape", action="append", type=parse_shape, required=True, metavar="MxN[:dtype]")
    ap.add_argument("--quick", action="store_true", help="a smaller search space for the block family")
    ap.add_argument("--top", type=int, default=0, help="rows per table (0 = all)")
    ap.add_argument("--save", metavar="JSON", help="write the best plan per shape (binding.load_tuned format)")
    ap.add_argument("--table", metavar="MD", help="write the measured tables as markdown")
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("tune: no GPU visible", file=sys.stderr)
        return 2
    doc = {"device": torch.cuda.get_device_properties(0).name, "plans": []}
    tables = []
    for M, N, dtype in args.shape:
        print(f"== {M}x{N} {dtype}", flush=True)
        results = tune_shape(M, N, dtype, args.quick)
        best = results[0]
        doc["plans"].append({"M": M, "N": N, "dtype": dtype, "plan": best["plan"], "us": best["us"],
                             "gbps": best["gbps"], "describe": best["describe"]})
        table = markdown_table(M, N, dtype, results, args.top)
        tables.append(table)
        print(table, flush=True)
    if args.save:
        with open(args.save, "w") as f:
            json.dump(doc, f, indent=1)
            f.write("\n")
    if args.table:
        with open(args.table, "w") as f:
            f.write("\n".join(tables))
    return 0


if __name__ == "__main__":
    sys.exit(main())
