"""Host-side checks of bench.py's contract pieces: the metric name, the one-GPU
guard, and the counter arithmetic behind roofline.traffic (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from memory_bound_row_rmsnorm_amd import workloads  # noqa: E402


def test_metric_name_of_the_default_workload():
    wl = workloads.WORKLOADS[workloads.HEADLINE]
    assert bench.metric_name("fwd", wl.M, wl.N, wl.dtype) == \
        "achieved HBM GB/s and % of MI355X peak, RMSNorm fwd 16384x512 bf16"
    assert bench.metric_name("bwd", 32768, 8192, "bf16").endswith("RMSNorm bwd 32768x8192 bf16")


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def _write_counters(d, name, kernel, counter, kernel_name, kib):
    path = os.path.join(d, f"{name}_{kernel}_{counter}_counter_collection.csv")
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for v in (kib, kib, kib * 1.5):         # the median ignores one outlier dispatch
            f.write(f"{kernel_name},{counter},{v}\n")


def test_traffic_is_scaled_by_the_copy_kernels_reading(tmp_path):
    """FETCH_SIZE reading half the bytes for the copy must double the kernel's reading too."""
    name = "rmsnorm_16384x512_bf16"
    wl = workloads.WORKLOADS[name]
    copy_bytes = wl.M * wl.N * 2
    _write_counters(tmp_path, name, "copy", "FETCH_SIZE", "__amd_rocclr_copyBuffer", copy_bytes / 2 / 1024)
    _write_counters(tmp_path, name, "copy", "WRITE_SIZE", "__amd_rocclr_copyBuffer", copy_bytes / 1024)
    _write_counters(tmp_path, name, "rmsnorm", "FETCH_SIZE", "rmsnorm_wave<...>", (copy_bytes + 1024) / 2 / 1024)
    _write_counters(tmp_path, name, "rmsnorm", "WRITE_SIZE", "rmsnorm_wave<...>", (copy_bytes + 65536) / 1024)
    t = bench.traffic_from_counters(wl, name, str(tmp_path))
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    assert t["fetch_bytes_per_launch"] == copy_bytes + 1024
    assert t["write_bytes_per_launch"] == copy_bytes + 65536
    assert t["traffic_bytes_per_launch"] == 2 * copy_bytes + 1024 + 65536
    assert t["kernel_source_sha256"] == bench.kernel_source_sha256()
    assert "resident_grid" not in t["plan"]


def test_stale_traffic_is_reported_as_null(tmp_path, monkeypatch):
    name = "rmsnorm_16384x512_bf16"
    plan = {"variant": 1, "grid": 1024, "resident_grid": 2048}
    (tmp_path / "profiles").mkdir()
    doc = {"kernel_source_sha256": "0" * 64, "plan": bench.plan_key(plan), "traffic_bytes_per_launch": 123}
    (tmp_path / "profiles" / f"traffic_{name}.json").write_text(json.dumps(doc))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: "1" * 64)
    assert bench.measured_traffic(name, plan) is None                  # other kernel sources
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: "0" * 64)
    assert bench.measured_traffic(name, plan) == 123
    assert bench.measured_traffic(name, dict(plan, grid=512)) is None   # another launch plan
    assert bench.measured_traffic("rmsnorm_64x512_bf16", plan) is None  # no summary at all


def test_copy_ceiling_library_rejects_bad_arguments_before_any_hip_call():
    """libcopy_ceiling.so (the practical ceiling bench.py --kernel hip_copy times) checks its
    arguments on the host; every call below fails before a launch."""
    lib = bench.load_copy_ceiling()
    a, b = 0x10000000, 0x20000000
    assert lib.copy_ceiling(a, b, 0, 4, 256, 0, None) == 0            # nothing to copy: no launch
    assert lib.copy_ceiling(a, b, 100, 4, 256, 0, None) == 1          # not a multiple of 16 bytes
    assert lib.copy_ceiling(a + 8, b, 1024, 4, 256, 0, None) == 1     # misaligned source
    assert lib.copy_ceiling(a, b, 1024, 3, 256, 0, None) == 1         # no such run length
    assert lib.copy_ceiling(a, b, 1024, 4, 100, 0, None) == 1         # workgroup not whole waves
    assert lib.copy_ceiling(a, a + 512, 1024, 4, 256, 0, None) == 1   # overlap
    assert lib.copy_ceiling(None, b, 1024, 4, 256, 0, None) == 1
    assert lib.copy_ceiling_sched(a, b, 0, 4, 256, 0, 0, None) == 0   # either schedule, nothing to copy
    assert lib.copy_ceiling_sched(a, b, 1024, 4, 256, 0, 2, None) == 1  # no such store schedule
    assert lib.copy_ceiling_sched(a, b, 100, 4, 256, 0, 0, None) == 1


def test_rotation_keeps_a_gib_of_other_x_between_two_touches():
    """Every timed launch reads an x last touched S - 1 sets earlier; S - 1 sets hold >= 1 GiB."""
    for x_bytes in (16 << 20, 512 << 20, 46_875_000 + 1, 64 << 20, 128 << 20, 1 << 30, 3 << 30):
        s = bench.rotation_sets(x_bytes)
        assert s >= 2 and (s - 1) * x_bytes >= bench.ROTATION_X_BYTES
        assert bench.inputs_label(s, x_bytes).startswith("cold in HBM")
    assert bench.rotation_sets(16 << 20) == 65
    assert bench.rotation_sets(512 << 20) == 3
    # tiny batches: the set count is capped, and the label says the rows may sit in a cache
    s = bench.rotation_sets(16 << 10)
    assert s == 4096 and bench.inputs_label(s, 16 << 10).startswith("warm")
    assert bench.inputs_label(20, 16 << 20).startswith("warm")


def _trace_row(name, start, dur, items, threads=256):
    return (f'"KERNEL_DISPATCH","Agent 1",1,0,1,1,1,"{name}",1,{start},{start + dur},0,0,8,0,16,'
            f'{threads},1,1,{items},1,1\n')


def test_trace_fit_recovers_intercept_and_rate(tmp_path):
    """Synthetic trace: t = 2 us + bytes / (7 TB/s) for the forward at several row counts (plus
    warm-up dispatches that must not count and another kernel that must be ignored)."""
    from memory_bound_row_rmsnorm_amd import binding

    wl = workloads.WORKLOADS[workloads.HEADLINE]
    rows = [1024, 4096, 16384, 65536]
    path = tmp_path / "k_kernel_trace.csv"
    t = 1_000_000
    with open(path, "w") as f:
        f.write('"Kind","Agent_Id","Queue_Id","Stream_Id","Thread_Id","Dispatch_Id","Kernel_Id","Kernel_Name",'
                '"Correlation_Id","Start_Timestamp","End_Timestamp","LDS_Block_Size","Scratch_Size","VGPR_Count",'
                '"Accum_VGPR_Count","SGPR_Count","Workgroup_Size_X","Workgroup_Size_Y","Workgroup_Size_Z",'
                '"Grid_Size_X","Grid_Size_Y","Grid_Size_Z"\n')
        for M in rows:
            p = binding.plan_query(M, wl.N, wl.dtype, cu_count=256)
            items = p.grid * p.block_threads
            ns = round(2000 + wl.with_rows(M).algorithmic_bytes() / 7e12 * 1e9)
            for i in range(5):            # warm-up: slower, and before the timed ones
                f.write(_trace_row("void rmsnorm_wave_exact<...>(...)", t, 3 * ns, items))
                t += 10 * ns
            for i in range(10):
                f.write(_trace_row("void rmsnorm_wave_exact<...>(...)", t, ns, items))
                f.write(_trace_row("__amd_rocclr_fillBufferAligned", t + ns, 100, items))
                t += 2 * ns
    r = bench.trace_fit(str(path), wl, rows, 10, "rmsnorm", 4, 256, fit_from=1024)
    assert r["fit"]["intercept_us"] == pytest.approx(2.0, abs=0.01)
    assert r["fit"]["rate_tb_per_s"] == pytest.approx(7.0, rel=1e-3)
    assert [q["M"] for q in r["points"]] == rows
    assert all(q["median_us"] == q["mean_us"] for q in r["points"])


def test_counter_hash_ignores_comments_and_layout():
    """Stored counters stay valid across edits to comments or layout of the kernel sources, and
    are voided by any change to the code itself (a string literal keeps its comment markers)."""
    base = 'int f(int a) { return a + 1; }  // add one\nconst char* s = "x//y";\n'
    assert bench.code_of(base) == bench.code_of('/* adds */ int f(int a)\n{\n    return a + 1;\n}\nconst char* s = "x//y";')
    assert bench.code_of(base) != bench.code_of(base.replace("a + 1", "a + 2"))
    assert bench.code_of(base) != bench.code_of(base.replace('"x//y"', '"x/y"'))
    assert "add one" not in bench.code_of(base) and '"x//y"' in bench.code_of(base)


def test_short_runs_take_more_timed_regions():
    """Each timed region is exactly `steps` launches; short runs take more regions so the median
    rests on enough of them (about 500 launches in all, at least 5 regions, at most 41)."""
    assert bench.regions_for(2000) == 5 and bench.regions_for(100) == 5
    assert bench.regions_for(20) == 25 and bench.regions_for(50) == 10
    assert bench.regions_for(1) == 41
