"""GPU tests of tuned dispatch: a registered plan is the one rmsnorm_fwd runs,
its results meet the same acceptance bar against the oracle, and the tuner's
measured best plan does too."""
from __future__ import annotations

import pytest
import torch

from memory_bound_row_rmsnorm_amd import workloads
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def bnd():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from memory_bound_row_rmsnorm_amd import binding
    binding.clear_tuned()
    yield binding
    binding.clear_tuned()


def run_and_check(bnd, wl, rows, what):
    x, w = workloads.make_inputs(wl, seed=5, rows=rows)
    xg, wg = x.to(DEV), w.to(DEV)
    y, rstd = bnd.rmsnorm_fwd(xg, wg, wl.eps, wl.offset)
    torch.cuda.synchronize()
    y_ref, r_ref = parity.oracle_for(x, w, wl.eps, wl.offset, wl.dtype)
    return parity.compare(y, rstd, y_ref, r_ref, wl.dtype, what), (xg, wg, y)


def test_registered_plan_is_used_and_correct(bnd):
    wl = workloads.WORKLOADS["rmsnorm_16384x512_bf16"]
    rows = 2048
    rule = bnd.plan_query(rows, wl.N, wl.dtype)
    tuned = rule.copy(lanes_per_row=64, vectors_per_lane=1, row_slots=2, block_threads=128, grid=rows // 4)
    bnd.set_tuned(rows, wl.N, wl.dtype, tuned)
    try:
        stats, (xg, wg, y) = run_and_check(bnd, wl, rows, "tuned plan")
        used = bnd.plan_query(rows, wl.N, wl.dtype, xg.data_ptr(), wg.data_ptr(), y.data_ptr())
        assert (used.row_slots, used.block_threads, used.grid) == (2, 128, rows // 4)
        print(stats, flush=True)
    finally:
        bnd.clear_tuned()


def test_tuner_best_plan_is_correct(bnd):
    from memory_bound_row_rmsnorm_amd import tune
    wl = workloads.WORKLOADS["rmsnorm_8192x3000_bf16_offset1"]
    rows = 1024
    print("CASE tune", rows, wl.N, flush=True)
    results = tune.tune_shape(rows, wl.N, wl.dtype, quick=True, log=lambda *a, **k: None)
    assert len(results) > 5
    assert all(r["gbps"] > 0 and r["vgprs"] > 0 and r["scratch_bytes"] == 0 for r in results)
    assert [r["us"] for r in results] == sorted(r["us"] for r in results)
    best = bnd.Plan()
    for f, v in results[0]["plan"].items():
        setattr(best, f, v)
    bnd.set_tuned(rows, wl.N, wl.dtype, best)
    try:
        stats, _ = run_and_check(bnd, wl, rows, f"tuned {results[0]['describe']}")
        print(results[0]["describe"], results[0]["us"], stats, flush=True)
    finally:
        bnd.clear_tuned()
