"""rmsnorm_bwd_noalloc (the backward for callers that cannot allocate: its dw partial rows live in
the library's per-GPU scratch array) against rmsnorm_bwd with a caller workspace, through the C ABI.

Two calls in a row, the second on a smaller input, so the scratch holds the first call's partial
rows when the second starts; where both entry points take the same plan the outputs must be
bit-identical, and where the scratch forces a smaller grid dw must meet the oracle's bar."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from memory_bound_row_rmsnorm_amd import workloads
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SCRATCH = 16 * 1024 * 1024


@pytest.fixture(scope="module")
def bnd():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from memory_bound_row_rmsnorm_amd import binding
    return binding


def inputs(wl, rows):
    x, w = workloads.make_inputs(wl, seed=3, rows=rows)
    dy = workloads.make_grad(wl, seed=3, rows=rows)
    _, r64 = parity.oracle_for(x, w, wl.eps, wl.offset, wl.dtype)       # rstd from the oracle forward
    return x, w, dy, r64.astype(np.float32)


def both(bnd, wl, x, w, dy, r32):
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    rg = torch.from_numpy(r32).to(DEV)
    dx_ws, dw_ws = bnd.rmsnorm_bwd(xg, wg, dyg, rg, wl.offset)
    dx_na = torch.full_like(xg, float("nan"))
    dw_na = torch.full((wl.N,), float("nan"), dtype=torch.float32, device=DEV)
    bnd.rmsnorm_bwd_noalloc_out(xg, wg, dyg, rg, dx_na, dw_na, wl.offset)
    torch.cuda.synchronize()
    plan = bnd.bwd_plan_query(x.shape[0], wl.N, wl.dtype, xg.data_ptr(), dyg.data_ptr(), dx_ws.data_ptr())
    return dx_ws.cpu(), dw_ws.cpu(), dx_na.cpu(), dw_na.cpu(), plan


def test_noalloc_matches_the_workspace_entry_point_on_two_calls(bnd):
    # first call: 8192 x 8192 bf16 -- its rule grid (512 partial rows of 32 KiB) fills the scratch
    big = workloads.WORKLOADS["rmsnorm_32768x8192_bf16_outliers"]
    small = workloads.WORKLOADS["rmsnorm_8192x3000_bf16_offset1"]
    for wl, rows in ((big, 8192), (small, 1000)):
        print("CASE noalloc", wl.name, rows, flush=True)
        x, w, dy, r32 = inputs(wl, rows)
        dx_ws, dw_ws, dx_na, dw_na, plan = both(bnd, wl, x, w, dy, r32)
        assert plan.grid * wl.N * 4 <= SCRATCH
        assert torch.equal(dx_na.view(torch.int16), dx_ws.view(torch.int16)), wl.name
        assert torch.equal(dw_na, dw_ws), wl.name
        _, dwe, dxe, dxs, dws = parity.oracle_bwd_for(x, w, dy, r32, wl.offset, wl.dtype)
        print(parity.compare_bwd(dx_na, dw_na, dxe, dxs, dwe, dws, wl.dtype, rows, plan.grid, wl.name), flush=True)


def test_noalloc_shrinks_the_grid_to_fit_its_scratch(bnd):
    """N = 65536 bf16 (the generic row pass): the rule's 512 partial rows of 256 KiB do not fit
    16 MiB, so 64 workgroups loop over the rows; dx stays bit-identical, dw meets the bar."""
    wl = workloads.WORKLOADS["rmsnorm_64x512_bf16"].__class__(
        "rows_65536_bf16", 512, 65536, "bf16", 1.0, 1.0, 1e-6, 0.0)
    print("CASE noalloc capped grid", wl.M, wl.N, flush=True)
    x, w, dy, r32 = inputs(wl, wl.M)
    dx_ws, dw_ws, dx_na, dw_na, plan = both(bnd, wl, x, w, dy, r32)
    assert plan.grid * wl.N * 4 > SCRATCH
    assert torch.equal(dx_na.view(torch.int16), dx_ws.view(torch.int16))
    _, dwe, dxe, dxs, dws = parity.oracle_bwd_for(x, w, dy, r32, wl.offset, wl.dtype)
    print(parity.compare_bwd(dx_na, dw_na, dxe, dxs, dwe, dws, wl.dtype, wl.M, SCRATCH // (wl.N * 4), "capped"),
          flush=True)


def test_noalloc_rejects_rows_wider_than_its_scratch(bnd):
    x = torch.zeros(2, SCRATCH // 4 + 8, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(x.shape[1], dtype=torch.bfloat16, device=DEV)
    r = torch.ones(2, dtype=torch.float32, device=DEV)
    with pytest.raises(bnd.RmsnormError) as e:
        bnd.rmsnorm_bwd_noalloc(x, w, x.clone(), r)
    assert e.value.status == 2
