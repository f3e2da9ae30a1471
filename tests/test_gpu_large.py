"""GPU parity for tensors beyond 4 GiB: rows whose byte offsets pass 2^31 and 2^32.

The workloads stay below 1 GiB per tensor, so a 32-bit byte offset anywhere in
a kernel's row addressing would pass every other test.  Here x (and y, dy, dx)
hold 2^31 + a few rows' worth of 16-bit elements (4 GiB and more; MI355X holds
288 GB).  Inputs are drawn on the device from seeded generators.  Checks:

  * forward, sampled rows (the first and last rows, the rows around the 2 GiB
    and 4 GiB byte offsets, random rows): y and rstd against the fp64 oracle,
    to the usual bar (1 ulp, rstd 1e-5);
  * forward, every row: the closed forms of the definition ("Rmsnorm Kernel
    Optimization", Overview): rstd^2 (mean x^2 + eps) = 1, and
    mean_j (y_j / (offset + w_j))^2 = mean x^2 / (mean x^2 + eps), within the
    rounding of y (2 u = 2^-7 for bf16) -- a row never written (y and rstd are
    NaN-filled first) or normalised with another row's rstd fails;
  * backward: dy is zero except on the sampled rows, so dx must be exactly zero
    on every other row (NaN-filled first), the sampled rows' dx must match the
    oracle, and dw (the other rows add exact zeros) must match the oracle over
    the sampled rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from memory_bound_row_rmsnorm_amd import workloads
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16}
U_2 = 2.0 ** -7          # twice the bf16 unit roundoff: the bound on (1 + d)^2 - 1 for y's rounding


@pytest.fixture(scope="module")
def bnd():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from memory_bound_row_rmsnorm_amd import binding
    return binding


def announce(*parts):
    print("CASE", *parts, flush=True)


def sample_rows(M: int, N: int, seed: int) -> np.ndarray:
    """The first and last rows, the rows around the first ones at 2 GiB and 4 GiB byte offsets,
    and random rows."""
    rows = set(range(4)) | set(range(M - 4, M))
    for boundary in (1 << 31, 1 << 32):
        c = boundary // (2 * N)
        rows |= set(range(c - 3, c + 3))
    rows |= set(np.random.default_rng(seed).integers(0, M, 24).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < M), dtype=np.int64)


def row_chunks(M: int, N: int, elems: int = 1 << 26):
    step = max(1, elems // N)
    for m0 in range(0, M, step):
        yield m0, min(M, m0 + step)


@pytest.mark.parametrize("M,N,dtype", [((1 << 21) + 37, 1024, "bf16"),     # wave family
                                       ((1 << 18) + 5, 8192, "bf16")])      # block family
def test_forward_beyond_4gib(bnd, M, N, dtype):
    eps, offset = 1e-6, 0.0
    plan = bnd.plan_query(M, N, dtype)
    announce("forward beyond 4 GiB", M, N, dtype, plan.as_dict())
    assert M * N * 2 > (1 << 32)
    x = workloads.fill_normal_(torch.empty(M, N, dtype=TORCH[dtype], device=DEV), seed=11)
    w = workloads.fill_normal_(torch.empty(N, dtype=TORCH[dtype], device=DEV), seed=12, sigma=0.1, mean=1.0)
    y = torch.full_like(x, float("nan"))
    r = torch.full((M,), float("nan"), dtype=torch.float32, device=DEV)
    bnd.rmsnorm_fwd_out(x, w, y, r, eps, offset)
    torch.cuda.synchronize()

    rows = sample_rows(M, N, seed=13)
    idx = torch.from_numpy(rows).to(DEV)
    xs = x.index_select(0, idx).cpu()
    y_ref, r_ref = parity.oracle_for(xs, w.cpu(), eps, offset, dtype)
    stats = parity.compare(y.index_select(0, idx), r.index_select(0, idx), y_ref, r_ref, dtype,
                           f"{M}x{N} sampled rows")

    g = w.float() + offset
    worst_r = worst_y = 0.0
    for m0, m1 in row_chunks(M, N):
        ms = x[m0:m1].float().pow(2).mean(1)
        rr = r[m0:m1]
        assert torch.isfinite(rr).all(), f"rows {m0}:{m1}: rstd not written"
        dev_r = (rr.double() ** 2 * (ms.double() + eps) - 1).abs().max().item()
        yy = (y[m0:m1].float() / g).pow(2).mean(1).double()
        assert torch.isfinite(yy).all(), f"rows {m0}:{m1}: y not written"
        dev_y = (yy - ms.double() / (ms.double() + eps)).abs().max().item()
        worst_r, worst_y = max(worst_r, dev_r), max(worst_y, dev_y)
        assert dev_r <= 1e-4, f"rows {m0}:{m1}: rstd^2 (ms + eps) off 1 by {dev_r}"
        assert dev_y <= U_2 + 1e-4, f"rows {m0}:{m1}: mean (y / g)^2 off by {dev_y}"
    print(M, N, dtype, stats, {"rstd_closed_form": worst_r, "mean_y2": worst_y}, flush=True)


def test_backward_beyond_4gib(bnd):
    M, N, dtype, offset = (1 << 21) + 37, 1024, "bf16", 0.0
    plan = bnd.bwd_plan_query(M, N, dtype)
    announce("backward beyond 4 GiB", M, N, dtype, plan.as_dict())
    td = TORCH[dtype]
    x = workloads.fill_normal_(torch.empty(M, N, dtype=td, device=DEV), seed=21)
    w = workloads.fill_normal_(torch.empty(N, dtype=td, device=DEV), seed=22, sigma=0.1, mean=1.0)
    rows = sample_rows(M, N, seed=23)
    idx = torch.from_numpy(rows).to(DEV)
    dy = torch.zeros_like(x)
    dy_rows = workloads.fill_normal_(torch.empty(len(rows), N, dtype=td, device=DEV), seed=24)
    dy.index_copy_(0, idx, dy_rows)
    gr = torch.Generator(device=DEV).manual_seed(25)
    rstd = torch.rand(M, generator=gr, device=DEV, dtype=torch.float32).mul_(1.5).add_(0.5)
    dx = torch.full_like(x, float("nan"))
    dw = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(bnd.bwd_workspace_size(M, N, dtype, x.data_ptr(), dy.data_ptr(), dx.data_ptr()),
                     dtype=torch.uint8, device=DEV)
    bnd.rmsnorm_bwd_out(x, w, dy, rstd, dx, dw, ws, offset)
    torch.cuda.synchronize()

    sampled = torch.zeros(M, dtype=torch.bool, device=DEV)
    sampled[idx] = True
    for m0, m1 in row_chunks(M, N):
        nonzero = (dx[m0:m1] != 0).any(1) & ~sampled[m0:m1]
        assert not nonzero.any(), (f"rows {m0}:{m1}: dx not exactly zero where dy is zero "
                                   f"(first row {m0 + int(nonzero.nonzero()[0])})")
    xb = workloads.to_bits(x.index_select(0, idx).cpu())
    dyb = workloads.to_bits(dy_rows.cpu())
    wb = workloads.to_bits(w.cpu())
    r_s = rstd.index_select(0, idx).cpu().numpy()
    _, dwe, dxe, dxs, dws = parity.oracle.rmsnorm_bwd(xb, wb, dyb, r_s, offset, dtype, want_exact=True)
    dx_worst = parity.compare_dx(dx.index_select(0, idx), dxe, dxs, dtype, "sampled rows")
    dw_worst = parity.compare_dw(dw, dwe, dws, M, plan.grid, "dw")
    print(M, N, dtype, {"dx_max_err_over_bound": dx_worst, "dw_max_err_over_bound": dw_worst}, flush=True)
