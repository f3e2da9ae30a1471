"""GPU parity of the backward: HIP kernels against the fp64 oracle backward,
through the C ABI, with the acceptance bar of tests/parity.py."""
from __future__ import annotations

import numpy as np
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
    return binding


def announce(*parts):
    print("CASE", *parts, flush=True)


def case(wl, rows, seed=0):
    """x, w, dy on the CPU and the rstd both sides use: the oracle forward's
    rstd rounded to fp32 (never a GPU output)."""
    x, w = workloads.make_inputs(wl, seed=seed, rows=rows)
    dy = workloads.make_grad(wl, seed=seed, rows=rows)
    _, r64 = parity.oracle_for(x, w, wl.eps, wl.offset, wl.dtype)
    return x, w, dy, r64.astype(np.float32)


def run_bwd(bnd, wl, x, w, dy, r32, plan=None, what=""):
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    rg = torch.from_numpy(r32).to(DEV)
    dx, dw = bnd.rmsnorm_bwd(xg, wg, dyg, rg, wl.offset, plan=plan)
    torch.cuda.synchronize()
    _, dwe, dxe, dxs, dws = parity.oracle_bwd_for(x, w, dy, r32, wl.offset, wl.dtype)
    p = plan or bnd.bwd_plan_query(x.shape[0], wl.N, wl.dtype, xg.data_ptr(), dyg.data_ptr(), dx.data_ptr())
    return parity.compare_bwd(dx, dw, dxe, dxs, dwe, dws, wl.dtype, x.shape[0], p.grid, what)


FULL = {"rmsnorm_64x512_bf16": None, "rmsnorm_16384x512_bf16": None, "rmsnorm_8192x3000_bf16_offset1": None,
        "rmsnorm_32768x8192_bf16_outliers": 4096, "rmsnorm_32768x8192_bf16_outlier_entries": 2048,
        "rmsnorm_262144x128_fp16": 65536,
        "rmsnorm_262144x128_bf16": 65536, "rmsnorm_4096x16384_fp16": 1024}


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_bwd_workload(bnd, name):
    wl = workloads.WORKLOADS[name]
    rows = FULL[name]
    announce("bwd", name, rows or wl.M)
    x, w, dy, r32 = case(wl, rows)
    stats = run_bwd(bnd, wl, x, w, dy, r32, what=name)
    print(name, stats, flush=True)


def bwd_candidates(bnd, M, N, dtype):
    base = bnd.bwd_plan_query(M, N, dtype)
    epv = 4 if dtype == "fp32" else 8
    out = []
    for pf in (0, 1):
        for lanes in (16, 32, 64):
            for vpl in (1, 2):
                for slots in (1, 2, 4):
                    for threads in (256, 512, 1024):
                        if lanes * vpl * epv >= N:
                            out.append(base.copy(variant=bnd.VARIANT_WAVE, lanes_per_row=lanes, vectors_per_lane=vpl,
                                                 row_slots=slots, block_threads=threads, prefetch=pf))
        for threads in (64, 128, 256, 512, 1024):
            for vpt in (1, 2):
                if threads * vpt * epv >= N:
                    out.append(base.copy(variant=bnd.VARIANT_BLOCK, block_threads=threads, vectors_per_lane=vpt,
                                         row_slots=1, prefetch=pf))
    for threads in (64, 256):
        out.append(base.copy(variant=bnd.VARIANT_GENERIC, block_threads=threads, prefetch=0))
    return out


@pytest.mark.parametrize("name", ["rmsnorm_16384x512_bf16", "rmsnorm_8192x3000_bf16_offset1",
                                  "rmsnorm_262144x128_fp16", "rmsnorm_4096x16384_fp16",
                                  "rmsnorm_32768x8192_bf16_outliers"])
def test_bwd_every_kernel(bnd, name):
    wl = workloads.WORKLOADS[name]
    M = 777 if wl.N <= 4096 else 97
    x, w, dy, r32 = case(wl, M, seed=3)
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    rg = torch.from_numpy(r32).to(DEV)
    dx_e = parity.oracle_bwd_for(x, w, dy, r32, wl.offset, wl.dtype)
    dwe = dx_e[1]
    ran = 0
    for plan in bwd_candidates(bnd, M, wl.N, wl.dtype):
        for grid in (1, 5, M):
            p = plan.copy(grid=grid)
            dx = torch.empty_like(xg)
            dw = torch.full((wl.N,), float("nan"), dtype=torch.float32, device=DEV)
            ws = torch.empty(grid * wl.N + 4, dtype=torch.float32, device=DEV)
            announce(name, p.as_dict())
            try:
                bnd.rmsnorm_bwd_out(xg, wg, dyg, rg, dx, dw, ws, wl.offset, plan=p)
            except bnd.RmsnormError as e:
                if e.status == 8:
                    continue
                raise
            torch.cuda.synchronize()
            parity.compare_bwd(dx, dw, dx_e[2], dx_e[3], dwe, dx_e[4], wl.dtype, M, grid, f"{name} {p.as_dict()}")
            ran += 1
    assert ran >= 12, ran


def test_bwd_in_place_and_stream(bnd):
    wl = workloads.WORKLOADS["rmsnorm_8192x3000_bf16_offset1"]
    announce("bwd in place")
    x, w, dy, r32 = case(wl, 300, seed=5)
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    rg = torch.from_numpy(r32).to(DEV)
    dw = torch.empty(wl.N, dtype=torch.float32, device=DEV)
    ws = torch.empty(bnd.bwd_workspace_size(300, wl.N, wl.dtype) // 4 + 4, dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        bnd.rmsnorm_bwd_out(xg, wg, dyg, rg, dyg, dw, ws, wl.offset)      # dx written over dy
    s.synchronize()
    e = parity.oracle_bwd_for(x, w, dy, r32, wl.offset, wl.dtype)
    p = bnd.bwd_plan_query(300, wl.N, wl.dtype)
    parity.compare_bwd(dyg, dw, e[2], e[3], e[1], e[4], wl.dtype, 300, p.grid, "in place")


@pytest.mark.parametrize("name", ["rmsnorm_16384x512_bf16", "rmsnorm_32768x8192_bf16_outliers",
                                  "rmsnorm_262144x128_fp16"])
def test_bwd_deterministic(bnd, name):
    wl = workloads.WORKLOADS[name]
    announce("bwd determinism", name)
    x, w, dy, r32 = case(wl, 2048, seed=7)
    args = [t.to(DEV) for t in (x, w, dy)] + [torch.from_numpy(r32).to(DEV)]
    dx0, dw0 = bnd.rmsnorm_bwd(*args, wl.offset)
    for _ in range(5):
        dx1, dw1 = bnd.rmsnorm_bwd(*args, wl.offset)
        assert torch.equal(dx0.view(torch.int16), dx1.view(torch.int16)) and torch.equal(dw0, dw1)


def test_bwd_end_to_end_from_gpu_forward(bnd):
    """GPU forward then GPU backward, against the oracle's fp64 forward and
    backward: the GPU rstd differs from the exact one by < 2e-7 relative,
    well inside the dx bound."""
    for name in ("rmsnorm_16384x512_bf16", "rmsnorm_4096x16384_fp16"):
        wl = workloads.WORKLOADS[name]
        announce("fwd+bwd", name)
        x, w = workloads.make_inputs(wl, seed=9, rows=512)
        dy = workloads.make_grad(wl, seed=9, rows=512)
        xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
        _, rg = bnd.rmsnorm_fwd(xg, wg, wl.eps, wl.offset)
        dx, dw = bnd.rmsnorm_bwd(xg, wg, dyg, rg, wl.offset)
        torch.cuda.synchronize()
        _, r64 = parity.oracle_for(x, w, wl.eps, wl.offset, wl.dtype)
        e = parity.oracle.rmsnorm_bwd(workloads.to_bits(x), workloads.to_bits(w), workloads.to_bits(dy), r64,
                                      wl.offset, wl.dtype, want_exact=True)
        p = bnd.bwd_plan_query(512, wl.N, wl.dtype)
        parity.compare_bwd(dx, dw, e[2], e[3], e[1], e[4], wl.dtype, 512, p.grid, f"fwd+bwd {name}")


def test_bwd_zero_rows_and_guards(bnd):
    announce("bwd M=0 and guard bands")
    x = torch.empty(0, 512, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(512, dtype=torch.bfloat16, device=DEV)
    r = torch.empty(0, dtype=torch.float32, device=DEV)
    dx, dw = bnd.rmsnorm_bwd(x, w, x, r)
    torch.cuda.synchronize()
    assert dx.shape == (0, 512) and torch.all(dw == 0)
    wl = workloads.WORKLOADS["rmsnorm_8192x3000_bf16_offset1"]
    x, w, dy, r32 = case(wl, 41, seed=11)
    M, N = 41, wl.N
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    rg = torch.from_numpy(r32).to(DEV)
    dxb = torch.full((M * N + 4096,), 0x5A5A, dtype=torch.int16, device=DEV)
    dwb = torch.full((N + 4096,), -3.0, dtype=torch.float32, device=DEV)
    dxv = dxb[:M * N].view(torch.bfloat16).view(M, N)
    dwv = dwb[:N]
    ws = torch.empty(bnd.bwd_workspace_size(M, N, wl.dtype) // 4 + 4, dtype=torch.float32, device=DEV)
    bnd.rmsnorm_bwd_out(xg, wg, dyg, rg, dxv, dwv, ws, wl.offset)
    torch.cuda.synchronize()
    assert torch.all(dxb[M * N:] == 0x5A5A) and torch.all(dwb[N:] == -3.0)
    e = parity.oracle_bwd_for(x, w, dy, r32, wl.offset, wl.dtype)
    p = bnd.bwd_plan_query(M, N, wl.dtype)
    parity.compare_bwd(dxv, dwv, e[2], e[3], e[1], e[4], wl.dtype, M, p.grid, "guards")


# ---------------------------------------------------------------------------
# fp32 input: four elements per 16-byte vector.  The oracle is the codec-free
# fp64 backward on the exactly widened inputs; the bar is one fp32 ulp of dx
# plus the same arithmetic term as for the 16-bit types.
# ---------------------------------------------------------------------------
def fp32_case(M, N, offset, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, N, generator=g) * 2.0
    w = 1.0 + 0.1 * torch.randn(N, generator=g)
    dy = torch.randn(M, N, generator=g)
    _, r64 = parity.oracle_fp32(x, w, 1e-6, offset)
    return x, w, dy, r64.astype(np.float32)


@pytest.mark.parametrize("M,N,offset", [(777, 128, 0.0), (777, 500, 1.0), (3000, 512, 0.0), (97, 4096, 1.0),
                                        (57, 8192, 0.0), (33, 1002, 1.0), (20, 8196, 0.0)])
def test_bwd_fp32_rule(bnd, M, N, offset):
    x, w, dy, r32 = fp32_case(M, N, offset, seed=N)
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    rg = torch.from_numpy(r32).to(DEV)
    p = bnd.bwd_plan_query(M, N, "fp32", xg.data_ptr(), dyg.data_ptr(), dyg.data_ptr())
    announce("bwd fp32", M, N, offset, p.as_dict())
    dx, dw = bnd.rmsnorm_bwd(xg, wg, dyg, rg, offset)
    torch.cuda.synchronize()
    _, dwe, dxe, dxs, dws = parity.oracle_bwd_for(x, w, dy, r32, offset, "fp32")
    stats = parity.compare_bwd(dx, dw, dxe, dxs, dwe, dws, "fp32", M, p.grid, f"bwd fp32 {M}x{N}")
    print("bwd fp32", M, N, stats, flush=True)


@pytest.mark.parametrize("M,N", [(777, 256), (300, 512), (97, 4096), (45, 8192)])
def test_bwd_fp32_every_kernel(bnd, M, N):
    x, w, dy, r32 = fp32_case(M, N, 1.0, seed=N + 1)
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    rg = torch.from_numpy(r32).to(DEV)
    _, dwe, dxe, dxs, dws = parity.oracle_bwd_for(x, w, dy, r32, 1.0, "fp32")
    ran = 0
    for plan in bwd_candidates(bnd, M, N, "fp32"):
        for grid in (1, 5, M):
            p = plan.copy(grid=grid)
            dx = torch.empty_like(xg)
            dw = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
            ws = torch.empty(grid * N + 4, dtype=torch.float32, device=DEV)
            announce("bwd fp32", M, N, p.as_dict())
            try:
                bnd.rmsnorm_bwd_out(xg, wg, dyg, rg, dx, dw, ws, 1.0, plan=p)
            except bnd.RmsnormError as e:
                if e.status == 8:
                    continue
                raise
            torch.cuda.synchronize()
            parity.compare_bwd(dx, dw, dxe, dxs, dwe, dws, "fp32", M, grid, f"bwd fp32 {M}x{N} {p.as_dict()}")
            ran += 1
    assert ran >= 12, ran
