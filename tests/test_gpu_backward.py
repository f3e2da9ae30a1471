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


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_bwd_workload_full_size(bnd, name):
    """Every workload at full size with the plan the benchmark times: every dx element and every dw
    column against the oracle, which runs over the rows in chunks (dw summed over the chunks in
    fp64)."""
    wl = workloads.WORKLOADS[name]
    M, N = wl.M, wl.N
    announce("bwd full-size", name, M, N, wl.dtype)
    x, w = workloads.make_inputs(wl, seed=0)
    dy = workloads.make_grad(wl, seed=0)
    _, r64 = parity.oracle_for(x, w, wl.eps, wl.offset, wl.dtype)
    r32 = r64.astype(np.float32)
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    rg = torch.from_numpy(r32).to(DEV)
    p = bnd.bwd_plan_query(M, N, wl.dtype, xg.data_ptr(), dyg.data_ptr(), xg.data_ptr())
    dx, dw = bnd.rmsnorm_bwd(xg, wg, dyg, rg, wl.offset)
    torch.cuda.synchronize()
    del xg, dyg
    dx = dx.cpu()
    xb, wb, dyb = workloads.to_bits(x), workloads.to_bits(w), workloads.to_bits(dy)
    rows = max(1, (1 << 24) // N)
    dwe = np.zeros(N)
    dws = np.zeros(N)
    dx_worst = 0.0
    for m0 in range(0, M, rows):
        m1 = min(M, m0 + rows)
        _, dw_c, ex, sc, ws_c = parity.oracle.rmsnorm_bwd(xb[m0:m1], wb, dyb[m0:m1], r32[m0:m1], wl.offset,
                                                          wl.dtype, want_exact=True)
        dx_worst = max(dx_worst, parity.compare_dx(dx[m0:m1], ex, sc, wl.dtype, f"{name} rows {m0}:{m1}"))
        dwe += dw_c
        dws += ws_c
    dw_worst = parity.compare_dw(dw, dwe, dws, M, p.grid, name)
    print(name, p.as_dict(), {"dx_max_err_over_bound": dx_worst, "dw_max_err_over_bound": dw_worst}, flush=True)


def bwd_candidates(bnd, M, N, dtype):
    base = bnd.bwd_plan_query(M, N, dtype)
    epv = 4 if dtype == "fp32" else 8
    out = []
    for pf in (0, 1):
        for lanes in (4, 8, 16, 32, 64):
            for vpl in (1, 2):
                for slots in (1, 2, 4):
                    for threads in (256, 512, 1024):
                        if lanes * vpl * epv >= N:
                            out.append(base.copy(variant=bnd.VARIANT_WAVE, lanes_per_row=lanes, vectors_per_lane=vpl,
                                                 row_slots=slots, block_threads=threads, prefetch=pf))
        for threads in (64, 128, 256, 512, 1024):
            for vpt in (1, 2):
                for rows in (1, 2, 4):             # rows per workgroup, threads / rows each
                    if threads // rows >= 64 and threads // rows * vpt * epv >= N:
                        out.append(base.copy(variant=bnd.VARIANT_BLOCK, block_threads=threads, vectors_per_lane=vpt,
                                             row_slots=rows, prefetch=pf))
    for threads in (256, 512, 1024):
        for vpt in (3, 4, 6):
            if threads * vpt * epv >= N:
                out.append(base.copy(variant=bnd.VARIANT_WIDE, block_threads=threads, vectors_per_lane=vpt,
                                     row_slots=1, prefetch=0))
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


@pytest.mark.parametrize("M,N,dtype", [(999, 16, "bf16"), (777, 40, "bf16"), (500, 64, "fp16"), (1000, 24, "bf16"),
                                       (333, 32, "fp32"), (300, 16, "fp32"), (129, 8, "fp16")])
def test_bwd_short_rows_every_kernel(bnd, M, N, dtype):
    """Rows of at most 8 vectors: the rule's plan (8-lane segments) and every compiled wave instance
    that covers the row, 4- and 8-lane segments included, at grids of 1, 5 and M."""
    x, w, dy, r32 = any_case(M, N, dtype, 1.0, seed=N + 11)
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    rg = torch.from_numpy(r32).to(DEV)
    _, dwe, dxe, dxs, dws = parity.oracle_bwd_for(x, w, dy, r32, 1.0, dtype)
    base = bnd.bwd_plan_query(M, N, dtype, xg.data_ptr(), dyg.data_ptr(), dyg.data_ptr())
    assert (base.variant, base.lanes_per_row) == (bnd.VARIANT_WAVE, 8), base.as_dict()
    dx, dw = bnd.rmsnorm_bwd(xg, wg, dyg, rg, 1.0)
    torch.cuda.synchronize()
    parity.compare_bwd(dx, dw, dxe, dxs, dwe, dws, dtype, M, base.grid, f"bwd short rule {M}x{N} {dtype}")
    ran, lanes_seen = 0, set()
    for plan in bwd_candidates(bnd, M, N, dtype):
        if plan.variant != bnd.VARIANT_WAVE:
            continue
        for grid in (1, 5, M):
            p = plan.copy(grid=grid)
            dx = torch.empty_like(xg)
            dw = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
            ws = torch.empty(grid * N + 4, dtype=torch.float32, device=DEV)
            announce("bwd short", M, N, dtype, p.as_dict())
            try:
                bnd.rmsnorm_bwd_out(xg, wg, dyg, rg, dx, dw, ws, 1.0, plan=p)
            except bnd.RmsnormError as e:
                if e.status == 8:
                    continue
                raise
            torch.cuda.synchronize()
            parity.compare_bwd(dx, dw, dxe, dxs, dwe, dws, dtype, M, grid, f"bwd short {M}x{N} {dtype} {p.as_dict()}")
            lanes_seen.add(p.lanes_per_row)
            ran += 1
    epv = EPV[dtype]
    assert 8 in lanes_seen and (4 in lanes_seen or N > 4 * epv), lanes_seen
    assert ran >= 24, ran


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
                                  "rmsnorm_262144x128_fp16", "rmsnorm_8192x3000_bf16_offset1"])
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


# ---------------------------------------------------------------------------
# Layouts: rows of x, dy and dx placed by strides (rmsnorm_bwd_ex).  Every case
# is compared with the oracle on the logical rows, and dx is written into a
# view of a sentinel-filled buffer whose other elements must not change.
# ---------------------------------------------------------------------------
SENT = {torch.bfloat16: (torch.int16, 0x7FC1), torch.float16: (torch.int16, 0x7E01),
        torch.float32: (torch.int32, 0x7FC00001)}


def _draw(shape, dtype, seed, sigma=1.0):
    g = torch.Generator().manual_seed(seed)
    return (sigma * torch.randn(*shape, generator=g)).to(dtype)


def _filled(numel, dtype):
    iv, val = SENT[dtype]
    t = torch.empty(numel, dtype=dtype, device=DEV)
    t.view(iv).fill_(val)
    return t


def _check_layout_bwd(bnd, x, w, dy, dx, dx_base, offset, what):
    dt = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[x.dtype]
    N = x.shape[-1]
    xc = x.cpu().reshape(-1, N)
    wc = w.cpu()
    dyc = dy.cpu().reshape(-1, N)
    M = xc.shape[0]
    if dt == "fp32":
        _, r64 = parity.oracle_fp32(xc, wc, 1e-6, offset)
    else:
        _, r64 = parity.oracle_for(xc, wc, 1e-6, offset, dt)
    r32 = r64.astype(np.float32)
    rg = torch.from_numpy(r32).to(DEV).reshape(x.shape[:-1])
    iv, val = SENT[x.dtype]
    before = dx_base.cpu().view(iv).clone()
    p = bnd.bwd_plan_query_ex(x, w, dy, out=dx)
    announce("bwd layout", what, p.as_dict())
    out, dw = bnd.rmsnorm_bwd_ex(x, w, dy, rg, offset, out=dx)
    torch.cuda.synchronize()
    _, dwe, dxe, dxs, dws = parity.oracle_bwd_for(xc, wc, dyc, r32, offset, dt)
    parity.compare_bwd(out.cpu().reshape(M, N), dw, dxe, dxs, dwe, dws, dt, M, p.grid, what)
    # nothing outside dx's view changed
    idx = torch.arange(dx_base.numel()).as_strided(dx.shape, dx.stride(), dx.storage_offset())
    mask = torch.zeros(dx_base.numel(), dtype=torch.bool)
    mask[idx.reshape(-1)] = True
    after = dx_base.cpu().view(iv)
    assert bool((after[~mask] == before[~mask]).all()), what
    return p


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_bwd_strided_rows(bnd, dtype):
    M, N = 300, 512
    xb = _draw((M, 768), dtype, 201).to(DEV)
    x = xb[:, 128:640]                                   # row stride 768
    w = (1.0 + 0.1 * _draw((N,), torch.float32, 202)).to(dtype).to(DEV)
    dyb = _draw((M, 1024), dtype, 203).to(DEV)
    dy = dyb[:, :N]                                      # row stride 1024
    dx_base = _filled(M * 640 + 64, dtype)
    dx = dx_base.as_strided((M, N), (640, 1), 32)        # row stride 640, 32 elements in
    p = _check_layout_bwd(bnd, x, w, dy, dx, dx_base, 1.0, f"strided 2-D {dtype}")
    assert p.variant == bnd.VARIANT_WAVE


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_bwd_qk_norm_heads(bnd, dtype):
    """Rows of head_dim inside a fused QKV projection output [B, S, 3, H, D]: q = [:, :, 0] has rows
    D apart within a token and 3*H*D apart between tokens (a 4-D view whose leading dimensions
    collapse into one batch stride)."""
    B, S, H, D = 2, 33, 8, 128
    qkv = _draw((B, S, 3, H, D), dtype, 211, 2.0).to(DEV)
    x = qkv[:, :, 0]
    dqkv = _draw((B, S, 3, H, D), dtype, 212).to(DEV)
    dy = dqkv[:, :, 0]
    w = (1.0 + 0.1 * _draw((D,), torch.float32, 213)).to(dtype).to(DEV)
    dx_base = _filled(B * S * 3 * H * D, dtype)
    dx = dx_base.view(B, S, 3, H, D)[:, :, 1]             # written into the k slot of another buffer
    _check_layout_bwd(bnd, x, w, dy, dx, dx_base, 0.0, f"qk-norm {dtype}")


@pytest.mark.parametrize("N", [512, 3000, 1002])
def test_bwd_batched_slices_and_interleaved(bnd, N):
    dtype = torch.bfloat16
    B, S = 4, 70
    big = _draw((B, S + 9, N), dtype, 221 + N).to(DEV)
    x = big[:, 3:3 + S]                                  # a sequence slice: batch stride (S + 9) N
    dy = _draw((S, B, N), dtype, 222 + N).to(DEV).transpose(0, 1)     # interleaved [S, B, N] view
    w = (0.1 * _draw((N,), torch.float32, 223 + N)).to(dtype).to(DEV)
    dx_base = _filled(B * (S + 2) * N + 8, dtype)
    dx = dx_base.as_strided((B, S, N), ((S + 2) * N, N, 1), 8)
    p = _check_layout_bwd(bnd, x, w, dy, dx, dx_base, 1.0, f"batched N={N}")
    if N % 8 == 0:
        assert p.variant != bnd.VARIANT_GENERIC


def test_bwd_layout_in_place(bnd):
    dtype = torch.float16
    B, S, N = 3, 50, 256
    x = _draw((B, S, N), dtype, 231, 30.0).to(DEV)
    buf = _draw((B, S + 5, N), dtype, 232).to(DEV)
    dy = buf[:, 2:2 + S]
    dy_copy = dy.clone()
    w = (1.0 + 0.1 * _draw((N,), torch.float32, 233)).to(dtype).to(DEV)
    xc = x.cpu().reshape(-1, N)
    _, r64 = parity.oracle_for(xc, w.cpu(), 1e-6, 0.0, "fp16")
    r32 = r64.astype(np.float32)
    rg = torch.from_numpy(r32).to(DEV).reshape(B, S)
    announce("bwd layout in place")
    out, dw = bnd.rmsnorm_bwd_ex(x, w, dy, rg, 0.0, out=dy)     # dx over dy, same layout
    torch.cuda.synchronize()
    _, dwe, dxe, dxs, dws = parity.oracle_bwd_for(xc, w.cpu(), dy_copy.cpu().reshape(-1, N), r32, 0.0, "fp16")
    p = bnd.bwd_plan_query_ex(x, w, dy, out=dy)
    parity.compare_bwd(out.cpu().reshape(-1, N), dw, dxe, dxs, dwe, dws, "fp16", B * S, p.grid, "in place layout")


# ---------------------------------------------------------------------------
# Rows off a 16-byte boundary: the shifted row pass (aligned chunks, weights
# shifted per row, dw kept per column across rows of different shifts).
# ---------------------------------------------------------------------------
TDT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
EPV = {"bf16": 8, "fp16": 8, "fp32": 4}


def any_case(M, N, dtype, offset, seed, sigma=2.0):
    """x, w, dy of `dtype` on the CPU and the rstd both sides use (the oracle
    forward's, rounded to fp32)."""
    g = torch.Generator().manual_seed(seed)
    x = (sigma * torch.randn(M, N, generator=g)).to(TDT[dtype])
    w = (1.0 + 0.1 * torch.randn(N, generator=g)).to(TDT[dtype])
    dy = torch.randn(M, N, generator=g).to(TDT[dtype])
    if dtype == "fp32":
        _, r64 = parity.oracle_fp32(x, w, 1e-6, offset)
    else:
        _, r64 = parity.oracle_for(x, w, 1e-6, offset, dtype)
    return x, w, dy, r64.astype(np.float32)


@pytest.mark.parametrize("M,N,dtype,offset", [
    (300, 3001, "bf16", 1.0), (777, 1001, "fp16", 0.0), (97, 8191, "bf16", 0.0),
    (33, 16377, "bf16", 1.0), (500, 17, "bf16", 0.0), (1000, 100, "fp16", 1.0),
    (2000, 257, "bf16", 1.0), (300, 1002, "fp32", 0.0), (50, 8189, "fp32", 1.0), (41, 4097, "fp32", 0.0),
    (3000, 249, "bf16", 0.0), (777, 61, "fp32", 1.0), (600, 505, "fp16", 0.0), (5000, 36, "bf16", 1.0),
    (4099, 300, "bf16", 1.0), (4099, 513, "bf16", 1.0), (1001, 1017, "fp16", 0.0), (777, 301, "fp32", 1.0),
    (333, 509, "fp32", 0.0), (2000, 506, "bf16", 0.0), (5600, 8193, "fp16", 1.0)])
def test_bwd_shifted_rule(bnd, M, N, dtype, offset):
    x, w, dy, r32 = any_case(M, N, dtype, offset, seed=N + M)
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    rg = torch.from_numpy(r32).to(DEV)
    p = bnd.bwd_plan_query(M, N, dtype, xg.data_ptr(), dyg.data_ptr(), dyg.data_ptr())
    announce("bwd shifted", M, N, dtype, offset, p.as_dict())
    epv = EPV[dtype]
    chunks = -(-(N + epv - 1) // epv)
    assert p.variant == (bnd.VARIANT_SHIFTED_WAVE if chunks <= 128 else bnd.VARIANT_SHIFTED)
    dx, dw = bnd.rmsnorm_bwd(xg, wg, dyg, rg, offset)
    dx2, dw2 = bnd.rmsnorm_bwd(xg, wg, dyg, rg, offset)
    torch.cuda.synchronize()
    _, dwe, dxe, dxs, dws = parity.oracle_bwd_for(x, w, dy, r32, offset, dtype)
    stats = parity.compare_bwd(dx, dw, dxe, dxs, dwe, dws, dtype, M, p.grid, f"bwd shifted {M}x{N} {dtype}")
    assert torch.equal(dx, dx2) and torch.equal(dw, dw2)          # the same bits on every run
    print("bwd shifted", M, N, dtype, stats, flush=True)


def shifted_wave_candidates(bnd, base, N, epv):
    out = []
    for pf in (0, 1):
        for lanes, vpl in ((8, 1), (16, 1), (32, 1), (64, 1), (64, 2)):
            for slots in (1, 2, 4):
                for threads in (256, 1024):
                    if lanes * vpl * epv >= N + epv - 1:
                        out.append(base.copy(variant=bnd.VARIANT_SHIFTED_WAVE, lanes_per_row=lanes,
                                             vectors_per_lane=vpl, row_slots=slots, block_threads=threads,
                                             prefetch=pf))
    return out


@pytest.mark.parametrize("M,N,dtype", [(97, 3001, "bf16"), (200, 1001, "fp16"), (60, 1003, "fp32"),
                                       (150, 33, "bf16"), (777, 100, "bf16"), (500, 250, "fp16"),
                                       (300, 61, "fp32"), (333, 505, "bf16"), (129, 513, "bf16"),
                                       (70, 301, "fp32"), (300, 36, "bf16"), (200, 20, "fp16"),
                                       (150, 29, "fp32")])
def test_bwd_shifted_every_kernel(bnd, M, N, dtype):
    x, w, dy, r32 = any_case(M, N, dtype, 1.0, seed=N + 7)
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    rg = torch.from_numpy(r32).to(DEV)
    _, dwe, dxe, dxs, dws = parity.oracle_bwd_for(x, w, dy, r32, 1.0, dtype)
    base = bnd.bwd_plan_query(M, N, dtype)
    epv = EPV[dtype]
    ran = 0
    for pf in (0, 1):
        for threads in (64, 128, 256, 512, 1024):
            for vpt in (1, 2, 3):
                if threads * vpt * epv < N + epv - 1 or threads * vpt * epv * 4 > 65536 or (vpt == 3 and pf):
                    continue    # does not cover the row, dw exceeds 64 KiB of LDS, or no such instance
                for grid in (1, 5, M):
                    p = base.copy(variant=bnd.VARIANT_SHIFTED, block_threads=threads, vectors_per_lane=vpt,
                                  prefetch=pf, grid=grid)
                    dx = torch.empty_like(xg)
                    dw = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
                    ws = torch.empty(grid * N + 4, dtype=torch.float32, device=DEV)
                    announce("bwd shifted", M, N, dtype, p.as_dict())
                    bnd.rmsnorm_bwd_out(xg, wg, dyg, rg, dx, dw, ws, 1.0, plan=p)
                    torch.cuda.synchronize()
                    parity.compare_bwd(dx, dw, dxe, dxs, dwe, dws, dtype, M, grid,
                                       f"bwd shifted {M}x{N} {dtype} {p.as_dict()}")
                    ran += 1
    for plan in shifted_wave_candidates(bnd, base, N, epv):
        for grid in (1, 3, M):
            p = plan.copy(grid=grid)
            dx = torch.empty_like(xg)
            dw = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
            ws = torch.empty(grid * N + 4, dtype=torch.float32, device=DEV)
            announce("bwd shifted wave", M, N, dtype, p.as_dict())
            try:
                bnd.rmsnorm_bwd_out(xg, wg, dyg, rg, dx, dw, ws, 1.0, plan=p)
            except bnd.RmsnormError as e:
                if e.status == 8:
                    continue
                raise
            torch.cuda.synchronize()
            parity.compare_bwd(dx, dw, dxe, dxs, dwe, dws, dtype, M, grid,
                               f"bwd shifted wave {M}x{N} {dtype} {p.as_dict()}")
            ran += 1
    assert ran >= 12, ran


def test_bwd_shifted_in_place(bnd):
    M, N = 300, 3001
    x, w, dy, r32 = any_case(M, N, "bf16", 1.0, seed=41)
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    rg = torch.from_numpy(r32).to(DEV)
    dw = torch.empty(N, dtype=torch.float32, device=DEV)
    ws = torch.empty(bnd.bwd_workspace_size(M, N, "bf16") // 4 + 4, dtype=torch.float32, device=DEV)
    announce("bwd shifted in place")
    bnd.rmsnorm_bwd_out(xg, wg, dyg, rg, dyg, dw, ws, 1.0)          # dx written over dy
    torch.cuda.synchronize()
    e = parity.oracle_bwd_for(x, w, dy, r32, 1.0, "bf16")
    p = bnd.bwd_plan_query(M, N, "bf16")
    assert p.variant == bnd.VARIANT_SHIFTED
    parity.compare_bwd(dyg, dw, e[2], e[3], e[1], e[4], "bf16", M, p.grid, "shifted in place")


@pytest.mark.parametrize("dtype,N", [("bf16", 1001), ("fp32", 1001), ("bf16", 100), ("fp32", 61)])
def test_bwd_shifted_edges_ignore_their_neighbours(bnd, dtype, N):
    """Rows 3 elements past a boundary with NaN between them (x and dy), w followed by NaN inside its
    last 16 bytes, dx into a sentinel buffer: the edge chunks' outside elements and w's tail must
    not reach c, dx or dw, and nothing outside dx's rows may change."""
    M, S = 120, N + 3 + 8
    tdt = TDT[dtype]
    x0, w0, dy0, _ = any_case(M, N, dtype, 1.0, seed=43)
    xb = torch.full((M, S), float("nan"), dtype=tdt)
    xb[:, 3:3 + N] = x0
    dyb = torch.full((M, S), float("nan"), dtype=tdt)
    dyb[:, 3:3 + N] = dy0
    wb = torch.full((N + 16,), float("nan"), dtype=tdt)
    wb[:N] = w0
    x, dy, w = xb.to(DEV)[:, 3:3 + N], dyb.to(DEV)[:, 3:3 + N], wb.to(DEV)[:N]
    dx_base = _filled(M * S + 16, tdt)
    dx = dx_base.as_strided((M, N), (S, 1), 3)
    p = _check_layout_bwd(bnd, x, w, dy, dx, dx_base, 1.0, f"shifted edges {dtype} {N}")
    assert p.variant in (bnd.VARIANT_SHIFTED, bnd.VARIANT_SHIFTED_WAVE)



# ---------------------------------------------------------------------------
# Aligned rows wider than x and dy can stay in registers: the wide row pass
# (two passes over each row, dw in registers).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,dtype,offset", [
    (40, 16392, "bf16", 1.0), (33, 18432, "bf16", 0.0), (20, 32768, "fp16", 1.0), (25, 24576, "fp32", 0.0),
    (30, 8196, "fp32", 1.0), (9, 20480, "bf16", 1.0), (300, 16400, "bf16", 0.0)])
def test_bwd_wide_rule(bnd, M, N, dtype, offset):
    x, w, dy, r32 = any_case(M, N, dtype, offset, seed=N + 2 * M)
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    rg = torch.from_numpy(r32).to(DEV)
    p = bnd.bwd_plan_query(M, N, dtype, xg.data_ptr(), dyg.data_ptr(), dyg.data_ptr())
    announce("bwd wide", M, N, dtype, offset, p.as_dict())
    assert p.variant == bnd.VARIANT_WIDE
    dx, dw = bnd.rmsnorm_bwd(xg, wg, dyg, rg, offset)
    dx2, dw2 = bnd.rmsnorm_bwd(xg, wg, dyg, rg, offset)
    torch.cuda.synchronize()
    _, dwe, dxe, dxs, dws = parity.oracle_bwd_for(x, w, dy, r32, offset, dtype)
    stats = parity.compare_bwd(dx, dw, dxe, dxs, dwe, dws, dtype, M, p.grid, f"bwd wide {M}x{N} {dtype}")
    assert torch.equal(dx, dx2) and torch.equal(dw, dw2)
    print("bwd wide", M, N, dtype, stats, flush=True)


@pytest.mark.parametrize("M,N,dtype", [(40, 24576, "bf16"), (21, 16392, "fp16"), (17, 12292, "fp32")])
def test_bwd_wide_every_kernel(bnd, M, N, dtype):
    x, w, dy, r32 = any_case(M, N, dtype, 1.0, seed=N + 11)
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    rg = torch.from_numpy(r32).to(DEV)
    _, dwe, dxe, dxs, dws = parity.oracle_bwd_for(x, w, dy, r32, 1.0, dtype)
    base = bnd.bwd_plan_query(M, N, dtype)
    epv = EPV[dtype]
    ran = 0
    for threads in (576, 768, 1024):
        for vpt in (3, 4, 5, 6):
            if threads * vpt * epv < N:
                continue
            for grid in (1, 5, M):
                p = base.copy(variant=bnd.VARIANT_WIDE, block_threads=threads, vectors_per_lane=vpt, grid=grid,
                              prefetch=0)
                dx = torch.empty_like(xg)
                dw = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
                ws = torch.empty(grid * N + 4, dtype=torch.float32, device=DEV)
                announce("bwd wide", M, N, dtype, p.as_dict())
                try:
                    bnd.rmsnorm_bwd_out(xg, wg, dyg, rg, dx, dw, ws, 1.0, plan=p)
                except bnd.RmsnormError as e:
                    if e.status == 8:
                        continue
                    raise
                torch.cuda.synchronize()
                parity.compare_bwd(dx, dw, dxe, dxs, dwe, dws, dtype, M, grid, f"bwd wide {M}x{N} {p.as_dict()}")
                ran += 1
    assert ran >= 6, ran


def test_bwd_wide_in_place(bnd):
    M, N = 50, 18432
    x, w, dy, r32 = any_case(M, N, "bf16", 1.0, seed=61)
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    rg = torch.from_numpy(r32).to(DEV)
    dw = torch.empty(N, dtype=torch.float32, device=DEV)
    ws = torch.empty(bnd.bwd_workspace_size(M, N, "bf16") // 4 + 4, dtype=torch.float32, device=DEV)
    announce("bwd wide in place")
    bnd.rmsnorm_bwd_out(xg, wg, dyg, rg, dyg, dw, ws, 1.0)          # dx written over dy
    torch.cuda.synchronize()
    e = parity.oracle_bwd_for(x, w, dy, r32, 1.0, "bf16")
    p = bnd.bwd_plan_query(M, N, "bf16")
    assert p.variant == bnd.VARIANT_WIDE
    parity.compare_bwd(dyg, dw, e[2], e[3], e[1], e[4], "bf16", M, p.grid, "wide in place")
