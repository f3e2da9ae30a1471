"""GPU parity of the general forward (rmsnorm_fwd_ex): strided 2-D rows, batched 3-D and 4-D
rows, broadcast rows, widths that are not a multiple of the 16-byte vector, fp32, in place, and
rstd left out.  Every case writes y into a view of a larger buffer filled with a sentinel and checks
that nothing outside the view changed."""
from __future__ import annotations

import itertools

import pytest
import torch

from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SENTINEL = {torch.bfloat16: 0x7FC1, torch.float16: 0x7E01, torch.float32: 0x7FC00001}
INT_VIEW = {torch.bfloat16: torch.int16, torch.float16: torch.int16, torch.float32: torch.int32}


@pytest.fixture(scope="module")
def bnd():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from memory_bound_row_rmsnorm_amd import binding
    return binding


def announce(*parts):
    print("CASE", *parts, flush=True)


def filled(numel: int, dtype) -> torch.Tensor:
    t = torch.empty(numel, dtype=dtype, device=DEV)
    t.view(INT_VIEW[dtype]).fill_(SENTINEL[dtype])
    return t


def view_mask(numel: int, shape, strides, offset) -> torch.Tensor:
    idx = torch.arange(numel).as_strided(shape, strides, offset)
    mask = torch.zeros(numel, dtype=torch.bool)
    mask[idx.reshape(-1)] = True
    return mask


def draw(shape, dtype, seed, sigma=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return (sigma * torch.randn(*shape, generator=g)).to(dtype)


def check(bnd, x: torch.Tensor, w: torch.Tensor, y: torch.Tensor, y_base: torch.Tensor, y_shape, y_strides,
          y_off, eps=1e-6, offset=0.0, what=""):
    """Run rmsnorm_fwd_ex into y (a view of y_base) and compare with the oracle on the logical rows."""
    plan = bnd.plan_query_ex(x, w, y)
    announce(what, tuple(x.shape), tuple(x.stride()), x.dtype, plan.as_dict()["variant_name"])
    out, rstd = bnd.rmsnorm_fwd_ex(x, w, eps, offset, out=y)
    torch.cuda.synchronize()
    assert out.data_ptr() == y.data_ptr()
    N = x.shape[-1]
    xc = x.cpu().contiguous().reshape(-1, N)
    wc = w.cpu()
    yc = out.cpu().contiguous().reshape(-1, N)
    if x.dtype == torch.float32:
        ye, re = parity.oracle_fp32(xc, wc, eps, offset)
        stats = parity.compare_fp32(yc, rstd.reshape(-1), ye, re, what)
    else:
        dt = "bf16" if x.dtype == torch.bfloat16 else "fp16"
        yr, rr = parity.oracle_for(xc, wc, eps, offset, dt)
        stats = parity.compare(yc, rstd.reshape(-1), yr, rr, dt, what)
    # nothing outside the view was written
    mask = view_mask(y_base.numel(), y_shape, y_strides, y_off)
    untouched = y_base.cpu().view(INT_VIEW[x.dtype])[~mask]
    expect = SENTINEL[x.dtype]
    assert bool((untouched == expect).all()), f"{what}: {int((untouched != expect).sum())} guard elements written"
    # rstd left out: the same y, nothing else written
    y2_base = filled(y_base.numel(), x.dtype)
    y2 = y2_base.as_strided(y_shape, y_strides, y_off)
    out2, none = bnd.rmsnorm_fwd_ex(x, w, eps, offset, want_rstd=False, out=y2)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(out2.cpu().view(INT_VIEW[x.dtype]), out.cpu().view(INT_VIEW[x.dtype])), what
    print(what, plan.as_dict()["variant_name"], stats, flush=True)
    return plan


def strided_case(bnd, dtype, M, N, x_ld, y_ld, seed, **kw):
    xb = draw((M * x_ld,), dtype, seed)
    x = xb.to(DEV).as_strided((M, N), (x_ld, 1), 0)
    w = (1.0 + 0.1 * draw((N,), torch.float32, seed + 1)).to(dtype).to(DEV)
    y_base = filled(M * y_ld + 64, dtype)
    y = y_base.as_strided((M, N), (y_ld, 1), 32)
    return check(bnd, x, w, y, y_base, (M, N), (y_ld, 1), 32, what=f"{M}x{N} ld {x_ld}/{y_ld}", **kw)


@pytest.mark.parametrize("dtype,M,N,x_ld,y_ld,family", [
    (torch.bfloat16, 1000, 512, 640, 576, "wave"),
    (torch.bfloat16, 777, 3001, 3008, 3016, "block"),       # ragged tail of 1 element
    (torch.float16, 1025, 100, 104, 112, "wave"),           # 16-lane rows, tail of 4
    (torch.bfloat16, 300, 8191, 8192, 8200, "block"),       # tail of 7
    (torch.float16, 64, 7, 8, 16, "wave"),                  # narrower than one vector
    (torch.bfloat16, 100, 4096, 4100, 4096, "generic"),     # x rows not 16-byte aligned
    (torch.float32, 333, 1027, 1028, 1032, "block"),        # fp32 tail of 3
    (torch.float32, 500, 130, 132, 136, "wave"),
])
def test_strided_rows(bnd, dtype, M, N, x_ld, y_ld, family):
    plan = strided_case(bnd, dtype, M, N, x_ld, y_ld, seed=11)
    assert plan.as_dict()["variant_name"] == family


@pytest.mark.parametrize("dtype,M,N", [
    (torch.float32, 4096, 512), (torch.float32, 64, 8192), (torch.float32, 8, 24576), (torch.float32, 300, 96),
    (torch.bfloat16, 500, 3001), (torch.float16, 333, 1234),        # contiguous ragged rows: generic kernel
])
def test_contiguous(bnd, dtype, M, N):
    sigma = 100.0 if dtype == torch.float16 else 1.0
    x = draw((M, N), dtype, 21, sigma).to(DEV)
    w = (1.0 + 0.1 * draw((N,), torch.float32, 22)).to(dtype).to(DEV)
    y_base = filled(M * N + 16, dtype)
    y = y_base.as_strided((M, N), (N, 1), 8)
    check(bnd, x, w, y, y_base, (M, N), (N, 1), 8, offset=1.0, what=f"contiguous {M}x{N}")


def test_batches_of_a_sliced_sequence(bnd):
    B, S_all, S, N = 4, 300, 257, 1024
    big = draw((B, S_all, N), torch.bfloat16, 31).to(DEV)
    x = big[:, 10:10 + S, :]                                   # rows 1024 apart, batches 300 * 1024 apart
    w = (1.0 + 0.1 * draw((N,), torch.float32, 32)).to(torch.bfloat16).to(DEV)
    y_base = filled(B * 260 * N, torch.bfloat16)
    shape, strides = (B, S, N), (260 * N, N, 1)
    y = y_base.as_strided(shape, strides, 0)
    plan = check(bnd, x, w, y, y_base, shape, strides, 0, what="3-D slice")
    assert plan.grid * plan.rows_per_trip < B * S               # one batch per grid row


def test_batches_interleaved(bnd):
    S, B, N = 257, 4, 1024
    base = draw((S, B, N), torch.bfloat16, 41).to(DEV)
    x = base.transpose(0, 1)                                   # [B, S, N] with strides (N, B * N, 1)
    w = (0.1 * draw((N,), torch.float32, 42)).to(torch.bfloat16).to(DEV)
    shape, strides = (B, S, N), (N, B * N, 1)
    y_base = filled(S * B * N, torch.bfloat16)
    y = y_base.as_strided(shape, strides, 0)
    check(bnd, x, w, y, y_base, shape, strides, 0, offset=1.0, what="3-D interleaved")


def test_four_dimensional_rows_collapse(bnd):
    shape = (2, 3, 64, 512)
    x = draw(shape, torch.float16, 51, 100.0).to(DEV)
    w = (1.0 + 0.1 * draw((512,), torch.float32, 52)).to(torch.float16).to(DEV)
    n = x.numel()
    y_base = filled(n, torch.float16)
    strides = (3 * 64 * 512, 64 * 512, 512, 1)
    y = y_base.as_strided(shape, strides, 0)
    check(bnd, x, w, y, y_base, shape, strides, 0, what="4-D contiguous")


def test_broadcast_rows(bnd):
    M, N = 1000, 512
    row = draw((1, N), torch.bfloat16, 61).to(DEV)
    x = row.expand(M, N)                                       # row stride 0
    w = (1.0 + 0.1 * draw((N,), torch.float32, 62)).to(torch.bfloat16).to(DEV)
    y_base = filled(M * N, torch.bfloat16)
    y = y_base.as_strided((M, N), (N, 1), 0)
    check(bnd, x, w, y, y_base, (M, N), (N, 1), 0, what="broadcast row")
    assert bool((y == y[0:1]).all())


def test_more_batches_than_one_launch_holds(bnd):
    B, N = 70000, 8                                            # 70000 batches of one row: two launches
    base = draw((B, 2, N), torch.float16, 71).to(DEV)
    x = base[:, :1, :]                                         # batch stride 16 elements
    w = (1.0 + 0.1 * draw((N,), torch.float32, 72)).to(torch.float16).to(DEV)
    shape, strides = (B, 1, N), (2 * N, N, 1)
    y_base = filled(B * 2 * N, torch.float16)
    y = y_base.as_strided(shape, strides, 0)
    check(bnd, x, w, y, y_base, shape, strides, 0, what="70000 batches")


def test_in_place_with_a_layout(bnd):
    M, N, ld = 513, 1000, 1008
    base = draw((M * ld,), torch.bfloat16, 81).to(DEV)
    x = base.as_strided((M, N), (ld, 1), 0)
    w = (1.0 + 0.1 * draw((N,), torch.float32, 82)).to(torch.bfloat16).to(DEV)
    before = base.cpu().clone()
    xc = x.cpu().contiguous()
    announce("in place", M, N, ld)
    out, rstd = bnd.rmsnorm_fwd_ex(x, w, 1e-6, 0.0, out=x)
    torch.cuda.synchronize()
    yr, rr = parity.oracle_for(xc, w.cpu(), 1e-6, 0.0, "bf16")
    parity.compare(out.cpu().contiguous(), rstd, yr, rr, "bf16", "in place")
    after = base.cpu()
    pad = view_mask(M * ld, (M, N), (ld, 1), 0)
    assert torch.equal(after.view(torch.int16)[~pad], before.view(torch.int16)[~pad])


def test_layout_errors_are_raised(bnd):
    x = torch.zeros(8, 64, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    y_overlapping = torch.zeros(8 * 32 + 64, dtype=torch.bfloat16, device=DEV).as_strided((8, 64), (32, 1), 0)
    with pytest.raises(bnd.RmsnormError) as e:
        bnd.rmsnorm_fwd_ex(x, w, out=y_overlapping)            # y rows overlap each other
    assert e.value.status == 2
    with pytest.raises(ValueError):
        bnd.rmsnorm_fwd_ex(x.t(), torch.ones(8, dtype=torch.bfloat16, device=DEV))   # last dim not unit stride


FP32_SWEEP_N = [1, 3, 4, 5, 63, 64, 65, 127, 128, 129, 255, 256, 511, 512, 513, 1023, 1024, 1025, 3000, 4097,
                8192, 16385, 24576]


@pytest.mark.parametrize("N", FP32_SWEEP_N)
def test_fp32_sweep(bnd, N):
    g = torch.Generator().manual_seed(N)
    for M in (1, 3, 65, 257):
        if M * N > 2_000_000:
            continue
        x = (torch.randn(M, N, generator=g) * 3)
        w = (torch.randn(N, generator=g) * 0.5)
        for offset in (0.0, 1.0):
            announce("fp32 sweep", M, N, offset)
            y, r = bnd.rmsnorm_fwd_ex(x.to(DEV), w.to(DEV), 1e-6, offset)
            torch.cuda.synchronize()
            ye, re = parity.oracle_fp32(x, w, 1e-6, offset)
            parity.compare_fp32(y, r, ye, re, f"fp32 sweep M={M} N={N} off={offset}")


# ---------------------------------------------------------------------------
# The shifted kernel: rows that do not start 16-byte aligned.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("N", [1, 7, 9, 100, 1001, 3001, 8191, 20001])
def test_shifted_every_instance(bnd, dtype, N):
    M = 37 if N < 8000 else 11
    sigma = 100.0 if dtype == torch.float16 else 1.0
    x = draw((M, N), dtype, 91, sigma).to(DEV)
    w = (1.0 + 0.1 * draw((N,), torch.float32, 92)).to(dtype).to(DEV)
    xc, wc = x.cpu(), w.cpu()
    if dtype == torch.float32:
        ref = parity.oracle_fp32(xc, wc, 1e-6, 1.0)
    else:
        dt = "bf16" if dtype == torch.bfloat16 else "fp16"
        ref = parity.oracle_for(xc, wc, 1e-6, 1.0, dt)
    base = bnd.plan_query_ex(x, w)
    es = x.element_size()
    epv = 16 // es
    if (N * es) % 16 == 0 or -(-(N + epv - 1) // epv) > 4096:
        # aligned rows take the vector kernels, rows wider than 4096 chunks the generic one
        assert base.as_dict()["variant_name"] != "shifted"
        return
    # the rule takes a shifted kernel from 16 elements up (the wave form up to 128 chunks); explicit
    # plans run the block form at any width
    nch = -(-(N + epv - 1) // epv)
    expect = "generic" if N < 16 else ("shifted_wave" if nch <= 128 else "shifted")
    assert base.as_dict()["variant_name"] == expect
    ran = 0
    for threads, vpt, grid, pf in itertools.product((64, 128, 256, 512, 1024), (1, 2, 3, 4), (M, 5), (0, 1)):
                p = base.copy(variant=bnd.VARIANT_SHIFTED, block_threads=threads, vectors_per_lane=vpt,
                              row_slots=1, prefetch=pf, grid=grid, xcd_group=1, max_blocks_per_cu=0)
                if bnd.plan_validate(M, N, x.dtype, p, x.data_ptr(), w.data_ptr(), x.data_ptr()) is None:
                    continue                     # does not cover N (the in-place pointers are equally aligned)
                y_base = filled(M * N + 16, dtype)
                y = y_base.as_strided((M, N), (N, 1), 8)
                announce("shifted", M, N, dtype, threads, vpt, grid, pf)
                out, rstd = bnd.rmsnorm_fwd_ex(x, w, 1e-6, 1.0, out=y, plan=p)
                torch.cuda.synchronize()
                what = f"shifted {M}x{N} {dtype} {threads}x{vpt} grid {grid} weights-with-row {pf}"
                if dtype == torch.float32:
                    parity.compare_fp32(out, rstd, ref[0], ref[1], what)
                else:
                    parity.compare(out, rstd, ref[0], ref[1], dt, what)
                mask = view_mask(y_base.numel(), (M, N), (N, 1), 8)
                assert bool((y_base.cpu().view(INT_VIEW[dtype])[~mask] == SENTINEL[dtype]).all()), what
                ran += 1
    assert ran >= (4 if N > 8000 else 12), ran


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("vectors,tail", [(1, 0), (2, 0), (3, 0), (4, 0), (5, 0), (8, 0), (4, 3), (8, 1)])
def test_narrow_wave_every_instance(bnd, dtype, vectors, tail):
    """Rows of at most 8 vectors: every 4- and 8-lane wave instance that covers the row (slots,
    workgroup sizes, next-trip prefetch, one trip and persistent grids), rows strided by a whole
    number of vectors, with a ragged tail of `tail` elements cut from the last vector."""
    es = torch.tensor([], dtype=dtype).element_size()
    epv = 16 // es
    if tail >= epv:
        return
    N = vectors * epv - tail
    ld = vectors * epv + epv                       # one spare vector between rows
    M = 301
    sigma = 100.0 if dtype == torch.float16 else 1.0
    xb = draw((M * ld,), dtype, 97 + N, sigma).to(DEV)
    x = xb.as_strided((M, N), (ld, 1), 0)
    w = (1.0 + 0.1 * draw((N,), torch.float32, 98)).to(dtype).to(DEV)
    xc, wc = x.cpu().contiguous(), w.cpu()
    if dtype == torch.float32:
        ref = parity.oracle_fp32(xc, wc, 1e-6, 1.0)
    else:
        dt = "bf16" if dtype == torch.bfloat16 else "fp16"
        ref = parity.oracle_for(xc, wc, 1e-6, 1.0, dt)
    y0_base = filled(M * ld + 16, dtype)
    y0 = y0_base.as_strided((M, N), (ld, 1), 8)
    base = bnd.plan_query_ex(x, w, y0)
    assert base.variant == bnd.VARIANT_WAVE and base.lanes_per_row == (4 if vectors <= 4 else 8), base.as_dict()
    check(bnd, x, w, y0, y0_base, (M, N), (ld, 1), 8, offset=1.0, what=f"narrow wave rule {M}x{N} ld {ld} {dtype}")
    ran, lanes_seen = 0, set()
    for lanes, slots, threads, pf in itertools.product((4, 8), (1, 2, 4), (64, 128, 256), (0, 1)):
        rows = threads // 64 * (64 // lanes) * slots
        for grid in (-(-M // rows), 2):
            p = base.copy(variant=bnd.VARIANT_WAVE, lanes_per_row=lanes, block_threads=threads, vectors_per_lane=1,
                          row_slots=slots, prefetch=pf, grid=grid, xcd_group=1, max_blocks_per_cu=0)
            y_base = filled(M * ld + 16, dtype)
            y = y_base.as_strided((M, N), (ld, 1), 8)
            what = f"narrow wave {M}x{N} ld {ld} {dtype} lanes {lanes} slots {slots} {threads} thr pf {pf} grid {grid}"
            announce(what)
            try:
                out, rstd = bnd.rmsnorm_fwd_ex(x, w, 1e-6, 1.0, out=y, plan=p)
            except bnd.RmsnormError as e:
                if e.status == 8:                # does not cover N, or no such instance
                    continue
                raise
            torch.cuda.synchronize()
            if dtype == torch.float32:
                parity.compare_fp32(out.cpu().contiguous(), rstd, ref[0], ref[1], what)
            else:
                parity.compare(out.cpu().contiguous(), rstd, ref[0], ref[1], dt, what)
            mask = view_mask(y_base.numel(), (M, N), (ld, 1), 8)
            assert bool((y_base.cpu().view(INT_VIEW[dtype])[~mask] == SENTINEL[dtype]).all()), what
            lanes_seen.add(lanes)
            ran += 1
    assert 8 in lanes_seen and (4 in lanes_seen or vectors > 4) and ran >= 20, (lanes_seen, ran)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("N", [9, 17, 29, 36, 61, 100, 129, 300, 505, 513, 1001, 1017])
def test_shifted_wave_every_instance(bnd, dtype, N):
    """The wave form of the shifted kernel: every compiled instance that covers N, one trip and
    persistent grids, next-trip prefetch on and off."""
    M = 37
    sigma = 100.0 if dtype == torch.float16 else 1.0
    x = draw((M, N), dtype, 93, sigma).to(DEV)
    w = (1.0 + 0.1 * draw((N,), torch.float32, 94)).to(dtype).to(DEV)
    xc, wc = x.cpu(), w.cpu()
    if dtype == torch.float32:
        ref = parity.oracle_fp32(xc, wc, 1e-6, 0.0)
    else:
        dt = "bf16" if dtype == torch.bfloat16 else "fp16"
        ref = parity.oracle_for(xc, wc, 1e-6, 0.0, dt)
    es = x.element_size()
    if (N * es) % 16 == 0:
        return                                   # aligned rows never take a shifted kernel
    base = bnd.plan_query_ex(x, w)
    ran = 0
    for lanes, vpl, slots, threads, pf in itertools.product((8, 16, 32, 64), (1, 2), (1, 2, 4), (64, 256), (0, 1)):
        rows = threads // 64 * (64 // lanes) * slots
        for grid in (-(-M // rows), 2):
            p = base.copy(variant=bnd.VARIANT_SHIFTED_WAVE, lanes_per_row=lanes, block_threads=threads,
                          vectors_per_lane=vpl, row_slots=slots, prefetch=pf, grid=grid, xcd_group=1,
                          max_blocks_per_cu=0)
            if bnd.plan_validate(M, N, x.dtype, p, x.data_ptr(), w.data_ptr(), x.data_ptr()) is None:
                continue                         # does not cover N, or no such instance
            y_base = filled(M * N + 16, dtype)
            y = y_base.as_strided((M, N), (N, 1), 8)
            announce("shifted wave", M, N, dtype, lanes, vpl, slots, threads, pf, grid)
            out, rstd = bnd.rmsnorm_fwd_ex(x, w, 1e-6, 0.0, out=y, plan=p)
            torch.cuda.synchronize()
            what = f"shifted wave {M}x{N} {dtype} lanes {lanes} vpl {vpl} slots {slots} {threads} thr pf {pf} grid {grid}"
            if dtype == torch.float32:
                parity.compare_fp32(out, rstd, ref[0], ref[1], what)
            else:
                parity.compare(out, rstd, ref[0], ref[1], dt, what)
            mask = view_mask(y_base.numel(), (M, N), (N, 1), 8)
            assert bool((y_base.cpu().view(INT_VIEW[dtype])[~mask] == SENTINEL[dtype]).all()), what
            ran += 1
    nch = -(-(N + 16 // es - 1) // (16 // es))
    assert ran >= (8 if nch > 128 else 16) or nch > 128, ran


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("N,lead", [(3001, 3), (1025, 1), (8191, 5), (300, 7), (129, 2), (1017, 6), (61, 3), (130, 5),
                                    (36, 3), (19, 1)])
def test_shifted_reads_whole_edge_chunks_but_uses_only_the_row(bnd, dtype, N, lead):
    """The shifted kernel loads the aligned 16 bytes around each row's ends, and w's last vector whole:
    NaN in those bytes (before the first row, after the last, after w) must not reach y or rstd, and
    sentinels around y must survive."""
    M = 29
    es = torch.tensor([], dtype=dtype).element_size()
    epv = 16 // es
    nan = float("nan")
    x_base = torch.full((M * N + 2 * epv + lead,), nan, dtype=dtype)
    x_base[lead:lead + M * N] = draw((M * N,), dtype, 101)
    x_base = x_base.to(DEV)
    x = x_base[lead:lead + M * N].view(M, N)
    w_base = torch.full((N + 2 * epv,), nan, dtype=dtype)
    w_base[:N] = (1.0 + 0.1 * draw((N,), torch.float32, 102)).to(dtype)
    w_base = w_base.to(DEV)
    w = w_base[:N]
    y_base = filled(M * N + 2 * epv + lead, dtype)
    y = y_base.as_strided((M, N), (N, 1), lead)
    plan = bnd.plan_query_ex(x, w, y)
    assert plan.as_dict()["variant_name"].startswith("shifted")
    xc, wc = x.cpu(), w.cpu()
    if dtype == torch.float32:
        ref = parity.oracle_fp32(xc, wc, 1e-6, 0.0)
    else:
        ref = parity.oracle_for(xc, wc, 1e-6, 0.0, "bf16")
    for pf in (0, 1):
        p = bnd.plan_validate(M, N, dtype, plan.copy(prefetch=pf), x.data_ptr(), w.data_ptr(), y.data_ptr())
        if p is None and pf == 1 and plan.variant == bnd.VARIANT_SHIFTED_WAVE:
            continue                             # the widest wave instance has no prefetching form
        assert p is not None
        y_base.copy_(filled(y_base.numel(), dtype))
        announce("shifted edges", M, N, dtype, lead, pf)
        out, rstd = bnd.rmsnorm_fwd_ex(x, w, 1e-6, 0.0, out=y, plan=p)
        torch.cuda.synchronize()
        what = f"shifted edges {M}x{N} {dtype} lead {lead} weights-with-row {pf}"
        assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(rstd).all()), what
        if dtype == torch.float32:
            parity.compare_fp32(out, rstd, ref[0], ref[1], what)
        else:
            parity.compare(out, rstd, ref[0], ref[1], "bf16", what)
        mask = view_mask(y_base.numel(), (M, N), (N, 1), lead)
        assert bool((y_base.cpu().view(INT_VIEW[dtype])[~mask] == SENTINEL[dtype]).all()), what


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_equally_misaligned_operands(bnd, dtype):
    M, N = 300, 512                                            # rows of 16-byte multiples, bases 1 element off
    xb = draw((M * N + 1,), dtype, 95).to(DEV)
    x = xb[1:].view(M, N)
    w = (1.0 + 0.1 * draw((N,), torch.float32, 96)).to(dtype).to(DEV)
    y_base = filled(M * N + 9, dtype)
    y = y_base.as_strided((M, N), (N, 1), 1)
    plan = check(bnd, x, w, y, y_base, (M, N), (N, 1), 1, what="misaligned bases")
    assert plan.as_dict()["variant_name"].startswith("shifted")


def test_shifted_in_place(bnd):
    M, N = 257, 3001
    x = draw((M, N), torch.float16, 97, 100.0).to(DEV)
    w = (1.0 + 0.1 * draw((N,), torch.float32, 98)).to(torch.float16).to(DEV)
    xc = x.cpu()
    announce("shifted in place", M, N)
    assert bnd.plan_query_ex(x, w, x).as_dict()["variant_name"] == "shifted"
    out, rstd = bnd.rmsnorm_fwd_ex(x, w, 1e-6, 0.0, out=x)
    torch.cuda.synchronize()
    yr, rr = parity.oracle_for(xc, w.cpu(), 1e-6, 0.0, "fp16")
    parity.compare(out, rstd, yr, rr, "fp16", "shifted in place")


# ---------------------------------------------------------------------------
# The wide kernel: aligned rows wider than the block family's registers hold.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,N,M", [(torch.bfloat16, 40968, 5), (torch.bfloat16, 65536, 5),
                                       (torch.float16, 49152, 4), (torch.bfloat16, 100003, 1),
                                       (torch.float32, 24580, 5), (torch.float32, 65537, 1)])
def test_wide_rows(bnd, dtype, N, M):
    """Rows of N elements at a row stride padded to whole 16-byte vectors (ragged N: the tail
    vector moves element by element)."""
    sigma = 100.0 if dtype == torch.float16 else 1.0
    epv = 16 // torch.tensor([], dtype=dtype).element_size()
    Np = -(-N // epv) * epv
    x = draw((M, Np), dtype, 301, sigma).to(DEV)[:, :N]
    w = (1.0 + 0.1 * draw((N,), torch.float32, 302)).to(dtype).to(DEV)
    xc, wc = x.cpu(), w.cpu()
    if dtype == torch.float32:
        ref = parity.oracle_fp32(xc, wc, 1e-6, 1.0)
    else:
        dt = "bf16" if dtype == torch.bfloat16 else "fp16"
        ref = parity.oracle_for(xc, wc, 1e-6, 1.0, dt)
    y_base = filled(M * Np + 16, dtype)
    y = y_base.as_strided((M, N), (Np, 1), 0)
    base = bnd.plan_query_ex(x, w, y)
    assert base.as_dict()["variant_name"] == "wide"
    ran = 0
    for threads, vpt, grid in itertools.product((256, 1024), (2, 4), (M, 2)):
        p = bnd.plan_validate(M, N, x.dtype, base.copy(block_threads=threads, vectors_per_lane=vpt, grid=grid),
                              x.data_ptr(), w.data_ptr(), y.data_ptr())
        assert p is not None
        y_base.copy_(filled(M * Np + 16, dtype))
        announce("wide", M, N, dtype, threads, vpt, grid)
        out, rstd = bnd.rmsnorm_fwd_ex(x, w, 1e-6, 1.0, out=y, plan=p)
        torch.cuda.synchronize()
        what = f"wide {M}x{N} {dtype} {threads}x{vpt} grid {grid}"
        if dtype == torch.float32:
            parity.compare_fp32(out, rstd, ref[0], ref[1], what)
        else:
            parity.compare(out, rstd, ref[0], ref[1], dt, what)
        mask = view_mask(y_base.numel(), (M, N), (Np, 1), 0)
        assert bool((y_base.cpu().view(INT_VIEW[dtype])[~mask] == SENTINEL[dtype]).all()), what
        ran += 1
    assert ran == 8
