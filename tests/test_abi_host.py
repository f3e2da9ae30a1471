"""The C-ABI library on the host: loads, exports what include/rmsnorm.h
declares, rejects bad arguments before any HIP call, and plans launches on the
host.  No kernel is launched here."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmsnorm.h")

bnd = pytest.importorskip("memory_bound_row_rmsnorm_amd.binding",
                          reason="librmsnorm_mi355x.so not built")
lib = bnd.lib

OK, NULL, SHAPE, DTYPE, SCALAR, OVERLAP, HIP, DEVICE, PLAN = range(9)
BF16, FP16, FP32 = 0, 1, 2
A = 0x10000000  # fake, 256-byte aligned, never dereferenced: every call below fails validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rmsnorm_[a-z_]+)\s*\(", text)))


def test_header_declarations_are_all_exported():
    names = declared_functions()
    assert names == sorted(bnd.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", bnd.LIBRARY], capture_output=True, text=True,
                        check=True).stdout
    exported = set(re.findall(r" T (rmsnorm_\w+)", nm))
    assert set(names) <= exported, set(names) - exported


def test_version_and_status_strings():
    assert lib.rmsnorm_version() == 10000
    for code, name in bnd.STATUS.items():
        assert bnd.status_string(code) == name
    assert bnd.status_string(99) == "RMSNORM_ERR_UNKNOWN"


def fwd(x=A, w=A + 0x1000000, y=A + 0x2000000, rstd=A + 0x3000000, M=4, N=512, eps=1e-6,
        offset=0.0, dtype=BF16):
    return lib.rmsnorm_fwd(x, w, y, rstd, M, N, eps, offset, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(M=-1), SHAPE),
    (dict(N=0), SHAPE),
    (dict(N=-5), SHAPE),
    (dict(M=1 << 40, N=1 << 40), SHAPE),
    (dict(dtype=3), DTYPE),
    (dict(dtype=-1), DTYPE),
    (dict(x=None), NULL),
    (dict(w=None), NULL),
    (dict(y=None), NULL),
    (dict(rstd=None), NULL),
    (dict(eps=-1e-6), SCALAR),
    (dict(eps=float("nan")), SCALAR),
    (dict(eps=float("inf")), SCALAR),
    (dict(offset=float("nan")), SCALAR),
    (dict(offset=float("-inf")), SCALAR),
    (dict(y=A + 16), OVERLAP),                      # y partially overlaps x
    (dict(y=A + 0x1000000 - 16), OVERLAP),          # y runs into w
    (dict(rstd=A + 8), OVERLAP),                    # rstd inside x
    (dict(rstd=A + 0x1000000 + 4), OVERLAP),        # rstd inside w
    (dict(rstd=A + 0x2000000 + 64), OVERLAP),       # rstd inside y
])
def test_argument_errors(kwargs, status):
    assert fwd(**kwargs) == status
    assert lib.rmsnorm_last_error().decode() != ""


def test_m_zero_is_a_noop_without_pointers():
    assert fwd(x=None, w=None, y=None, rstd=None, M=0) == OK
    assert lib.rmsnorm_last_error().decode() == ""


def test_m_zero_still_checks_shape_and_scalars():
    assert fwd(M=0, N=0) == SHAPE
    assert fwd(M=0, eps=-1.0) == SCALAR


def test_errors_are_checked_before_plans():
    p = bnd.Plan()
    assert lib.rmsnorm_fwd_with_plan(A, A, A + 16, A + 0x3000000, 4, 512, 1e-6, 0.0, BF16,
                                     ctypes.byref(p), None) == OVERLAP
    assert lib.rmsnorm_fwd_with_plan(A, A + 0x1000000, A + 0x2000000, A + 0x3000000, 4, 512, 1e-6,
                                     0.0, BF16, None, None) == NULL


def host_plan(M, N, dtype=BF16, x=None, w=None, y=None, cu=256):
    p = bnd.Plan()
    st = lib.rmsnorm_plan_query(M, N, dtype, x, w, y, cu, ctypes.byref(p))
    assert st == OK, bnd.status_string(st) + " " + lib.rmsnorm_last_error().decode()
    return p


def covers(p, N):
    if p.variant == bnd.VARIANT_GENERIC:
        return True
    return p.lanes_per_row * p.vectors_per_lane * p.vec_elems >= N


@pytest.mark.parametrize("M,N", [(64, 512), (16384, 512), (8192, 3000), (32768, 8192),
                                 (262144, 128), (4096, 16384), (1, 8), (7, 256), (100, 1024),
                                 (3, 4096), (5, 40960)])
def test_host_plans_cover_the_row_one_trip_per_workgroup(M, N):
    for dtype in (BF16, FP16):
        p = host_plan(M, N, dtype)
        assert p.variant in (bnd.VARIANT_WAVE, bnd.VARIANT_BLOCK)
        assert p.vec_elems == 8 and covers(p, N)
        # no more vectors per lane than the row needs
        assert (p.vectors_per_lane - 1) * p.lanes_per_row * 8 < N
        assert p.block_threads % 64 == 0 and 64 <= p.block_threads <= 1024
        groups = -(-M // p.rows_per_trip)
        assert p.grid == groups and p.trips == 1 and p.prefetch == 0
        per_cu = 2048 // p.block_threads
        if p.max_blocks_per_cu:
            per_cu = min(per_cu, p.max_blocks_per_cu)
        assert p.resident_grid == 256 * per_cu
        assert 1 <= p.xcd_group <= 256


def test_planner_choices_for_the_workloads():
    p = host_plan(16384, 512)             # rows of exactly 64 vectors: half-wave rows, 8 KiB per wave
    assert (p.variant, p.lanes_per_row, p.vectors_per_lane, p.row_slots) == (bnd.VARIANT_WAVE, 32, 2, 4)
    assert p.rows_per_trip == 32 and p.grid == 512 and p.block_threads == 256
    p = host_plan(16383, 512)             # fewer rows: 64-lane rows, 4 rows per wave
    assert (p.lanes_per_row, p.vectors_per_lane, p.row_slots, p.grid) == (64, 1, 4, 1024)
    p = host_plan(16384, 504)             # one vector short of that: 64-lane rows, masked
    assert (p.lanes_per_row, p.vectors_per_lane, p.row_slots) == (64, 1, 4)
    p = host_plan(16384, 256, FP32)       # 64 fp32 vectors
    assert (p.lanes_per_row, p.vectors_per_lane, p.row_slots) == (32, 2, 4)
    p = host_plan(262144, 128, FP16)        # several rows per slot: 2 KiB per wave, 2-wave workgroups
    assert (p.variant, p.lanes_per_row, p.row_slots, p.block_threads) == (bnd.VARIANT_WAVE, 16, 2, 128)
    assert p.rows_per_trip == 16 and p.grid == 262144 // 16
    p = host_plan(64, 256)
    assert (p.lanes_per_row, p.row_slots, p.block_threads) == (32, 2, 128)
    # rows of at most 8 vectors: 8-lane segments (2 KiB per wave), at most 4: 4-lane ones (4 KiB)
    p = host_plan(262144, 64)
    assert (p.lanes_per_row, p.vectors_per_lane, p.row_slots, p.block_threads) == (8, 1, 2, 128)
    assert p.rows_per_trip == 32 and p.grid == 262144 // 32
    p = host_plan(262144, 40)
    assert (p.lanes_per_row, p.row_slots) == (8, 2)
    p = host_plan(262144, 32)
    assert (p.lanes_per_row, p.vectors_per_lane, p.row_slots, p.block_threads) == (4, 1, 4, 128)
    assert p.rows_per_trip == 128 and p.grid == 262144 // 128
    p = host_plan(1000, 8)
    assert (p.lanes_per_row, p.row_slots) == (4, 4)
    p = host_plan(1000, 72)
    assert (p.lanes_per_row, p.row_slots) == (16, 2)
    assert (host_plan(1000, 32, FP32).lanes_per_row, host_plan(1000, 16, FP32).lanes_per_row) == (8, 4)
    p = host_plan(100, 1024)
    assert (p.lanes_per_row, p.vectors_per_lane, p.row_slots) == (64, 2, 2)
    p = host_plan(32768, 8192)            # 512 MiB of x: about 1 MiB of rows per XCD group
    assert (p.variant, p.block_threads, p.vectors_per_lane) == (bnd.VARIANT_BLOCK, 256, 4)
    assert (p.xcd_group, p.max_blocks_per_cu) == (64, 3)  # contiguous exact-width rows: capped at 3
    assert host_plan(16383, 8192).xcd_group == 8          # just under 256 MiB of x: 128 KiB groups
    assert p.resident_grid == 256 * 3
    p = host_plan(32768, 8000)            # not an exact width: the block family's cap of 64 KiB of rows
    assert (p.block_threads, p.vectors_per_lane, p.max_blocks_per_cu) == (256, 4, 4)
    p = host_plan(8192, 3000)
    assert (p.variant, p.block_threads, p.vectors_per_lane) == (bnd.VARIANT_BLOCK, 256, 2)
    assert (p.xcd_group, p.max_blocks_per_cu) == (16, 0)
    p = host_plan(4096, 16384, FP16)      # contiguous rows of exactly 2048 vectors: the exact-width block form
    assert (p.variant, p.block_threads, p.vectors_per_lane) == (bnd.VARIANT_BLOCK, 256, 8)
    assert (p.xcd_group, p.max_blocks_per_cu) == (8, 3)
    p = host_plan(4096, 16376, FP16)      # one vector short: the 1024-thread block plan
    assert (p.variant, p.block_threads, p.vectors_per_lane) == (bnd.VARIANT_BLOCK, 1024, 2)
    p = host_plan(3, 40960)
    assert (p.block_threads, p.vectors_per_lane, p.max_blocks_per_cu) == (1024, 5, 0)
    assert host_plan(3, 49152).variant == bnd.VARIANT_WIDE        # six 16-bit vectors per thread do not fit
    p = host_plan(4096, 12288)
    assert (p.variant, p.block_threads, p.vectors_per_lane) == (bnd.VARIANT_BLOCK, 512, 3)
    for M, N in ((16384, 512), (262144, 128), (64, 256)):
        p = host_plan(M, N)
        assert (p.xcd_group, p.max_blocks_per_cu) == (1, 0)


def test_every_aligned_width_takes_a_16_byte_kernel():
    """No width the 16-byte kernels can hold falls through to the generic kernel:
    up to 1024 x 5 vectors of 8 for 16-bit rows, 1024 x 6 vectors of 4 for fp32."""
    for dtype, epv, widest in (("bf16", 8, 1024 * 5 * 8), ("fp16", 8, 1024 * 5 * 8), ("fp32", 4, 1024 * 6 * 4)):
        for N in range(epv, widest + 1, epv):
            p = query_ex(1024, N, dtype)
            assert p.variant in (bnd.VARIANT_WAVE, bnd.VARIANT_BLOCK), (dtype, N)
            assert p.lanes_per_row * p.vectors_per_lane * epv >= N, (dtype, N)


@pytest.mark.parametrize("N,dtype", [(40968, "bf16"), (49152, "bf16"), (1 << 17, "fp16"), (1 << 20, "bf16"),
                                     (24580, "fp32"), (65536, "fp32")])
def test_rows_wider_than_the_registers_take_the_wide_kernel(N, dtype):
    p = query_ex(64, N, dtype)
    assert (p.variant, p.block_threads, p.vectors_per_lane, p.rows_per_trip) == (bnd.VARIANT_WIDE, 1024, 2, 1)
    assert p.vec_elems == (4 if dtype == "fp32" else 8) and p.grid == 64


def test_a_single_ragged_row_takes_the_vector_kernels():
    """One row: its stride never applies, so a ragged width still moves as 16-byte vectors plus a
    tail vector."""
    assert query_ex(1, 3001).variant == bnd.VARIANT_BLOCK
    assert query_ex(1, 1001).variant == bnd.VARIANT_WAVE
    assert query_ex(1, 100003).variant == bnd.VARIANT_WIDE
    assert query_ex(2, 3001).variant == bnd.VARIANT_SHIFTED         # two rows: the second starts unaligned


def test_huge_row_counts_loop_with_prefetch():
    """A dispatch takes fewer than 2^32 work-items: the grid is capped at (2^32 - 1) // threads
    and the workgroups loop, loading the next trip ahead."""
    p = host_plan(1 << 40, 8192)
    assert p.block_threads == 256 and p.grid == (2 ** 32 - 1) // 256
    assert p.grid * p.block_threads < 2 ** 32 and p.trips > 1 and p.prefetch == 1


@pytest.mark.parametrize("M,N,dtype", [(1 << 24, 2048, BF16), (1 << 24, 16384, FP16), (1 << 30, 512, BF16),
                                       (1 << 33, 3000, BF16), (1 << 31, 3001, BF16), (1 << 33, 3, BF16)])
def test_grids_stay_below_2_to_32_work_items(M, N, dtype):
    """16.8M rows of 2048 bf16 (137 GB of x and y, which fits in 288 GB) ask for 2^24 workgroups of
    256 threads: the plan caps the grid and loops instead of failing at launch."""
    p = host_plan(M, N, dtype=dtype)
    assert p.grid * p.block_threads < 2 ** 32 and p.grid < 2 ** 31
    assert p.grid * p.rows_per_trip * p.trips >= M


def test_plans_past_2_to_32_work_items_are_rejected():
    M, N = 1 << 24, 2048
    p = host_plan(M, N)
    args = (A, A + (1 << 40), A + (2 << 40), A + (3 << 40), M, N, 1e-6, 0.0, BF16)
    out = bnd.Plan()
    for grid, status in ((p.grid, OK), (p.grid + 1, PLAN), (1 << 24, PLAN)):
        q = p.copy(grid=grid)
        assert lib.rmsnorm_plan_validate(M, N, BF16, args[0], args[1], args[2], ctypes.byref(q), 256,
                                         ctypes.byref(out)) == status, grid


@pytest.mark.parametrize("N", [257, 3001, 1025, 32761])
def test_ragged_contiguous_rows_take_a_shifted_kernel(N):
    p = host_plan(10, N)                       # rows start a varying distance past a 16-byte boundary
    assert p.variant in (bnd.VARIANT_SHIFTED, bnd.VARIANT_SHIFTED_WAVE) and p.vec_elems == 8
    assert p.lanes_per_row * p.vectors_per_lane * 8 >= N + 7
    assert p.rows_per_trip == (1 if p.variant == bnd.VARIANT_SHIFTED
                               else p.block_threads // 64 * (64 // p.lanes_per_row) * p.row_slots)
    f = host_plan(10, N, dtype=FP16, x=A + 2, y=A + 2 + 0x1000000)    # equally misaligned x and y
    assert f.variant == p.variant


@pytest.mark.parametrize("N,threads,vpt,prefetch", [(1018, 64, 3, 1), (3001, 128, 3, 1), (6001, 256, 3, 1),
                                                    (8191, 512, 3, 0), (16383, 1024, 3, 0), (32761, 1024, 4, 0)])
def test_shifted_rule(N, threads, vpt, prefetch):
    """Rows wider than 128 chunks: the fewest threads holding the row's chunks at most 3 per thread;
    weights fetched with the row up to 256 threads."""
    p = host_plan(10, N)
    assert (p.variant, p.block_threads, p.vectors_per_lane, p.prefetch) == (bnd.VARIANT_SHIFTED, threads, vpt,
                                                                            prefetch)


@pytest.mark.parametrize("N,dtype,lanes,vpl", [(17, BF16, 8, 1), (57, BF16, 8, 1), (58, BF16, 16, 1),
                                               (121, BF16, 16, 1), (129, BF16, 32, 1),
                                               (249, BF16, 32, 1), (257, BF16, 64, 1), (505, BF16, 64, 1),
                                               (513, BF16, 64, 2), (1017, BF16, 64, 2), (130, FP16, 32, 1),
                                               (29, FP32, 8, 1), (61, FP32, 16, 1), (509, FP32, 64, 2)])
def test_shifted_wave_rule(N, dtype, lanes, vpl):
    """Rows of 16 elements up to 128 chunks: a row per segment of 8, 16, 32 or 64 lanes (the fewest
    that hold its chunks, up to 64), four slots per wave (two with 8- and 16-lane rows)."""
    p = host_plan(100000, N, dtype=dtype)
    slots = 2 if lanes <= 16 else 4
    assert (p.variant, p.lanes_per_row, p.vectors_per_lane, p.row_slots) == (bnd.VARIANT_SHIFTED_WAVE, lanes, vpl,
                                                                            slots)
    rows = 4 * (64 // lanes) * slots
    assert p.rows_per_trip == rows and p.grid == -(-100000 // rows) and p.trips == 1


@pytest.mark.parametrize("N,x,w", [(512, A + 2, None), (512, A + 8, None),   # x and y not equally aligned
                                   (3001, None, A + 2),                        # w not 16-byte aligned
                                   (49161, None, None),                        # unaligned, over 4096 chunks
                                   (7, None, None), (15, None, None)])          # short unaligned rows
def test_unaligned_or_very_wide_rows_take_the_generic_kernel(N, x, w):
    p = host_plan(10, N, x=x, w=w)
    assert p.variant == bnd.VARIANT_GENERIC and p.vec_elems == 1


def test_plans_that_do_not_fit_are_rejected_before_launch():
    good = host_plan(100, 512)
    bad = [
        good.copy(vectors_per_lane=0),                                      # no such kernel
        good.copy(variant=bnd.VARIANT_WAVE, lanes_per_row=16, vectors_per_lane=1),  # covers 128 < 512
        good.copy(block_threads=96),
        good.copy(block_threads=2048),
        good.copy(grid=0),
        good.copy(variant=7),
        good.copy(variant=bnd.VARIANT_BLOCK, block_threads=64, vectors_per_lane=8),  # not compiled
        good.copy(xcd_group=0),
        good.copy(xcd_group=257),
        good.copy(max_blocks_per_cu=1),
        good.copy(max_blocks_per_cu=33),
        good.copy(max_blocks_per_cu=-2),
        good.copy(prefetch=2),
    ]
    args = (A, A + 0x1000000, A + 0x2000000, A + 0x3000000, 100, 512, 1e-6, 0.0, BF16)
    for p in bad:
        assert lib.rmsnorm_fwd_with_plan(*args, ctypes.byref(p), None) == PLAN, p.as_dict()
    # a wave plan needs N % 8 == 0 and 16-byte alignment
    p = good.copy()
    assert lib.rmsnorm_fwd_with_plan(A, A + 0x1000000, A + 0x2000000, A + 0x3000000, 100, 511,
                                     1e-6, 0.0, BF16, ctypes.byref(p), None) == PLAN
    assert lib.rmsnorm_fwd_with_plan(A + 2, A + 0x1000000, A + 0x2000000, A + 0x3000000, 100, 512,
                                     1e-6, 0.0, BF16, ctypes.byref(p), None) == PLAN


def test_plan_query_validates():
    p = bnd.Plan()
    assert lib.rmsnorm_plan_query(-1, 8, BF16, None, None, None, 256, ctypes.byref(p)) == SHAPE
    assert lib.rmsnorm_plan_query(1, 8, 5, None, None, None, 256, ctypes.byref(p)) == DTYPE
    assert lib.rmsnorm_plan_query(1, 8, BF16, None, None, None, 256, None) == NULL


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------
X, W, DY, R, DX, DW, WS = (A + k * 0x1000000 for k in range(7))


def bwd(x=X, w=W, dy=DY, rstd=R, dx=DX, dw=DW, M=4, N=512, offset=0.0, dtype=BF16, ws=WS,
        ws_bytes=1 << 24):
    return lib.rmsnorm_bwd(x, w, dy, rstd, dx, dw, M, N, offset, dtype, ws, ws_bytes, None)


def bwd_noalloc(x=X, w=W, dy=DY, rstd=R, dx=DX, dw=DW, M=4, N=512, offset=0.0, dtype=BF16):
    return lib.rmsnorm_bwd_noalloc(x, w, dy, rstd, dx, dw, M, N, offset, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(M=-1), SHAPE),
    (dict(N=0), SHAPE),
    (dict(dtype=7), DTYPE),
    (dict(dw=None), NULL),
    (dict(x=None), NULL),
    (dict(offset=float("nan")), SCALAR),
    (dict(dx=X), OVERLAP),
    (dict(dw=DX + 64), OVERLAP),
    (dict(N=4 * 1024 * 1024 + 8, M=1), SHAPE),     # one partial row of N fp32 exceeds the 16 MiB scratch
])
def test_bwd_noalloc_argument_errors(kwargs, status):
    """rmsnorm_bwd_noalloc checks its arguments, and that a partial row fits its scratch, before
    any HIP call (these calls make none)."""
    assert bwd_noalloc(**kwargs) == status


def test_bwd_noalloc_scratch_limit_is_the_header_constant():
    text = open(HEADER).read()
    assert re.search(r"#define RMSNORM_BWD_SCRATCH_BYTES \(16 \* 1024 \* 1024\)", text)
    for N in (4 * 1024 * 1024 + 1, 4 * 1024 * 1024 + 8, 1 << 23):
        assert bwd_noalloc(N=N, M=1) == SHAPE, N


@pytest.mark.parametrize("kwargs,status", [
    (dict(M=-1), SHAPE),
    (dict(N=0), SHAPE),
    (dict(dtype=7), DTYPE),
    (dict(dtype=3), DTYPE),                # not a dtype code
    (dict(dw=None), NULL),
    (dict(x=None), NULL),
    (dict(dy=None), NULL),
    (dict(rstd=None), NULL),
    (dict(dx=None), NULL),
    (dict(w=None), NULL),
    (dict(offset=float("inf")), SCALAR),
    (dict(dx=X), OVERLAP),                 # dx on x
    (dict(dx=DY + 16), OVERLAP),           # dx partially over dy
    (dict(dw=X + 64), OVERLAP),            # dw inside x
    (dict(dw=DX + 64), OVERLAP),           # dw inside dx
    (dict(ws=None), NULL),
    (dict(ws_bytes=100), SHAPE),           # workspace too small
    (dict(ws=DX + 32), OVERLAP),           # workspace over dx
    (dict(ws=WS + 4), PLAN),               # workspace not 16-byte aligned
])
def test_bwd_argument_errors(kwargs, status):
    assert bwd(**kwargs) == status, lib.rmsnorm_last_error().decode()
    assert lib.rmsnorm_last_error().decode() != ""


@pytest.mark.parametrize("N,variant,lanes,vpl", [(128, 1, 32, 1), (512, 1, 64, 2), (4096, 2, 512, 2),
                                               (8192, 2, 1024, 2), (8196, 6, 1024, 3), (8200, 6, 1024, 3),
                                               (24576, 6, 1024, 6), (24580, 3, 0, 0),
                                               (1002, 4, 128, 2), (8189, 4, 1024, 2), (8190, 3, 0, 0)])
def test_bwd_fp32_plans(N, variant, lanes, vpl):
    """fp32 rows: four elements per 16-byte vector, so the wave family holds 512 and the block
    family 8192 elements, the wide family 24576 and the shifted family rows of up to 2048 chunks;
    wider rows take the generic kernel."""
    p = bnd.Plan()
    assert lib.rmsnorm_bwd_plan_query(4096, N, FP32, None, None, None, 256, ctypes.byref(p)) == OK
    assert p.variant == variant
    if variant != 3:
        assert (p.vec_elems, p.lanes_per_row, p.vectors_per_lane) == (4, lanes, vpl)


def test_bwd_plans_and_workspace():
    def plan(M, N, dtype=BF16, x=None):
        p = bnd.Plan()
        st = lib.rmsnorm_bwd_plan_query(M, N, dtype, x, None, None, 256, ctypes.byref(p))
        assert st == OK, lib.rmsnorm_last_error().decode()
        return p

    def ws(M, N, dtype=BF16, x=None):
        b = ctypes.c_int64()
        assert lib.rmsnorm_bwd_workspace_size(M, N, dtype, x, None, None, ctypes.byref(b)) == OK
        return b.value

    # grid = min(trips, 4096 waves' worth of workgroups, 3M/32); prefetch when a workgroup makes several
    # trips and the grid is at most one workgroup per unit
    p = plan(16384, 512)
    assert (p.variant, p.lanes_per_row, p.vectors_per_lane, p.block_threads) == (bnd.VARIANT_WAVE, 64, 1, 1024)
    assert (p.row_slots, p.grid, p.rows_per_trip, p.trips, p.prefetch) == (1, 256, 16, 4, 1)
    assert ws(16384, 512) == 256 * 512 * 4
    p = plan(262144, 128, FP16)
    assert (p.variant, p.lanes_per_row, p.row_slots, p.grid, p.prefetch) == (bnd.VARIANT_WAVE, 16, 2, 256, 1)
    for n in (16, 40, 64):                 # rows of at most 8 vectors: 8-lane segments, two slots
        p = plan(262144, n)
        assert (p.variant, p.lanes_per_row, p.row_slots, p.grid, p.prefetch) == (bnd.VARIANT_WAVE, 8, 2, 256, 1)
        assert p.rows_per_trip == 256
    p = plan(32768, 8192)
    assert (p.variant, p.block_threads, p.vectors_per_lane, p.grid) == (bnd.VARIANT_BLOCK, 512, 2, 512)
    assert p.prefetch == 0 and ws(32768, 8192) == 512 * 8192 * 4      # two workgroups per unit: no prefetch
    p = plan(8192, 3000)                  # rows of 256 threads, four to a workgroup, next trip ahead
    assert (p.variant, p.block_threads, p.lanes_per_row, p.row_slots, p.vectors_per_lane) == \
        (bnd.VARIANT_BLOCK, 1024, 256, 4, 2)
    assert (p.rows_per_trip, p.grid, p.prefetch, p.trips) == (4, 256, 1, 8)
    assert ws(8192, 3000) == 256 * 3000 * 4
    p = plan(100, 2048)                   # 25 trips of 4 rows, 3M/32 = 9 workgroups
    assert (p.row_slots, p.grid, p.prefetch) == (4, 9, 1)
    p = plan(4096, 4096, FP32)            # 3M/32 = 384 rounds down to whole CUs: 256, next row ahead
    assert (p.block_threads, p.row_slots, p.grid, p.prefetch) == (512, 1, 256, 1)
    p = plan(4096, 16384, FP16)
    assert (p.variant, p.block_threads, p.vectors_per_lane, p.grid, p.prefetch) == (bnd.VARIANT_BLOCK, 1024, 2, 256, 1)
    assert plan(64, 8192).grid == 6                              # 3M/32 bounds the workspace traffic
    p = plan(10, 16392)                                          # wider than registers hold: two passes
    assert (p.variant, p.block_threads, p.vectors_per_lane, p.prefetch) == (bnd.VARIANT_WIDE, 1024, 3, 0)
    assert (plan(4096, 32768).variant, plan(4096, 32768).vectors_per_lane) == (bnd.VARIANT_WIDE, 4)
    assert plan(10, 32776).variant == bnd.VARIANT_GENERIC      # wider than the 16-byte kernels hold
    assert plan(10, 511).variant == bnd.VARIANT_SHIFTED_WAVE      # 65 chunks: two per lane of a wave
    assert plan(10, 1018).variant == bnd.VARIANT_SHIFTED           # 129 chunks: one row per workgroup
    assert plan(10, 512, x=A + 2).variant == bnd.VARIANT_GENERIC
    assert plan(3, 512).grid == 1                               # 3 rows fit one 8-wave workgroup
    assert ws(0, 512) == 0
    for M, N in ((16384, 512), (32768, 8192), (77, 3000), (5, 7)):
        p = plan(M, N)
        cover = p.variant == bnd.VARIANT_GENERIC or p.lanes_per_row * p.vectors_per_lane * 8 >= N
        assert cover and p.grid * p.trips * p.rows_per_trip >= M


def test_bwd_plans_that_do_not_fit_are_rejected():
    good = bnd.Plan()
    assert lib.rmsnorm_bwd_plan_query(100, 512, BF16, None, None, None, 256, ctypes.byref(good)) == OK
    for p in (good.copy(row_slots=4, prefetch=1),   # the 4-slot wave shape has no prefetching form
              good.copy(prefetch=2), good.copy(xcd_group=2), good.copy(max_blocks_per_cu=4),
              good.copy(vectors_per_lane=3), good.copy(block_threads=1024, lanes_per_row=16, row_slots=1,
                                                       vectors_per_lane=1),
              good.copy(variant=bnd.VARIANT_BLOCK, block_threads=64, vectors_per_lane=4)):
        st = lib.rmsnorm_bwd_with_plan(X, W, DY, R, DX, DW, 100, 512, 0.0, BF16, ctypes.byref(p), WS,
                                       1 << 24, None)
        assert st == PLAN, (p.as_dict(), lib.rmsnorm_last_error().decode())


# ---------------------------------------------------------------------------
# Tuned dispatch and plan validation (host only)
# ---------------------------------------------------------------------------
@pytest.fixture
def clean_tuned():
    bnd.clear_tuned()
    yield
    bnd.clear_tuned()


def test_plan_validate_matches_what_launches_accept():
    p = bnd.plan_query(16384, 512, "bf16", cu_count=256)
    v = bnd.plan_validate(16384, 512, "bf16", p.copy(lanes_per_row=64, vectors_per_lane=1, row_slots=2, grid=2048),
                          cu_count=256)
    assert (v.rows_per_trip, v.trips, v.resident_grid) == (8, 1, 2048)
    assert bnd.plan_validate(16384, 512, "bf16", p.copy(vectors_per_lane=7), cu_count=256) is None
    assert bnd.plan_validate(16384, 512, "bf16", p, x_ptr=A + 2, cu_count=256) is None      # unaligned x
    with pytest.raises(bnd.RmsnormError):
        bnd.plan_validate(16384, 0, "bf16", p, cu_count=256)                                  # bad shape raises


def test_bwd_plan_validate_fills_the_derived_fields():
    p = bnd.bwd_plan_query(8192, 3000, "bf16", cu_count=256)
    assert bnd.bwd_plan_validate(8192, 3000, "bf16", p, cu_count=256).as_dict() == p.as_dict()
    v = bnd.bwd_plan_validate(8192, 3000, "bf16", p.copy(row_slots=2, block_threads=512, grid=512), cu_count=256)
    assert (v.lanes_per_row, v.rows_per_trip, v.trips) == (256, 2, 8)     # 8192 rows / (512 x 2 a trip)
    assert bnd.bwd_plan_validate(8192, 3000, "bf16", p.copy(row_slots=3), cu_count=256) is None
    assert bnd.bwd_plan_validate(8192, 3000, "bf16", p.copy(xcd_group=8), cu_count=256) is None
    assert bnd.bwd_plan_validate(8192, 3000, "bf16", p.copy(block_threads=128, row_slots=1), cu_count=256) is None  # 2048 < 3000
    with pytest.raises(bnd.RmsnormError):
        bnd.bwd_plan_validate(8192, 0, "bf16", p, cu_count=256)                               # bad shape raises


def test_tuned_plan_replaces_the_rule_for_exactly_its_shape(clean_tuned):
    rule = bnd.plan_query(16384, 512, "bf16", cu_count=256)
    tuned = rule.copy(lanes_per_row=64, vectors_per_lane=1, row_slots=2, block_threads=128, grid=4096)
    bnd.set_tuned(16384, 512, "bf16", tuned)
    assert bnd.tuned_count() == 1
    got = bnd.plan_query(16384, 512, "bf16", cu_count=256)
    assert (got.row_slots, got.block_threads, got.grid) == (2, 128, 4096)
    assert bnd.plan_query(16384, 512, "fp16", cu_count=256).row_slots == rule.row_slots   # other dtype
    assert bnd.plan_query(16385, 512, "bf16", cu_count=256).block_threads == rule.block_threads
    # a tuned plan that does not fit the call's pointers falls back to the rule, without an error
    fb = bnd.plan_query(16384, 512, "bf16", x_ptr=A + 2, cu_count=256)
    assert fb.variant == bnd.VARIANT_GENERIC and lib.rmsnorm_last_error() == b""
    bnd.set_tuned(16384, 512, "bf16", tuned.copy(row_slots=4, block_threads=256, grid=1024))  # replace
    assert bnd.tuned_count() == 1 and bnd.plan_query(16384, 512, "bf16", cu_count=256).row_slots == 4
    bnd.clear_tuned()
    assert bnd.tuned_count() == 0
    assert bnd.plan_query(16384, 512, "bf16", cu_count=256).block_threads == rule.block_threads


def test_tuned_plans_are_validated(clean_tuned):
    rule = bnd.plan_query(4096, 512, "bf16", cu_count=256)
    for bad in (rule.copy(vectors_per_lane=7), rule.copy(block_threads=96), rule.copy(grid=0),
                rule.copy(lanes_per_row=16)):                  # 16 lanes x 1 vector do not cover 512 columns
        with pytest.raises(bnd.RmsnormError) as e:
            bnd.set_tuned(4096, 512, "bf16", bad)
        assert e.value.status == PLAN
    assert lib.rmsnorm_plan_set_tuned(0, 512, BF16, ctypes.byref(rule)) == SHAPE
    assert lib.rmsnorm_plan_set_tuned(4096, 512, BF16, None) == NULL
    assert bnd.tuned_count() == 0


def test_load_tuned_reads_the_tuner_format(clean_tuned, tmp_path):
    import json
    rule = bnd.plan_query(8192, 3000, "bf16", cu_count=256)
    plan = {f: getattr(rule, f) for f in bnd.PLAN_FIELDS}
    plan["xcd_group"] = 4
    path = tmp_path / "t.json"
    path.write_text(json.dumps({"device": "test", "plans": [{"M": 8192, "N": 3000, "dtype": "bf16", "plan": plan}]}))
    assert bnd.load_tuned(str(path)) == 1
    assert bnd.plan_query(8192, 3000, "bf16", cu_count=256).xcd_group == 4


def test_tuner_search_space_is_valid_and_contains_the_rule():
    tune = pytest.importorskip("memory_bound_row_rmsnorm_amd.tune")
    for M, N, dtype in ((16384, 512, "bf16"), (32768, 8192, "bf16"), (8192, 3000, "bf16"), (262144, 128, "fp16"),
                        (4096, 16384, "fp16"), (100, 1000, "bf16")):
        cands = tune.candidates(M, N, dtype, quick=True)
        keys = {tuple(getattr(p, f) for f in bnd.PLAN_FIELDS) for p in cands}
        assert len(keys) == len(cands) > 3
        rule = bnd.plan_query(M, N, dtype, cu_count=256)
        assert all(bnd.plan_validate(M, N, dtype, p, cu_count=256) is not None for p in cands)
        fam = {p.variant for p in cands}
        assert rule.variant in fam and bnd.VARIANT_GENERIC in fam


# ---------------------------------------------------------------------------
# Strided / batched layouts, optional rstd, fp32 (host only)
# ---------------------------------------------------------------------------
def fwd_ex(x=A, w=A + 0x1000000, y=A + 0x2000000, rstd=A + 0x3000000, M=4, N=512, dtype=BF16,
           layout=None, plan=None):
    lay = ctypes.byref(bnd.Layout(*layout)) if layout is not None else None
    return lib.rmsnorm_fwd_ex(x, w, y, rstd, M, N, 1e-6, 0.0, dtype, lay,
                              ctypes.byref(plan) if plan is not None else None, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(layout=(0, -1, 0, 512, 0)), SHAPE),               # negative stride
    (dict(layout=(3, 512, 4096, 512, 4096)), SHAPE),        # M = 4 is not a multiple of 3 rows
    (dict(layout=(0, 512, 0, 256, 0)), SHAPE),              # y rows overlap each other
    (dict(layout=(2, 512, 512, 512, 512)), SHAPE),          # y batches overlap (neither order is disjoint)
    (dict(x=None), NULL),
    (dict(dtype=3), DTYPE),
    (dict(y=A, layout=(0, 1024, 0, 512, 0)), OVERLAP),       # in place needs the same layout
    (dict(y=A + 0x1000, layout=(0, 1024, 0, 1024, 0)), OVERLAP),   # spans overlap (x spans 7168 bytes)
    (dict(rstd=A + 3 * 1024 * 2 + 16, layout=(0, 1024, 0, 512, 0)), OVERLAP),  # rstd inside x's span
])
def test_fwd_ex_argument_errors(kwargs, status):
    assert fwd_ex(**kwargs) == status, lib.rmsnorm_last_error().decode()
    assert lib.rmsnorm_last_error().decode() != ""


def test_fwd_ex_accepts_null_rstd_and_valid_layouts():
    # valid calls get past every check: on a machine without a GPU they stop at the device
    for kw in (dict(rstd=None), dict(layout=(0, 1024, 0, 512, 0)), dict(y=A, layout=(0, 1024, 0, 1024, 0)),
               dict(layout=(2, 1024, 4096, 512, 1024)),       # batch-major y
               dict(layout=(2, 512, 2048, 1024, 512)),        # row-major interleaved y
               dict(layout=(0, 0, 0, 512, 0)),                # x broadcast: every row reads row 0
               dict(dtype=2)):
        st = fwd_ex(**kw)
        assert st in (HIP, DEVICE), (kw, st, lib.rmsnorm_last_error().decode())


def query_ex(M, N, dtype="bf16", x=A, w=A, y=A, layout=None):
    p = bnd.Plan()
    lay = ctypes.byref(bnd.Layout(*layout)) if layout is not None else None
    st = lib.rmsnorm_plan_query_ex(M, N, bnd.DTYPE_NAMES[dtype], x, w, y, lay, 256, ctypes.byref(p))
    assert st == OK, lib.rmsnorm_last_error().decode()
    return p


def test_layouts_choose_the_vector_kernels_when_rows_stay_aligned():
    assert query_ex(4096, 512, layout=(0, 1024, 0, 512, 0)).variant == bnd.VARIANT_WAVE
    assert query_ex(4096, 512, layout=(0, 516, 0, 512, 0)).variant == bnd.VARIANT_GENERIC   # x rows 8-byte aligned
    # ragged widths on aligned rows: the vector kernels with their tail path
    p = query_ex(4096, 3001, layout=(0, 3008, 0, 3008, 0))
    assert p.variant == bnd.VARIANT_BLOCK and p.block_threads * p.vectors_per_lane * 8 >= 3001
    assert query_ex(4096, 3001).variant == bnd.VARIANT_SHIFTED      # contiguous rows of 3001 are unaligned
    assert query_ex(4096, 3001, layout=(0, 3001, 0, 3002, 0)).variant == bnd.VARIANT_GENERIC   # y differs
    assert query_ex(4096, 100, layout=(0, 104, 0, 104, 0)).variant == bnd.VARIANT_WAVE
    # batches: the plan covers one batch's rows
    p = query_ex(8 * 1000, 512, layout=(1000, 512, 1024 * 512, 512, 1000 * 512))
    assert p.variant == bnd.VARIANT_WAVE and p.grid * p.rows_per_trip >= 1000 and p.grid * p.rows_per_trip < 8000
    # batches that continue the row stride collapse into one batch of all rows
    p = query_ex(8 * 1000, 512, layout=(1000, 512, 1000 * 512, 512, 1000 * 512))
    assert p.grid * p.rows_per_trip >= 8000


def test_fp32_plans():
    p = query_ex(16384, 512, "fp32")
    assert (p.variant, p.vec_elems, p.lanes_per_row, p.vectors_per_lane) == (bnd.VARIANT_WAVE, 4, 64, 2)
    p = query_ex(32768, 8192, "fp32")
    assert (p.variant, p.vec_elems, p.block_threads, p.vectors_per_lane) == (bnd.VARIANT_BLOCK, 4, 1024, 2)
    p = query_ex(4, 24576, "fp32")
    assert (p.variant, p.vectors_per_lane) == (bnd.VARIANT_BLOCK, 6)
    assert query_ex(4, 24576, "bf16").variant == bnd.VARIANT_BLOCK          # 1024 x 3 vectors of 8
    assert query_ex(4, 45056, "bf16").variant == bnd.VARIANT_WIDE           # wider than 1024 x 5 x 8
    assert query_ex(4, 130, "fp32", layout=(0, 132, 0, 132, 0)).variant == bnd.VARIANT_WAVE


def test_widest_instances_refuse_ragged_widths():
    # fp32 1024 x 6 has no tail path: a ragged row that needs it takes the wide kernel, which has one
    assert query_ex(4, 24576 - 3, "fp32", layout=(0, 24576, 0, 24576, 0)).variant == bnd.VARIANT_WIDE
    assert query_ex(4, 24576, "fp32").vectors_per_lane == 6
    assert query_ex(4, 40960 - 3, layout=(0, 40960, 0, 40960, 0)).vectors_per_lane == 5   # bf16 1024 x 5 has one
    p = bnd.plan_query(4, 24576, "fp32", cu_count=256)
    ragged = bnd.plan_validate(4, 24573, "fp32", p, cu_count=256)
    assert ragged is None                                   # an explicit plan is refused, not run wrong


# ---------------------------------------------------------------------------
# Backward with layouts (host checks and plans; no kernel runs)
# ---------------------------------------------------------------------------
def bwd_ex_status(M, N, lay, dtype=BF16, x=A, dy=None, dx=None, ws_bytes=1 << 30):
    dy = dy if dy is not None else A + 0x40000000
    dx = dx if dx is not None else A + 0x80000000
    return lib.rmsnorm_bwd_ex(x, A + 0xC0000000, dy, A + 0xD0000000, dx, A + 0xE0000000, M, N, 0.0, dtype,
                              ctypes.byref(lay) if lay is not None else None, None, A + 0xF0000000, ws_bytes, None)


@pytest.mark.parametrize("lay,M,N,status", [
    (bnd.BwdLayout(7, 64, 0, 64, 0, 64, 0), 64, 64, SHAPE),              # M not a multiple of rows
    (bnd.BwdLayout(0, 64, 0, 64, 0, 32, 0), 64, 64, SHAPE),              # dx rows overlap
    (bnd.BwdLayout(4, 64, 256, 64, 256, 64, 128), 64, 64, SHAPE),        # dx batches overlap
    (bnd.BwdLayout(0, -1, 0, 64, 0, 64, 0), 64, 64, SHAPE),              # negative stride
    (bnd.BwdLayout(2, 64, 256, 64, 256, 64, 256), 1 << 31, 64, SHAPE),   # several batches and M >= 2^31
])
def test_bwd_ex_layout_errors(lay, M, N, status):
    assert bwd_ex_status(M, N, lay) == status, lib.rmsnorm_last_error().decode()
    assert lib.rmsnorm_last_error().decode() != ""


def test_bwd_ex_in_place_needs_the_same_layout():
    lay = bnd.BwdLayout(0, 512, 0, 1024, 0, 512, 0)
    assert bwd_ex_status(64, 512, lay, dy=A + 0x40000000, dx=A + 0x40000000) == OVERLAP
    lay = bnd.BwdLayout(0, 512, 0, 1024, 0, 1024, 0)
    st = bwd_ex_status(64, 512, lay, dy=A + 0x40000000, dx=A + 0x40000000)
    assert st == HIP, lib.rmsnorm_last_error().decode()          # accepted: fails only at the device
    assert bwd_ex_status(64, 512, bnd.BwdLayout(0, 512, 0, 512, 0, 512, 0), dx=A + 16) == OVERLAP   # dx over x


def bwd_plan_ex(M, N, lay, dtype=BF16, x=A, w=A, dy=A, dx=A):
    p = bnd.Plan()
    st = lib.rmsnorm_bwd_plan_query_ex(M, N, dtype, x, w, dy, dx, ctypes.byref(lay) if lay is not None else None,
                                       256, ctypes.byref(p))
    assert st == OK, lib.rmsnorm_last_error().decode()
    return p


def test_bwd_ex_plans():
    contiguous = bwd_plan_ex(4096, 512, None)
    assert bwd_plan_ex(4096, 512, bnd.BwdLayout(0, 512, 0, 512, 0, 512, 0)).as_dict() == contiguous.as_dict()
    # a strided view that keeps rows aligned still takes the vector kernels
    p = bwd_plan_ex(4096, 512, bnd.BwdLayout(32, 1536, 32 * 1536, 512, 32 * 512, 2048, 32 * 2048))
    assert p.variant == bnd.VARIANT_WAVE and p.as_dict() == contiguous.as_dict()
    # a row stride that breaks 16-byte alignment takes the generic kernel
    assert bwd_plan_ex(4096, 512, bnd.BwdLayout(0, 516, 0, 512, 0, 512, 0)).variant == bnd.VARIANT_GENERIC
    assert bwd_plan_ex(4096, 512, bnd.BwdLayout(32, 512, 32 * 512 + 4, 512, 32 * 512, 512, 32 * 512)).variant == \
        bnd.VARIANT_GENERIC
    b = ctypes.c_int64()
    lay = bnd.BwdLayout(32, 1536, 32 * 1536, 512, 32 * 512, 2048, 32 * 2048)
    assert lib.rmsnorm_bwd_workspace_size_ex(4096, 512, BF16, A, A, A, A, ctypes.byref(lay), ctypes.byref(b)) == OK
    assert b.value == p.grid * 512 * 4


def test_bwd_shifted_plans():
    """Rows off a 16-byte boundary take the shifted row pass when x, dy and dx sit equally far past
    a boundary on every row and w is aligned: the fewest threads (64 to 1024) holding the row's
    chunks at most 2 per thread, rows of 16 to 2048 chunks."""
    p = bwd_plan_ex(8192, 3001, None)
    assert (p.variant, p.block_threads, p.vectors_per_lane, p.vec_elems) == (bnd.VARIANT_SHIFTED, 256, 2, 8)
    assert (p.lanes_per_row, p.rows_per_trip, p.grid, p.prefetch) == (256, 1, 768, 0)
    # 1025 chunks: 512 x 3 when the rows fill two 512-thread workgroups per unit, else 1024 x 2
    p = bwd_plan_ex(32768, 8191, None)
    assert (p.variant, p.block_threads, p.vectors_per_lane, p.grid, p.prefetch) == \
        (bnd.VARIANT_SHIFTED, 512, 3, 512, 0)
    p = bwd_plan_ex(4096, 8191, None)
    assert (p.variant, p.block_threads, p.vectors_per_lane, p.grid, p.prefetch) == \
        (bnd.VARIANT_SHIFTED, 1024, 2, 256, 1)
    assert (bwd_plan_ex(32768, 12281, None).block_threads, bwd_plan_ex(32768, 12282, None).block_threads) == \
        (512, 1024)                                # 1536 and 1537 chunks
    # rows of at most 128 chunks: a row per 8/16/32/64-lane segment, one chunk per lane (two per lane
    # of a 64-lane wave above 64 chunks)
    p = bwd_plan_ex(100, 17, None)                 # 3 chunks
    assert (p.variant, p.lanes_per_row, p.vectors_per_lane, p.row_slots, p.block_threads) == \
        (bnd.VARIANT_SHIFTED_WAVE, 8, 1, 1, 1024)
    # 5-6 chunks: eight rows per wave, up to 32 waves per compute unit (512 workgroups)
    p = bwd_plan_ex(262144, 36, None)
    assert (p.lanes_per_row, p.row_slots, p.rows_per_trip, p.grid, p.prefetch) == (8, 1, 128, 512, 0)
    # 13 chunks: one slot of four rows per wave, up to 64 waves per compute unit (1024 workgroups)
    p = bwd_plan_ex(262144, 100, None)
    assert (p.lanes_per_row, p.row_slots, p.rows_per_trip, p.grid, p.prefetch) == (16, 1, 64, 1024, 0)
    p = bwd_plan_ex(16384, 249, None)              # 32 chunks: 512 trips, one per workgroup
    assert (p.variant, p.lanes_per_row, p.row_slots, p.grid) == (bnd.VARIANT_SHIFTED_WAVE, 32, 1, 512)
    p = bwd_plan_ex(262144, 257, None)             # 33 chunks: a row per wave, two slots
    assert (p.variant, p.lanes_per_row, p.row_slots, p.grid, p.prefetch) == (bnd.VARIANT_SHIFTED_WAVE, 64, 2, 256, 0)
    p = bwd_plan_ex(16384, 505, None)              # 64 chunks: one per lane
    assert (p.variant, p.lanes_per_row, p.vectors_per_lane) == (bnd.VARIANT_SHIFTED_WAVE, 64, 1)
    # 65 to 128 chunks: a row per wave, two chunks per lane, one slot
    for n in (506, 513, 1001, 1017):               # 65, 65, 126 and 128 chunks
        p = bwd_plan_ex(16384, n, None)
        assert (p.variant, p.lanes_per_row, p.vectors_per_lane, p.row_slots, p.prefetch, p.grid) == \
            (bnd.VARIANT_SHIFTED_WAVE, 64, 2, 1, 0, 256), n
    p = bwd_plan_ex(16384, 1018, None)             # 129 chunks: one row per workgroup, two per thread
    assert (p.variant, p.block_threads, p.vectors_per_lane) == (bnd.VARIANT_SHIFTED, 128, 2)
    assert bwd_plan_ex(16, 16377, None).variant == bnd.VARIANT_SHIFTED      # 2048 chunks
    assert bwd_plan_ex(16, 16378, None).variant == bnd.VARIANT_GENERIC      # 2049
    assert bwd_plan_ex(100, 15, None).variant == bnd.VARIANT_GENERIC        # shorter than 16 elements
    assert bwd_plan_ex(100, 16, None).variant == bnd.VARIANT_WAVE
    # x, dy and dx must share the distance past a boundary; w must be aligned
    assert bwd_plan_ex(100, 3001, None, dx=A + 2).variant == bnd.VARIANT_GENERIC
    assert bwd_plan_ex(100, 3001, None, dy=A + 4).variant == bnd.VARIANT_GENERIC
    assert bwd_plan_ex(100, 3001, None, w=A + 2).variant == bnd.VARIANT_GENERIC
    assert bwd_plan_ex(100, 3001, None, x=A + 1, dy=A + 1, dx=A + 1).variant == bnd.VARIANT_GENERIC
    # aligned rows on equally offset bases are shifted too (every row one element in: 65 chunks)
    p = bwd_plan_ex(100, 512, None, x=A + 2, dy=A + 0x100002, dx=A + 0x200002)
    assert (p.variant, p.lanes_per_row, p.vectors_per_lane) == (bnd.VARIANT_SHIFTED_WAVE, 64, 2)
    assert bwd_plan_ex(100, 2048, None, x=A + 2, dy=A + 0x100002, dx=A + 0x200002).variant == \
        bnd.VARIANT_SHIFTED
    # strides may differ by whole 16-byte vectors, not by less
    lay = bnd.BwdLayout(0, 3001, 0, 3009, 0, 3017, 0)
    assert bwd_plan_ex(100, 3001, lay).variant == bnd.VARIANT_SHIFTED
    lay = bnd.BwdLayout(0, 3001, 0, 3002, 0, 3001, 0)
    assert bwd_plan_ex(100, 3001, lay).variant == bnd.VARIANT_GENERIC
    lay = bnd.BwdLayout(4, 3001, 4 * 3001 + 8, 3001, 4 * 3001 + 8, 3001, 4 * 3001 + 1)
    assert bwd_plan_ex(100, 3001, lay).variant == bnd.VARIANT_GENERIC    # batch strides out of phase
    lay = bnd.BwdLayout(4, 3001, 4 * 3001 + 8, 3001, 4 * 3001 + 16, 3001, 4 * 3001 + 24)
    assert bwd_plan_ex(100, 3001, lay).variant == bnd.VARIANT_SHIFTED


def test_bwd_shifted_plans_that_do_not_fit_are_rejected():
    good = bwd_plan_ex(100, 3001, None)
    base = dict(x=A, w=A, dy=A + 0x10000000, dx=A + 0x20000000)
    sw = bwd_plan_ex(100, 300, None)
    for p, N in ((good.copy(vectors_per_lane=3), 3001),                   # no such instance
                 (sw.copy(lanes_per_row=32), 300),                         # 32 lanes x 1 chunk < 39
                 (sw.copy(lanes_per_row=128), 300),
                 (sw.copy(lanes_per_row=32, vectors_per_lane=2), 300),     # two chunks only with 64 lanes
                 (sw.copy(vectors_per_lane=2, row_slots=2, prefetch=1), 300),  # no such instance
                 (sw.copy(row_slots=4, prefetch=1, lanes_per_row=16), 100),  # no such instance
                 (sw, 512),                                                # aligned rows
                 (good.copy(block_threads=128, lanes_per_row=128), 3001),  # 128 x 2 chunks < 376
                 (good.copy(prefetch=2), 3001),
                 (good, 3000)):                                            # aligned rows: not shifted
        st = lib.rmsnorm_bwd_with_plan(base["x"], base["w"], base["dy"], A + 0x30000000, base["dx"],
                                       A + 0x40000000, 100, N, 0.0, BF16, ctypes.byref(p), A + 0x50000000,
                                       1 << 24, None)
        assert st == PLAN, (p.as_dict(), N, lib.rmsnorm_last_error().decode())


def test_bwd_wide_plans_that_do_not_fit_are_rejected():
    good = bnd.Plan()
    assert lib.rmsnorm_bwd_plan_query(100, 24576, BF16, None, None, None, 256, ctypes.byref(good)) == OK
    assert (good.variant, good.vectors_per_lane, good.grid) == (bnd.VARIANT_WIDE, 3, 9)
    for p, N in ((good.copy(prefetch=1), 24576),                  # no prefetching form
                 (good.copy(vectors_per_lane=5), 24576),          # not compiled for 16-bit data
                 (good.copy(block_threads=512), 24576),           # 512 x 3 vectors < 3072
                 (good, 24580)):                                  # rows not 16-byte aligned
        st = lib.rmsnorm_bwd_with_plan(X, W, DY, R, DX, DW, 100, N, 0.0, BF16, ctypes.byref(p), WS, 1 << 24, None)
        assert st == PLAN, (p.as_dict(), N, lib.rmsnorm_last_error().decode())


# ---------------------------------------------------------------------------
# The instance a launch runs: the exact-width wave form where the call fits it.
# ---------------------------------------------------------------------------
EXACT_WIDTHS = [("bf16", 128), ("bf16", 256), ("bf16", 512), ("bf16", 1024), ("fp16", 512), ("fp32", 64),
                ("fp32", 512)]


@pytest.mark.parametrize("dtype,N", EXACT_WIDTHS)
def test_exact_widths_launch_the_exact_wave_form(dtype, N):
    for M in (1, 7, 16384, 262144):
        q = bnd.kernel_query(M, N, dtype, A, A, A + (1 << 30), resources=False)
        assert q["kernel"].startswith("rmsnorm_wave_exact<"), (M, N, dtype, q)
        plan = bnd.plan_query(M, N, dtype, cu_count=256)
        shape = f",{plan.lanes_per_row},{plan.vectors_per_lane},{plan.row_slots},{plan.block_threads // 64}>"
        assert q["kernel"].endswith(shape), (q, plan.as_dict())


def test_other_launches_keep_the_general_instance():
    M, N = 16384, 512
    base = bnd.plan_query(M, N, "bf16", cu_count=256)

    def name(plan=None, n=N, m=M):
        return bnd.kernel_query(m, n, "bf16", A, A, A + (1 << 30), plan=plan, resources=False)["kernel"]

    assert name() == "rmsnorm_wave_exact<BF16,32,2,4,4>"
    lanes64 = base.copy(lanes_per_row=64, vectors_per_lane=1, grid=1024)
    assert name(lanes64) == "rmsnorm_wave_exact<BF16,64,1,4,4>"
    # a persistent grid, a remap, prefetching: the general instance
    assert name(base.copy(grid=64)).startswith("rmsnorm_wave<")
    assert name(base.copy(xcd_group=2)).startswith("rmsnorm_wave<")
    assert name(lanes64.copy(prefetch=1)).startswith("rmsnorm_wave<")
    # a width below the plan's full row (masked columns); a single ragged row (a tail vector;
    # several ragged contiguous rows start unaligned and take a shifted kernel)
    assert name(n=504).startswith("rmsnorm_wave<")
    assert name(n=500, m=1).startswith("rmsnorm_wave<")
    # no exact form for this segment shape or workgroup size
    assert name(lanes64.copy(row_slots=8)).startswith("rmsnorm_wave<")
    assert name(base.copy(block_threads=512, grid=512)).startswith("rmsnorm_wave<")
    # the block family has its own exact forms (rows of exactly 1024 vectors here); a width
    # below the plan's full row, a persistent grid or prefetching keep the general instance
    assert name(n=8192) == "rmsnorm_block_exact<BF16,4,256>"
    assert name(n=8000).startswith("rmsnorm_block<")
    blk = bnd.plan_query(M, 8192, "bf16", cu_count=256)
    assert name(blk.copy(grid=1024), n=8192).startswith("rmsnorm_block<")
    assert name(blk.copy(grid=M + 1), n=8192).startswith("rmsnorm_block<")   # a workgroup past the rows
    assert name(blk.copy(prefetch=1, grid=1024), n=8192).startswith("rmsnorm_block<")
    with pytest.raises(bnd.RmsnormError):
        name(m=0)


def test_exact_form_row_limit():
    """The exact form has no loop: it runs while one grid of fewer than 2^32 work-items covers the
    rows (32 rows per 256-thread workgroup at N = 512, well inside its 32-bit row numbers); one
    row more and the grid loops in the general instance."""
    limit = (2 ** 32 - 1) // 256 * 32
    assert limit < (1 << 31) - (1 << 16)
    below = bnd.kernel_query(limit, 512, "bf16", A, A, A + (1 << 40), resources=False)["kernel"]
    at = bnd.kernel_query(limit + 1, 512, "bf16", A, A, A + (1 << 40), resources=False)["kernel"]
    assert below.startswith("rmsnorm_wave_exact<"), below
    assert at.startswith("rmsnorm_wave<"), at


def test_exact_block_form_is_planned_only_where_it_fits():
    """256 threads x 8 vectors exist only as the exact-width block form: contiguous rows of
    exactly 16384 16-bit elements in one batch, one trip."""
    q = bnd.kernel_query(4096, 16384, "fp16", A, A, A + (1 << 30), resources=False)
    assert q["kernel"] == "rmsnorm_block_exact<FP16,8,256>", q
    base = bnd.plan_query(4096, 16384, "bf16", cu_count=256)
    assert (base.block_threads, base.vectors_per_lane) == (256, 8)
    # a persistent grid or a ragged width cannot take it
    assert bnd.plan_validate(4096, 16384, "bf16", base, cu_count=256) is not None
    assert bnd.plan_validate(4096, 16384, "bf16", base.copy(grid=1024), cu_count=256) is None
    assert bnd.plan_validate(4096, 16384, "bf16", base.copy(grid=4097), cu_count=256) is None   # exactly M
    assert bnd.plan_validate(4096, 16000, "bf16", base, cu_count=256) is None
    # rows of a strided layout: the rule plans the 1024-thread block family instead
    lay = bnd.Layout(0, 20000, 0, 16384, 0)
    p = bnd.Plan()
    assert lib.rmsnorm_plan_query_ex(4096, 16384, BF16, A, A, A + (1 << 30), bnd.ctypes.byref(lay), 256,
                                     bnd.ctypes.byref(p)) == OK
    assert (p.block_threads, p.vectors_per_lane) == (1024, 2)
    # fp32 keeps its rule
    assert bnd.plan_query(4096, 8192, "fp32", cu_count=256).vectors_per_lane != 8


@pytest.mark.parametrize("dtype,N", [("bf16", 8192), ("fp16", 8192), ("fp32", 4096)])
def test_exact_block_form_256x4(dtype, N):
    """Contiguous rows of exactly 1024 vectors run the 256 x 4 exact-width block form, capped at
    3 workgroups per CU; a strided layout or several batches keep the block family and its cap."""
    code = {"bf16": BF16, "fp16": FP16, "fp32": FP32}[dtype]
    q = bnd.kernel_query(32768, N, dtype, A, A, A + (1 << 31), resources=False)
    assert q["kernel"] == f"rmsnorm_block_exact<{ {'bf16': 'BF16', 'fp16': 'FP16', 'fp32': 'F32'}[dtype] },4,256>", q
    p = host_plan(32768, N, code)
    assert (p.block_threads, p.vectors_per_lane, p.max_blocks_per_cu) == (256, 4, 3)
    lay = bnd.Layout(0, N + 64, 0, N, 0)
    ps = bnd.Plan()
    assert lib.rmsnorm_plan_query_ex(32768, N, code, A, A, A + (1 << 31), bnd.ctypes.byref(lay), 256,
                                     bnd.ctypes.byref(ps)) == OK
    assert (ps.block_threads, ps.vectors_per_lane, ps.max_blocks_per_cu) == (256, 4, 4)
