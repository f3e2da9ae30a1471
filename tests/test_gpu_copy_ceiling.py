"""The copy the benchmark measures the forward against (libcopy_ceiling.so,
bench.py --kernel hip_copy) copies exactly: every run length, workgroup size
and a grid small enough to loop, over sizes that end inside a run."""
from __future__ import annotations

import pytest
import torch

import bench

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.mark.parametrize("serial", [1, 0])
@pytest.mark.parametrize("vpl", [1, 2, 4, 8])
@pytest.mark.parametrize("threads", [64, 256, 1024])
def test_copy_ceiling_copies_exactly(vpl, threads, serial):
    lib = bench.load_copy_ceiling()
    g = torch.Generator(device=DEV).manual_seed(vpl * 1000 + threads)
    for nbytes in (16, 16 * 1000 + 48, (1 << 24) + 16 * 7):
        for grid in (0, 3):
            print("CASE copy", vpl, threads, serial, nbytes, grid, flush=True)
            src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g, device=DEV, dtype=torch.int32)
            dst = torch.full((nbytes // 4 + 8,), 0x5A5A5A5A, device=DEV, dtype=torch.int32)
            st = lib.copy_ceiling_sched(src.data_ptr(), dst.data_ptr(), nbytes, vpl, threads, grid, serial,
                                        torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            assert st == 0
            assert torch.equal(dst[: nbytes // 4], src)
            assert bool((dst[nbytes // 4:] == 0x5A5A5A5A).all()), "wrote past the end"
