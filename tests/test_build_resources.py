"""Every compiled kernel instance keeps within its register budget: no scratch and no spilled
registers, read from the compiler's resource remarks that the build writes next to the library
(``memory_bound_row_rmsnorm_amd/_build/kernel_resources.txt``).  CPU only."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REMARKS = os.path.join(ROOT, "memory_bound_row_rmsnorm_amd", "_build", "kernel_resources.txt")


def parse(path):
    kernels, cur = {}, None
    with open(path) as f:
        for line in f:
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                cur = m.group(1)
                kernels[cur] = {}
                continue
            m = re.search(r"remark:\s+(VGPRs|VGPRs Spill|SGPRs Spill|ScratchSize \[bytes/lane\]|"
                          r"Occupancy \[waves/SIMD\]): (\d+)", line)
            if cur and m:
                kernels[cur][m.group(1)] = int(m.group(2))
    return kernels


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(REMARKS):
        pytest.skip("library not built here (the build writes the remarks)")
    k = parse(REMARKS)
    assert k, "no kernel remarks found"
    return k


def test_every_family_is_compiled(kernels):
    names = " ".join(kernels)
    for family in ("rmsnorm_wave", "rmsnorm_block", "rmsnorm_wide", "rmsnorm_shifted", "rmsnorm_shifted_wave",
                   "rmsnorm_generic", "rmsnorm_bwd_wave", "rmsnorm_bwd_block", "rmsnorm_bwd_shifted", "rmsnorm_bwd_generic",
                   "rmsnorm_dw_reduce"):
        assert family in names, family


def test_no_scratch_and_no_spills(kernels):
    bad = {name: r for name, r in kernels.items()
           if r.get("ScratchSize [bytes/lane]", 0) or r.get("VGPRs Spill", 0) or r.get("SGPRs Spill", 0)}
    assert not bad, bad


def test_register_budget_of_1024_thread_workgroups(kernels):
    # every kernel is launched with up to 1024 threads: 128 VGPRs at most
    over = {name: r["VGPRs"] for name, r in kernels.items() if r.get("VGPRs", 0) > 128}
    assert not over, over
