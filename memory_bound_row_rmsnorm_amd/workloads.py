"""Seeded synthetic workloads for the row RMSNorm forward.

This module only draws inputs: it holds none of the normalisation's arithmetic
and imports neither the HIP binding nor the oracle, so both sides of a parity
check can take their inputs from it.

Recipe (every workload, every seed):
  1. ``g = torch.Generator('cpu').manual_seed(seed)``
  2. ``zx = torch.randn(M, N, generator=g)`` then ``zw = torch.randn(N, generator=g)``;
     for the outlier-channel workload also ``cols = torch.randperm(N, generator=g)[:k]``
     with ``k = round(0.01 * N)``; for the outlier-entry workload instead
     ``hit = torch.rand(M, N, generator=g) < 0.01``.
  3. ``x = sigma * zx`` (outlier columns, or outlier entries, multiplied by 50,
     in fp32), cast once to the dtype; ``w = w_mean + 0.1 * zw`` cast once to
     the dtype.

The shapes, dtypes, value spreads, eps and offset are those of the row RMSNorm
workloads the pages discuss: the 16384 x 512 bf16 shape measured in "Why cutile's
rmsnorm required full register" (opening report), Llama-style (offset 0) and
Gemma3-style (offset 1) weights from that report's kernel listing, a hidden size
that is not a power of two and a large-magnitude fp16 case whose 16-bit
sum of squares would overflow ("Rmsnorm Kernel Optimization", Common Pitfalls),
and small hidden sizes that call for several rows per program (same page, Key
Optimizations).
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np
import torch

TORCH_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    dtype: str          # "bf16" | "fp16" | "fp32"
    x_sigma: float      # x ~ N(0, sigma^2)
    w_mean: float       # w = w_mean + 0.1 * N(0, 1)
    eps: float
    offset: float
    outlier_channels: bool = False   # 1% of the columns scaled by 50
    outlier_entries: bool = False    # each entry scaled by 50 with probability 0.01

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    def algorithmic_bytes(self) -> int:
        """x read once, y written once, w read once, fp32 rstd written once."""
        s = self.elem_bytes
        return 2 * self.M * self.N * s + self.N * s + 4 * self.M

    def with_rows(self, M: int) -> "Workload":
        return dataclasses.replace(self, M=M)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("rmsnorm_64x512_bf16", 64, 512, "bf16", 1.0, 1.0, 1e-6, 0.0),
        Workload("rmsnorm_16384x512_bf16", 16384, 512, "bf16", 1.0, 1.0, 1e-6, 0.0),
        Workload("rmsnorm_8192x3000_bf16_offset1", 8192, 3000, "bf16", 2.0, 0.0, 1e-6, 1.0),
        Workload("rmsnorm_32768x8192_bf16_outliers", 32768, 8192, "bf16", 1.0, 1.0, 1e-5, 0.0,
                 outlier_channels=True),
        Workload("rmsnorm_32768x8192_bf16_outlier_entries", 32768, 8192, "bf16", 1.0, 1.0, 1e-5, 0.0,
                 outlier_entries=True),
        Workload("rmsnorm_262144x128_fp16", 262144, 128, "fp16", 100.0, 1.0, 1e-6, 0.0),
        Workload("rmsnorm_262144x128_bf16", 262144, 128, "bf16", 1.0, 1.0, 1e-6, 0.0),
        Workload("rmsnorm_4096x16384_fp16", 4096, 16384, "fp16", 100.0, 1.0, 1e-6, 0.0),
    ]
}

HEADLINE = "rmsnorm_16384x512_bf16"


def outlier_count(N: int) -> int:
    return int(round(0.01 * N))


def make_inputs(wl: Workload, seed: int = 0, rows: int | None = None):
    """Draw (x, w) as CPU tensors of the workload's dtype.

    ``rows`` draws only the first ``rows`` rows of the same recipe with the same
    generator state order (x first, then w), so w differs from the full-size
    draw; use it for reduced-size cases, not for sampling a full-size run.
    """
    M = wl.M if rows is None else rows
    g = torch.Generator("cpu").manual_seed(seed)
    zx = torch.randn(M, wl.N, generator=g, dtype=torch.float32)
    zw = torch.randn(wl.N, generator=g, dtype=torch.float32)
    x = zx.mul_(wl.x_sigma)
    if wl.outlier_channels:
        cols = torch.randperm(wl.N, generator=g)[: outlier_count(wl.N)]
        x[:, cols] *= 50.0
    if wl.outlier_entries:
        hit = torch.rand(M, wl.N, generator=g) < 0.01
        x[hit] *= 50.0
    w = zw.mul_(0.1).add_(wl.w_mean)
    td = TORCH_DTYPES[wl.dtype]
    return x.to(td), w.to(td)


def make_grad(wl: Workload, seed: int = 0, rows: int | None = None) -> torch.Tensor:
    """Upstream gradient dy for the backward: N(0, 1) in the workload's dtype,
    from its own generator (seed + 1000003) so it is independent of x and w."""
    M = wl.M if rows is None else rows
    g = torch.Generator("cpu").manual_seed(seed + 1000003)
    return torch.randn(M, wl.N, generator=g, dtype=torch.float32).to(TORCH_DTYPES[wl.dtype])


def fill_normal_(t: torch.Tensor, seed: int, sigma: float = 1.0, mean: float = 0.0,
                 chunk: int = 1 << 26) -> torch.Tensor:
    """Fill ``t`` in place with mean + sigma * N(0, 1), drawn in fp32 on the tensor's own device
    from a generator seeded with ``seed``, ``chunk`` elements at a time, then rounded to t's dtype.
    For tensors too large to draw on the host (several GiB of rows)."""
    g = torch.Generator(device=t.device).manual_seed(seed)
    flat = t.view(-1)
    for i in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - i)
        z = torch.randn(n, generator=g, device=t.device, dtype=torch.float32)
        flat[i:i + n] = z.mul_(sigma).add_(mean)
    return t


def to_bits(t: torch.Tensor) -> np.ndarray:
    """Bit patterns of a CPU 16-bit tensor as a uint16 numpy array (no copy of values)."""
    if t.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"expected a 16-bit float tensor, got {t.dtype}")
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(b: np.ndarray, dtype: str) -> torch.Tensor:
    """CPU tensor of the given 16-bit dtype from uint16 bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(TORCH_DTYPES[dtype])


def sha256_of(t: torch.Tensor) -> str:
    return hashlib.sha256(to_bits(t).tobytes()).hexdigest()
