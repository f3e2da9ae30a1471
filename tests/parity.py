"""Comparison of GPU results with the oracle.

Acceptance, written here once:
  * y: every element within 1 unit in the last place of the oracle's rounded
    value.  Distances count representable values between two patterns, with
    +0 and -0 equal (the ordered-integer view of a sign-magnitude format).
    Both NaN counts as equal; NaN against a number fails.
  * rstd: |rstd_gpu - rstd_oracle| <= 1e-5 * rstd_oracle.

Why 1 ulp: the kernels compute in fp32 and round once; the oracle computes in
fp64 and rounds once.  The fp32 path is within a few fp32 ulps (about 1e-6
relative) of the exact value, far inside one bf16 (2^-8) or fp16 (2^-11)
ulp, but an exact value that sits within that distance of a rounding midpoint
may round to either neighbour.  So one ulp is the tightest bar any fp32 path
can meet; a bar of 0 ulp would fail on about 1e-4 of the elements.
The rstd bound covers fp32 summation of up to 16384 squares (relative error
below (N/64 + 8) * 2^-24 for the tree the kernels use) plus the hardware
reciprocal square root (about 1 fp32 ulp).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from memory_bound_row_rmsnorm_amd import workloads

Y_ULP_TOL = 1
RSTD_RTOL = 1e-5

NAN_MASK = {"bf16": (0x7F80, 0x007F), "fp16": (0x7C00, 0x03FF)}


def ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def is_nan(bits: np.ndarray, dtype: str) -> np.ndarray:
    e, f = NAN_MASK[dtype]
    return ((bits & e) == e) & ((bits & f) != 0)


def ulp_distance(a: np.ndarray, b: np.ndarray, dtype: str) -> np.ndarray:
    d = np.abs(ordered(a) - ordered(b))
    na, nb = is_nan(a, dtype), is_nan(b, dtype)
    d = np.where(na & nb, 0, d)
    return np.where(na ^ nb, 1 << 20, d)


def gpu_bits(t: torch.Tensor) -> np.ndarray:
    return workloads.to_bits(t.cpu())


def compare(y_gpu: torch.Tensor, rstd_gpu: torch.Tensor, y_ref: np.ndarray, rstd_ref: np.ndarray,
            dtype: str, what: str = "") -> dict:
    """Assert the acceptance bar; return statistics."""
    yb = gpu_bits(y_gpu).reshape(y_ref.shape)
    r = rstd_gpu.cpu().numpy().astype(np.float64)
    dist = ulp_distance(yb, y_ref, dtype)
    worst = int(dist.max()) if dist.size else 0
    if worst > Y_ULP_TOL:
        idx = np.unravel_index(int(np.argmax(dist)), dist.shape)
        raise AssertionError(
            f"{what}: y off by {worst} ulp at {idx}: gpu 0x{int(yb[idx]):04x} oracle 0x{int(y_ref[idx]):04x} "
            f"({int(np.sum(dist > Y_ULP_TOL))} elements beyond {Y_ULP_TOL} ulp)")
    with np.errstate(invalid="ignore"):
        rel = np.abs(r - rstd_ref) / np.abs(rstd_ref)
    both_inf = np.isinf(r) & np.isinf(rstd_ref)
    rel = np.where(both_inf, 0.0, rel)
    bad = ~(rel <= RSTD_RTOL)
    if bad.any():
        m = int(np.argmax(np.where(bad, 1, 0)))
        raise AssertionError(f"{what}: rstd row {m}: gpu {r[m]!r} oracle {rstd_ref[m]!r} "
                             f"(relative {rel[m]:.3e}, {int(bad.sum())} rows beyond {RSTD_RTOL})")
    return {
        "elements": int(dist.size),
        "exact_fraction": float(np.mean(dist == 0)) if dist.size else 1.0,
        "one_ulp": int(np.sum(dist == 1)),
        "rstd_max_rel": float(rel.max()) if rel.size else 0.0,
    }


def oracle_for(x_cpu: torch.Tensor, w_cpu: torch.Tensor, eps: float, offset: float, dtype: str):
    return oracle.rmsnorm_fwd(workloads.to_bits(x_cpu), workloads.to_bits(w_cpu), eps, offset, dtype)
