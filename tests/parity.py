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


# ---------------------------------------------------------------------------
# Backward.  dx can cancel (r g dy against r^3 c x), so a bound relative to dx
# itself is meaningless where it nearly vanishes; the bar is relative to the
# size of the terms it is computed from:
#   |dx_gpu - dx_exact| <= ulp_dtype(dx_exact) + 2^-16 * (|r g dy| + |r^3 x| mean_j |dy g x|)
# one ulp for the single rounding to the dtype, and 2^-16 (about 1.5e-5) for
# fp32 products and the additions in c: at most 32 in sequence per thread (rows
# of up to 32768 elements in the 16-byte kernels), a 6-level wave tree and 16
# waves (first-order bound (32 + 6 + 16) * 2^-24, with a factor 4 to spare).
#   |dw_gpu - dw_exact| <= 2 K 2^-24 sum_m |dy x r| + 2^-23 |dw_exact|
# where K = ceil(M / G) + G + 64 bounds the sequential fp32 additions along
# any one column (rows of one workgroup, its waves and segments, then the G
# partial rows), with a factor 2 to spare, plus the final rounding.
# Both sides use the same rstd values.
# ---------------------------------------------------------------------------
FRAC_BITS = {"bf16": 7, "fp16": 10, "fp32": 23}
MIN_EXP = {"bf16": -126, "fp16": -14, "fp32": -126}


def ulp_of(v: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the dtype's values at v: 2^(floor(log2 |v|) - fraction bits), and the subnormal
    spacing 2^(min exponent - fraction bits) at and below the smallest normal (zero included).
    2^floor(log2 |v|) is |v| with its fp64 fraction bits cleared."""
    a = np.ascontiguousarray(np.abs(np.asarray(v, dtype=np.float64)))
    p2 = (a.view(np.uint64) & np.uint64(0x7FF0000000000000)).view(np.float64)
    return np.maximum(p2, 2.0 ** MIN_EXP[dtype]) * 2.0 ** -FRAC_BITS[dtype]


def compare_dx(dx_gpu: torch.Tensor, dx_exact: np.ndarray, dx_scale: np.ndarray, dtype: str,
               what: str = "") -> float:
    """dx against the oracle's exact dx with the bound above; returns the largest error / bound."""
    if dtype == "fp32":
        dxg = dx_gpu.cpu().double().numpy().reshape(dx_exact.shape)
    else:
        dxg = oracle.decode(gpu_bits(dx_gpu).reshape(dx_exact.shape), dtype)
    err = np.abs(dxg - dx_exact)
    bound = ulp_of(dx_exact, dtype) + 2.0 ** -16 * dx_scale
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(int(np.argmax(np.where(bad, err / bound, 0))), err.shape)
        raise AssertionError(f"{what}: dx off at {i}: gpu {dxg[i]!r} exact {dx_exact[i]!r} bound {bound[i]!r} "
                             f"({int(bad.sum())} elements out of bound)")
    return float(np.max(err / bound)) if err.size else 0.0


def compare_dw(dw_gpu: torch.Tensor, dw_exact: np.ndarray, dw_scale: np.ndarray, M: int, G: int,
               what: str = "") -> float:
    """dw against the oracle's dw with the bound above (G = the row pass's grid); returns the
    largest error / bound."""
    dwg = dw_gpu.cpu().numpy().astype(np.float64)
    K = -(-M // max(G, 1)) + G + 64
    wbound = 2 * K * 2.0 ** -24 * dw_scale + 2.0 ** -23 * np.abs(dw_exact) + 1e-30
    werr = np.abs(dwg - dw_exact)
    wbad = ~(werr <= wbound)
    if wbad.any():
        j = int(np.argmax(np.where(wbad, werr / wbound, 0)))
        raise AssertionError(f"{what}: dw[{j}] gpu {dwg[j]!r} exact {dw_exact[j]!r} bound {wbound[j]!r} "
                             f"({int(wbad.sum())} columns out of bound)")
    return float(np.max(werr / wbound)) if werr.size else 0.0


def compare_bwd(dx_gpu: torch.Tensor, dw_gpu: torch.Tensor, dx_exact: np.ndarray, dx_scale: np.ndarray,
                dw_exact: np.ndarray, dw_scale: np.ndarray, dtype: str, M: int, G: int, what: str = "") -> dict:
    return {"dx_max_err_over_bound": compare_dx(dx_gpu, dx_exact, dx_scale, dtype, what),
            "dw_max_err_over_bound": compare_dw(dw_gpu, dw_exact, dw_scale, M, G, what)}


def oracle_bwd_for(x_cpu, w_cpu, dy_cpu, rstd_f32: np.ndarray, offset: float, dtype: str):
    """Oracle backward on the same rstd values the GPU receives: (dx bits or None for fp32, dw,
    dx before rounding, dx term scale, dw term scale).  fp32 inputs widen to fp64 exactly and take
    the codec-free backward; the bar is then one fp32 ulp of dx plus the arithmetic term."""
    r = np.asarray(rstd_f32, dtype=np.float64)
    if dtype == "fp32":
        ex, dw, sc, ws = oracle.rmsnorm_bwd_f64(x_cpu.double().numpy(), w_cpu.double().numpy(),
                                                dy_cpu.double().numpy(), r, float(np.float32(offset)))
        return None, dw, ex, sc, ws
    return oracle.rmsnorm_bwd(workloads.to_bits(x_cpu), workloads.to_bits(w_cpu), workloads.to_bits(dy_cpu),
                              r, offset, dtype, want_exact=True)


# ---------------------------------------------------------------------------
# fp32 input.  The oracle's fp64 forward gives y_exact; the bar is relative
# to it, derived from the kernels' fp32 arithmetic:
#   sum of squares: at most 24 sequential FMAs per lane, 6 butterfly and
#     readlane levels, 15 cross-wave additions: relative error < 46 * 2^-24;
#   mean and eps: 1/N rounded, one FMA: 2 * 2^-24;
#   rsqrt: hardware, about 1 ulp: 2 * 2^-24, plus half the mean's error;
#   offset + w, x * r, (x r) g: three roundings: 3 * 2^-24.
# First order that is under 30 * 2^-24; the bar takes 64 * 2^-24 (3.8e-6),
# plus 2^-140 absolute where y_exact is subnormal in fp32.  rstd: as for the
# 16-bit types.
# ---------------------------------------------------------------------------
F32_REL = 64 * 2.0 ** -24
F32_ABS = 2.0 ** -140


def oracle_fp32(x_cpu: torch.Tensor, w_cpu: torch.Tensor, eps: float, offset: float):
    """(y_exact, rstd) in fp64 for fp32 inputs, with eps and offset taken as fp32."""
    e = float(np.float32(eps))
    o = float(np.float32(offset))
    return oracle.rmsnorm_fwd_f64(x_cpu.double().numpy(), w_cpu.double().numpy(), e, o)


def compare_fp32(y_gpu: torch.Tensor, rstd_gpu, y_exact: np.ndarray, rstd_ref: np.ndarray, what: str = "") -> dict:
    y = y_gpu.cpu().double().numpy().reshape(y_exact.shape)
    err = np.abs(y - y_exact)
    bound = F32_REL * np.abs(y_exact) + F32_ABS
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(int(np.argmax(np.where(bad, err / bound, 0))), err.shape)
        raise AssertionError(f"{what}: y off at {i}: gpu {y[i]!r} exact {y_exact[i]!r} bound {bound[i]!r} "
                             f"({int(bad.sum())} elements out of bound)")
    stats = {"elements": int(y.size), "max_err_over_bound": float(np.max(err / bound)) if y.size else 0.0}
    if rstd_gpu is not None:
        r = rstd_gpu.cpu().numpy().astype(np.float64).reshape(rstd_ref.shape)
        rel = np.abs(r - rstd_ref) / np.abs(rstd_ref)
        if not np.all(rel <= RSTD_RTOL):
            m = int(np.argmax(rel))
            raise AssertionError(f"{what}: rstd row {m}: gpu {r[m]!r} oracle {rstd_ref[m]!r}")
        stats["rstd_max_rel"] = float(rel.max()) if rel.size else 0.0
    return stats
