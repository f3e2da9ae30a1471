"""Pins for the fp64 oracle: checks against what the pages and mathematics fix.

Every function here takes an ``oracle.Oracle`` and raises AssertionError when
the oracle disagrees with something independent of it:

  * exact decodes of every 16-bit pattern by Python's ``struct`` (binary16) and
    by reinterpreting the pattern as the top half of a binary32 (bfloat16);
  * numpy's correctly rounded float64 -> float16 cast, and torch's float32 ->
    bfloat16 cast on values exact in float32 (a single rounding there);
  * exact rational arithmetic (``fractions.Fraction``) for the whole forward on
    tiny inputs, including an exact nearest-even decision that never evaluates
    a square root;
  * hand-worked fixtures in ``tests/golden/``;
  * closed forms and invariants of the formula: constant rows, N = 1, unit
    weights, power-of-two scale invariance, sign symmetry, offset equivalence,
    row independence;
  * P3's correctness expression ("Rmsnorm Kernel Optimization", Verification)
    evaluated by torch in float64;
  * for the backward (derived, not on the pages): central finite differences
    of the fp64 forward, torch's float64 autograd of the same expression, and
    identities of the derivative (orthogonality to x at eps = 0, oddness,
    homogeneity and additivity in dy, closed forms for one row and for a
    constant row).

The same functions run against deliberately mutated copies of the oracle in
``test_oracle_mutants.py``: each plausible mistake must trip at least one pin.
"""
from __future__ import annotations

import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "rmsnorm_handworked.json")

FORMATS = {
    # exponent bits, fraction bits
    "bf16": (8, 7),
    "fp16": (5, 10),
}


# --------------------------------------------------------------------------
# independent exact decoding
# --------------------------------------------------------------------------
def exact_value(bits: int, dtype: str) -> Fraction | float:
    """Exact value of one 16-bit pattern via struct (returns float for inf/nan)."""
    if dtype == "bf16":
        v = struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
    else:
        v = struct.unpack("<e", struct.pack("<H", bits & 0xFFFF))[0]
    if math.isnan(v) or math.isinf(v):
        return v
    return Fraction(v)


def fp32(v: float) -> float:
    """The fp32 value a float argument becomes at the C boundary."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


_POS_CACHE: dict[str, list[Fraction]] = {}


def positive_ladder(dtype: str) -> list[Fraction]:
    """All finite non-negative values in pattern order, plus 2^(emax+1) as the
    overflow rung (its pattern index equals the +infinity pattern)."""
    if dtype not in _POS_CACHE:
        E, P = FORMATS[dtype]
        inf_bits = ((1 << E) - 1) << P
        vals = [exact_value(b, dtype) for b in range(inf_bits)]
        bias = (1 << (E - 1)) - 1
        vals.append(Fraction(2) ** (bias + 1))
        _POS_CACHE[dtype] = vals
    return _POS_CACHE[dtype]


def exact_rne_of_ratio(a: Fraction, b: Fraction, dtype: str):
    """Nearest-even pattern of y = a / sqrt(b) (b > 0), decided exactly.

    Returns (pattern, near_tie) where near_tie is True when y lies within a
    relative 1e-12 of a rounding midpoint, where an fp64 evaluation may
    legitimately land on either side.
    """
    sign = 0x8000 if a < 0 else 0
    a = abs(a)
    if a == 0:
        return sign, False
    a2 = a * a
    ladder = positive_ladder(dtype)
    # largest k with ladder[k] <= y  <=>  ladder[k]^2 * b <= a^2
    lo, hi = 0, len(ladder) - 1
    if ladder[hi] ** 2 * b <= a2:
        return sign | (len(ladder) - 1), False  # at or past the overflow rung
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if ladder[mid] ** 2 * b <= a2:
            lo = mid
        else:
            hi = mid
    m = (ladder[lo] + ladder[lo + 1]) / 2
    lhs = m * m * b
    near = abs(a2 - lhs) <= Fraction(1, 10 ** 12) * lhs
    if a2 > lhs:
        k = lo + 1
    elif a2 < lhs:
        k = lo
    else:
        k = lo if lo % 2 == 0 else lo + 1
    return sign | k, near


def is_nan_bits(b: int, dtype: str) -> bool:
    E, P = FORMATS[dtype]
    return ((b >> P) & ((1 << E) - 1)) == (1 << E) - 1 and (b & ((1 << P) - 1)) != 0


def same_value_bits(a: int, b: int) -> bool:
    """Bitwise equal, with +0 and -0 taken as equal."""
    return a == b or ((a & 0x7FFF) == 0 and (b & 0x7FFF) == 0)


# --------------------------------------------------------------------------
# codec pins
# --------------------------------------------------------------------------
def pin_decode_all_patterns(o):
    for dtype in ("bf16", "fp16"):
        bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        got = o.decode(bits, dtype)
        for b in range(65536):
            ref = exact_value(b, dtype)
            g = got[b]
            if isinstance(ref, float) and math.isnan(ref):
                assert math.isnan(g), (dtype, hex(b), g)
            else:
                assert g == float(ref), (dtype, hex(b), g, ref)
                if ref == 0:
                    assert math.copysign(1.0, g) == (-1.0 if b & 0x8000 else 1.0), (dtype, hex(b))


def pin_encode_roundtrip(o):
    for dtype in ("bf16", "fp16"):
        bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        vals = o.decode(bits, dtype)
        back = o.encode(vals, dtype)
        for b in range(65536):
            if is_nan_bits(b, dtype):
                assert is_nan_bits(int(back[b]), dtype), (dtype, hex(b), hex(back[b]))
            else:
                assert int(back[b]) == b, (dtype, hex(b), hex(back[b]))


def pin_encode_midpoints(o):
    """Exact midpoints tie to the even pattern; one fp64 ulp either side decides."""
    for dtype in ("bf16", "fp16"):
        ladder = positive_ladder(dtype)
        n = len(ladder) - 1
        ks = np.arange(n)                         # pairs (k, k+1), k+1 may be the overflow rung
        lo = np.array([float(ladder[k]) for k in ks])
        hi = np.array([float(ladder[k + 1]) for k in ks])
        mid = (lo + hi) / 2                       # exact: one more bit than the format
        tie = o.encode(mid, dtype).astype(np.int64)
        up = o.encode(np.nextafter(mid, np.inf), dtype).astype(np.int64)
        down = o.encode(np.nextafter(mid, 0.0), dtype).astype(np.int64)
        even = np.where(ks % 2 == 0, ks, ks + 1)
        assert np.array_equal(tie, even), dtype
        assert np.array_equal(up, ks + 1), dtype
        assert np.array_equal(down, ks), dtype
        # mirror image for negative values
        ntie = o.encode(-mid, dtype).astype(np.int64)
        assert np.array_equal(ntie, even | 0x8000), dtype


def pin_encode_specials(o):
    cases = {
        "bf16": [(0.0, 0x0000), (-0.0, 0x8000), (math.inf, 0x7F80), (-math.inf, 0xFF80),
                 (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000), (1.5 * 2.0 ** -134, 0x0001),
                 (3.3895313892515355e38, 0x7F7F), (1e300, 0x7F80), (-1e300, 0xFF80),
                 (5e-324, 0x0000)],
        "fp16": [(0.0, 0x0000), (-0.0, 0x8000), (math.inf, 0x7C00), (-math.inf, 0xFC00),
                 (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000), (1.5 * 2.0 ** -25, 0x0001),
                 (65504.0, 0x7BFF), (65519.99, 0x7BFF), (65520.0, 0x7C00), (1e300, 0x7C00),
                 (2.0 ** -14, 0x0400), (5e-324, 0x0000)],
    }
    for dtype, pairs in cases.items():
        got = o.encode(np.array([v for v, _ in pairs]), dtype)
        for (v, want), g in zip(pairs, got):
            assert int(g) == want, (dtype, v, hex(g), hex(want))
        nan = o.encode(np.array([math.nan]), dtype)
        assert is_nan_bits(int(nan[0]), dtype), (dtype, hex(nan[0]))


def pin_encode_vs_numpy_fp16(o, seed=1234, n=200_000):
    rng = np.random.default_rng(seed)
    mags = np.exp(rng.uniform(np.log(1e-9), np.log(7e4), size=n))
    vals = mags * rng.choice([-1.0, 1.0], size=n)
    got = o.encode(vals, "fp16")
    ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref), int(np.sum(got != ref))


def pin_encode_vs_torch_bf16(o, seed=4321, n=200_000):
    """Values exact in float32: torch's float32 -> bfloat16 cast rounds once."""
    g = torch.Generator().manual_seed(seed)
    mags = torch.exp(torch.empty(n, dtype=torch.float64).uniform_(math.log(1e-30), math.log(1e30),
                                                                  generator=g))
    sgn = torch.where(torch.rand(n, generator=g) < 0.5, -1.0, 1.0).to(torch.float64)
    v32 = (mags * sgn).to(torch.float32)
    ref = v32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = o.encode(v32.to(torch.float64).numpy(), "bf16")
    assert np.array_equal(got, ref), int(np.sum(got != ref))


# --------------------------------------------------------------------------
# forward pins
# --------------------------------------------------------------------------
def _bits(vals, dtype):
    """Patterns of values that must be exact in the dtype (checked)."""
    arr = np.asarray(vals, dtype=np.float64)
    out = np.empty(arr.shape, dtype=np.uint16)
    flat = out.reshape(-1)
    for i, v in enumerate(arr.reshape(-1)):
        if dtype == "fp16":
            b = int(np.array([v]).astype(np.float16).view(np.uint16)[0])
        else:
            b = struct.unpack("<I", struct.pack("<f", v))[0] >> 16
        assert float(exact_value(b, dtype)) == v, (v, dtype)
        flat[i] = b
    return out


def pin_golden(o):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        dtype, N = c["dtype"], c["N"]
        x = np.array([[int(h, 16) for h in c["x"]]], dtype=np.uint16)
        w = np.array([int(h, 16) for h in c["w"]], dtype=np.uint16)
        assert x.shape == (1, N) and w.shape == (N,), c["name"]
        y, r = o.rmsnorm_fwd(x, w, c["eps"], c["offset"], dtype)
        want = [int(h, 16) for h in c["y"]]
        got = [int(v) for v in y[0]]
        assert got == want, (c["name"], [hex(g) for g in got], c["y"])
        b = Fraction(c["ms_plus_eps"])
        rf = Fraction(float(r[0]))
        assert abs(rf * rf * b - 1) <= Fraction(1, 2 ** 50), (c["name"], float(r[0]))


def pin_constant_rows(o):
    for dtype in ("bf16", "fp16"):
        for N in (1, 3, 8, 100, 513):
            for c in (-3.0, 0.5, 1.0, 7.0, 0.0078125):
                for eps in (0.0, 1e-6, 0.25):
                    for offset in (0.0, 1.0):
                        w = o.encode(np.linspace(-2, 2, N) if N > 1 else np.array([0.75]), dtype)
                        # c * fl(1/|c|) == sign(c) exactly in fp64 for these c
                        x = np.tile(_bits([c], dtype), (2, N))
                        y, r, ye = o.rmsnorm_fwd(x, w, eps, offset, dtype, want_exact=True)
                        e = fp32(eps)
                        want_r = 1.0 / math.sqrt(c * c + e)
                        assert abs(r[0] - want_r) <= 4e-16 * want_r, (dtype, N, c, eps)
                        wv = o.decode(w, dtype)
                        # y_j = c / sqrt(c^2 + eps) * (offset + w_j)
                        yx = c * want_r * (fp32(offset) + wv)
                        assert np.allclose(ye[0], yx, rtol=1e-14, atol=0), (dtype, N, c, eps)
                        if eps == 0.0:
                            # exactly sign(c) * (offset + w_j), one rounding
                            want = o.encode(math.copysign(1.0, c) * (fp32(offset) + wv), dtype)
                            assert all(same_value_bits(int(a), int(b))
                                       for a, b in zip(y[1], want)), (dtype, N, c, offset)


def pin_n_equals_one(o):
    rng = np.random.default_rng(7)
    for dtype in ("bf16", "fp16"):
        xv = rng.uniform(-30, 30, size=64)
        x = o.encode(xv, dtype).reshape(64, 1)
        x[x & 0x7FFF == 0] = o.encode(np.array([1.5]), dtype)[0]
        w = _bits([0.25], dtype)            # offset + w exact: no rounding tie to land on
        for offset in (0.0, 1.0):
            y, r = o.rmsnorm_fwd(x, w, 0.0, offset, dtype)
            xd = o.decode(x[:, 0], dtype)
            assert np.array_equal(r, 1.0 / np.abs(xd)), dtype
            want = o.encode(np.sign(xd) * (offset + o.decode(w, dtype)[0]), dtype)
            assert np.array_equal(y[:, 0], want), (dtype, offset)


def pin_unit_weight_mean_square(o):
    """w = 1, offset 0: mean(y_exact^2) = ms / (ms + eps); about 1 once rounded."""
    rng = np.random.default_rng(11)
    for dtype in ("bf16", "fp16"):
        for N in (7, 64, 1000):
            x = o.encode(rng.normal(0, 3, size=(4, N)), dtype)
            w = o.encode(np.ones(N), dtype)
            for eps in (1e-6, 1.0):
                y, r, ye = o.rmsnorm_fwd(x, w, eps, 0.0, dtype, want_exact=True)
                xd = o.decode(x, dtype)
                ms = np.mean(xd * xd, axis=1)
                target = ms / (ms + fp32(eps))
                assert np.allclose(np.mean(ye * ye, axis=1), target, rtol=1e-12), (dtype, N, eps)
                if eps == 1e-6:
                    yr = o.decode(y, dtype)
                    assert np.all(np.abs(np.mean(yr * yr, axis=1) - 1.0) < 2.0 ** -7), (dtype, N)


def pin_power_of_two_scale(o):
    """x -> 2^j x with eps = 0: y bitwise unchanged, rstd scaled by exactly 2^-j."""
    rng = np.random.default_rng(13)
    for dtype in ("bf16", "fp16"):
        z = rng.normal(0, 1, size=(5, 77))
        z = np.sign(z) * np.maximum(np.abs(z), 0.05)     # stay clear of fp16 subnormals
        x = o.encode(z, dtype)
        w = o.encode(rng.normal(1, 0.1, size=77), dtype)
        y0, r0 = o.rmsnorm_fwd(x, w, 0.0, 0.0, dtype)
        for j in (-3, 2, 5):
            xs = o.encode(o.decode(x, dtype) * 2.0 ** j, dtype)
            assert np.array_equal(o.decode(xs, dtype), o.decode(x, dtype) * 2.0 ** j)
            y1, r1 = o.rmsnorm_fwd(xs, w, 0.0, 0.0, dtype)
            assert np.array_equal(y0, y1), (dtype, j)
            assert np.array_equal(r1, r0 * 2.0 ** -j), (dtype, j)
        # eps > 0: the difference shrinks as eps -> 0 (scale 16 > 1)
        xs = o.encode(o.decode(x, dtype) * 16.0, dtype)
        diffs = []
        for eps in (1e-1, 1e-3, 1e-5):
            _, _, ya = o.rmsnorm_fwd(x, w, eps, 0.0, dtype, want_exact=True)
            _, _, yb = o.rmsnorm_fwd(xs, w, eps, 0.0, dtype, want_exact=True)
            diffs.append(np.max(np.abs(ya - yb)))
        assert diffs[0] > diffs[1] > diffs[2], diffs


def pin_sign_symmetry(o):
    rng = np.random.default_rng(17)
    for dtype in ("bf16", "fp16"):
        x = o.encode(rng.normal(0, 2, size=(6, 45)), dtype)
        w = o.encode(rng.normal(0, 1, size=45), dtype)
        for offset in (0.0, 1.0):
            y0, r0 = o.rmsnorm_fwd(x, w, 1e-6, offset, dtype)
            y1, r1 = o.rmsnorm_fwd(x ^ np.uint16(0x8000), w, 1e-6, offset, dtype)
            assert np.array_equal(r0, r1), dtype
            assert all(same_value_bits(int(a), int(b) ^ 0x8000)
                       for a, b in zip(y0.reshape(-1), y1.reshape(-1))), (dtype, offset)


def pin_offset_equivalence(o):
    """offset 1 with w equals offset 0 with 1 + w when 1 + w is exact in the dtype."""
    rng = np.random.default_rng(19)
    for dtype in ("bf16", "fp16"):
        N = 96
        k = rng.integers(-60, 60, size=N)
        wv = k / 128.0                      # 1 + k/128 is exact in bf16 and fp16
        w = _bits(wv, dtype)
        w1 = _bits(1.0 + wv, dtype)
        x = o.encode(rng.normal(0, 1, size=(3, N)), dtype)
        ya, ra = o.rmsnorm_fwd(x, w, 1e-6, 1.0, dtype)
        yb, rb = o.rmsnorm_fwd(x, w1, 1e-6, 0.0, dtype)
        assert np.array_equal(ra, rb) and np.array_equal(ya, yb), dtype


def pin_rstd_invariant(o):
    """r^2 (mean(x^2) + eps) = 1 to fp64 accuracy."""
    rng = np.random.default_rng(23)
    for dtype in ("bf16", "fp16"):
        x = o.encode(rng.normal(0, 5, size=(8, 300)), dtype)
        w = o.encode(np.ones(300), dtype)
        for eps in (1e-6, 0.5):
            _, r = o.rmsnorm_fwd(x, w, eps, 0.0, dtype)
            xd = o.decode(x, dtype)
            ms = np.sum(xd * xd, axis=1) / 300
            assert np.allclose(r * r * (ms + fp32(eps)), 1.0, rtol=0, atol=1e-13), (dtype, eps)


def pin_row_independence(o):
    """Rows of wildly different magnitude give the same result alone or together."""
    rng = np.random.default_rng(29)
    for dtype, (small, big) in (("bf16", (2.0 ** -20, 2.0 ** 20)), ("fp16", (2.0 ** -6, 2.0 ** 6))):
        for N in (1, 13, 127, 300):
            z = rng.normal(0, 1, size=(6, N))
            z *= np.where(np.arange(6) % 2 == 0, small, big)[:, None]
            x = o.encode(z, dtype)
            w = o.encode(rng.normal(1, 0.1, size=N), dtype)
            y, r = o.rmsnorm_fwd(x, w, 1e-6, 0.0, dtype)
            for m in range(6):
                y1, r1 = o.rmsnorm_fwd(x[m:m + 1], w, 1e-6, 0.0, dtype)
                assert np.array_equal(y1[0], y[m]) and r1[0] == r[m], (dtype, N, m)


def _random_patterns(rng, shape, dtype, spread):
    """Random finite patterns: random sign and fraction, exponent within +-spread
    binades of 1, a few zeros and (fp16) subnormals."""
    E, P = FORMATS[dtype]
    bias = (1 << (E - 1)) - 1
    e = rng.integers(bias - spread, bias + spread + 1, size=shape)
    f = rng.integers(0, 1 << P, size=shape)
    s = rng.integers(0, 2, size=shape)
    b = (s << 15) | (e << P) | f
    z = rng.random(shape)
    b = np.where(z < 0.04, s << 15, b)                              # zeros
    b = np.where((z >= 0.04) & (z < 0.07), (s << 15) | f, b)        # subnormals
    return b.astype(np.uint16)


def pin_bruteforce_exact(o, seed=31, trials=120):
    """Whole forward in exact rationals on tiny inputs; nearest-even decided
    without evaluating a square root (compare y^2 against squared midpoints)."""
    rng = np.random.default_rng(seed)
    near_ties = 0
    checked = 0
    for t in range(trials):
        dtype = ("bf16", "fp16")[t % 2]
        M = int(rng.integers(1, 5))
        N = int(rng.integers(1, 17))
        spread = 4 if dtype == "fp16" else 12
        x = _random_patterns(rng, (M, N), dtype, spread)
        w = _random_patterns(rng, (N,), dtype, 3)
        eps = float((0.0, 1e-6, 0.3, float(rng.uniform(0, 2)))[t % 4])
        offset = float((0.0, 1.0, fp32(float(rng.uniform(-1, 1))))[t % 3])
        xf = [[exact_value(int(b), dtype) for b in row] for row in x]
        wf = [exact_value(int(b), dtype) for b in w]
        e = Fraction(fp32(eps))
        off = Fraction(fp32(offset))
        for m in range(M):
            if eps == 0.0 and all(v == 0 for v in xf[m]):
                x[m, 0] = 0x3C00 if dtype == "fp16" else 0x3F80
                xf[m][0] = Fraction(1)
        y, r = o.rmsnorm_fwd(x, w, eps, offset, dtype)
        for m in range(M):
            ss = sum(v * v for v in xf[m])
            b = ss / N + e
            rf = Fraction(float(r[m]))
            assert abs(rf * rf * b - 1) <= Fraction(N + 8, 2 ** 52), (t, m, float(r[m]))
            for j in range(N):
                a = xf[m][j] * (off + wf[j])
                want, near = exact_rne_of_ratio(a, b, dtype)
                if near:
                    near_ties += 1
                    continue
                checked += 1
                assert same_value_bits(int(y[m, j]), want), (t, dtype, m, j, hex(y[m, j]), hex(want))
    assert checked > 1000 and near_ties <= 2, (checked, near_ties)


def pin_torch_fp64_expression(o):
    """x * rsqrt(mean(x^2) + eps) * (offset + w), evaluated by torch in float64."""
    rng = np.random.default_rng(37)
    for dtype in ("bf16", "fp16"):
        for N in (5, 128, 3000):
            x = o.encode(rng.normal(0, 4, size=(4, N)), dtype)
            w = o.encode(rng.normal(0.5, 0.3, size=N), dtype)
            for eps, offset in ((1e-6, 0.0), (1e-2, 1.0)):
                _, r, ye = o.rmsnorm_fwd(x, w, eps, offset, dtype, want_exact=True)
                td = torch.bfloat16 if dtype == "bf16" else torch.float16
                xt = torch.from_numpy(x.view(np.int16)).view(td).to(torch.float64)
                wt = torch.from_numpy(w.view(np.int16)).view(td).to(torch.float64)
                rt = torch.rsqrt(xt.pow(2).mean(-1, keepdim=True) + fp32(eps))
                ref = (xt * rt * (fp32(offset) + wt)).numpy()
                assert np.allclose(r, rt[:, 0].numpy(), rtol=1e-13, atol=0), (dtype, N)
                assert np.allclose(ye, ref, rtol=1e-13, atol=1e-300), (dtype, N, eps)


# --------------------------------------------------------------------------
# backward pins.  The pages keep rstd for a backward pass without printing
# one; the oracle's backward is the derivative of its forward, so it is pinned
# against finite differences of that forward, against torch's float64
# autograd, and against identities of the derivative.
# --------------------------------------------------------------------------
def _bwd_case(o, rng, M, N, dtype, eps, offset, xscale=1.0):
    x = o.encode(rng.normal(0, xscale, size=(M, N)), dtype)
    w = o.encode(rng.normal(0.3, 0.5, size=N), dtype)
    dy = o.encode(rng.normal(0, 1, size=(M, N)), dtype)
    xd, wd, dyd = o.decode(x, dtype), o.decode(w, dtype), o.decode(dy, dtype)
    _, r = o.rmsnorm_fwd_f64(xd, wd, fp32(eps), fp32(offset))
    return x, w, dy, xd, wd, dyd, r


def pin_bwd_forward_f64_matches(o):
    """The fp64-input forward used for finite differences equals the codec forward."""
    rng = np.random.default_rng(41)
    for dtype in ("bf16", "fp16"):
        x = o.encode(rng.normal(0, 2, size=(5, 33)), dtype)
        w = o.encode(rng.normal(1, 0.1, size=33), dtype)
        for eps, offset in ((1e-6, 0.0), (0.25, 1.0)):
            _, r, ye = o.rmsnorm_fwd(x, w, eps, offset, dtype, want_exact=True)
            y2, r2 = o.rmsnorm_fwd_f64(o.decode(x, dtype), o.decode(w, dtype), fp32(eps), fp32(offset))
            assert np.array_equal(r, r2) and np.array_equal(ye, y2), (dtype, eps)


def pin_bwd_finite_differences(o):
    """dx and dw against central differences of L = sum(dy * y) through the fp64 forward."""
    rng = np.random.default_rng(43)
    for dtype in ("bf16", "fp16"):
        for M, N, eps, offset in ((3, 7, 1e-6, 0.0), (2, 16, 0.5, 1.0), (1, 1, 1e-3, 0.0), (4, 5, 0.0, 1.0)):
            x, w, dy, xd, wd, dyd, r = _bwd_case(o, rng, M, N, dtype, eps, offset)
            _, dw, dxe, _, _ = o.rmsnorm_bwd(x, w, dy, r, offset, dtype, want_exact=True)
            e, off = fp32(eps), fp32(offset)

            def loss(xx, ww):
                y, _ = o.rmsnorm_fwd_f64(xx, ww, e, off)
                return float(np.sum(dyd * y))

            fd_x = np.empty_like(xd)
            for idx in np.ndindex(*xd.shape):
                h = 1e-6 * max(1.0, abs(xd[idx]))
                xp, xm = xd.copy(), xd.copy()
                xp[idx] += h
                xm[idx] -= h
                fd_x[idx] = (loss(xp, wd) - loss(xm, wd)) / (2 * h)
            fd_w = np.empty_like(wd)
            for j in range(N):
                h = 1e-6 * max(1.0, abs(wd[j]))
                wp, wm = wd.copy(), wd.copy()
                wp[j] += h
                wm[j] -= h
                fd_w[j] = (loss(xd, wp) - loss(xd, wm)) / (2 * h)
            sx = np.max(np.abs(fd_x)) + 1.0
            sw = np.max(np.abs(fd_w)) + 1.0
            assert np.allclose(dxe, fd_x, rtol=1e-6, atol=1e-7 * sx), (dtype, M, N, np.max(np.abs(dxe - fd_x)))
            assert np.allclose(dw, fd_w, rtol=1e-6, atol=1e-7 * sw), (dtype, M, N, np.max(np.abs(dw - fd_w)))


def pin_bwd_torch_autograd(o):
    """torch float64 autograd of x * rsqrt(mean(x^2) + eps) * (offset + w)."""
    rng = np.random.default_rng(47)
    for dtype in ("bf16", "fp16"):
        for M, N, eps, offset in ((6, 128, 1e-6, 0.0), (3, 3000, 1e-2, 1.0), (17, 9, 0.0, 0.0)):
            x, w, dy, xd, wd, dyd, r = _bwd_case(o, rng, M, N, dtype, eps, offset)
            _, dw, dxe, _, _ = o.rmsnorm_bwd(x, w, dy, r, offset, dtype, want_exact=True)
            xt = torch.tensor(xd, requires_grad=True)
            wt = torch.tensor(wd, requires_grad=True)
            y = xt * torch.rsqrt(xt.pow(2).mean(-1, keepdim=True) + fp32(eps)) * (fp32(offset) + wt)
            y.backward(torch.tensor(dyd))
            assert np.allclose(dxe, xt.grad.numpy(), rtol=1e-9, atol=1e-12 * np.max(np.abs(dxe))), (dtype, M, N)
            assert np.allclose(dw, wt.grad.numpy(), rtol=1e-9, atol=1e-12 * np.max(np.abs(dw))), (dtype, M, N)


def pin_bwd_identities(o):
    """sum_k dx_k x_k = r N c eps / (ms + eps) (zero at eps = 0: the output does
    not change along x); dx and dw are odd and homogeneous in dy: exact
    under dy -> -dy and dy -> 2 dy; additive in dy; M = 1 gives dw = dy x r."""
    rng = np.random.default_rng(53)
    for dtype in ("bf16", "fp16"):
        for eps, offset in ((0.0, 0.0), (0.3, 1.0)):
            x, w, dy, xd, wd, dyd, r = _bwd_case(o, rng, 5, 40, dtype, eps, offset)
            _, dw, dxe, _, _ = o.rmsnorm_bwd(x, w, dy, r, offset, dtype, want_exact=True)
            g = fp32(offset) + wd
            ms = np.mean(xd * xd, axis=1)
            c = np.mean(dyd * g * xd, axis=1)
            lhs = np.sum(dxe * xd, axis=1)
            rhs = r * 40 * c * fp32(eps) / (ms + fp32(eps))
            scale = np.sum(np.abs(dxe * xd), axis=1)
            assert np.all(np.abs(lhs - rhs) <= 1e-12 * scale), (dtype, eps, lhs, rhs)
            # dy -> -dy and dy -> 2 dy (exact in the dtype and in fp64)
            _, dwn, dxn, _, _ = o.rmsnorm_bwd(x, w, dy ^ np.uint16(0x8000), r, offset, dtype, want_exact=True)
            assert np.array_equal(dxn, -dxe) and np.array_equal(dwn, -dw)
            dy2 = o.encode(2.0 * dyd, dtype)
            assert np.array_equal(o.decode(dy2, dtype), 2.0 * dyd)
            _, dw2, dx2, _, _ = o.rmsnorm_bwd(x, w, dy2, r, offset, dtype, want_exact=True)
            assert np.allclose(dx2, 2.0 * dxe, rtol=1e-15, atol=0) and np.allclose(dw2, 2.0 * dw, rtol=1e-15, atol=0)
            # additivity on small-integer gradients (sums exact in the dtype)
            a = rng.integers(-8, 9, size=(5, 40)).astype(np.float64)
            b = rng.integers(-8, 9, size=(5, 40)).astype(np.float64)
            outs = [o.rmsnorm_bwd(x, w, o.encode(v, dtype), r, offset, dtype, want_exact=True) for v in (a, b, a + b)]
            sc = outs[2][3]
            assert np.all(np.abs(outs[0][2] + outs[1][2] - outs[2][2]) <= 1e-13 * (sc + 1e-300)), dtype
            assert np.allclose(outs[0][1] + outs[1][1], outs[2][1], rtol=1e-13, atol=1e-13 * np.max(outs[2][4]))
        # one row: dw_j = dy_j x_j r exactly in fp64
        x, w, dy, xd, wd, dyd, r = _bwd_case(o, rng, 1, 64, dtype, 1e-6, 0.0)
        _, dw = o.rmsnorm_bwd(x, w, dy, r, 0.0, dtype)
        assert np.array_equal(dw, dyd[0] * xd[0] * r[0]), dtype
        # zero upstream gradient
        dx0, dw0 = o.rmsnorm_bwd(x, w, np.zeros_like(dy), r, 0.0, dtype)
        assert np.all((dx0 & 0x7FFF) == 0) and np.all(dw0 == 0)


def pin_bwd_constant_row(o):
    """x = c, w = 1, offset 0, dy = 1: dx_k = r eps / (c^2 + eps) (zero at eps 0), dw_j = M c r."""
    for dtype in ("bf16", "fp16"):
        for c in (1.5, -3.0):
            for eps in (0.0, 0.25):
                N, M = 12, 3
                x = np.tile(_bits([c], dtype), (M, N))
                w = _bits(np.ones(N), dtype)
                dy = _bits(np.ones((M, N)), dtype)
                e = fp32(eps)
                r = np.full(M, 1.0 / math.sqrt(c * c + e))
                dx, dw, dxe, _, _ = o.rmsnorm_bwd(x, w, dy, r, 0.0, dtype, want_exact=True)
                want = r[0] * e / (c * c + e)
                assert np.allclose(dxe, want, rtol=1e-14, atol=1e-15), (dtype, c, eps)
                assert np.allclose(dw, M * c * r[0], rtol=1e-15, atol=0), (dtype, c, eps)


def pin_bwd_f64_path(o):
    """The fp64-input backward (the fp32 path's oracle): equal, bit for bit, to the codec backward on
    16-bit inputs; against central differences of the fp64 forward and torch float64 autograd on
    fp32 inputs; dw of one row is dy x r exactly."""
    rng = np.random.default_rng(59)
    for dtype in ("bf16", "fp16"):
        x, w, dy, xd, wd, dyd, r = _bwd_case(o, rng, 4, 37, dtype, 1e-6, 1.0)
        _, dw, dxe, dxs, dws = o.rmsnorm_bwd(x, w, dy, r, 1.0, dtype, want_exact=True)
        ex, dw2, sc, ws = o.rmsnorm_bwd_f64(xd, wd, dyd, r, fp32(1.0))
        assert np.array_equal(ex, dxe) and np.array_equal(dw2, dw), dtype
        assert np.array_equal(sc, dxs) and np.array_equal(ws, dws), dtype
    f32 = lambda a: np.asarray(a, dtype=np.float32).astype(np.float64)
    for M, N, eps, offset in ((3, 7, 1e-6, 0.0), (2, 16, 0.5, 1.0), (1, 1, 1e-3, 0.0)):
        xd = f32(rng.normal(0, 3, size=(M, N)))
        wd = f32(rng.normal(0.3, 0.5, size=N))
        dyd = f32(rng.normal(0, 1, size=(M, N)))
        e, off = fp32(eps), fp32(offset)
        _, r = o.rmsnorm_fwd_f64(xd, wd, e, off)
        dxe, dw, _, _ = o.rmsnorm_bwd_f64(xd, wd, dyd, r, off)

        def loss(xx, ww):
            y, _ = o.rmsnorm_fwd_f64(xx, ww, e, off)
            return float(np.sum(dyd * y))

        fd_x = np.empty_like(xd)
        for idx in np.ndindex(*xd.shape):
            h = 1e-6 * max(1.0, abs(xd[idx]))
            xp, xm = xd.copy(), xd.copy()
            xp[idx] += h
            xm[idx] -= h
            fd_x[idx] = (loss(xp, wd) - loss(xm, wd)) / (2 * h)
        fd_w = np.empty_like(wd)
        for j in range(N):
            h = 1e-6 * max(1.0, abs(wd[j]))
            wp, wm = wd.copy(), wd.copy()
            wp[j] += h
            wm[j] -= h
            fd_w[j] = (loss(xd, wp) - loss(xd, wm)) / (2 * h)
        assert np.allclose(dxe, fd_x, rtol=1e-6, atol=1e-7 * (np.max(np.abs(fd_x)) + 1.0)), (M, N)
        assert np.allclose(dw, fd_w, rtol=1e-6, atol=1e-7 * (np.max(np.abs(fd_w)) + 1.0)), (M, N)
        xt = torch.tensor(xd, requires_grad=True)
        wt = torch.tensor(wd, requires_grad=True)
        y = xt * torch.rsqrt(xt.pow(2).mean(-1, keepdim=True) + e) * (off + wt)
        y.backward(torch.tensor(dyd))
        assert np.allclose(dxe, xt.grad.numpy(), rtol=1e-9, atol=1e-12 * np.max(np.abs(dxe))), (M, N)
        assert np.allclose(dw, wt.grad.numpy(), rtol=1e-9, atol=1e-12 * np.max(np.abs(dw))), (M, N)
        if M == 1:
            assert np.array_equal(dw, dyd[0] * xd[0] * r[0])


def pin_fp32_path(o):
    """fp32 inputs: the oracle's fp64 forward, then one IEEE round-to-nearest-even to binary32.

    The rounding step is numpy's float64 -> float32 cast; pinned here on exact
    midpoints (ties to even), one fp64 ulp either side of them, overflow at
    FLT_MAX + half an ulp, and gradual underflow.  The fp64 forward on fp32
    inputs is pinned by a constant row with eps = 0 (y = sign(c) (offset + w)
    exactly) and by the brute-force rational result on tiny rows.
    """
    one = np.float64(1.0)
    ulp = 2.0 ** -23
    mids = np.array([1 + ulp / 2, 1 + 3 * ulp / 2, -(1 + ulp / 2), 2 ** -126 * (1 + ulp / 2)])
    want = np.array([1.0, 1 + 2 * ulp, -1.0, 2 ** -126], dtype=np.float32)
    assert np.array_equal(mids.astype(np.float32), want), mids.astype(np.float32)
    above = np.nextafter(one + ulp / 2, np.inf)
    below = np.nextafter(one + 3 * ulp / 2, -np.inf)
    assert np.float32(above) == np.float32(1 + ulp) and np.float32(below) == np.float32(1 + ulp)
    fmax = float(np.finfo(np.float32).max)
    assert np.isinf(np.float32(fmax + 2.0 ** (127 - 24))) and np.float32(np.nextafter(fmax + 2.0 ** (127 - 24), 0)) == fmax
    tiny = 2.0 ** -149
    assert np.float32(tiny * 1.5) == np.float32(2 * tiny) and np.float32(tiny * 0.5) == 0.0 and np.float32(tiny * 2.5) == np.float32(2 * tiny)
    # constant rows of a power of two, eps = 0: r = 1/|c| and y = sign(c) * (offset + w), all exact
    rng = np.random.default_rng(7)
    for c in (4.0, -0.25, 2.0 ** -70, -(2.0 ** 90)):
        w = np.float32(rng.standard_normal(33)).astype(np.float64)
        for off in (0.0, 1.0):
            y, r = o.rmsnorm_fwd_f64(np.full((2, 33), c), w, 0.0, off)
            assert np.array_equal(y, np.broadcast_to(np.sign(c) * (off + w), y.shape)), (c, off)
            assert np.all(r == 1.0 / abs(c)), (c, r)
    # tiny rows against exact rationals: the rounded fp32 result is the nearest binary32 value
    from fractions import Fraction
    for trial in range(40):
        N = int(rng.integers(1, 9))
        x = np.float32(rng.standard_normal((1, N)) * 4).astype(np.float64)
        w = np.float32(rng.standard_normal(N)).astype(np.float64)
        y, _ = o.rmsnorm_fwd_f64(x, w, 0.0, 0.0)
        y32 = y.astype(np.float32)
        ss = sum(Fraction(v) ** 2 for v in x[0])
        for j in range(N):
            num = Fraction(x[0, j]) * Fraction(w[j])           # y = num / sqrt(ss / N)
            # exact y^2 = num^2 * N / ss; compare squares of the neighbours of y32
            y2 = num * num * N / ss
            cand = float(y32[0, j])
            lo, hi = np.nextafter(np.float32(cand), np.float32(-np.inf)), np.nextafter(np.float32(cand), np.float32(np.inf))
            for other in (lo, hi):
                mid = (Fraction(cand) + Fraction(float(other))) / 2
                # y32 must be at least as close to the exact value as each neighbour: the exact
                # value lies on y32's side of the midpoint (signs agree with num)
                if num > 0:
                    assert (mid * mid <= y2) == (float(other) < cand) or mid * mid == y2, (trial, j)
                elif num < 0:
                    assert (mid * mid <= y2) == (float(other) > cand) or mid * mid == y2, (trial, j)


ALL_PINS = [
    pin_decode_all_patterns,
    pin_encode_roundtrip,
    pin_encode_midpoints,
    pin_encode_specials,
    pin_encode_vs_numpy_fp16,
    pin_encode_vs_torch_bf16,
    pin_golden,
    pin_constant_rows,
    pin_n_equals_one,
    pin_unit_weight_mean_square,
    pin_power_of_two_scale,
    pin_sign_symmetry,
    pin_offset_equivalence,
    pin_rstd_invariant,
    pin_row_independence,
    pin_bruteforce_exact,
    pin_torch_fp64_expression,
    pin_bwd_forward_f64_matches,
    pin_bwd_finite_differences,
    pin_bwd_torch_autograd,
    pin_bwd_identities,
    pin_bwd_constant_row,
    pin_bwd_f64_path,
    pin_fp32_path,
]
