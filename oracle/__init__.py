"""Plain fp64 CPU oracle for the row RMSNorm forward and backward (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never does, and the oracle never imports the product path.

The arithmetic lives in ``rmsnorm_oracle.c`` (plain C, fp64, OpenMP over rows);
this module only builds it with gcc and marshals numpy arrays.  The formula it
follows is stated in that file's header, with the passages of "Rmsnorm Kernel
Optimization" (Overview) and "Why cutile's rmsnorm required full register"
(kernel listing of the opening report) it comes from.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "rmsnorm_oracle.c")
LIBRARY = os.path.join(_HERE, "librmsnorm_oracle.so")

DTYPE_CODES = {"bf16": 0, "fp16": 1}

_U16P = ctypes.POINTER(ctypes.c_uint16)
_F64P = ctypes.POINTER(ctypes.c_double)


def compile_oracle(src: str, out: str, verbose: bool = False) -> str:
    """gcc, fp64, no fast-math, no FMA contraction, OpenMP over rows."""
    tmp = f"{out}.{os.getpid()}.tmp"       # concurrent builders never share a temporary
    cmd = [
        "gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math",
        "-o", tmp, src, "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    return compile_oracle(SOURCE, LIBRARY, verbose)


def _code(dtype: str) -> int:
    if dtype not in DTYPE_CODES:
        raise ValueError(f"dtype must be one of {sorted(DTYPE_CODES)}, got {dtype!r}")
    return DTYPE_CODES[dtype]


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bit patterns, got {a.dtype}")
    return a


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_decode.argtypes = [ctypes.c_uint16, ctypes.c_int]
        lib.oracle_decode.restype = ctypes.c_double
        lib.oracle_encode_rne.argtypes = [ctypes.c_double, ctypes.c_int]
        lib.oracle_encode_rne.restype = ctypes.c_uint16
        lib.oracle_decode_array.argtypes = [_U16P, _F64P, ctypes.c_int64, ctypes.c_int]
        lib.oracle_decode_array.restype = None
        lib.oracle_encode_array.argtypes = [_F64P, _U16P, ctypes.c_int64, ctypes.c_int]
        lib.oracle_encode_array.restype = None
        lib.oracle_rmsnorm_fwd.argtypes = [
            _U16P, _U16P, ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_float,
            ctypes.c_int, _U16P, _F64P, _F64P,
        ]
        lib.oracle_rmsnorm_fwd.restype = ctypes.c_int
        lib.oracle_rmsnorm_fwd_f64.argtypes = [
            _F64P, _F64P, ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_double,
            _F64P, _F64P,
        ]
        lib.oracle_rmsnorm_fwd_f64.restype = ctypes.c_int
        lib.oracle_rmsnorm_bwd.argtypes = [
            _U16P, _U16P, _U16P, _F64P, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
            ctypes.c_int, _U16P, _F64P, _F64P, _F64P, _F64P,
        ]
        lib.oracle_rmsnorm_bwd.restype = ctypes.c_int
        lib.oracle_rmsnorm_bwd_f64.argtypes = [
            _F64P, _F64P, _F64P, _F64P, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            _F64P, _F64P, _F64P, _F64P,
        ]
        lib.oracle_rmsnorm_bwd_f64.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        self.path = path
        self._lib = lib

    def decode(self, bits, dtype: str) -> np.ndarray:
        """Exact fp64 values of 16-bit patterns."""
        b = _u16(bits)
        out = np.empty(b.shape, dtype=np.float64)
        self._lib.oracle_decode_array(b.ctypes.data_as(_U16P), out.ctypes.data_as(_F64P),
                                      b.size, _code(dtype))
        return out

    def encode(self, values, dtype: str) -> np.ndarray:
        """Round fp64 values to 16-bit patterns, nearest-even, in one step."""
        v = np.ascontiguousarray(values, dtype=np.float64)
        out = np.empty(v.shape, dtype=np.uint16)
        self._lib.oracle_encode_array(v.ctypes.data_as(_F64P), out.ctypes.data_as(_U16P),
                                      v.size, _code(dtype))
        return out

    def rmsnorm_fwd(self, x_bits, w_bits, eps: float, offset: float, dtype: str,
                    want_exact: bool = False):
        """Oracle forward on host arrays of 16-bit patterns.

        x_bits: uint16 [M, N]; w_bits: uint16 [N].  eps and offset are taken as
        fp32, as the kernels receive them.  Returns (y_bits uint16 [M, N],
        rstd float64 [M]) and, if ``want_exact``, y before rounding
        (float64 [M, N]).
        """
        x = _u16(x_bits)
        w = _u16(w_bits)
        if x.ndim != 2 or w.ndim != 1 or w.shape[0] != x.shape[1]:
            raise ValueError(f"shape mismatch: x {x.shape}, w {w.shape}")
        M, N = x.shape
        y = np.empty((M, N), dtype=np.uint16)
        rstd = np.empty((M,), dtype=np.float64)
        ye = np.empty((M, N), dtype=np.float64) if want_exact else None
        rc = self._lib.oracle_rmsnorm_fwd(
            x.ctypes.data_as(_U16P), w.ctypes.data_as(_U16P), M, N,
            ctypes.c_float(eps), ctypes.c_float(offset), _code(dtype),
            y.ctypes.data_as(_U16P), rstd.ctypes.data_as(_F64P),
            ye.ctypes.data_as(_F64P) if ye is not None else None)
        if rc != 0:
            raise ValueError(f"oracle rejected arguments (M={M}, N={N}, dtype={dtype})")
        if want_exact:
            return y, rstd, ye
        return y, rstd

    def rmsnorm_fwd_f64(self, x, w, eps: float, offset: float):
        """fp64 forward on fp64 inputs (no codec): returns (y [M, N], rstd [M])."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        w = np.ascontiguousarray(w, dtype=np.float64)
        M, N = x.shape
        y = np.empty((M, N), dtype=np.float64)
        r = np.empty((M,), dtype=np.float64)
        rc = self._lib.oracle_rmsnorm_fwd_f64(x.ctypes.data_as(_F64P), w.ctypes.data_as(_F64P),
                                              M, N, eps, offset, y.ctypes.data_as(_F64P),
                                              r.ctypes.data_as(_F64P))
        if rc != 0:
            raise ValueError("oracle rejected arguments")
        return y, r

    def rmsnorm_bwd(self, x_bits, w_bits, dy_bits, rstd, offset: float, dtype: str,
                    want_exact: bool = False):
        """Oracle backward.  x_bits, dy_bits uint16 [M, N]; w_bits uint16 [N];
        rstd [M] (taken as given, widened to fp64).  Returns (dx_bits uint16
        [M, N], dw float64 [N]) and, if ``want_exact``, also dx before
        rounding, the per-element term scale of dx and the per-column term
        scale of dw (see rmsnorm_oracle.c)."""
        x, w, dy = _u16(x_bits), _u16(w_bits), _u16(dy_bits)
        if x.ndim != 2 or dy.shape != x.shape or w.shape != (x.shape[1],):
            raise ValueError(f"shape mismatch: x {x.shape}, dy {dy.shape}, w {w.shape}")
        M, N = x.shape
        r = np.ascontiguousarray(rstd, dtype=np.float64)
        if r.shape != (M,):
            raise ValueError(f"rstd must have shape [{M}]")
        dx = np.empty((M, N), dtype=np.uint16)
        dw = np.empty((N,), dtype=np.float64)
        ex = np.empty((M, N), dtype=np.float64) if want_exact else None
        sc = np.empty((M, N), dtype=np.float64) if want_exact else None
        ws = np.empty((N,), dtype=np.float64) if want_exact else None
        ptr = lambda a: a.ctypes.data_as(_F64P) if a is not None else None
        rc = self._lib.oracle_rmsnorm_bwd(
            x.ctypes.data_as(_U16P), w.ctypes.data_as(_U16P), dy.ctypes.data_as(_U16P),
            r.ctypes.data_as(_F64P), M, N, ctypes.c_float(offset), _code(dtype),
            dx.ctypes.data_as(_U16P), dw.ctypes.data_as(_F64P), ptr(ex), ptr(sc), ptr(ws))
        if rc != 0:
            raise ValueError(f"oracle rejected arguments (M={M}, N={N}, dtype={dtype})")
        if want_exact:
            return dx, dw, ex, sc, ws
        return dx, dw

    def rmsnorm_bwd_f64(self, x, w, dy, rstd, offset: float):
        """Backward on fp64 inputs (fp32 values widen exactly), no codec.
        Returns (dx before rounding, dw, dx term scale, dw term scale), all
        float64; ``offset`` is used as given (pass an fp32 value)."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        dy = np.ascontiguousarray(dy, dtype=np.float64)
        w = np.ascontiguousarray(w, dtype=np.float64)
        if x.ndim != 2 or dy.shape != x.shape or w.shape != (x.shape[1],):
            raise ValueError(f"shape mismatch: x {x.shape}, dy {dy.shape}, w {w.shape}")
        M, N = x.shape
        r = np.ascontiguousarray(rstd, dtype=np.float64)
        if r.shape != (M,):
            raise ValueError(f"rstd must have shape [{M}]")
        ex = np.empty((M, N), dtype=np.float64)
        dw = np.empty((N,), dtype=np.float64)
        sc = np.empty((M, N), dtype=np.float64)
        ws = np.empty((N,), dtype=np.float64)
        rc = self._lib.oracle_rmsnorm_bwd_f64(
            x.ctypes.data_as(_F64P), w.ctypes.data_as(_F64P), dy.ctypes.data_as(_F64P), r.ctypes.data_as(_F64P),
            M, N, float(offset), ex.ctypes.data_as(_F64P), dw.ctypes.data_as(_F64P), sc.ctypes.data_as(_F64P),
            ws.ctypes.data_as(_F64P))
        if rc != 0:
            raise ValueError(f"oracle rejected arguments (M={M}, N={N})")
        return ex, dw, sc, ws

    def max_threads(self) -> int:
        """Threads the OpenMP loop uses (OMP_NUM_THREADS, else all cores)."""
        return int(self._lib.oracle_max_threads())

    def set_threads(self, n: int) -> None:
        """Threads for later calls (timing only; results do not depend on it)."""
        self._lib.oracle_set_threads(int(n))


_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from ``rmsnorm_oracle.c`` (rebuilt when the source is newer)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        _default = Oracle(LIBRARY)
    return _default


def decode(bits, dtype: str) -> np.ndarray:
    return default().decode(bits, dtype)


def encode(values, dtype: str) -> np.ndarray:
    return default().encode(values, dtype)


def rmsnorm_fwd(x_bits, w_bits, eps: float, offset: float, dtype: str, want_exact: bool = False):
    return default().rmsnorm_fwd(x_bits, w_bits, eps, offset, dtype, want_exact)


def rmsnorm_fwd_f64(x, w, eps: float, offset: float):
    return default().rmsnorm_fwd_f64(x, w, eps, offset)


def rmsnorm_bwd(x_bits, w_bits, dy_bits, rstd, offset: float, dtype: str, want_exact: bool = False):
    return default().rmsnorm_bwd(x_bits, w_bits, dy_bits, rstd, offset, dtype, want_exact)


def rmsnorm_bwd_f64(x, w, dy, rstd, offset: float):
    return default().rmsnorm_bwd_f64(x, w, dy, rstd, offset)


def max_threads() -> int:
    return default().max_threads()
