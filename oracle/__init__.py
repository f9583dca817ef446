"""Binary64 CPU oracle for row-wise LayerNorm / RMSNorm / fused add+RMSNorm,
forward and backward.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product package.  It shares no
code with the HIP path; see oracle.c for the definitions and the passages
each one follows.

Arrays are numpy.  Storage formats: bfloat16 and IEEE binary16 tensors are
carried as uint16 bit patterns, fp32 as float32.  The math functions take and return float64.

Parity status: every function here is pinned by tests/test_oracle_*.py
against closed forms, invariants, finite differences, brute force or exact
rational arithmetic (see the docstring of each test module).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_i64 = ctypes.c_int64
_dbl = ctypes.c_double
_P = ctypes.c_void_p

_SIGNATURES = {
    "orc_ln_fwd": [_i64, _i64, _P, _i64, _P, _P, _dbl, _P, _i64, _P, _P],
    "orc_rms_fwd": [_i64, _i64, _P, _i64, _P, _dbl, _P, _i64, _P],
    "orc_fused_add_rms_fwd": [_i64, _i64, _P, _i64, _P, _i64, _P, _dbl,
                              _P, _i64, _P, _i64, _P],
    "orc_ln_bwd": [_i64, _i64, _P, _i64, _P, _i64, _P, _dbl, _P, _i64,
                   _P, _P, _P, _P],
    "orc_rms_bwd": [_i64, _i64, _P, _i64, _P, _i64, _P, _dbl, _P, _i64,
                    _P, _P],
    "orc_fused_add_rms_bwd": [_i64, _i64, _P, _i64, _P, _i64, _P, _P, _P,
                              _i64, _P, _i64, _P],
    "orc_welford": [_P, _i64, _P, _P, _P],
    "orc_welford_merge": [_dbl, _dbl, _dbl, _dbl, _dbl, _dbl, _P, _P, _P],
    "orc_bf16_decode": [_P, _P, _i64],
    "orc_bf16_encode": [_P, _P, _i64],
    "orc_f32_encode": [_P, _P, _i64],
    "orc_f16_decode": [_P, _P, _i64],
    "orc_f16_encode": [_P, _P, _i64],
    "orc_num_threads": [],
    "orc_set_threads": [ctypes.c_int],
}


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def eps_at_boundary(eps: float) -> float:
    """eps as the C boundary carries it: a binary32 value, widened exactly.
    (Reading: the pages leave eps's type open; the library takes a float, so
    the oracle uses the same binary32 value.)"""
    return float(np.float32(eps))


class Oracle:
    """ctypes view of one build of oracle.c (the default build, or a test's
    deliberately mutated copy)."""

    def __init__(self, lib_path: str = LIB_PATH):
        if lib_path == LIB_PATH and not os.path.exists(lib_path):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(lib_path)
        for name, args in _SIGNATURES.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_int if name == "orc_num_threads" else None
        self.lib = lib
        self.path = lib_path

    def num_threads(self) -> int:
        return int(self.lib.orc_num_threads())

    def set_threads(self, n: int) -> None:
        """OpenMP threads for later calls (the CPU baseline's 1-thread run)."""
        self.lib.orc_set_threads(int(n))

    # ------------------------------------------------------------ codec --
    def bf16_decode(self, bits):
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, dtype=np.float64)
        self.lib.orc_bf16_decode(_p(bits), _p(out), bits.size)
        return out

    def bf16_encode(self, v):
        v = _f64(v)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.orc_bf16_encode(_p(v), _p(out), v.size)
        return out

    def f16_decode(self, bits):
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, dtype=np.float64)
        self.lib.orc_f16_decode(_p(bits), _p(out), bits.size)
        return out

    def f16_encode(self, v):
        v = _f64(v)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.orc_f16_encode(_p(v), _p(out), v.size)
        return out

    def f32_encode(self, v):
        v = _f64(v)
        out = np.empty(v.shape, dtype=np.float32)
        self.lib.orc_f32_encode(_p(v), _p(out), v.size)
        return out

    def decode(self, a, dtype: str):
        """Storage array -> float64 (exact)."""
        if dtype == "bf16":
            return self.bf16_decode(a)
        if dtype == "f16":
            return self.f16_decode(a)
        if dtype == "f32":
            return np.asarray(a, dtype=np.float32).astype(np.float64)
        raise ValueError(dtype)

    def encode(self, v, dtype: str):
        """float64 -> storage array, one correctly rounded step (RNE)."""
        if dtype == "bf16":
            return self.bf16_encode(v)
        if dtype == "f16":
            return self.f16_encode(v)
        if dtype == "f32":
            return self.f32_encode(v)
        raise ValueError(dtype)

    # ---------------------------------------------------------- forward --
    def ln_fwd(self, x, gamma, beta, eps):
        """LayerNorm forward.  Returns (y, mean, rstd), all float64."""
        x = _f64(x)
        N, H = x.shape
        gamma = _f64(gamma)
        beta = None if beta is None else _f64(beta)
        y = np.empty_like(x)
        mean = np.empty(N)
        rstd = np.empty(N)
        self.lib.orc_ln_fwd(N, H, _p(x), H, _p(gamma), _p(beta), float(eps),
                            _p(y), H, _p(mean), _p(rstd))
        return y, mean, rstd

    def rms_fwd(self, x, gamma, eps):
        """RMSNorm forward.  Returns (y, rstd)."""
        x = _f64(x)
        N, H = x.shape
        gamma = _f64(gamma)
        y = np.empty_like(x)
        rstd = np.empty(N)
        self.lib.orc_rms_fwd(N, H, _p(x), H, _p(gamma), float(eps), _p(y), H,
                             _p(rstd))
        return y, rstd

    def fused_add_rms_fwd(self, x, res, gamma, eps):
        """Fused residual add + RMSNorm forward.  Returns (y, h, rstd) with h
        the exact (unrounded) x + res."""
        x = _f64(x)
        res = _f64(res)
        N, H = x.shape
        gamma = _f64(gamma)
        y = np.empty_like(x)
        h = np.empty_like(x)
        rstd = np.empty(N)
        self.lib.orc_fused_add_rms_fwd(N, H, _p(x), H, _p(res), H, _p(gamma),
                                       float(eps), _p(y), H, _p(h), H,
                                       _p(rstd))
        return y, h, rstd

    # --------------------------------------------------------- backward --
    def ln_bwd(self, dy, x, gamma, eps):
        """LayerNorm backward.  Returns (dx, dgamma, dbeta, mean, rstd); the
        statistics are recomputed from x in binary64."""
        dy = _f64(dy)
        x = _f64(x)
        N, H = x.shape
        gamma = _f64(gamma)
        dx = np.empty_like(x)
        dg = np.empty(H)
        db = np.empty(H)
        mean = np.empty(N)
        rstd = np.empty(N)
        self.lib.orc_ln_bwd(N, H, _p(dy), H, _p(x), H, _p(gamma), float(eps),
                            _p(dx), H, _p(dg), _p(db), _p(mean), _p(rstd))
        return dx, dg, db, mean, rstd

    def rms_bwd(self, dy, x, gamma, eps):
        """RMSNorm backward.  Returns (dx, dgamma, rstd)."""
        dy = _f64(dy)
        x = _f64(x)
        N, H = x.shape
        gamma = _f64(gamma)
        dx = np.empty_like(x)
        dg = np.empty(H)
        rstd = np.empty(N)
        self.lib.orc_rms_bwd(N, H, _p(dy), H, _p(x), H, _p(gamma), float(eps),
                             _p(dx), H, _p(dg), _p(rstd))
        return dx, dg, rstd

    def fused_add_rms_bwd(self, dy, h, gamma, rstd, dh_in=None):
        """Fused add+RMSNorm backward at the stored h with the forward's
        saved rstd.  Returns (dx, dgamma); dx is also the residual's
        gradient."""
        dy = _f64(dy)
        h = _f64(h)
        N, H = h.shape
        gamma = _f64(gamma)
        rstd = _f64(rstd)
        dh_in = None if dh_in is None else _f64(dh_in)
        dx = np.empty_like(h)
        dg = np.empty(H)
        self.lib.orc_fused_add_rms_bwd(N, H, _p(dy), H, _p(h), H, _p(gamma),
                                       _p(rstd), _p(dh_in), H, _p(dx), H, _p(dg))
        return dx, dg

    # ---------------------------------------------------------- welford --
    def welford(self, x):
        """Sequential Welford over a 1-D array: (count, mean, M2)."""
        x = _f64(x).ravel()
        n, m, q = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        self.lib.orc_welford(_p(x), x.size, ctypes.byref(n), ctypes.byref(m),
                             ctypes.byref(q))
        return n.value, m.value, q.value

    def welford_merge(self, a, b):
        """Parallel merge of two (count, mean, M2) states."""
        n, m, q = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        self.lib.orc_welford_merge(float(a[0]), float(a[1]), float(a[2]),
                                   float(b[0]), float(b[1]), float(b[2]),
                                   ctypes.byref(n), ctypes.byref(m),
                                   ctypes.byref(q))
        return n.value, m.value, q.value


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def __getattr__(name):
    # module-level shortcuts: oracle.ln_fwd(...) etc. use the default build.
    # Submodule names fall through to the import system (the first
    # `from oracle import build` in a fresh tree runs before liboracle.so
    # exists, so it must not try to load it).
    if name.startswith("_") or name in ("build",):
        raise AttributeError(name)
    return getattr(default(), name)
