"""ctypes front end of the fp64 sequential oracle (ssd_oracle.c).

TEST INFRASTRUCTURE ONLY. Inputs are float64 arrays that hold the exact
values the scan under test reads (widened from bf16 or fp32 storage).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

_lib = None


def ensure_built() -> str:
    if not os.path.exists(_build.LIB) or (
            os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
        _build.build()
    return _build.LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(ensure_built())
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_int64)
        i32 = ctypes.c_int32
        lib.ssd_oracle_scan.restype = ctypes.c_int
        lib.ssd_oracle_scan.argtypes = [i32, lp, i32, i32, i32, i32, i32,
                                        dp, dp, dp, dp, dp, i32, dp, dp, dp,
                                        dp, dp, dp, lp, dp, i32]
        lib.ssd_oracle_threads.restype = ctypes.c_int
        lib.ssd_oracle_set_threads.restype = None
        lib.ssd_oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def threads() -> int:
    return int(_load().ssd_oracle_threads())


def set_threads(n: int) -> None:
    """Threads of later scans (timing of the oracle itself; results do not
    depend on it)."""
    _load().ssd_oracle_set_threads(int(n))


def _dptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


@dataclass
class ScanResult:
    y: np.ndarray               # [T, H, P]
    final_state: np.ndarray     # [S, H, P, N]
    boundary_state: np.ndarray  # [S, H, P, N] state at the last multiple of Q
    boundary_len: np.ndarray    # [S] tokens after that boundary
    chunk_states: np.ndarray | None  # [S, max_chunks, H, P, N]


def scan(x, dt, A, B, C, cu, chunk_size, D=None, dt_bias=None,
         dt_softplus=True, init=None, max_chunks=0) -> ScanResult:
    """Sequential fp64 recurrence over a varlen pack.

    x[T,H,P], dt[T,H], B/C[T,G,N], A/D/dt_bias[H], cu[S+1], init[S,H,P,N].
    """
    x, dt, B, C = _f64(x), _f64(dt), _f64(B), _f64(C)
    A, D, dt_bias, init = _f64(A), _f64(D), _f64(dt_bias), _f64(init)
    cu = np.ascontiguousarray(cu, dtype=np.int64)
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    S = cu.shape[0] - 1
    assert dt.shape == (T, H) and B.shape == (T, G, N) and C.shape == (T, G, N)
    assert cu[-1] == T and cu[0] == 0
    y = np.zeros((T, H, P))
    fin = np.zeros((S, H, P, N))
    bnd = np.zeros((S, H, P, N))
    blen = np.zeros(S, dtype=np.int64)
    cs = np.zeros((S, max_chunks, H, P, N)) if max_chunks > 0 else None
    rc = _load().ssd_oracle_scan(
        S, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, G, P, N,
        int(chunk_size), _dptr(x), _dptr(dt), _dptr(A), _dptr(D),
        _dptr(dt_bias), int(bool(dt_softplus)), _dptr(B), _dptr(C),
        _dptr(init), _dptr(y), _dptr(fin), _dptr(bnd),
        blen.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _dptr(cs),
        int(max_chunks))
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_scan failed with {rc}")
    return ScanResult(y, fin, bnd, blen, cs)
