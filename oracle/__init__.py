"""Python face of the CPU oracle (oracle.cpp).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It shares no code with the HIP
library; it takes plain numpy arrays and returns plain numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, ERR_ARG, ERR_COORD_RANGE, ERR_DUPLICATE = 0, -1, -2, -3


class OracleError(RuntimeError):
    def __init__(self, status: int):
        names = {ERR_ARG: "bad argument", ERR_COORD_RANGE: "coordinate out of range",
                 ERR_DUPLICATE: "duplicate coordinate"}
        super().__init__(f"oracle status {status}: {names.get(status, 'unknown')}")
        self.status = status


def build(force: bool = True) -> str:
    """Compile oracle.cpp with g++ into liboracle.so next to it."""
    if force or not os.path.exists(_LIB):
        cmd = ["g++", "-O3", "-march=x86-64-v3", "-fopenmp", "-shared", "-fPIC", "-std=c++17",
               _SRC, "-o", _LIB + ".tmp"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        lib.oracle_build_map.argtypes = [p, i64, i32, i32, i32, i32, i32, p]
        lib.oracle_build_map.restype = ctypes.c_int
        lib.oracle_conv.argtypes = [p, p, p, p, i64, i32, i32, i32, i32, p]
        lib.oracle_conv.restype = None
        lib.oracle_linear.argtypes = [p, p, p, i64, i32, i32, p]
        lib.oracle_linear.restype = None
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on (n >= 1)."""
    _load().oracle_set_num_threads(int(n))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def build_map(coords, batch: int, grid, ksize: int = 3) -> np.ndarray:
    """[N, ksize^3] int32 neighbour map by dictionary lookup; raises OracleError on bad input."""
    c = np.ascontiguousarray(np.asarray(coords, dtype=np.int32).reshape(-1, 4))
    n = c.shape[0]
    taps = ksize ** 3
    out = np.empty((n, taps), dtype=np.int32)
    st = _load().oracle_build_map(_ptr(c), n, int(batch), int(grid[0]), int(grid[1]),
                                  int(grid[2]), int(ksize), _ptr(out))
    if st != OK:
        raise OracleError(st)
    return out


def conv(x, w, bias, nbr, flip: bool = False) -> np.ndarray:
    """fp64 Y = bias + sum over taps of X[nbr[:, t]] @ W[t]; inputs are upcast exactly."""
    X = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    W = np.ascontiguousarray(np.asarray(w, dtype=np.float64))
    M = np.ascontiguousarray(np.asarray(nbr, dtype=np.int32))
    n, cin = X.shape
    taps, wcin, cout = W.shape
    assert wcin == cin and M.shape == (n, taps)
    B = None if bias is None else np.ascontiguousarray(np.asarray(bias, dtype=np.float64))
    Y = np.empty((n, cout), dtype=np.float64)
    _load().oracle_conv(_ptr(X), _ptr(W), None if B is None else _ptr(B), _ptr(M), n, taps,
                        cin, cout, int(bool(flip)), _ptr(Y))
    return Y


def linear(x, w, bias) -> np.ndarray:
    """fp64 per-voxel linear map Y = X @ W + bias (W is [cin, cout] or [1, cin, cout])."""
    X = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    W = np.asarray(w, dtype=np.float64)
    if W.ndim == 3:
        W = W[0]
    W = np.ascontiguousarray(W)
    n, cin = X.shape
    assert W.shape[0] == cin
    cout = W.shape[1]
    B = None if bias is None else np.ascontiguousarray(np.asarray(bias, dtype=np.float64))
    Y = np.empty((n, cout), dtype=np.float64)
    _load().oracle_linear(_ptr(X), _ptr(W), None if B is None else _ptr(B), n, cin, cout,
                          _ptr(Y))
    return Y
