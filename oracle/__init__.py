"""fp64 CPU oracle for the block-dequant GEMV -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module. The product library never does, and the
two share no code: this wrapper loads ``oracle/liboracle.so`` built from the
plain C in ``oracle/oracle.c`` and nothing else.

Every function returns float64 numpy arrays: ``y`` (the product) and ``a``
(sum of |w_k * x_k| per output, the scale of the acceptance tolerance).
Canonical block bytes in, as produced by the seeded generators: GGUF-style
Q8_0 (34 B per 32 weights) and Q4_0 (18 B per 32 weights) blocks, or fp16
row-major weights.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

Q8_0, Q4_0, F16, Q4_K, Q6_K = 1, 2, 3, 4, 5
KINDS = {"q8_0": Q8_0, "q4_0": Q4_0, "f16": F16, "q4_k": Q4_K, "q6_k": Q6_K}


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (plain -O2, no vector intrinsics, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib(path: str | None = None):
    """Load (building first if needed) the oracle shared library."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        _lib = _declare(ctypes.CDLL(build()))
    return _lib


def _declare(L):
    i64, i32, vp, dp, fp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    L.oracle_half_to_double.restype = ctypes.c_double
    L.oracle_silu.argtypes = [ctypes.c_double]
    L.oracle_silu.restype = ctypes.c_double
    L.oracle_gemv.argtypes = [i32, vp, fp, dp, dp, i64, i64, i32]
    L.oracle_gemv.restype = i32
    L.oracle_gemv_range.argtypes = [i32, vp, fp, dp, dp, i64, i64, i64, i64]
    L.oracle_gemv_range.restype = i32
    L.oracle_gemv_rows.argtypes = [i32, vp, fp, vp, i64, dp, dp, i64, i64]
    L.oracle_gemv_rows.restype = i32
    L.oracle_gateup_silu.argtypes = [i32, vp, vp, fp, dp, dp, dp, dp, dp, i64, i64, i32]
    L.oracle_gateup_silu.restype = i32
    L.oracle_verify.argtypes = [i32, vp, fp, dp, dp, i64, i64, i32, i32]
    L.oracle_gemv_epilogue.argtypes = [i32, vp, fp, fp, fp, dp, dp, i64, i64, i32]
    L.oracle_gemv_epilogue.restype = i32
    L.oracle_verify.restype = i32
    L.oracle_rmsnorm.argtypes = [fp, fp, ctypes.c_double, dp, i64]
    L.oracle_rmsnorm.restype = i32
    L.oracle_gemv_rmsnorm.argtypes = [i32, vp, fp, fp, ctypes.c_double, dp, dp, i64, i64]
    L.oracle_gemv_rmsnorm.restype = i32
    L.oracle_gateup_silu_rmsnorm.argtypes = [i32, vp, vp, fp, fp, ctypes.c_double, dp, dp, dp, dp, dp, i64, i64]
    L.oracle_gateup_silu_rmsnorm.restype = i32
    return L


def _kind(kind) -> int:
    return KINDS[kind] if isinstance(kind, str) else int(kind)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check_w(kind: int, w: np.ndarray, N: int, K: int):
    w = np.ascontiguousarray(w)
    if kind == Q8_0:
        need = N * (K // 32) * 34
    elif kind == Q4_0:
        need = N * (K // 32) * 18
    elif kind == Q4_K:
        need = N * (K // 256) * 144
    elif kind == Q6_K:
        need = N * (K // 256) * 210
    else:
        need = N * K * 2
    if w.nbytes != need:
        raise ValueError(f"weight buffer has {w.nbytes} bytes, expected {need}")
    return w


def gemv(kind, w: np.ndarray, x: np.ndarray, N: int, K: int, threads: int = 1, L=None):
    """y[n] = sum_k W[n,k] x[k] in fp64, plus a[n] = sum_k |W[n,k] x[k]|."""
    L = L or lib()
    k = _kind(kind)
    w = _check_w(k, w, N, K)
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.size == K
    y = np.empty(N, np.float64)
    a = np.empty(N, np.float64)
    rc = L.oracle_gemv(k, _ptr(w), _ptr(x), _ptr(y), _ptr(a), N, K, threads)
    if rc:
        raise ValueError("oracle_gemv rejected its arguments")
    return y, a


def gemv_rows(kind, w: np.ndarray, x: np.ndarray, rows, N: int, K: int, L=None):
    """The same product for a chosen list of rows only (for very large N)."""
    L = L or lib()
    k = _kind(kind)
    w = _check_w(k, w, N, K)
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    y = np.empty(rows.size, np.float64)
    a = np.empty(rows.size, np.float64)
    rc = L.oracle_gemv_rows(k, _ptr(w), _ptr(x), _ptr(rows), rows.size, _ptr(y), _ptr(a), N, K)
    if rc:
        raise ValueError("oracle_gemv_rows rejected its arguments")
    return y, a


def gateup_silu(kind, gate: np.ndarray, up: np.ndarray, x: np.ndarray, N_ff: int, K: int,
                threads: int = 1, L=None):
    """out[n] = silu(g[n]) * u[n]; also returns g, u and their magnitude sums."""
    L = L or lib()
    k = _kind(kind)
    gate = _check_w(k, gate, N_ff, K)
    up = _check_w(k, up, N_ff, K)
    x = np.ascontiguousarray(x, dtype=np.float32)
    out, g, u, ag, au = (np.empty(N_ff, np.float64) for _ in range(5))
    rc = L.oracle_gateup_silu(k, _ptr(gate), _ptr(up), _ptr(x), _ptr(out), _ptr(g), _ptr(u),
                              _ptr(ag), _ptr(au), N_ff, K, threads)
    if rc:
        raise ValueError("oracle_gateup_silu rejected its arguments")
    return out, g, u, ag, au


def gemv_epilogue(kind, w: np.ndarray, x: np.ndarray, N: int, K: int, bias=None, residual=None,
                  threads: int = 1, L=None):
    """out[n] = sum_k W[n][k] x[k] + bias[n] + residual[n] (either may be None); also the
    product's magnitude sums."""
    L = L or lib()
    k = _kind(kind)
    w = _check_w(k, w, N, K)
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    r = None if residual is None else np.ascontiguousarray(residual, dtype=np.float32)
    for v in (b, r):
        if v is not None and v.shape != (N,):
            raise ValueError("bias and residual must have N entries")
    out = np.empty(N, np.float64)
    a = np.empty(N, np.float64)
    rc = L.oracle_gemv_epilogue(k, _ptr(w), _ptr(x), None if b is None else _ptr(b), None if r is None else _ptr(r),
                                _ptr(out), _ptr(a), N, K, threads)
    if rc:
        raise ValueError("oracle_gemv_epilogue rejected its arguments")
    return out, a


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float, L=None) -> np.ndarray:
    """gamma * x / sqrt(mean(x^2) + eps) in fp64 (eps is used as given, e.g. an fp32 value)."""
    L = L or lib()
    x = np.ascontiguousarray(x, dtype=np.float32)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    if gamma.shape != x.shape:
        raise ValueError("gamma must have K entries")
    out = np.empty(x.size, np.float64)
    if L.oracle_rmsnorm(_ptr(x), _ptr(gamma), float(eps), _ptr(out), x.size):
        raise ValueError("oracle_rmsnorm rejected its arguments")
    return out


def gemv_rmsnorm(kind, w: np.ndarray, x: np.ndarray, gamma: np.ndarray, eps: float, N: int, K: int, L=None):
    """y = W rmsnorm(x) in fp64 (the normalised activation exact in double), and a = sum |W xn|."""
    L = L or lib()
    k = _kind(kind)
    w = _check_w(k, w, N, K)
    x = np.ascontiguousarray(x, dtype=np.float32)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    assert x.size == K and gamma.size == K
    y = np.empty(N, np.float64)
    a = np.empty(N, np.float64)
    if L.oracle_gemv_rmsnorm(k, _ptr(w), _ptr(x), _ptr(gamma), float(eps), _ptr(y), _ptr(a), N, K):
        raise ValueError("oracle_gemv_rmsnorm rejected its arguments")
    return y, a


def gateup_silu_rmsnorm(kind, gate: np.ndarray, up: np.ndarray, x: np.ndarray, gamma: np.ndarray, eps: float,
                        N_ff: int, K: int, L=None):
    """out = silu(Wgate xn) * (Wup xn) with xn = rmsnorm(x); also g, u and their magnitude sums."""
    L = L or lib()
    k = _kind(kind)
    gate = _check_w(k, gate, N_ff, K)
    up = _check_w(k, up, N_ff, K)
    x = np.ascontiguousarray(x, dtype=np.float32)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    out, g, u, ag, au = (np.empty(N_ff, np.float64) for _ in range(5))
    if L.oracle_gateup_silu_rmsnorm(k, _ptr(gate), _ptr(up), _ptr(x), _ptr(gamma), float(eps), _ptr(out), _ptr(g),
                                    _ptr(u), _ptr(ag), _ptr(au), N_ff, K):
        raise ValueError("oracle_gateup_silu_rmsnorm rejected its arguments")
    return out, g, u, ag, au


def verify(kind, w: np.ndarray, X: np.ndarray, N: int, K: int, threads: int = 1, L=None):
    """Y[m] = W X[m] for each activation row m (each row is its own M=1 product)."""
    L = L or lib()
    k = _kind(kind)
    w = _check_w(k, w, N, K)
    X = np.ascontiguousarray(X, dtype=np.float32)
    M = X.shape[0]
    Y = np.empty((M, N), np.float64)
    A = np.empty((M, N), np.float64)
    rc = L.oracle_verify(k, _ptr(w), _ptr(X), _ptr(Y), _ptr(A), N, K, M, threads)
    if rc:
        raise ValueError("oracle_verify rejected its arguments")
    return Y, A


def half_to_double(bits: int, L=None) -> float:
    return (L or lib()).oracle_half_to_double(bits)


def silu(g: float, L=None) -> float:
    return (L or lib()).oracle_silu(g)


# ---- acceptance bounds (stated once, used by every parity test) ----------

def linear_tol(a: np.ndarray) -> np.ndarray:
    """|y_gpu - y_ref| <= 1e-5 * sum_k |w_k x_k| + 1e-7 for every linear output."""
    return 1e-5 * a + 1e-7


def epilogue_tol(a: np.ndarray, bias=None, residual=None, out=None, f16: bool = False) -> np.ndarray:
    """Bound for an epilogue output: the linear bound widened by the magnitudes of
    the fp32 addends (each addition rounds once in fp32), plus, for an fp16
    output, the fp16 rounding of the fp32 value (at most 2^-11 of its magnitude,
    or 2^-25 in the subnormal range)."""
    mag = np.asarray(a, np.float64).copy()
    for v in (bias, residual):
        if v is not None:
            mag = mag + np.abs(np.asarray(v, np.float64))
    tol = linear_tol(mag)
    if f16:
        tol = tol + 2.0 ** -11 * (np.abs(np.asarray(out, np.float64)) + tol) + 2.0 ** -25
    return tol


def silu_tol(g: np.ndarray, u: np.ndarray, ag: np.ndarray, au: np.ndarray, out: np.ndarray) -> np.ndarray:
    """Bound for out = silu(g) * u given the linear bounds tg, tu on g and u.

    silu' is at most 1.0998 in magnitude, so the gate error moves silu by at most
    1.1*tg; the product then adds |silu(g)|*tu, and a relative 1e-6 covers the
    fp32 exp, divide and multiply of the epilogue.
    """
    tg = linear_tol(ag)
    tu = linear_tol(au)
    s = g / (1.0 + np.exp(-g))
    return 1.1 * tg * (np.abs(u) + tu) + np.abs(s) * tu + 1e-6 * np.abs(out) + 1e-7
