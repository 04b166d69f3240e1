"""Shared helpers of the GPU parity tests (device side via the C ABI, oracle on the CPU)."""
from __future__ import annotations

import os
import sys

import numpy as np

import oracle as O

THREADS = max(1, min(256, len(os.sched_getaffinity(0))))   # the CPUs this process may run on


def announce(msg: str):
    """Name the case on the real stderr before each GPU step (survives output capture)."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def to_dev(a: np.ndarray):
    torch = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def empty_f32(n: int, fill: float | None = None):
    torch = torch_dev()
    t = torch.empty(n, dtype=torch.float32, device="cuda")
    if fill is not None:
        t.fill_(fill)
    return t


def sync():
    torch_dev().cuda.synchronize()


def assert_linear(y_gpu: np.ndarray, y_ref: np.ndarray, a_ref: np.ndarray, ctx: str):
    """|y_gpu - y_ref| <= 1e-5 * sum|w x| + 1e-7 for every output."""
    y_gpu = np.asarray(y_gpu, np.float64)
    assert y_gpu.shape == y_ref.shape, ctx
    assert np.all(np.isfinite(y_gpu)), f"{ctx}: non-finite outputs"
    err = np.abs(y_gpu - y_ref)
    tol = O.linear_tol(a_ref)
    bad = np.flatnonzero(err > tol)
    if bad.size:
        i = bad[np.argmax(err[bad] / tol[bad])]
        raise AssertionError(f"{ctx}: {bad.size}/{y_ref.size} outputs out of tolerance; worst row {i}: "
                             f"gpu {y_gpu[i]!r} ref {y_ref[i]!r} err {err[i]:.3e} tol {tol[i]:.3e}")
    return float(np.max(err / tol)) if err.size else 0.0


def assert_silu(y_gpu, out, g, u, ag, au, ctx: str):
    y_gpu = np.asarray(y_gpu, np.float64)
    assert np.all(np.isfinite(y_gpu)), f"{ctx}: non-finite outputs"
    err = np.abs(y_gpu - out)
    tol = O.silu_tol(g, u, ag, au, out)
    bad = np.flatnonzero(err > tol)
    if bad.size:
        i = bad[np.argmax(err[bad] / tol[bad])]
        raise AssertionError(f"{ctx}: {bad.size}/{out.size} outputs out of tolerance; worst {i}: "
                             f"gpu {y_gpu[i]!r} ref {out[i]!r} err {err[i]:.3e} tol {tol[i]:.3e}")
    return float(np.max(err / tol)) if err.size else 0.0


def run_qgemv(kind: str, canon: np.ndarray, x: np.ndarray, N: int, K: int, canary: int = 0):
    """Pack on the device, run qgemv_<kind>, return y (and the canary tail if asked)."""
    import block_dequant_gemv_amd as qg
    packed = qg.pack_weights(kind, canon, N, K)
    xd = to_dev(x.astype(np.float32))
    y = empty_f32(N + canary, fill=12345.0)
    qg.qgemv(kind, packed, xd, y, N, K)
    sync()
    out = y.cpu().numpy()
    return (out[:N], out[N:]) if canary else out
