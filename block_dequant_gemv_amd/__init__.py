"""Python binding of libqgemv.so, the MI355X block-dequant GEMV library.

A thin ctypes layer over the C ABI in include/qgemv.h: the functions have the
same names and arguments, take torch tensors (device memory) or numpy arrays
(host memory) and only marshal pointers, sizes and the HIP stream. Every step
of the computation runs in the library's HIP kernels; there is no fallback.
If the library is not built, or a call fails, an exception is raised.

Build the library with ``python -m block_dequant_gemv_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

Q8_0 = 1
Q4_0 = 2
Q4_K = 3
Q6_K = 4
QTYPES = {"q8_0": Q8_0, "q4_0": Q4_0, "q4_k": Q4_K, "q6_k": Q6_K}

QG_OK, QG_EINVAL, QG_EALIGN, QG_EUNSUPPORTED, QG_EHIP = range(5)
QG_OUT_F32, QG_OUT_F16 = 0, 1

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqgemv.so")

# every function declared in include/qgemv.h
SYMBOLS = (
    "qg_packed_size", "qg_pack", "qg_pack_rows", "qg_pack_gateup",
    "qg_pack_host", "qg_unpack_host", "qg_pack_gateup_host",
    "qgemv_q8_0", "qgemv_q4_0", "qgemv_q4_k", "qgemv_q6_k", "qgemv_epilogue", "gemv_f16_splitk", "qgemv_fused_gateup_silu", "qgemv_verify",
    "qg_rmsnorm", "qgemv_rmsnorm", "qgemv_rmsnorm_gateup_silu", "qg_prefill_workspace_size", "qgemm_prefill",
    "qgemm_prefill_noalloc",
    "qg_status_str", "qg_last_error", "qg_plan_info", "qg_f16_plan_info", "qg_time_next_launch", "qg_reload_tuning",
    "qg_probe_stream", "qg_probe_empty",
)


class QGError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


_lib = None


def lib():
    """Load libqgemv.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run python -m block_dequant_gemv_amd.build")
        # torch bundles its own HIP runtime under the same soname as ROCm's. Load
        # torch first so that libqgemv binds to that one runtime: the library
        # receives torch's device pointers and streams, and two runtimes in one
        # process would each try to own the device.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        sig = {
            "qg_packed_size": ([i32, i64, i64], sz),
            "qg_pack": ([i32, vp, vp, i64, i64, vp], i32),
            "qg_pack_rows": ([i32, vp, vp, i64, i64, i64, i64, vp], i32),
            "qg_pack_gateup": ([i32, vp, vp, vp, i64, i64, vp], i32),
            "qg_pack_host": ([i32, vp, vp, i64, i64], i32),
            "qg_unpack_host": ([i32, vp, vp, i64, i64], i32),
            "qg_pack_gateup_host": ([i32, vp, vp, vp, i64, i64], i32),
            "qgemv_q8_0": ([vp, vp, vp, i64, i64, vp], i32),
            "qgemv_q4_0": ([vp, vp, vp, i64, i64, vp], i32),
            "qgemv_q4_k": ([vp, vp, vp, i64, i64, vp], i32),
            "qgemv_q6_k": ([vp, vp, vp, i64, i64, vp], i32),
            "qgemv_epilogue": ([i32, vp, vp, vp, vp, vp, i32, i64, i64, vp], i32),
            "qg_rmsnorm": ([vp, vp, ctypes.c_float, vp, i64, vp], i32),
            "qg_prefill_workspace_size": ([i32, i64, i64, i64], sz),
            "qgemm_prefill": ([i32, vp, vp, vp, i64, i64, i64, vp, sz, vp], i32),
            "qgemm_prefill_noalloc": ([i32, vp, vp, vp, i64, i64, i64, vp], i32),
            "qgemv_rmsnorm": ([i32, vp, vp, vp, ctypes.c_float, vp, i64, i64, vp], i32),
            "qgemv_rmsnorm_gateup_silu": ([i32, vp, vp, vp, ctypes.c_float, vp, i64, i64, vp], i32),
            "gemv_f16_splitk": ([vp, vp, vp, i64, i64, vp], i32),
            "qgemv_fused_gateup_silu": ([i32, vp, vp, vp, i64, i64, vp], i32),
            "qgemv_verify": ([i32, vp, vp, vp, i64, i64, i32, vp], i32),
            "qg_status_str": ([i32], ctypes.c_char_p),
            "qg_last_error": ([], ctypes.c_char_p),
            "qg_plan_info": ([i32, i64, i64, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i64),
                              ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i64)], i32),
            "qg_f16_plan_info": ([i64, i64, vp, vp, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                  ctypes.POINTER(i64)], i32),
            "qg_time_next_launch": ([vp, vp], i32),
            "qg_probe_stream": ([vp, sz, vp, vp], i32),
            "qg_probe_empty": ([vp], i32),
            "qg_reload_tuning": ([], i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _qtype(q) -> int:
    return QTYPES[q] if isinstance(q, str) else int(q)


def _check(fn: str, status: int):
    if status != QG_OK:
        raise QGError(fn, status, lib().qg_last_error().decode())


def _stream(stream):
    """hipStream_t of `stream` (None = torch's current stream on the current device)."""
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev(t, name: str, dtype=None):
    """Device pointer of a contiguous torch CUDA tensor (None passes NULL through)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (CUDA/HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    return t.data_ptr()


def _host(a: np.ndarray, name: str):
    if not isinstance(a, np.ndarray) or not a.flags.c_contiguous:
        raise ValueError(f"{name} must be a C-contiguous numpy array")
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32():
    import torch
    return torch.float32


# ---- packing ---------------------------------------------------------------

def qg_packed_size(qtype, N: int, K: int) -> int:
    return int(lib().qg_packed_size(_qtype(qtype), N, K))


def qg_pack(qtype, canonical, packed, N: int, K: int, stream=None):
    _check("qg_pack", lib().qg_pack(_qtype(qtype), _dev(canonical, "canonical"), _dev(packed, "packed"),
                                    N, K, _stream(stream)))


def qg_pack_rows(qtype, canonical, packed, N_total: int, row0: int, nrows: int, K: int, stream=None):
    _check("qg_pack_rows", lib().qg_pack_rows(_qtype(qtype), _dev(canonical, "canonical"), _dev(packed, "packed"),
                                              N_total, row0, nrows, K, _stream(stream)))


def qg_pack_gateup(qtype, gate, up, packed, N_ff: int, K: int, stream=None):
    _check("qg_pack_gateup", lib().qg_pack_gateup(_qtype(qtype), _dev(gate, "gate"), _dev(up, "up"),
                                                  _dev(packed, "packed"), N_ff, K, _stream(stream)))


def qg_pack_host(qtype, canonical: np.ndarray, N: int, K: int) -> np.ndarray:
    out = np.empty(qg_packed_size(qtype, N, K), np.uint8)
    _check("qg_pack_host", lib().qg_pack_host(_qtype(qtype), _host(canonical, "canonical"), _host(out, "packed"),
                                              N, K))
    return out


def qg_unpack_host(qtype, packed: np.ndarray, N: int, K: int) -> np.ndarray:
    q = _qtype(qtype)
    row = {Q8_0: (K // 32) * 34, Q4_0: (K // 32) * 18, Q4_K: (K // 256) * 144, Q6_K: (K // 256) * 210}[q]
    out = np.empty(N * row, np.uint8)
    _check("qg_unpack_host", lib().qg_unpack_host(_qtype(qtype), _host(packed, "packed"), _host(out, "canonical"),
                                                  N, K))
    return out


def qg_pack_gateup_host(qtype, gate: np.ndarray, up: np.ndarray, N_ff: int, K: int) -> np.ndarray:
    out = np.empty(qg_packed_size(qtype, 2 * N_ff, K), np.uint8)
    _check("qg_pack_gateup_host", lib().qg_pack_gateup_host(_qtype(qtype), _host(gate, "gate"), _host(up, "up"),
                                                            _host(out, "packed"), N_ff, K))
    return out


# ---- GEMVs -----------------------------------------------------------------

def qgemv_q8_0(w_packed, x, y, N: int, K: int, stream=None):
    _check("qgemv_q8_0", lib().qgemv_q8_0(_dev(w_packed, "w_packed"), _dev(x, "x", _f32()), _dev(y, "y", _f32()),
                                          N, K, _stream(stream)))


def qgemv_q4_0(w_packed, x, y, N: int, K: int, stream=None):
    _check("qgemv_q4_0", lib().qgemv_q4_0(_dev(w_packed, "w_packed"), _dev(x, "x", _f32()), _dev(y, "y", _f32()),
                                          N, K, _stream(stream)))


def qgemv_q4_k(w_packed, x, y, N: int, K: int, stream=None):
    _check("qgemv_q4_k", lib().qgemv_q4_k(_dev(w_packed, "w_packed"), _dev(x, "x", _f32()), _dev(y, "y", _f32()),
                                          N, K, _stream(stream)))


def qgemv_q6_k(w_packed, x, y, N: int, K: int, stream=None):
    _check("qgemv_q6_k", lib().qgemv_q6_k(_dev(w_packed, "w_packed"), _dev(x, "x", _f32()), _dev(y, "y", _f32()),
                                          N, K, _stream(stream)))


def qgemv_epilogue(qtype, w_packed, x, y, N: int, K: int, bias=None, residual=None, stream=None):
    """y = ((W x) + bias) + residual; y's dtype (float32 or float16) selects the output type."""
    import torch
    if y.dtype not in (torch.float32, torch.float16):
        raise ValueError(f"y must be float32 or float16, got {y.dtype}")
    out_type = QG_OUT_F16 if y.dtype == torch.float16 else QG_OUT_F32
    _check("qgemv_epilogue",
           lib().qgemv_epilogue(_qtype(qtype), _dev(w_packed, "w_packed"), _dev(x, "x", _f32()),
                                _dev(bias, "bias", _f32()), _dev(residual, "residual", _f32()), _dev(y, "y"),
                                out_type, N, K, _stream(stream)))


def qg_rmsnorm(x, gamma, eps: float, out, K: int, stream=None):
    _check("qg_rmsnorm", lib().qg_rmsnorm(_dev(x, "x", _f32()), _dev(gamma, "gamma", _f32()), float(eps),
                                          _dev(out, "out", _f32()), K, _stream(stream)))


def qgemv_rmsnorm(qtype, w_packed, x, gamma, eps: float, y, N: int, K: int, stream=None):
    _check("qgemv_rmsnorm", lib().qgemv_rmsnorm(_qtype(qtype), _dev(w_packed, "w_packed"), _dev(x, "x", _f32()),
                                                _dev(gamma, "gamma", _f32()), float(eps), _dev(y, "y", _f32()),
                                                N, K, _stream(stream)))


def qgemv_rmsnorm_gateup_silu(qtype, w_gateup_packed, x, gamma, eps: float, y, N_ff: int, K: int, stream=None):
    _check("qgemv_rmsnorm_gateup_silu",
           lib().qgemv_rmsnorm_gateup_silu(_qtype(qtype), _dev(w_gateup_packed, "w_gateup_packed"),
                                           _dev(x, "x", _f32()), _dev(gamma, "gamma", _f32()), float(eps),
                                           _dev(y, "y", _f32()), N_ff, K, _stream(stream)))


def qg_prefill_workspace_size(qtype, N: int, K: int, M: int) -> int:
    return int(lib().qg_prefill_workspace_size(_qtype(qtype), N, K, M))


def qgemm_prefill(qtype, w_packed, X, Y, N: int, K: int, M: int, workspace=None, stream=None):
    """Y[M][N] = X W^T on the matrix cores. `workspace` is a uint8 device tensor of at
    least qg_prefill_workspace_size(qtype, N, K, M) bytes (allocated here with torch if None)."""
    import torch
    if workspace is None:
        workspace = torch.empty(qg_prefill_workspace_size(qtype, N, K, M), dtype=torch.uint8, device=X.device)
    _check("qgemm_prefill", lib().qgemm_prefill(_qtype(qtype), _dev(w_packed, "w_packed"), _dev(X, "X", _f32()),
                                                _dev(Y, "Y", _f32()), N, K, M, _dev(workspace, "workspace"),
                                                workspace.numel() * workspace.element_size(), _stream(stream)))
    return workspace


QG_PREFILL_NOALLOC_MAX_BYTES = 64 << 20


def qgemm_prefill_noalloc(qtype, w_packed, X, Y, N: int, K: int, M: int, stream=None):
    """qgemm_prefill on the library's own per-GPU scratch array (no workspace,
    nothing allocated); shapes whose workspace exceeds QG_PREFILL_NOALLOC_MAX_BYTES
    are refused."""
    _check("qgemm_prefill_noalloc",
           lib().qgemm_prefill_noalloc(_qtype(qtype), _dev(w_packed, "w_packed"), _dev(X, "X", _f32()),
                                       _dev(Y, "Y", _f32()), N, K, M, _stream(stream)))


def gemv_f16_splitk(w_f16, x, y, N: int, K: int, stream=None):
    _check("gemv_f16_splitk", lib().gemv_f16_splitk(_dev(w_f16, "w_f16"), _dev(x, "x", _f32()), _dev(y, "y", _f32()),
                                                    N, K, _stream(stream)))


def qgemv_fused_gateup_silu(qtype, w_gateup_packed, x, y, N_ff: int, K: int, stream=None):
    _check("qgemv_fused_gateup_silu",
           lib().qgemv_fused_gateup_silu(_qtype(qtype), _dev(w_gateup_packed, "w_gateup_packed"),
                                         _dev(x, "x", _f32()), _dev(y, "y", _f32()), N_ff, K, _stream(stream)))


def qgemv_verify(qtype, w_packed, X, Y, N: int, K: int, M: int, stream=None):
    _check("qgemv_verify", lib().qgemv_verify(_qtype(qtype), _dev(w_packed, "w_packed"), _dev(X, "X", _f32()),
                                              _dev(Y, "Y", _f32()), N, K, M, _stream(stream)))


def qgemv(qtype, w_packed, x, y, N: int, K: int, stream=None):
    """qgemv_q8_0, qgemv_q4_0, qgemv_q4_k or qgemv_q6_k by qtype."""
    {Q8_0: qgemv_q8_0, Q4_0: qgemv_q4_0, Q4_K: qgemv_q4_k, Q6_K: qgemv_q6_k}[_qtype(qtype)](w_packed, x, y, N, K,
                                                                                         stream)


# ---- diagnostics -----------------------------------------------------------

def qg_status_str(status: int) -> str:
    return lib().qg_status_str(status).decode()


def qg_last_error() -> str:
    return lib().qg_last_error().decode()


def qg_plan_info(qtype, N: int, K: int, M: int = 1, rmsnorm: bool = False) -> dict:
    w = ctypes.c_int()
    g = ctypes.c_int64()
    xl = ctypes.c_int()
    ps = ctypes.c_int()
    lds = ctypes.c_int64()
    _check("qg_plan_info", lib().qg_plan_info(_qtype(qtype), N, K, M, 1 if rmsnorm else 0, ctypes.byref(w),
                                              ctypes.byref(g), ctypes.byref(xl), ctypes.byref(ps),
                                              ctypes.byref(lds)))
    return {"split_k_ways": w.value, "workgroups": g.value, "x_in_lds": bool(xl.value),
            "persistent": bool(ps.value), "lds_bytes": lds.value}


F16_FORMS = {0: "lane-split", 1: "row", 2: "split-K row"}


def qg_f16_plan_info(N: int, K: int, w_addr: int = 0, x_addr: int = 0) -> dict:
    """The form gemv_f16_splitk takes for this shape; w_addr and x_addr are the
    addresses whose alignment it inspects (0: 16-byte aligned)."""
    f = ctypes.c_int()
    wv = ctypes.c_int()
    g = ctypes.c_int64()
    _check("qg_f16_plan_info", lib().qg_f16_plan_info(N, K, w_addr or 0x10000, x_addr or 0x10000, ctypes.byref(f),
                                                      ctypes.byref(wv), ctypes.byref(g)))
    return {"form": F16_FORMS[f.value], "waves": wv.value, "workgroups": g.value}


def qg_reload_tuning():
    """Re-read the QG_* launch-shape overrides from the environment."""
    _check("qg_reload_tuning", lib().qg_reload_tuning())


def qg_time_next_launch(start_event, stop_event):
    """Bind two timing events (torch.cuda.Event that have been recorded once, so
    that they exist, or raw hipEvent_t ints) to the next GEMV kernel this thread
    launches; None, None clears."""
    def handle(e):
        if e is None or isinstance(e, int):
            return e
        if not e.cuda_event:
            raise ValueError("record the event once before binding it (torch creates it lazily)")
        return e.cuda_event
    _check("qg_time_next_launch", lib().qg_time_next_launch(handle(start_event), handle(stop_event)))


# ---- load-time helpers (torch allocates; the library packs) ------------------

def upload(a: np.ndarray, device="cuda"):
    """Copy a host numpy array to a new device tensor (torch is the allocator)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def pack_weights(qtype, canonical: np.ndarray, N: int, K: int, device="cuda", stream=None):
    """Upload canonical blocks and re-tile them on the device; returns the packed uint8 tensor."""
    import torch
    canon_d = upload(canonical.view(np.uint8), device)
    packed = torch.empty(qg_packed_size(qtype, N, K), dtype=torch.uint8, device=device)
    qg_pack(qtype, canon_d, packed, N, K, stream)
    torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
    return packed


def pack_concat(qtype, parts: list, K: int, device="cuda", stream=None):
    """Pack canonical row blocks [(canonical, rows), ...] into one concatenated weight (e.g. QKV)."""
    import torch
    N = sum(r for _, r in parts)
    packed = torch.empty(qg_packed_size(qtype, N, K), dtype=torch.uint8, device=device)
    row0 = 0
    keep = []
    for canon, rows in parts:
        c = upload(canon.view(np.uint8), device)
        keep.append(c)
        qg_pack_rows(qtype, c, packed, N, row0, rows, K, stream)
        row0 += rows
    torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
    return packed


def pack_gateup(qtype, gate: np.ndarray, up: np.ndarray, N_ff: int, K: int, device="cuda", stream=None):
    """Upload gate and up projections and fuse them into one packed weight."""
    import torch
    g = upload(gate.view(np.uint8), device)
    u = upload(up.view(np.uint8), device)
    packed = torch.empty(qg_packed_size(qtype, 2 * N_ff, K), dtype=torch.uint8, device=device)
    qg_pack_gateup(qtype, g, u, packed, N_ff, K, stream)
    torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
    return packed


def bound_call(name: str, *args):
    """A zero-argument callable for one C-ABI call with its arguments already
    marshalled (raw pointers, sizes, stream handle): for timed loops, where
    re-checking torch tensors on every launch would dominate small calls."""
    fn = getattr(lib(), name)

    def call():
        st = fn(*args)
        if st:
            _check(name, st)
    return call
