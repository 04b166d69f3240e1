"""Host-side tests of libqgemv: symbols, argument checks, the packer (no GPU needed).

None of these makes a compute call: every entry point below is given arguments
that its host-side checks reject before any HIP call is made.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import block_dequant_gemv_amd as qg
from block_dequant_gemv_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qg.LIB_PATH):
        from block_dequant_gemv_amd import build
        build.build()
    return qg.lib()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(q\w+|gemv_\w+)\s*\(", src)))


def test_header_and_binding_agree():
    assert sorted(qg.SYMBOLS) == header_functions()


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", qg.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in header_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


def test_status_strings(L):
    for s in range(5):
        assert qg.qg_status_str(s).startswith("QG_")
    assert "unknown" in qg.qg_status_str(99)


def test_packed_size(L):
    # N % 8 == 0, K % 1024 == 0: the packed form is exactly the canonical bytes
    for kind, bb in (("q8_0", 34), ("q4_0", 18)):
        for N, K in ((1024, 1024), (4096, 1024), (17408, 5120), (5120, 17408)):
            assert qg.qg_packed_size(kind, N, K) == N * (K // 32) * bb
    # ragged: padding rows up to a multiple of 8 and 256-byte plane alignment
    # 9 rows -> 2 tiles of 8 rows; quant plane 16 rows * 2 blocks * 16 B = 512,
    # scale plane 16 * 2 * 2 B = 64 -> 256 after alignment
    assert qg.qg_packed_size("q4_0", 9, 64) == 512 + 256
    assert qg.qg_packed_size("q8_0", 9, 64) == 1024 + 256
    for bad in ((0, 32), (-1, 32), (8, 33), (8, 0)):
        assert qg.qg_packed_size("q8_0", *bad) == 0
    assert qg.qg_packed_size(7, 8, 32) == 0
    # Q4_K: 148 bytes per 256 weights (16 B of nibbles + 2 B of sc/mn per 32, and
    # 4 B of d/dmin per 256) when the planes need no padding; K % 256 == 0
    for N, K in ((1024, 1024), (4096, 1024), (17408, 5120), (5120, 17408)):
        assert qg.qg_packed_size("q4_k", N, K) == N * (K // 256) * 148
    # 8 x 256: quant 1024, scale 128 -> 256, super 32 -> 256
    assert qg.qg_packed_size("q4_k", 8, 256) == 1024 + 256 + 256
    for bad in ((8, 32), (8, 1056), (8, 0)):
        assert qg.qg_packed_size("q4_k", *bad) == 0
    # Q6_K: as canonical, 210 bytes per 256 weights (24 B of quants + 2 B of
    # scales per 32, 2 B of d per 256); 8 x 256: quant 1536, scale 128 -> 256,
    # super 16 -> 256
    for N, K in ((1024, 1024), (4096, 1024), (17408, 5120), (5120, 17408)):
        assert qg.qg_packed_size("q6_k", N, K) == N * (K // 256) * 210
    assert qg.qg_packed_size("q6_k", 8, 256) == 1536 + 256 + 256
    for bad in ((8, 32), (8, 1056), (8, 0)):
        assert qg.qg_packed_size("q6_k", *bad) == 0


FAKE = 0x10000  # a 64 KiB-aligned address that is never dereferenced


def call(L, name, *args):
    return getattr(L, name)(*args)


def test_argument_checks_return_codes_without_gpu(L):
    null = None
    f = FAKE
    # null pointers
    assert call(L, "qgemv_q8_0", null, f, f + 4096, 8, 32, null) == qg.QG_EINVAL
    assert call(L, "qgemv_q4_0", f, null, f + 4096, 8, 32, null) == qg.QG_EINVAL
    assert call(L, "gemv_f16_splitk", f, f + 4096, null, 8, 32, null) == qg.QG_EINVAL
    # bad sizes
    assert call(L, "qgemv_q8_0", f, f + (1 << 20), f + (2 << 20), 8, 48, null) == qg.QG_EINVAL
    assert call(L, "qgemv_q4_0", f, f + (1 << 20), f + (2 << 20), 0, 64, null) == qg.QG_EINVAL
    assert call(L, "gemv_f16_splitk", f, f + (1 << 20), f + (2 << 20), 8, -1, null) == qg.QG_EINVAL
    # misalignment
    assert call(L, "qgemv_q8_0", f + 8, f + (1 << 20), f + (2 << 20), 8, 32, null) == qg.QG_EALIGN
    assert call(L, "qgemv_q8_0", f, f + (1 << 20) + 4, f + (2 << 20), 8, 32, null) == qg.QG_EALIGN
    assert call(L, "qgemv_q8_0", f, f + (1 << 20), f + (2 << 20) + 2, 8, 32, null) == qg.QG_EALIGN
    assert call(L, "gemv_f16_splitk", f + 1, f + (1 << 20), f + (2 << 20), 8, 32, null) == qg.QG_EALIGN
    # overlapping output
    assert call(L, "qgemv_q8_0", f, f + (1 << 20), f + (1 << 20) + 16, 8, 32, null) == qg.QG_EINVAL
    assert call(L, "qgemv_q4_0", f, f + (1 << 20), f + 64, 8, 32, null) == qg.QG_EINVAL
    assert call(L, "gemv_f16_splitk", f, f + (1 << 20), f + (1 << 20), 8, 32, null) == qg.QG_EINVAL
    # unsupported qtype / row count
    assert call(L, "qgemv_verify", 1, f, f + (1 << 20), f + (2 << 20), 8, 32, 1, null) == qg.QG_EUNSUPPORTED
    assert call(L, "qgemv_verify", 1, f, f + (1 << 20), f + (2 << 20), 8, 32, 7, null) == qg.QG_EUNSUPPORTED
    assert call(L, "qgemv_verify", 5, f, f + (1 << 20), f + (2 << 20), 8, 32, 2, null) == qg.QG_EUNSUPPORTED
    # Q4_K / Q6_K: every GEMV form, K a multiple of 256; not the prefill GEMM
    for qt in (qg.Q4_K, qg.Q6_K):
        assert call(L, "qgemv_verify", qt, f, f + (1 << 20), f + (2 << 20), 8, 1056, 2, null) == qg.QG_EINVAL
        assert call(L, "qgemv_fused_gateup_silu", qt, f, f + (1 << 20), f + (2 << 20), 8, 1056,
                    null) == qg.QG_EINVAL
        assert call(L, "qgemv_epilogue", qt, f, f + (1 << 20), null, null, f + (2 << 20), qg.QG_OUT_F32, 8, 1056,
                    null) == qg.QG_EINVAL
        assert call(L, "qgemm_prefill", qt, f, f + (1 << 20), f + (2 << 20), 8, 256, 16, f + (3 << 20), 1 << 20,
                    null) == qg.QG_EUNSUPPORTED
        assert qg.qg_prefill_workspace_size(qt, 8, 256, 16) == 0
    assert call(L, "qgemv_q4_k", f, f + (1 << 20), f + (2 << 20), 8, 32, null) == qg.QG_EINVAL
    assert call(L, "qgemv_q4_k", f, f + (1 << 20), f + (2 << 20), 8, 1056, null) == qg.QG_EINVAL
    assert call(L, "qgemv_q4_k", f + 8, f + (1 << 20), f + (2 << 20), 8, 256, null) == qg.QG_EALIGN
    assert call(L, "qgemv_q4_k", f, f + (1 << 20), f + (1 << 20), 8, 256, null) == qg.QG_EINVAL
    assert call(L, "qgemv_q6_k", f, f + (1 << 20), f + (2 << 20), 8, 1056, null) == qg.QG_EINVAL
    assert call(L, "qgemv_q6_k", f + 8, f + (1 << 20), f + (2 << 20), 8, 256, null) == qg.QG_EALIGN
    assert call(L, "qgemv_q6_k", f, f + (1 << 20), f + (1 << 20), 8, 256, null) == qg.QG_EINVAL
    assert call(L, "qgemv_fused_gateup_silu", 5, f, f + (1 << 20), f + (2 << 20), 8, 32, null) == qg.QG_EUNSUPPORTED
    assert call(L, "qgemv_fused_gateup_silu", 1, f, f + (1 << 20), f + (2 << 20), 0, 32, null) == qg.QG_EINVAL
    # verify: the M x K activations must not overlap the M x N outputs
    assert call(L, "qgemv_verify", 2, f, f + (1 << 20), f + (1 << 20) + 4 * 32 * 3, 8, 32, 4, null) == qg.QG_EINVAL
    # packers
    assert call(L, "qg_pack", 1, null, f, 8, 32, null) == qg.QG_EINVAL
    assert call(L, "qg_pack", 1, f, f + 8, 8, 32, null) == qg.QG_EALIGN
    assert call(L, "qg_pack_rows", 2, f, f + (1 << 20), 8, 6, 4, 32, null) == qg.QG_EINVAL
    assert call(L, "qg_pack_gateup", 2, f, null, f + (1 << 20), 8, 32, null) == qg.QG_EINVAL
    assert call(L, "qg_pack", 1, f, f + 16, 8, 32, null) == qg.QG_EINVAL  # overlap
    msg = qg.qg_last_error()
    assert "overlap" in msg


def _alignment_cases():
    """(call, argument builder, {pointer: documented alignment}) for every entry
    point that checks alignment, as include/qgemv.h states it. The builder takes
    a dict of pointers; the output always overlaps the activations (or the
    packed buffer the canonical one), so a call whose alignment checks pass
    fails the overlap check that follows them, before any HIP call."""
    import ctypes as C
    e = C.c_float(1e-6)
    N, K = 8, 256
    return [
        ("qgemv_q8_0", lambda p: (p["w"], p["x"], p["y"], N, K, None), {"w": 16, "x": 16, "y": 4}),
        ("qgemv_q4_0", lambda p: (p["w"], p["x"], p["y"], N, K, None), {"w": 16, "x": 16, "y": 4}),
        ("qgemv_q4_k", lambda p: (p["w"], p["x"], p["y"], N, K, None), {"w": 16, "x": 16, "y": 4}),
        ("qgemv_q6_k", lambda p: (p["w"], p["x"], p["y"], N, K, None), {"w": 16, "x": 16, "y": 4}),
        ("qgemv_epilogue", lambda p: (2, p["w"], p["x"], p["b"], p["r"], p["y"], qg.QG_OUT_F32, N, K, None),
         {"w": 16, "x": 16, "b": 4, "r": 4, "y": 4}),
        ("qgemv_epilogue", lambda p: (1, p["w"], p["x"], None, None, p["y"], qg.QG_OUT_F16, N, K, None),
         {"w": 16, "x": 16, "y": 2}),
        ("qgemv_fused_gateup_silu", lambda p: (3, p["w"], p["x"], p["y"], N, K, None), {"w": 16, "x": 16, "y": 4}),
        ("qgemv_verify", lambda p: (4, p["w"], p["x"], p["y"], N, K, 3, None), {"w": 16, "x": 16, "y": 4}),
        ("qgemv_rmsnorm", lambda p: (1, p["w"], p["x"], p["g"], e, p["y"], N, K, None),
         {"w": 16, "x": 16, "g": 16, "y": 4}),
        ("qgemv_rmsnorm_gateup_silu", lambda p: (2, p["w"], p["x"], p["g"], e, p["y"], N, K, None),
         {"w": 16, "x": 16, "g": 16, "y": 4}),
        ("gemv_f16_splitk", lambda p: (p["w"], p["x"], p["y"], N, K, None), {"w": 2, "x": 4, "y": 4}),
        ("qgemm_prefill", lambda p: (1, p["w"], p["x"], p["y"], N, K, 4, p["s"], 1 << 20, None),
         {"w": 16, "x": 4, "y": 4, "s": 256}),
        ("qg_rmsnorm", lambda p: (p["x"], p["g"], e, p["y"], K, None), {"x": 4, "g": 4, "y": 4}),
        ("qg_pack", lambda p: (1, p["c"], p["p"], N, K, None), {"p": 16}),
        ("qg_pack_rows", lambda p: (2, p["c"], p["p"], N, 0, N, K, None), {"p": 16}),
        ("qg_pack_gateup", lambda p: (1, p["c"], p["c2"], p["p"], N, K, None), {"p": 16}),
    ]


def test_documented_alignment_is_exactly_what_is_checked(L):
    # every pointer at exactly its documented alignment passes the alignment
    # checks (the call then fails on the deliberate overlap: QG_EINVAL), and at
    # half of it is refused with QG_EALIGN
    f = FAKE
    base = {"w": f, "x": f + (1 << 20), "g": f + (2 << 20), "b": f + (3 << 20), "r": f + (4 << 20),
            "s": f + (5 << 20), "c": f + (6 << 20), "c2": f + (7 << 20)}
    base["y"] = base["x"] + 64          # overlaps x
    base["p"] = base["c"] + 64          # overlaps the canonical input
    for name, args, align in _alignment_cases():
        for arg, a in align.items():
            for off, want in ((a, qg.QG_EINVAL), (a // 2, qg.QG_EALIGN)):
                ptrs = dict(base)
                ptrs[arg] = base[arg] + off
                got = call(L, name, *args(ptrs))
                assert got == want, (name, arg, off, got, qg.qg_last_error())
                if want == qg.QG_EINVAL:
                    assert "overlap" in qg.qg_last_error() or "workspace" in qg.qg_last_error(), (name, arg)


def test_probe_argument_checks_without_gpu(L):
    f = FAKE
    pr = lambda *a: call(L, "qg_probe_stream", *a)  # noqa: E731
    assert pr(None, 1024, f, None) == qg.QG_EINVAL
    assert pr(f, 1024, None, None) == qg.QG_EINVAL
    assert pr(f, 0, f + (1 << 20), None) == qg.QG_EINVAL
    assert pr(f, 1000, f + (1 << 20), None) == qg.QG_EINVAL          # not a multiple of 1 KiB
    assert pr(f + 8, 1024, f + (1 << 20), None) == qg.QG_EALIGN
    assert pr(f, 1024, f + (1 << 20) + 2, None) == qg.QG_EALIGN
    assert pr(f, 4096, f + 1024, None) == qg.QG_EINVAL               # sink inside buf
    assert "overlap" in qg.qg_last_error()


def test_epilogue_argument_checks_without_gpu(L):
    f = FAKE
    w, x, y, b, r = f, f + (1 << 20), f + (2 << 20), f + (3 << 20), f + (4 << 20)
    ep = lambda *a: call(L, "qgemv_epilogue", *a)  # noqa: E731
    # (qtype, w, x, bias, residual, y, out_type, N, K, stream)
    assert ep(1, None, x, b, r, y, 0, 8, 32, None) == qg.QG_EINVAL          # null weights
    assert ep(1, w, x, b, r, None, 0, 8, 32, None) == qg.QG_EINVAL          # null output
    assert ep(5, w, x, b, r, y, 0, 8, 32, None) == qg.QG_EUNSUPPORTED       # unknown qtype
    assert ep(1, w, x, b, r, y, 2, 8, 32, None) == qg.QG_EUNSUPPORTED       # unknown output type
    assert ep(2, w, x, b, r, y, 0, 8, 48, None) == qg.QG_EINVAL             # K % 32
    assert ep(1, w, x, b + 2, r, y, 0, 8, 32, None) == qg.QG_EALIGN         # bias alignment
    assert ep(1, w, x, b, r + 1, y, 0, 8, 32, None) == qg.QG_EALIGN         # residual alignment
    assert ep(1, w, x, b, r, y + 2, 0, 8, 32, None) == qg.QG_EALIGN         # fp32 output alignment
    assert ep(1, w, x, b, r, y + 1, 1, 8, 32, None) == qg.QG_EALIGN         # fp16 output alignment
    assert ep(1, w, x, y + 16, r, y, 0, 8, 32, None) == qg.QG_EINVAL        # y overlaps bias
    assert ep(1, w, x, b, y + 4, y, 0, 8, 32, None) == qg.QG_EINVAL         # y overlaps residual, shifted
    assert ep(1, w, x, b, y, y, 1, 8, 32, None) == qg.QG_EINVAL             # in place needs fp32 output
    assert ep(1, w, y - 16, b, r, y, 1, 8, 32, None) == qg.QG_EINVAL        # y overlaps x
    assert "overlap" in qg.qg_last_error()


def test_rmsnorm_argument_checks_without_gpu(L):
    import ctypes as C
    f = FAKE
    w, x, g, y = f, f + (1 << 20), f + (2 << 20), f + (3 << 20)
    e = C.c_float
    rn = lambda *a: call(L, "qg_rmsnorm", *a)  # noqa: E731
    gn = lambda *a: call(L, "qgemv_rmsnorm", *a)  # noqa: E731
    gu = lambda *a: call(L, "qgemv_rmsnorm_gateup_silu", *a)  # noqa: E731
    # qg_rmsnorm(x, gamma, eps, out, K, stream)
    assert rn(None, g, e(1e-6), y, 8, None) == qg.QG_EINVAL
    assert rn(x, g, e(1e-6), y, 0, None) == qg.QG_EINVAL
    assert rn(x, g, e(-1.0), y, 8, None) == qg.QG_EINVAL
    assert rn(x, g, e(float("inf")), y, 8, None) == qg.QG_EINVAL
    assert rn(x, g, e(float("nan")), y, 8, None) == qg.QG_EINVAL
    assert rn(x + 2, g, e(1e-6), y, 8, None) == qg.QG_EALIGN
    assert rn(x, g, e(1e-6), x + 16, 8, None) == qg.QG_EINVAL      # out overlaps x
    assert rn(x, g, e(1e-6), g, 8, None) == qg.QG_EINVAL           # out is gamma
    # qgemv_rmsnorm(qtype, w, x, gamma, eps, y, N, K, stream)
    assert gn(1, w, x, None, e(1e-6), y, 8, 32, None) == qg.QG_EINVAL
    assert gn(1, w, x, g + 4, e(1e-6), y, 8, 32, None) == qg.QG_EALIGN
    assert gn(2, w, x, g, e(-1e-3), y, 8, 32, None) == qg.QG_EINVAL
    assert gn(2, w, x, g, e(1e-6), y, 8, 40960 + 32, None) == qg.QG_EUNSUPPORTED
    # the normalised copy lives in LDS next to the kernel's static arrays: K <= 39936
    assert gn(2, w, x, g, e(1e-6), y, 8, 40960, None) == qg.QG_EUNSUPPORTED
    assert gn(2, w, x, g, e(1e-6), y, 8, 39936 + 32, None) == qg.QG_EUNSUPPORTED
    assert gu(1, w, x, g, e(1e-6), y, 8, 40960, None) == qg.QG_EUNSUPPORTED
    assert gn(2, w, x, y - 16, e(1e-6), y, 8, 32, None) == qg.QG_EINVAL   # y overlaps gamma
    assert gn(5, w, x, g, e(1e-6), y, 8, 32, None) == qg.QG_EUNSUPPORTED
    assert gn(1, w, x, g, e(1e-6), y, 8, 48, None) == qg.QG_EINVAL
    # qgemv_rmsnorm_gateup_silu(qtype, w, x, gamma, eps, y, N_ff, K, stream)
    assert gu(1, w, x, g, e(1e-6), y, 0, 32, None) == qg.QG_EINVAL
    assert gu(1, w, x, None, e(1e-6), y, 8, 32, None) == qg.QG_EINVAL
    assert gu(2, w, x, g, e(1e-6), y, 8, 65536, None) == qg.QG_EUNSUPPORTED


def test_gemm_argument_checks_without_gpu(L):
    f = FAKE
    w, x, y, ws = f, f + (1 << 24), f + (2 << 24), f + (3 << 24)
    # 20 rows padded to 32 (two 16-row tiles): one 256-byte block of row factors and 32 x 1024 x 4
    # bytes of split activations; K below 16 chunks of 4 blocks is never split, and a 64-row
    # weight with 16 chunks or more is split into ranges of at least two chunks (128 blocks -> 16),
    # each range with its M x N partial sums
    need = qg.qg_prefill_workspace_size("q8_0", 64, 1024, 20)
    assert need == 256 + 32 * 1024 * 4
    with_split = qg.qg_prefill_workspace_size("q8_0", 64, 4096, 20)
    assert with_split == 256 + 32 * 4096 * 4 + 16 * 20 * 64 * 4
    # 70 rows: five 16-row tiles in groups of one, two or four (80, 96 or 128 padded rows); a weight
    # with enough row blocks is not split (no partial sums)
    lm = qg.qg_prefill_workspace_size("q4_0", 248320, 5120, 70)
    assert (lm - 512) % (5120 * 4) == 0 and (lm - 512) // (5120 * 4) in (80, 96, 128)
    assert qg.qg_prefill_workspace_size("q8_0", 64, 1024, 0) == 0
    assert qg.qg_prefill_workspace_size("q8_0", 64, 1000, 4) == 0
    assert qg.qg_prefill_workspace_size(3, 64, 1024, 4) == 0
    gm = lambda *a: call(L, "qgemm_prefill", *a)  # noqa: E731
    # (qtype, w, X, Y, N, K, M, workspace, workspace_bytes, stream)
    assert gm(1, w, x, y, 64, 1024, 0, ws, need, None) == qg.QG_EINVAL            # M = 0
    assert gm(1, w, x, y, 64, 1024, 20, None, need, None) == qg.QG_EINVAL         # no workspace
    assert gm(1, w, x, y, 64, 1024, 20, ws, need - 4, None) == qg.QG_EINVAL       # workspace too small
    assert "qg_prefill_workspace_size" in qg.qg_last_error()
    assert gm(1, w, x, y, 64, 1024, 20, ws + 16, need, None) == qg.QG_EALIGN      # workspace alignment
    assert gm(1, w + 8, x, y, 64, 1024, 20, ws, need, None) == qg.QG_EALIGN       # weight alignment
    assert gm(1, w, x + 2, y, 64, 1024, 20, ws, need, None) == qg.QG_EALIGN       # X alignment
    assert gm(2, w, x, x + 64, 64, 1024, 20, ws, need, None) == qg.QG_EINVAL      # Y overlaps X
    assert gm(2, w, x, y, 64, 1024, 20, y + 256, need, None) == qg.QG_EINVAL      # workspace overlaps Y
    assert gm(2, w, x, y, 64, 1024, 20, x, need, None) == qg.QG_EINVAL            # workspace overlaps X
    assert gm(5, w, x, y, 64, 1024, 20, ws, need, None) == qg.QG_EUNSUPPORTED     # unknown qtype
    assert gm(1, w, x, y, 64, 1000, 20, ws, need, None) == qg.QG_EINVAL           # K % 32


def test_prefill_noalloc_checks_without_gpu(L):
    # qgemm_prefill_noalloc: the prefill GEMM's checks, and shapes whose workspace
    # exceeds the library's per-GPU scratch are refused before any HIP call
    f = FAKE
    w, x, y = f, f + (1 << 24), f + (2 << 24)
    na = lambda *a: call(L, "qgemm_prefill_noalloc", *a)  # noqa: E731
    # (qtype, w, X, Y, N, K, M, stream)
    assert na(1, w, x, y, 64, 1024, 0, None) == qg.QG_EINVAL                     # M = 0
    assert na(1, None, x, y, 64, 1024, 20, None) == qg.QG_EINVAL                 # null weights
    assert na(1, w + 8, x, y, 64, 1024, 20, None) == qg.QG_EALIGN                # weight alignment
    assert na(1, w, x + 2, y, 64, 1024, 20, None) == qg.QG_EALIGN                # X alignment
    assert na(2, w, x, x + 64, 64, 1024, 20, None) == qg.QG_EINVAL               # Y overlaps X
    assert na(3, w, x, y, 64, 1024, 20, None) == qg.QG_EUNSUPPORTED              # Q4_K: GEMV only
    assert na(1, w, x, y, 64, 1000, 20, None) == qg.QG_EINVAL                    # K % 32
    # Q4_0 5120 x 17408 at M = 1024: 1024 x 17408 x 4 bytes of split activations alone (71 MB)
    need = qg.qg_prefill_workspace_size("q4_0", 5120, 17408, 1024)
    assert need > qg.QG_PREFILL_NOALLOC_MAX_BYTES
    assert na(2, w, x, f + (1 << 34), 5120, 17408, 1024, None) == qg.QG_EUNSUPPORTED
    assert "qg_prefill_workspace_size" in qg.qg_last_error()


def test_time_next_launch_arguments(L):
    # host-only: binding or clearing events makes no HIP call
    f = FAKE
    assert call(L, "qg_time_next_launch", f, None) == qg.QG_EINVAL
    assert call(L, "qg_time_next_launch", None, f) == qg.QG_EINVAL
    assert call(L, "qg_time_next_launch", None, None) == qg.QG_OK
    # a failed call clears a binding: the fake events are never handed to HIP
    assert call(L, "qg_time_next_launch", f, f + 64) == qg.QG_OK
    assert call(L, "qgemv_q8_0", None, f, f + 4096, 8, 32, None) == qg.QG_EINVAL
    assert call(L, "qg_time_next_launch", None, None) == qg.QG_OK


def test_plan_info_split_is_independent_of_m(L):
    # the decode GEMV and the verify GEMV of a weight must add in the same order:
    # same form, same K split, whatever M is
    for kind in ("q8_0", "q4_0"):
        for N, K in ((1, 32), (100, 2080), (1024, 2048), (1024, 3072), (5120, 17408), (17408, 5120),
                     (4096, 1024), (248320, 5120), (151936, 1024), (64, 65536), (8, 32 * 1024 * 40)):
            p1 = qg.qg_plan_info(kind, N, K, 1)
            for M in range(2, 7):
                pm = qg.qg_plan_info(kind, N, K, M)
                assert (pm["split_k_ways"], pm["persistent"]) == (p1["split_k_ways"], p1["persistent"]), (N, K, M)
    # the LM heads run one wavefront per tile; the mid-size matrices the persistent form
    assert not qg.qg_plan_info("q4_0", 248320, 5120)["persistent"]
    assert not qg.qg_plan_info("q8_0", 151936, 1024)["persistent"]
    p = qg.qg_plan_info("q4_0", 5120, 17408)
    assert p["persistent"] and p["split_k_ways"] > 1 and 17 % p["split_k_ways"] == 0


def test_plan_info_three_segments_get_three_wavefronts(L):
    # a row tile of exactly three 1024-weight segments is split over three
    # wavefronts (one segment each), for every type and every M; two or four
    # segments keep the power-of-two split
    for kind in ("q8_0", "q4_0", "q4_k", "q6_k"):
        for N in (1, 77, 1024, 2048):
            for M in range(1, 7):
                assert qg.qg_plan_info(kind, N, 3072, M)["split_k_ways"] == 3, (kind, N, M)
    assert qg.qg_plan_info("q8_0", 1024, 2048)["split_k_ways"] == 2
    assert qg.qg_plan_info("q8_0", 1024, 4096)["split_k_ways"] == 4
    # the one-wavefront-per-tile form with 2048 tiles or more: no split
    p = qg.qg_plan_info("q8_0", 8 * 4096, 3072)
    assert not p["persistent"] and p["split_k_ways"] == 1


def test_plan_info_long_rows_split_eight_ways_over_staged_activations(L):
    # few row tiles and 16 or more segments: eight wavefronts per tile at every M,
    # taking their activations from one staged copy whenever it fits in LDS
    for kind in ("q8_0", "q4_0", "q4_k", "q6_k"):
        for N, K in ((640, 17408), (1280, 8192), (24, 32768)):
            for M in (1, 4, 6):
                p = qg.qg_plan_info(kind, N, K, M)
                assert not p["persistent"] and p["split_k_ways"] == 8, (kind, N, K, M, p)
        assert qg.qg_plan_info(kind, 640, 17408)["x_in_lds"]
        assert qg.qg_plan_info(kind, 1280, 8192, 2)["x_in_lds"]
        # 16 segments but 4096 row tiles: one wavefront per tile
        assert qg.qg_plan_info(kind, 8 * 4096, 16384)["split_k_ways"] == 1
        # M K 4 bytes over the 160 KiB of LDS (M >= 3 at K = 17408): every row from L2
        assert qg.qg_plan_info(kind, 640, 17408, 2)["x_in_lds"]
        assert not any(qg.qg_plan_info(kind, 640, 17408, M)["x_in_lds"] for M in (3, 4, 5, 6))


LDS_PER_CU = 160 * 1024


def test_plan_lds_fits_a_cu(L):
    # every plan's LDS (static arrays plus the staged activations, partials and
    # phases) fits the 160 KiB of a gfx950 CU, at every M, for the RMSNorm
    # prologue too; shapes at and around the boundaries of each form
    shapes = [(8, 1024), (1280, 8192), (640, 17408), (24, 32768), (5120, 17408), (2001, 17408), (17408, 5120),
              (1024, 39936), (5120, 39936), (8, 40960), (640, 40960), (2048, 16384), (248320, 5120)]
    for kind in ("q8_0", "q4_0", "q4_k", "q6_k"):
        for N, K in shapes:
            for M in range(1, 7):
                p = qg.qg_plan_info(kind, N, K, M)
                assert 0 < p["lds_bytes"] <= LDS_PER_CU, (kind, N, K, M, p)
            if K <= 39936:
                p = qg.qg_plan_info(kind, N, K, 1, rmsnorm=True)
                assert p["x_in_lds"] and p["lds_bytes"] <= LDS_PER_CU, (kind, N, K, p)


def test_plan_staged_copy_at_the_lds_boundary(L):
    # 1280 x 8192 at M = 5: the 5 staged rows take exactly 160 KiB and the eight
    # split-K wavefronts' partials 1280 bytes more, so the rows come from L2
    for kind in ("q8_0", "q4_0", "q4_k", "q6_k"):
        p = qg.qg_plan_info(kind, 1280, 8192, 5)
        assert p["split_k_ways"] == 8 and not p["x_in_lds"], (kind, p)
        assert p["lds_bytes"] <= LDS_PER_CU
        # four rows (128 KiB + 1 KiB) still fit
        assert qg.qg_plan_info(kind, 1280, 8192, 4)["x_in_lds"]
    # Q4_K stages each row's 32-weight block sums after its activations: 4 rows x 8
    # segments x (4096 + 128) bytes, next to the eight wavefronts' partials
    p = qg.qg_plan_info("q4_k", 1280, 8192, 4)
    assert p["lds_bytes"] == 4 * 8 * 4224 + 8 * 4 * 8 * 4, p
    # the RMSNorm kernels add the sums up per unit: their staged copy is the activations alone
    for N in (8, 1024, 24000):
        pk = qg.qg_plan_info("q4_k", N, 39936, 1, rmsnorm=True)
        assert pk == qg.qg_plan_info("q4_0", N, 39936, 1, rmsnorm=True), (N, pk)
    # the RMSNorm prologue: K = 39936 (39 segments) fits next to the largest
    # static array; 40960 does not, for any form
    for kind in ("q8_0", "q4_0", "q4_k", "q6_k"):
        for N in (8, 1024, 5120, 17408, 248320):
            p = qg.qg_plan_info(kind, N, 39936, 1, rmsnorm=True)
            assert p["x_in_lds"] and p["lds_bytes"] <= LDS_PER_CU, (kind, N, p)
            with pytest.raises(qg.QGError) as err:
                qg.qg_plan_info(kind, N, 40960, 1, rmsnorm=True)
            assert err.value.status == qg.QG_EUNSUPPORTED
    # a persistent RMSNorm plan whose partials do not fit next to the staged copy
    # takes the one-wavefront-per-tile form instead of being refused: 24000 rows
    # are 3000 tiles, 12 per CU, each split in 13 K ranges, 4992 bytes of
    # partials next to 156 KiB of activations (5120 rows, 3 tiles per CU, fit)
    p = qg.qg_plan_info("q4_0", 24000, 39936, 1, rmsnorm=True)
    assert not p["persistent"] and p["x_in_lds"], p
    assert qg.qg_plan_info("q4_0", 24000, 39936, 1)["persistent"]
    assert qg.qg_plan_info("q4_0", 5120, 39936, 1, rmsnorm=True)["persistent"]
    with pytest.raises(qg.QGError):
        qg.qg_plan_info("q4_0", 5120, 1024, 2, rmsnorm=True)      # the prologue takes M = 1


def test_f16_form_rule_as_documented(L):
    # gemv_f16_splitk: fewer than 1024 rows with K % 8 == 0, K <= 32768 and
    # aligned w, x: split-K row form; else K = 512 L (L <= 16): row form; else
    # the lane-split form; misaligned w or x (or K % 8 != 0) always the last
    f = 0x10000
    for N, K in ((48, 5120), (256, 5120), (1, 8), (1023, 32768), (640, 1000)):
        p = qg.qg_f16_plan_info(N, K)
        assert p["form"] == "split-K row" and p["workgroups"] == N, (N, K, p)
        assert p["waves"] == -(-(K // 8) // 256) and p["waves"] <= 16
    # row form: 4 rows per workgroup, 8 from 4096 rows on
    for N, K in ((1024, 5120), (4095, 5120), (2049, 8192), (4096, 5120), (5120, 5120), (17408, 512)):
        p = qg.qg_f16_plan_info(N, K)
        assert p["form"] == "row" and p["waves"] == (4 if N < 4096 else 8), (N, K, p)
        assert p["workgroups"] == -(-N // p["waves"]), (N, K, p)
    for N, K in ((1023, 32776), (5120, 1000), (1024, 8200), (5120, 8704), (300, 7)):
        assert qg.qg_f16_plan_info(N, K)["form"] == "lane-split", (N, K)
    for N, K in ((48, 5120), (5120, 5120)):
        assert qg.qg_f16_plan_info(N, K, w_addr=f + 8)["form"] == "lane-split"
        assert qg.qg_f16_plan_info(N, K, x_addr=f + 4)["form"] == "lane-split"
    with pytest.raises(qg.QGError):
        qg.qg_f16_plan_info(0, 8)


def test_tuning_overrides_are_read_on_reload(L, monkeypatch):
    # the launch-shape overrides are read once and on qg_reload_tuning(), not per call
    assert qg.qg_plan_info("q4_0", 5120, 17408)["persistent"]
    monkeypatch.setenv("QG_PERSIST", "0")
    assert qg.qg_plan_info("q4_0", 5120, 17408)["persistent"]        # not re-read yet
    qg.qg_reload_tuning()
    assert not qg.qg_plan_info("q4_0", 5120, 17408)["persistent"]
    monkeypatch.delenv("QG_PERSIST")
    qg.qg_reload_tuning()
    assert qg.qg_plan_info("q4_0", 5120, 17408)["persistent"]


SHAPES = [(1, 32), (3, 64), (8, 1024), (9, 1056), (17, 2048), (24, 3104), (5, 5120)]
# Q4_K: K % 256 == 0; ragged last segments of 8, 16 and 24 blocks
Q4_K_SHAPES = [(1, 256), (3, 512), (8, 1024), (9, 1280), (17, 2048), (24, 2304), (5, 5120), (2, 1792)]


@pytest.mark.parametrize("kind,N,K", [(k, n, kk) for k in ("q8_0", "q4_0") for n, kk in SHAPES] +
                         [(k, n, kk) for k in ("q4_k", "q6_k") for n, kk in Q4_K_SHAPES])
def test_pack_unpack_roundtrip(L, kind, N, K):
    canon = W.matrix(kind, N, K, np.random.default_rng(N * 7 + K))
    packed = qg.qg_pack_host(kind, canon, N, K)
    assert packed.size == qg.qg_packed_size(kind, N, K)
    back = qg.qg_unpack_host(kind, packed, N, K)
    assert np.array_equal(back, canon)
    # the packed form holds at least the canonical bytes
    assert packed.size >= canon.size and canon.size == W.matrix_bytes(kind, N, K)


def test_q6_k_pack_places_every_field(L):
    # One row, K = 256: d lands in the super plane (row 0, slot 0), block j's two
    # int8 scales (weights 32j..32j+15 and 32j+16..32j+31) as bytes 0 and 1 of
    # its scale-plane entry, and each weight's 6-bit quant splits into a nibble
    # in the Q4_0 arrangement of quant unit 0 and a 2-bit part at its bit pair in
    # the row's dwords of quant unit 4 (rows 0-1: row 0 in bytes 0..7).
    N, K = 1, 256
    s_off = 8 * 8 * 24          # quant plane: 8 rows x 8 blocks x 24 B
    u_off = s_off + 256
    canon = np.zeros(210, np.uint8)
    canon[192:208] = np.arange(-8, 8, dtype=np.int8).view(np.uint8)
    canon[208:210] = [0x34, 0x12]
    packed = qg.qg_pack_host("q6_k", canon, N, K)
    assert list(packed[u_off:u_off + 2]) == [0x34, 0x12]
    for j in range(8):
        assert packed[s_off + j * 8].view(np.int8) == 2 * j - 8
        assert packed[s_off + j * 8 + 1].view(np.int8) == 2 * j - 7
    # one tile, one segment of nb = 8 blocks: unit u of slot 0, block j at ((u * 2 + 0) * 8 + j) * 16

    def hi_pos(e):
        f = e % 8
        p = (f % 2) * 16 + 4 + 4 * ((f // 2) % 2) + 2 * (f // 4)
        return (p + 24 * (e // 8)) % 32
    assert sorted(hi_pos(e) // 2 for e in range(16)) == list(range(16))   # the 16 bit pairs, once each
    for w, q in ((0, 1), (5, 47), (31, 60), (33, 17), (70, 63), (100, 32), (130, 5), (255, 40)):
        c = canon.copy()
        h, r = divmod(w, 128)
        g, l = divmod(r, 32)
        c[64 * h + 32 * (g % 2) + l] |= (q & 15) << (4 * (g // 2))
        c[128 + 32 * h + l] |= (q >> 4) << (2 * g)
        p = qg.qg_pack_host("q6_k", c, N, K)
        j, e = divmod(w, 32)
        lo = int.from_bytes(bytes(p[((0 * 2) * 8 + j) * 16 + 4 * (e // 8):][:4]), "little")
        assert (lo >> (4 * ((e % 8) // 2 + 4 * (e % 2)))) & 15 == q & 15, (w, q)
        hi = int.from_bytes(bytes(p[((4 * 2) * 8 + j) * 16 + 4 * (e // 16):][:4]), "little")
        assert (hi >> hi_pos(e % 16)) & 3 == q >> 4, (w, q)
        # nothing else set in the quant plane
        bits = int(np.unpackbits(p[:s_off]).sum())
        assert bits == bin(q & 15).count("1") + bin(q >> 4).count("1"), (w, q)


def _q4_k_centre(d_bits: int, dmin_bits: int, sc: int, mn: int) -> int:
    """The load-time centre of a Q4_K sub-block, from its definition in exact
    rational arithmetic: dmin*mn / (d*sc) rounded to the nearest integer (ties
    down), clamped to 0..15; 0 when d*sc is 0."""
    from fractions import Fraction
    f16 = lambda b: Fraction(float(np.array([b], np.uint16).view(np.float16)[0]))  # noqa: E731
    a, b = f16(d_bits) * sc, f16(dmin_bits) * mn
    if a == 0:
        return 0
    r = b / a
    c = int(np.floor(r))
    if r - c > Fraction(1, 2):
        c += 1
    return min(15, max(0, c))


def test_q4_k_centre_values(L):
    # the centre stored in the low 4 bits of the scale word, against its definition
    cases = [(0x3C00, 0x3C00, 1, 0), (0x3C00, 0x3C00, 2, 15), (0x3C00, 0x3C00, 2, 16), (0x3C00, 0x3C00, 2, 17),
             (0x3C00, 0x4000, 16, 32), (0x3C00, 0x3C00, 1, 63), (0x3C00, 0x3C00, 0, 5), (0x0000, 0x3C00, 9, 9),
             (0xBC00, 0x3C00, 4, 20), (0x3C00, 0xBC00, 4, 20), (0xBC00, 0xBC00, 4, 20), (0x0001, 0x0003, 63, 21),
             (0x7BFF, 0x0001, 63, 63), (0x0001, 0x7BFF, 63, 63), (0x3555, 0x2AAA, 7, 11)]
    rng = np.random.default_rng(5)
    for _ in range(300):
        cases.append((int(rng.integers(0, 0x7C00)) | (0x8000 if rng.random() < 0.1 else 0),
                      int(rng.integers(0, 0x7C00)), int(rng.integers(0, 64)), int(rng.integers(0, 64))))
    for d, dmin, sc, mn in cases:
        canon = np.zeros(144, np.uint8)
        canon[0:4] = [d & 255, d >> 8, dmin & 255, dmin >> 8]
        canon[4] = sc
        canon[8] = mn
        packed = qg.qg_pack_host("q4_k", canon, 1, 256)
        word = int(packed[1024]) | (int(packed[1025]) << 8)
        assert word & 15 == _q4_k_centre(d, dmin, sc, mn), (hex(d), hex(dmin), sc, mn, word & 15)
        assert (word >> 4) & 63 == sc and word >> 10 == mn
        assert np.array_equal(qg.qg_unpack_host("q4_k", packed, 1, 256), canon)


def test_q4_k_pack_places_every_field(L):
    # One row, K = 256: each field of the canonical super-block, set alone, lands
    # where the kernel reads it: d and dmin in the super plane (row 0, slot 0),
    # sub-block j's 6-bit scale and min in bits 4-9 and 10-15 of its scale-plane
    # word (bits 0-3: the centre), and its nibbles in the Q4_0 arrangement of
    # quant-plane block j.
    N, K = 1, 256
    size = qg.qg_packed_size("q4_k", N, K)
    q_bytes, s_off = 8 * 8 * 16, 1024
    u_off = s_off + 256
    for j in range(8):
        for sc, mn in ((1, 0), (0, 1), (63, 0), (0, 63), (37, 50)):
            canon = np.zeros(144, np.uint8)
            canon[0:4] = [0x11, 0x22, 0x33, 0x44]
            u = canon[4:16]
            if j < 4:
                u[j] |= sc
                u[j + 4] |= mn
            else:
                u[j + 4] |= (sc & 15) | ((mn & 15) << 4)
                u[j - 4] |= (sc >> 4) << 6
                u[j] |= (mn >> 4) << 6
            packed = qg.qg_pack_host("q4_k", canon, N, K)
            assert packed.size == size
            assert list(packed[u_off:u_off + 4]) == [0x11, 0x22, 0x33, 0x44]
            # scale plane: (slot 0 * nb + j) * 4 rows * 2 B, row 0
            word = int(packed[s_off + j * 8]) | (int(packed[s_off + j * 8 + 1]) << 8)
            assert word == _q4_k_centre(0x2211, 0x4433, sc, mn) | (sc << 4) | (mn << 10), (j, sc, mn, hex(word))
            assert not packed[:q_bytes].any()
    # weight 64 g + l (l < 32) is the low nibble of byte 32 g + l: sub-block 2 g,
    # element l; weight 64 g + 32 + l the high nibble: sub-block 2 g + 1
    for w in (0, 5, 31, 32, 63, 64, 100, 255):
        canon = np.zeros(144, np.uint8)
        g, l = w // 64, w % 64
        canon[16 + 32 * g + (l % 32)] = 0x0F if l < 32 else 0xF0
        packed = qg.qg_pack_host("q4_k", canon, N, K)
        j, e = 2 * g + (l >= 32), l % 32
        # row 0 is slot 0, b 0 of the only tile: block j's 16 B sit at j * 16
        blk = packed[j * 16: j * 16 + 16]
        dw = int.from_bytes(bytes(blk[4 * (e // 8): 4 * (e // 8) + 4]), "little")
        pos = (e % 8) // 2 + 4 * ((e % 8) % 2)
        assert (dw >> (4 * pos)) & 0xF == 0xF
        assert int(np.unpackbits(packed[:q_bytes]).sum()) == 4


@pytest.mark.parametrize("kind", ["q8_0", "q4_0"])
def test_pack_is_a_permutation_of_bytes(L, kind):
    # The packed planes hold exactly the canonical quants (Q8_0 bytes XOR 0x80,
    # Q4_0 nibbles moved within their block) and scales, plus zeros for the
    # padding rows of the last tile.
    N, K = 13, 1088
    canon = W.matrix(kind, N, K, np.random.default_rng(3))
    packed = qg.qg_pack_host(kind, canon, N, K)
    bb, qb = (34, 32) if kind == "q8_0" else (18, 16)
    KB = K // 32
    rows_pad = (N + 7) // 8 * 8
    blocks = canon.reshape(-1, bb)
    qplane = packed[: rows_pad * KB * qb]
    soff = (qplane.size + 255) // 256 * 256
    splane = packed[soff: soff + rows_pad * KB * 2].copy().view("<u2")
    pad_blocks = (rows_pad - N) * KB
    if kind == "q8_0":
        want_q = np.concatenate([blocks[:, 2:].reshape(-1) ^ 0x80, np.zeros(pad_blocks * qb, np.uint8)])
        got_q = qplane
    else:
        q = blocks[:, 2:].reshape(-1)
        want_q = np.concatenate([q & 0xF, q >> 4, np.zeros(pad_blocks * 32, np.uint8)])
        got_q = np.concatenate([qplane & 0xF, qplane >> 4])
    assert np.array_equal(np.sort(want_q), np.sort(got_q))
    want_s = np.concatenate([blocks[:, 0:2].copy().view("<u2").reshape(-1), np.zeros(pad_blocks, np.uint16)])
    assert np.array_equal(np.sort(want_s), np.sort(splane))
    assert not packed[qplane.size:soff].any() and not packed[soff + splane.size * 2:].any()


@pytest.mark.parametrize("kind", ["q8_0", "q4_0"])
def test_gateup_host_pack_interleaves_rows(L, kind):
    N_ff, K = 11, 2048
    rng = np.random.default_rng(21)
    gate = W.matrix(kind, N_ff, K, rng)
    up = W.matrix(kind, N_ff, K, rng)
    bb = 34 if kind == "q8_0" else 18
    inter = np.stack([gate.reshape(N_ff, -1), up.reshape(N_ff, -1)], axis=1).reshape(-1)
    assert inter.size == 2 * N_ff * (K // 32) * bb
    assert np.array_equal(qg.qg_pack_gateup_host(kind, gate, up, N_ff, K), qg.qg_pack_host(kind, inter, 2 * N_ff, K))
