"""Parity at the full sizes of the five workload configurations, with the same
entry points (and therefore launch plans) that bench.py times.

Every output row is checked against the fp64 oracle (the oracle runs on up to
16 host threads); verify rows are also compared with memcmp against M=1.
"""
import numpy as np
import pytest

import block_dequant_gemv_amd as qg
import oracle as O
from block_dequant_gemv_amd.workloads import Workload
from gpu_helpers import THREADS, announce, assert_linear, assert_silu, empty_f32, sync, to_dev

pytestmark = pytest.mark.gpu


def _gemv_case(wl: Workload, name: str):
    _, kind, N, K, _ = wl.entry(name)
    canon = wl.weight(name)
    x = wl.x(name)
    announce(f"config {wl.cfg} {name}: {kind} {N}x{K}")
    if kind == "f16":
        y = empty_f32(N)
        qg.gemv_f16_splitk(to_dev(canon), to_dev(x), y, N, K)
    else:
        packed = qg.pack_weights(kind, canon, N, K)
        y = empty_f32(N)
        qg.qgemv(kind, packed, to_dev(x), y, N, K)
    sync()
    y_ref, a_ref = O.gemv(kind, canon, x, N, K, threads=THREADS)
    return assert_linear(y.cpu().numpy(), y_ref, a_ref, f"config {wl.cfg} {name}")


def _gateup_case(wl: Workload, gate: str, up: str):
    _, kind, N_ff, K, _ = wl.entry(gate)
    g, u = wl.weight(gate), wl.weight(up)
    x = wl.x(gate)
    announce(f"config {wl.cfg} fused gate|up: {kind} 2x{N_ff}x{K}")
    packed = qg.pack_gateup(kind, g, u, N_ff, K)
    y = empty_f32(N_ff)
    qg.qgemv_fused_gateup_silu(kind, packed, to_dev(x), y, N_ff, K)
    sync()
    out, gg, uu, ag, au = O.gateup_silu(kind, g, u, x, N_ff, K, threads=THREADS)
    return assert_silu(y.cpu().numpy(), out, gg, uu, ag, au, f"config {wl.cfg} gate|up")


def test_config0_q8_0_1024():
    _gemv_case(Workload(0), "w")


def test_config1_qwen3_decode_set():
    wl = Workload(1)
    # fused QKV: three projections packed into one concatenated weight
    K = 1024
    parts = [(wl.weight(n), wl.entry(n)[2]) for n in ("q_proj", "k_proj", "v_proj")]
    x = wl.x("q_proj")
    announce("config 1 fused QKV 4096x1024")
    packed = qg.pack_concat("q8_0", parts, K)
    y = empty_f32(4096)
    qg.qgemv_q8_0(packed, to_dev(x), y, 4096, K)
    sync()
    y = y.cpu().numpy()
    row0 = 0
    for canon, rows in parts:
        y_ref, a_ref = O.gemv("q8_0", canon, x, rows, K, threads=THREADS)
        assert_linear(y[row0:row0 + rows], y_ref, a_ref, f"QKV rows {row0}..{row0 + rows}")
        row0 += rows
    _gemv_case(wl, "o_proj")
    _gateup_case(wl, "gate", "up")
    _gemv_case(wl, "down")
    _gemv_case(wl, "lm_head")


def test_config2_q4_0_27b_shapes():
    wl = Workload(2)
    _gateup_case(wl, "gate", "up")
    wl.drop("gate")
    wl.drop("up")
    _gemv_case(wl, "down")
    _gemv_case(wl, "lm_head")


def test_config3_f16_splitk():
    wl = Workload(3)
    for name in ("square", "thin", "small"):
        _gemv_case(wl, name)


@pytest.mark.parametrize("name", ["q4_0_w", "q8_0_w"])
def test_config4_verify(name):
    wl = Workload(4)
    _, kind, N, K, _ = wl.entry(name)
    canon = wl.weight(name)
    packed = qg.pack_weights(kind, canon, N, K)
    X = wl.x(name, M=6)
    Xd = to_dev(X)
    ones = []
    for m in range(6):
        y = empty_f32(N)
        qg.qgemv(kind, packed, Xd[m].contiguous(), y, N, K)
        ones.append(y)
    sync()
    ones = [o.cpu().numpy() for o in ones]
    Y_ref, A_ref = O.verify(kind, canon, X, N, K, threads=THREADS)
    for m in range(6):
        assert_linear(ones[m], Y_ref[m], A_ref[m], f"config 4 {name} M=1 row {m}")
    for M in range(2, 7):
        announce(f"config 4 verify {name} M={M}")
        Y = empty_f32(M * N)
        qg.qgemv_verify(kind, packed, Xd[:M].contiguous(), Y, N, K, M)
        sync()
        Yh = Y.cpu().numpy().reshape(M, N)
        for m in range(M):
            assert Yh[m].tobytes() == ones[m].tobytes(), f"{name} M={M} row {m} differs from M=1"
