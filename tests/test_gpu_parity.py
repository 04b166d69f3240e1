"""GPU parity of every entry point against the fp64 oracle, at sizes the oracle
finishes quickly that still span several tiles, ragged row tiles, ragged
K segments, split-K plans and the global-memory activation path."""
import numpy as np
import pytest

import block_dequant_gemv_amd as qg
import oracle as O
from block_dequant_gemv_amd import workloads as W
from gpu_helpers import (THREADS, announce, assert_linear, assert_silu, empty_f32, run_qgemv, sync,
                         to_dev, torch_dev)

pytestmark = pytest.mark.gpu

# (N, K): single block; under one tile; exactly one tile; a tile + 1 row; ragged
# last segment; several segments; 3 segments (split 2 ways); c0 shape; 160
# blocks per row; 17 segments (split 4 ways); activations too large for LDS;
# then two shapes that the planner gives the persistent form (>= 2048 tile x
# segment units under 4096 tiles): 251 tiles with a ragged last row tile and a
# ragged 3-block last segment (9 ranges, fewer tiles than CUs), and 413 tiles
# of 5 segments (two tiles on some workgroups).
SHAPES = [(1, 32), (7, 64), (8, 1024), (9, 1056), (33, 2080), (100, 3072), (1024, 1024), (257, 5120),
          (640, 17408), (24, 32768), (50, 25632), (2001, 8288), (3300, 5120)]


@pytest.mark.parametrize("kind", ["q8_0", "q4_0"])
@pytest.mark.parametrize("N,K", SHAPES)
def test_qgemv_matches_oracle(kind, N, K):
    rng = np.random.default_rng(1000 + N + K)
    canon = W.matrix(kind, N, K, rng)
    x = W.activation(K, rng)
    announce(f"qgemv_{kind} N={N} K={K} plan={qg.qg_plan_info(kind, N, K)}")
    y, tail = run_qgemv(kind, canon, x, N, K, canary=37)
    assert np.all(tail == 12345.0), "wrote past y[N-1]"
    y_ref, a_ref = O.gemv(kind, canon, x, N, K, threads=THREADS)
    assert_linear(y, y_ref, a_ref, f"{kind} {N}x{K}")


@pytest.mark.parametrize("kind", ["q8_0", "q4_0"])
def test_pack_device_equals_host(kind):
    torch = torch_dev()
    for N, K in ((1, 32), (9, 1056), (100, 3072), (37, 5120)):
        canon = W.matrix(kind, N, K, np.random.default_rng(N + K))
        announce(f"qg_pack {kind} N={N} K={K}")
        packed = qg.pack_weights(kind, canon, N, K)
        assert np.array_equal(packed.cpu().numpy(), qg.qg_pack_host(kind, canon, N, K)), (N, K)
    # load-time concatenation (fused QKV)
    K = 1024
    parts = [(W.matrix(kind, n, K, np.random.default_rng(n)), n) for n in (20, 9, 11)]
    announce(f"qg_pack_rows {kind} concat")
    packed = qg.pack_concat(kind, parts, K)
    cat = np.concatenate([p for p, _ in parts])
    assert np.array_equal(packed.cpu().numpy(), qg.qg_pack_host(kind, cat, 40, K))
    # gate|up fusion
    N_ff = 13
    gate, up = (W.matrix(kind, N_ff, K, np.random.default_rng(s)) for s in (1, 2))
    announce(f"qg_pack_gateup {kind}")
    packed = qg.pack_gateup(kind, gate, up, N_ff, K)
    assert np.array_equal(packed.cpu().numpy(), qg.qg_pack_gateup_host(kind, gate, up, N_ff, K))
    del torch


@pytest.mark.parametrize("kind", ["q8_0", "q4_0"])
def test_closed_forms_exact_on_gpu(kind):
    # all-equal quants, equal scales, x = 1: y = c * d * K exactly (every partial sum is exact)
    K, N = 5120, 16
    if kind == "q4_0":
        blk = bytes([0x00, 0x38]) + bytes([0xFF] * 16)          # d = 0.5, v = 7
        expect = 7 * 0.5 * K
    else:
        blk = bytes([0x00, 0x34]) + bytes([3] * 32)             # d = 0.25, q = 3
        expect = 3 * 0.25 * K
    canon = np.frombuffer(blk * (N * K // 32), np.uint8).copy()
    announce(f"closed form {kind}")
    y = run_qgemv(kind, canon, np.ones(K, np.float32), N, K)
    assert np.all(y == expect)
    # subnormal scale 2^-24 with q = 127 (Q8_0) / v = 7 (Q4_0): no flush to zero
    if kind == "q8_0":
        blk = bytes([0x01, 0x00]) + bytes([127] * 32)
        expect = K * 127 * 2.0 ** -24
    else:
        blk = bytes([0x01, 0x00]) + bytes([0xFF] * 16)
        expect = K * 7 * 2.0 ** -24
    canon = np.frombuffer(blk * (N * K // 32), np.uint8).copy()
    y = run_qgemv(kind, canon, np.ones(K, np.float32), N, K)
    assert np.all(y == np.float32(expect))


def test_q8_0_full_int8_range_and_zero_scales():
    N, K = 64, 2048
    rng = np.random.default_rng(8)
    canon = W.q8_0_matrix(N, K, rng).reshape(-1, 34)
    canon[:, 2:] = rng.integers(-128, 128, size=(canon.shape[0], 32), dtype=np.int8).view(np.uint8)
    canon[::5, 0:2] = 0                       # some zero scales
    canon[1::7, 0:2] = [0x01, 0x80]           # some negative subnormal scales (-2^-24)
    canon = canon.reshape(-1)
    x = W.activation(K, rng)
    announce("q8_0 int8 range")
    y = run_qgemv("q8_0", canon, x, N, K)
    y_ref, a_ref = O.gemv("q8_0", canon, x, N, K)
    assert_linear(y, y_ref, a_ref, "q8_0 int8 range")


@pytest.mark.parametrize("kind,N_ff,K", [(k, n, kk) for k in ("q8_0", "q4_0")
                                         for n, kk in ((1, 32), (7, 1056), (3072, 1024), (512, 3072), (300, 5120),
                                                       (100, 17408), (2101, 5120), (10000, 1024))] +
                         [(k, n, kk) for k in ("q4_k", "q6_k") for n, kk in ((7, 1280), (512, 3072), (300, 5120),
                                                                            (2101, 5120))])
def test_fused_gateup_silu_matches_oracle(kind, N_ff, K):
    rng = np.random.default_rng(77 + N_ff + K)
    gate = W.matrix(kind, N_ff, K, rng)
    up = W.matrix(kind, N_ff, K, rng)
    x = W.activation(K, rng)
    announce(f"gateup {kind} N_ff={N_ff} K={K}")
    packed = qg.pack_gateup(kind, gate, up, N_ff, K)
    y = empty_f32(N_ff + 5, fill=-7.0)
    qg.qgemv_fused_gateup_silu(kind, packed, to_dev(x), y, N_ff, K)
    sync()
    y = y.cpu().numpy()
    assert np.all(y[N_ff:] == -7.0)
    out, g, u, ag, au = O.gateup_silu(kind, gate, up, x, N_ff, K, threads=THREADS)
    assert_silu(y[:N_ff], out, g, u, ag, au, f"gateup {kind} {N_ff}x{K}")


@pytest.mark.parametrize("N,K", [(5120, 5120), (256, 5120), (48, 5120), (1, 1), (3, 7), (100, 1000),
                                 (33, 1001), (2049, 64), (600, 24)])
def test_f16_splitk_matches_oracle(N, K):
    rng = np.random.default_rng(N * 31 + K)
    w = W.f16_matrix(N, K, rng)
    x = W.activation(K, rng)
    announce(f"gemv_f16_splitk N={N} K={K}")
    y = empty_f32(N + 3, fill=5.0)
    qg.gemv_f16_splitk(to_dev(w), to_dev(x), y, N, K)
    sync()
    y = y.cpu().numpy()
    assert np.all(y[N:] == 5.0)
    y_ref, a_ref = O.gemv("f16", w, x, N, K, threads=THREADS)
    assert_linear(y[:N], y_ref, a_ref, f"f16 {N}x{K}")


def test_f16_splitk_misaligned_pointers():
    torch = torch_dev()
    N, K = 40, 512
    rng = np.random.default_rng(4)
    w = W.f16_matrix(N, K, rng)
    x = W.activation(K, rng)
    # weights starting 2 bytes into a buffer and x starting 4 bytes in: slow path
    wbuf = torch.zeros(N * K + 1, dtype=torch.int16, device="cuda")
    wbuf[1:] = torch.from_numpy(w.view(np.int16)).to("cuda")
    xbuf = torch.zeros(K + 1, dtype=torch.float32, device="cuda")
    xbuf[1:] = torch.from_numpy(x).to("cuda")
    y = empty_f32(N)
    announce("gemv_f16_splitk misaligned")
    qg.lib()
    st = qg.lib().gemv_f16_splitk(wbuf.data_ptr() + 2, xbuf.data_ptr() + 4, y.data_ptr(), N, K,
                                  torch.cuda.current_stream().cuda_stream)
    assert st == 0, qg.qg_last_error()
    sync()
    y_ref, a_ref = O.gemv("f16", w, x, N, K)
    assert_linear(y.cpu().numpy(), y_ref, a_ref, "f16 misaligned")


@pytest.mark.parametrize("kind", ["q8_0", "q4_0"])
def test_run_to_run_bitwise_determinism(kind):
    torch = torch_dev()
    for N, K in ((1024, 1024), (640, 17408)):
        rng = np.random.default_rng(99)
        canon = W.matrix(kind, N, K, rng)
        x = to_dev(W.activation(K, rng))
        packed = qg.pack_weights(kind, canon, N, K)
        announce(f"determinism {kind} {N}x{K}")
        outs = []
        for _ in range(10):
            y = empty_f32(N)
            qg.qgemv(kind, packed, x, y, N, K)
            outs.append(y)
        sync()
        ref = outs[0].cpu().numpy().tobytes()
        assert all(o.cpu().numpy().tobytes() == ref for o in outs[1:])
    w = W.f16_matrix(48, 5120, np.random.default_rng(5))
    wd, xd = to_dev(w), to_dev(W.activation(5120, np.random.default_rng(6)))
    outs = []
    for _ in range(10):
        y = empty_f32(48)
        qg.gemv_f16_splitk(wd, xd, y, 48, 5120)
        outs.append(y)
    sync()
    assert all(torch.equal(o, outs[0]) for o in outs[1:])


def test_timed_launch_matches_untimed_launch():
    # binding timing events to a launch changes neither the kernel nor its output,
    # and the binding is used by exactly one call
    torch = torch_dev()
    N, K = 1000, 2048
    rng = np.random.default_rng(77)
    for kind in ("q8_0", "q4_0"):
        canon = W.matrix(kind, N, K, rng)
        packed = qg.pack_weights(kind, canon, N, K)
        xd = to_dev(W.activation(K, rng))
        y0, y1, y2 = empty_f32(N), empty_f32(N), empty_f32(N)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for e in ev:
            e.record()
        announce(f"timed launch {kind} {N}x{K}")
        qg.qgemv(kind, packed, xd, y0, N, K)
        qg.qg_time_next_launch(ev[0], ev[1])
        qg.qgemv(kind, packed, xd, y1, N, K)
        qg.qgemv(kind, packed, xd, y2, N, K)
        sync()
        ms = ev[0].elapsed_time(ev[1])
        assert 0.0 < ms < 1000.0, ms
        a0, a1, a2 = (t.cpu().numpy() for t in (y0, y1, y2))
        assert a0.tobytes() == a1.tobytes() == a2.tobytes()
