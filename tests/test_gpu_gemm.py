"""GPU parity of the small-M GEMM (qgemm_prefill, matrix cores) against the fp64
oracle: Y[m] = W X[m] for every activation row, within the linear bound
1e-5 * sum|w x| + 1e-7 of each output. Shapes span several row tiles and
workgroups, a ragged last weight tile, a ragged last K segment and a ragged
last chunk of it, M below, at and across the 16-row activation tile and the
64-row activation group, every group width (QG_GEMM_MT = 1..4), 1, 2, 4 and 8
wavefronts of 1 and 2 row groups per workgroup and the K split across
workgroups (with its partial sums added in a fixed order)."""
import os

import numpy as np
import pytest

import block_dequant_gemv_amd as qg
import oracle as O
from block_dequant_gemv_amd import workloads as W
from gpu_helpers import THREADS, announce, assert_linear, sync, to_dev, torch_dev

pytestmark = pytest.mark.gpu

# (N, K, M); M = 80 runs two groups of four activation tiles, the second with
# three zero tiles, over a ragged 33-block K (its last chunk holds one block).
# The activation split holds a row in registers up to K = 32768, 1, 2 or 4 lane
# runs per thread (K <= 8192, <= 16384, <= 32768: 12288 and 17408 take the
# last two), and splits longer rows in two passes (40960)
SHAPES = [(4096, 1024, 16), (1024, 3072, 8), (300, 2080, 20), (33, 1056, 1), (257, 5120, 40), (2048, 17408, 3),
          (1000, 1024, 64), (17408, 5120, 32), (300, 1056, 80), (100, 12288, 5), (64, 40960, 3)]


def _run(kind, packed, X, N, K, M, tail=0, ws=None):
    torch = torch_dev()
    Y = torch.full((M * N + tail,), -9.0, dtype=torch.float32, device="cuda")
    ws = qg.qgemm_prefill(kind, packed, to_dev(X), Y, N, K, M, workspace=ws)
    sync()
    out = Y.cpu().numpy()
    return out[:M * N].reshape(M, N), out[M * N:], ws


@pytest.mark.parametrize("kind", ["q8_0", "q4_0"])
@pytest.mark.parametrize("N,K,M", SHAPES)
def test_gemm_matches_oracle(kind, N, K, M):
    rng = np.random.default_rng(7000 + N + K + M)
    canon = W.matrix(kind, N, K, rng)
    X = W.activation(K, rng, M=M).reshape(M, K)
    packed = qg.pack_weights(kind, canon, N, K)
    announce(f"qgemm_prefill {kind} N={N} K={K} M={M}")
    Y, tail, _ = _run(kind, packed, X, N, K, M, tail=9)
    assert np.all(tail == -9.0), "wrote past Y"
    Y_ref, A_ref = O.verify(kind, canon, X, N, K, threads=THREADS)
    for m in range(M):
        assert_linear(Y[m], Y_ref[m], A_ref[m], f"gemm {kind} {N}x{K} M={M} row {m}")


@pytest.mark.parametrize("kind", ["q8_0", "q4_0"])
def test_gemm_pass_widths_and_determinism(kind):
    N, K, M = 640, 5120, 72
    rng = np.random.default_rng(31)
    canon = W.matrix(kind, N, K, rng)
    X = W.activation(K, rng, M=M).reshape(M, K)
    packed = qg.pack_weights(kind, canon, N, K)
    Y_ref, A_ref = O.verify(kind, canon, X, N, K, threads=THREADS)
    outs = {}
    try:
        for mt in ("1", "2", "3", "4"):
            os.environ["QG_GEMM_MT"] = mt
            qg.qg_reload_tuning()
            announce(f"qgemm_prefill {kind} groups of {mt} activation tiles")
            Y, _, ws = _run(kind, packed, X, N, K, M)
            Y2, _, _ = _run(kind, packed, X, N, K, M, ws=ws)
            assert np.array_equal(Y.view(np.uint32), Y2.view(np.uint32)), "run-to-run bits differ"
            for m in range(M):
                assert_linear(Y[m], Y_ref[m], A_ref[m], f"gemm {kind} MT={mt} row {m}")
            outs[mt] = Y
    finally:
        os.environ.pop("QG_GEMM_MT", None)
        qg.qg_reload_tuning()
    # the group width changes which workgroup computes a row, not its operations
    same = [np.array_equal(outs[mt].view(np.uint32), outs["1"].view(np.uint32)) for mt in ("2", "3", "4")]
    assert all(same), f"group widths 2, 3, 4 against 1: bit-equal {same}"


@pytest.mark.parametrize("kind", ["q8_0", "q4_0"])
def test_gemm_launch_shapes(kind):
    # every (row groups, workgroup size, K split) against the oracle; the K split
    # changes the rounding of a row, the other knobs only who computes it
    N, K, M = 300, 5120, 20
    rng = np.random.default_rng(77)
    canon = W.matrix(kind, N, K, rng)
    X = W.activation(K, rng, M=M).reshape(M, K)
    packed = qg.pack_weights(kind, canon, N, K)
    Y_ref, A_ref = O.verify(kind, canon, X, N, K, threads=THREADS)
    knobs = ("QG_GEMM_ROWGROUPS", "QG_GEMM_WAVES", "QG_GEMM_KSPLIT", "QG_GEMM_MT")
    by_split = {}
    try:
        for rg, gw, ks in ((1, 4, 1), (2, 4, 1), (2, 8, 1), (1, 8, 1), (2, 1, 1), (2, 2, 1), (1, 4, 2), (2, 2, 3),
                           (2, 8, 5), (1, 1, 5)):
            for kk in knobs:
                os.environ.pop(kk, None)
            os.environ.update(QG_GEMM_ROWGROUPS=str(rg), QG_GEMM_WAVES=str(gw), QG_GEMM_KSPLIT=str(ks))
            qg.qg_reload_tuning()
            announce(f"qgemm_prefill {kind} rowgroups={rg} waves={gw} ksplit={ks}")
            Y, tail, _ = _run(kind, packed, X, N, K, M, tail=5)
            assert np.all(tail == -9.0)
            for m in range(M):
                assert_linear(Y[m], Y_ref[m], A_ref[m], f"gemm {kind} rg={rg} g={gw} ks={ks} row {m}")
            if ks in by_split:
                assert np.array_equal(Y.view(np.uint32), by_split[ks].view(np.uint32)), \
                    "launch shape changed the bits at a fixed K split"
            by_split[ks] = Y
    finally:
        for kk in knobs:
            os.environ.pop(kk, None)
        qg.qg_reload_tuning()


@pytest.mark.parametrize("kind", ["q8_0", "q4_0"])
def test_gemm_row_scaling_handles_dynamic_range(kind):
    # rows of very different magnitude (1e-6 .. 1e6, and an all-zero row): each row
    # gets its own power-of-two scale before the fp16 split, so every row keeps
    # the relative accuracy of the linear bound
    N, K, M = 512, 2048, 6
    rng = np.random.default_rng(5)
    canon = W.matrix(kind, N, K, rng)
    X = W.activation(K, rng, M=M).reshape(M, K)
    X = X * np.array([1e-6, 1.0, 1e6, 3e-3, 0.0, 2.0 ** 20], np.float32)[:, None]
    X[5, ::7] *= np.float32(1e-3)     # a wide spread inside one row as well
    packed = qg.pack_weights(kind, canon, N, K)
    announce(f"qgemm_prefill {kind} dynamic range")
    Y, _, _ = _run(kind, packed, X.astype(np.float32), N, K, M)
    Y_ref, A_ref = O.verify(kind, canon, X.astype(np.float32), N, K, threads=THREADS)
    for m in range(M):
        assert_linear(Y[m], Y_ref[m], A_ref[m], f"gemm {kind} dynamic range row {m}")
    assert np.all(Y[4] == 0.0)


def test_gemm_closed_form_exact():
    # all-equal quants and scales with X = 1: every partial sum is an exact small
    # integer multiple of d, so the GEMM returns c * d * K exactly in every output
    torch = torch_dev()
    K, N, M = 5120, 64, 17
    for kind, blk, expect in (("q4_0", bytes([0x00, 0x38]) + bytes([0xFF] * 16), 7 * 0.5 * K),
                              ("q8_0", bytes([0x00, 0x34]) + bytes([3] * 32), 3 * 0.25 * K)):
        canon = np.frombuffer(blk * (N * K // 32), np.uint8).copy()
        packed = qg.pack_weights(kind, canon, N, K)
        announce(f"qgemm_prefill closed form {kind}")
        Y, _, _ = _run(kind, packed, np.ones((M, K), np.float32), N, K, M)
        assert np.all(Y == expect), (kind, Y.min(), Y.max())
    del torch


@pytest.mark.parametrize("kind", ["q8_0", "q4_0"])
def test_gemm_unaligned_activations_same_bits(kind):
    # X only 4-byte aligned (the documented minimum) takes the activation split's
    # scalar loads; the split's arithmetic is the same, so Y is the same bits as
    # with a 16-byte-aligned X, and within the bound of the oracle
    torch = torch_dev()
    N, K, M = 300, 2080, 20
    rng = np.random.default_rng(77)
    canon = W.matrix(kind, N, K, rng)
    X = W.activation(K, rng, M=M).reshape(M, K)
    packed = qg.pack_weights(kind, canon, N, K)
    announce(f"qgemm_prefill {kind} unaligned X")
    Y_al, _, ws = _run(kind, packed, X, N, K, M)
    buf = torch.empty(M * K + 4, dtype=torch.float32, device="cuda")
    Xu = buf[1:1 + M * K]
    assert Xu.data_ptr() % 16 == 4
    Xu.copy_(torch.from_numpy(X.reshape(-1)))
    Y = torch.full((M * N,), -9.0, dtype=torch.float32, device="cuda")
    qg.qgemm_prefill(kind, packed, Xu, Y, N, K, M, workspace=ws)
    sync()
    Y_un = Y.cpu().numpy().reshape(M, N)
    assert np.array_equal(Y_un.view(np.uint32), Y_al.view(np.uint32))
    Y_ref, A_ref = O.verify(kind, canon, X, N, K, threads=THREADS)
    for m in range(M):
        assert_linear(Y_un[m], Y_ref[m], A_ref[m], f"gemm {kind} unaligned X row {m}")
