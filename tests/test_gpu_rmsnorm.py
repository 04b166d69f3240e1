"""GPU parity of the RMSNorm calls against the fp64 oracle: the standalone
qg_rmsnorm, and the GEMVs with the RMSNorm fused into their prologue
(qgemv_rmsnorm, qgemv_rmsnorm_gateup_silu) in both launch forms.

Tolerances. The oracle keeps the normalised activation exact in double. The
GPU's normalised value carries the fp32 error of the sum of squares (a chain of
at most K/1024 + 22 additions), of the square root and division (correctly
rounded) and of two multiplies: at most about 24 units of 2^-24 relative. That
is added to the GEMV's own <= 60 units, so the linear bound 1e-5 * sum|w xn| +
1e-7 (= 168 units) still holds for the fused product; the standalone norm is
checked against 1e-5 of each element's magnitude.
"""
import numpy as np
import pytest

import block_dequant_gemv_amd as qg
import oracle as O
from block_dequant_gemv_amd import workloads as W
from gpu_helpers import THREADS, announce, assert_linear, assert_silu, empty_f32, sync, to_dev

pytestmark = pytest.mark.gpu

EPS = np.float32(1e-6)


def _gamma(K, rng):
    return (1.0 + 0.25 * rng.standard_normal(K)).astype(np.float32)


@pytest.mark.parametrize("K", [1, 7, 32, 1024, 5120, 17408, 100003])
def test_rmsnorm_matches_oracle(K):
    rng = np.random.default_rng(K)
    x = W.activation(K, rng)
    g = _gamma(K, rng)
    out = empty_f32(K + 3, fill=9.0)
    announce(f"qg_rmsnorm K={K}")
    qg.qg_rmsnorm(to_dev(x), to_dev(g), float(EPS), out[:K], K)
    sync()
    got = out.cpu().numpy()
    assert np.all(got[K:] == 9.0), "wrote past out[K-1]"
    ref = O.rmsnorm(x, g, float(EPS))
    err = np.abs(got[:K].astype(np.float64) - ref)
    assert np.all(err <= 1e-5 * np.abs(ref) + 1e-30), float(np.max(err / (np.abs(ref) + 1e-30)))


# (N, K): fused QKV (tile form), a ragged shape, a three-way K split (1024x3072),
# the persistent form (3300x5120, 5120x17408 with its K ranges), and K = 17408
# in the tile form (68 KiB staged)
SHAPES = [(4096, 1024), (33, 2080), (1024, 3072), (3300, 5120), (5120, 17408), (640, 17408)]


@pytest.mark.parametrize("kind,N,K", [(k, n, kk) for k in ("q8_0", "q4_0") for n, kk in SHAPES] +
                         [(k, n, kk) for k in ("q4_k", "q6_k") for n, kk in ((4096, 1024), (3300, 5120), (640, 17408))])
def test_gemv_rmsnorm_matches_oracle(kind, N, K):
    rng = np.random.default_rng(500 + N + K)
    canon = W.matrix(kind, N, K, rng)
    x = W.activation(K, rng)
    g = _gamma(K, rng)
    packed = qg.pack_weights(kind, canon, N, K)
    y = empty_f32(N + 4, fill=-5.0)
    announce(f"qgemv_rmsnorm {kind} {N}x{K} plan={qg.qg_plan_info(kind, N, K)}")
    qg.qgemv_rmsnorm(kind, packed, to_dev(x), to_dev(g), float(EPS), y[:N], N, K)
    sync()
    got = y.cpu().numpy()
    assert np.all(got[N:] == -5.0), "wrote past y[N-1]"
    y_ref, a_ref = O.gemv_rmsnorm(kind, canon, x, g, float(EPS), N, K)
    assert_linear(got[:N], y_ref, a_ref, f"rmsnorm gemv {kind} {N}x{K}")


# The largest K the prologue takes (39 segments, 156 KiB staged next to the
# kernels' static arrays), in each form: one wavefront per tile with eight
# split-K wavefronts (40 rows), the persistent form (1024 and 5120 rows, 13 K
# ranges), and 24000 rows, whose persistent partials would not fit next to the
# staged copy, so the plan takes the tile form (one wavefront per tile).
@pytest.mark.parametrize("N,persistent", [(40, False), (1024, True), (5120, True), (24000, False)])
def test_gemv_rmsnorm_largest_k(N, persistent):
    kind, K = "q4_0", 39936
    plan = qg.qg_plan_info(kind, N, K, 1, rmsnorm=True)
    assert plan["persistent"] == persistent and plan["x_in_lds"] and plan["lds_bytes"] <= 160 * 1024, plan
    rng = np.random.default_rng(700 + N)
    canon = W.matrix(kind, N, K, rng)
    x = W.activation(K, rng)
    g = _gamma(K, rng)
    packed = qg.pack_weights(kind, canon, N, K)
    y = empty_f32(N + 4, fill=-5.0)
    announce(f"qgemv_rmsnorm {kind} {N}x{K} plan={plan}")
    qg.qgemv_rmsnorm(kind, packed, to_dev(x), to_dev(g), float(EPS), y[:N], N, K)
    sync()
    got = y.cpu().numpy()
    assert np.all(got[N:] == -5.0), "wrote past y[N-1]"
    y_ref, a_ref = O.gemv_rmsnorm(kind, canon, x, g, float(EPS), N, K)
    assert_linear(got[:N], y_ref, a_ref, f"rmsnorm gemv {kind} {N}x{K}")


@pytest.mark.parametrize("kind,N_ff,K", [(k, n, kk) for k in ("q8_0", "q4_0")
                                         for n, kk in ((3072, 1024), (100, 5120), (17408, 5120))] +
                         [(k, 300, 5120) for k in ("q4_k", "q6_k")])
def test_gateup_rmsnorm_matches_oracle(kind, N_ff, K):
    rng = np.random.default_rng(900 + N_ff + K)
    gate, up = W.matrix(kind, N_ff, K, rng), W.matrix(kind, N_ff, K, rng)
    x = W.activation(K, rng)
    g = _gamma(K, rng)
    packed = qg.pack_gateup(kind, gate, up, N_ff, K)
    y = empty_f32(N_ff)
    announce(f"qgemv_rmsnorm_gateup_silu {kind} N_ff={N_ff} K={K}")
    qg.qgemv_rmsnorm_gateup_silu(kind, packed, to_dev(x), to_dev(g), float(EPS), y, N_ff, K)
    sync()
    out, gg, uu, ag, au = O.gateup_silu_rmsnorm(kind, gate, up, x, g, float(EPS), N_ff, K)
    assert_silu(y.cpu().numpy(), out, gg, uu, ag, au, f"rmsnorm gate|up {kind} {N_ff}x{K}")


def test_rmsnorm_closed_forms_on_gpu():
    # x = 1, eps = 3, gamma = 2: the normalised activation is exactly 1, so the fused
    # product equals the plain product on x = 1 bit for bit (same kernel, same sums),
    # and the standalone norm returns exactly 1; x = 0 with eps > 0 gives exactly 0
    rng = np.random.default_rng(12)
    for kind, N, K in (("q8_0", 4096, 1024), ("q4_0", 3300, 5120)):
        canon = W.matrix(kind, N, K, rng)
        packed = qg.pack_weights(kind, canon, N, K)
        ones, twos = to_dev(np.ones(K, np.float32)), to_dev(np.full(K, 2.0, np.float32))
        y_norm, y_plain, out = empty_f32(N), empty_f32(N), empty_f32(K)
        announce(f"rmsnorm closed forms {kind} {N}x{K}")
        qg.qgemv_rmsnorm(kind, packed, ones, twos, 3.0, y_norm, N, K)
        qg.qgemv(kind, packed, ones, y_plain, N, K)
        qg.qg_rmsnorm(ones, twos, 3.0, out, K)
        sync()
        assert y_norm.cpu().numpy().tobytes() == y_plain.cpu().numpy().tobytes()
        assert np.all(out.cpu().numpy() == 1.0)
        zeros = to_dev(np.zeros(K, np.float32))
        qg.qgemv_rmsnorm(kind, packed, zeros, twos, 1e-6, y_norm, N, K)
        sync()
        assert np.all(y_norm.cpu().numpy() == 0.0)
