"""GPU parity of the super-block GEMVs (qgemv_q4_k, qgemv_q6_k) against the fp64
oracle: shapes that span several row tiles, ragged row tiles, ragged last
segments of 8, 16 and 24 blocks, split-K plans, the global-memory activation
path and the persistent form; the device packer against the host packer; exact
closed forms (subnormal d; for Q4_K the min term alone, for Q6_K scale -128 and
the quant extremes); every forced launch shape; and the same bits run to run.

Tolerance: the linear bound 1e-5 * sum |w x| + 1e-7 of the other types, with
sum |w x| from the oracle. Q6_K scales each 16-weight sum of (q - 32) x by its
int8 scale, then by d. Q4_K sums each sub-block as d*sc * sum((q - c) x) +
(d*sc*c - dmin*mn) * sum(x) around a load-time centre c, whose two terms are
bounded by 3 |w| per weight, so its rounding scales with sum |w x| too; the
cancellation cases (d*sc*q = dmin*mn exactly, large scales) are checked below
against the same bound."""
import itertools
import os

import numpy as np
import pytest

import block_dequant_gemv_amd as qg
import oracle as O
from block_dequant_gemv_amd import workloads as W
from gpu_helpers import THREADS, announce, assert_linear, empty_f32, run_qgemv, sync, to_dev

pytestmark = pytest.mark.gpu

# (N, K), K % 256 == 0: one super-block; under one tile; one tile; a tile + 1
# row with an 8-block last segment; 16- and 24-block last segments; 3 full
# segments; 5 segments; 17 segments (split-K); activations too large for LDS;
# then the persistent form: 251 tiles with a ragged row tile and an 8-block last
# segment, and 413 tiles of 5 segments.
SHAPES = [(1, 256), (7, 512), (8, 1024), (9, 1280), (33, 1536), (40, 1792), (100, 3072), (257, 5120),
          (640, 17408), (24, 32768), (2001, 8448), (3300, 5120)]


KINDS = ["q4_k", "q6_k"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("N,K", SHAPES)
def test_kquant_matches_oracle(kind, N, K):
    rng = np.random.default_rng(4000 + N + K)
    canon = W.matrix(kind, N, K, rng)
    x = W.activation(K, rng)
    announce(f"qgemv_{kind} N={N} K={K} plan={qg.qg_plan_info(kind, N, K)}")
    y, tail = run_qgemv(kind, canon, x, N, K, canary=37)
    assert np.all(tail == 12345.0), "wrote past y[N-1]"
    y_ref, a_ref = O.gemv(kind, canon, x, N, K, threads=THREADS)
    assert_linear(y, y_ref, a_ref, f"{kind} {N}x{K}")


@pytest.mark.parametrize("kind", KINDS)
def test_kquant_pack_device_equals_host(kind):
    for N, K in ((1, 256), (9, 1280), (100, 3072), (37, 5120), (5, 1792)):
        canon = W.matrix(kind, N, K, np.random.default_rng(N + K))
        announce(f"qg_pack {kind} N={N} K={K}")
        packed = qg.pack_weights(kind, canon, N, K)
        assert np.array_equal(packed.cpu().numpy(), qg.qg_pack_host(kind, canon, N, K)), (N, K)
    # load-time concatenation of row ranges
    K = 1024
    parts = [(W.matrix(kind, n, K, np.random.default_rng(n)), n) for n in (20, 9, 11)]
    announce(f"qg_pack_rows {kind} concat")
    packed = qg.pack_concat(kind, parts, K)
    cat = np.concatenate([p for p, _ in parts])
    assert np.array_equal(packed.cpu().numpy(), qg.qg_pack_host(kind, cat, 40, K))


def _superblock(d: int, dmin: int, sc: int, mn: int, q: int) -> bytes:
    """One canonical Q4_K super-block with every sub-block's scale sc and min mn
    and every quant q (the 6-bit fields packed as the format stores them)."""
    u = bytearray(12)
    for j in range(8):
        if j < 4:
            u[j] |= sc
            u[j + 4] |= mn
        else:
            u[j + 4] |= (sc & 15) | ((mn & 15) << 4)
            u[j - 4] |= (sc >> 4) << 6
            u[j] |= (mn >> 4) << 6
    return d.to_bytes(2, "little") + dmin.to_bytes(2, "little") + bytes(u) + bytes([q | (q << 4)] * 128)


@pytest.mark.parametrize("d,dmin,sc,mn,q,w", [
    (0x3800, 0x3400, 3, 2, 7, 10.0),               # 0.5 * 3 * 7 - 0.25 * 2
    (0x0001, 0x0000, 63, 0, 15, 945 * 2.0 ** -24),  # subnormal d, no flush to zero
    (0x0000, 0x3C00, 0, 63, 15, -63.0),            # the min term alone
    (0x3C00, 0x3C00, 63, 63, 0, -63.0),            # q = 0: only -dmin * mn remains
    (0x3C00, 0x4000, 16, 32, 4, 0.0),              # 1 * 16 * 4 - 2 * 32: the terms cancel exactly
    (0x5400, 0x5400, 7, 56, 8, 0.0),               # 64 * 7 * 8 - 64 * 56, large scales
    (0x4800, 0x3C00, 1, 63, 15, 57.0),             # 8 * 1 * 15 - 1 * 63: centre 8 (63 / 8 rounded)
    (0x3C00, 0x3C00, 1, 63, 15, -48.0),            # 15 - 63: centre 63 clamped to 15
])
def test_q4_k_closed_forms_exact_on_gpu(d, dmin, sc, mn, q, w):
    # every weight equal, x = 1: y = w * K exactly (every partial sum is exact)
    N, K = 16, 5120
    canon = np.frombuffer(_superblock(d, dmin, sc, mn, q) * (N * K // 256), np.uint8).copy()
    announce(f"q4_k closed form d={d:#x} dmin={dmin:#x} sc={sc} mn={mn} q={q}")
    y = run_qgemv("q4_k", canon, np.ones(K, np.float32), N, K)
    assert np.all(y == np.float32(w * K)), (y[:4], w * K)
    y_ref, _ = O.gemv("q4_k", canon, np.ones(K, np.float32), N, K)
    assert np.all(y_ref == w * K)


def _superblock_fields(d: int, dmin: int, sc, mn, q) -> bytes:
    """One canonical Q4_K super-block from per-sub-block scales sc[8] and mins
    mn[8] and per-weight quants q[256]: weight 64 g + l sits in the low nibble
    and weight 64 g + 32 + l in the high nibble of quant byte 32 g + l."""
    u = bytearray(12)
    for j in range(8):
        if j < 4:
            u[j] |= int(sc[j])
            u[j + 4] |= int(mn[j])
        else:
            u[j + 4] |= (int(sc[j]) & 15) | ((int(mn[j]) & 15) << 4)
            u[j - 4] |= (int(sc[j]) >> 4) << 6
            u[j] |= (int(mn[j]) >> 4) << 6
    qs = bytearray(128)
    for g in range(4):
        for ln in range(32):
            qs[32 * g + ln] = int(q[64 * g + ln]) | (int(q[64 * g + 32 + ln]) << 4)
    return d.to_bytes(2, "little") + dmin.to_bytes(2, "little") + bytes(u) + bytes(qs)


def test_q4_k_cancelling_terms_within_contract_bound():
    # Sub-blocks whose two weight terms d*sc*q and dmin*mn cancel, with large
    # scales: dmin*mn / (d*sc) is 8 or 8 - 1/sc and every quant is 7, 8 or 9, so
    # each weight is 0 or +-d*sc (or within d*sc/sc of it) while d*sc*q and
    # dmin*mn are about 8 d*sc each. Random activations. Row 0 has every weight
    # exactly 0 (mn = 8 sc, q = 8): its output must be exactly 0, with the
    # 1e-7 absolute floor as the whole tolerance.
    N, K = 40, 5120
    rng = np.random.default_rng(31)
    nsb = K // 256
    blocks = []
    for n in range(N):
        for _ in range(nsb):
            d = int(rng.choice([0x4800, 0x4A00, 0x3C00, 0x5400]))   # 8, 12, 1, 64
            sc = rng.integers(1, 8, size=8)
            if n == 0:
                mn, q = 8 * sc, np.full(256, 8)
            else:
                mn = 8 * sc - rng.integers(0, 2, size=8)
                q = rng.integers(7, 10, size=256)
            blocks.append(_superblock_fields(d, d, sc, mn, q))
    canon = np.frombuffer(b"".join(blocks), np.uint8).copy()
    x = W.activation(K, rng)
    announce("q4_k cancelling terms")
    y = run_qgemv("q4_k", canon, x, N, K)
    y_ref, a_ref = O.gemv("q4_k", canon, x, N, K, threads=THREADS)
    assert y_ref[0] == 0.0 and a_ref[0] == 0.0
    assert y[0] == 0.0, y[0]
    assert_linear(y, y_ref, a_ref, "q4_k cancelling terms")
    # the same rows as verify activations: memcmp-equal to M = 1 per row
    X = W.activation(K, rng, M=3)
    packed = qg.pack_weights("q4_k", canon, N, K)
    Y = empty_f32(3 * N)
    qg.qgemv_verify("q4_k", packed, to_dev(X), Y, N, K, 3)
    ones = []
    for m in range(3):
        ym = empty_f32(N)
        qg.qgemv("q4_k", packed, to_dev(X[m]), ym, N, K)
        ones.append(ym)
    sync()
    Yh = Y.cpu().numpy().reshape(3, N)
    Y_ref, A_ref = O.verify("q4_k", canon, X, N, K, threads=THREADS)
    for m in range(3):
        assert Yh[m].tobytes() == ones[m].cpu().numpy().tobytes()
        assert_linear(Yh[m], Y_ref[m], A_ref[m], f"q4_k cancelling terms, verify row {m}")


def _q6_k_superblock(d: int, sc: int, q: int) -> bytes:
    """One canonical Q6_K super-block with every scale sc and every quant q."""
    lo, hi = q & 15, q >> 4
    return bytes([lo | (lo << 4)] * 128) + bytes([hi * 0x55] * 64) + bytes([sc & 255] * 16) + d.to_bytes(2, "little")


@pytest.mark.parametrize("d,sc,q,w", [
    (0x3800, 3, 40, 12.0),                         # 0.5 * 3 * (40 - 32)
    (0x0001, -128, 63, -3968 * 2.0 ** -24),        # subnormal d, scale -128, q = 63
    (0x3C00, 127, 0, -4064.0),                     # q = 0: 127 * -32
    (0x3C00, -1, 32, 0.0),                         # q = 32 is zero
])
def test_q6_k_closed_forms_exact_on_gpu(d, sc, q, w):
    # every weight equal, x = 1: y = w * K exactly (every partial sum is exact)
    N, K = 16, 5120
    canon = np.frombuffer(_q6_k_superblock(d, sc, q) * (N * K // 256), np.uint8).copy()
    announce(f"q6_k closed form d={d:#x} sc={sc} q={q}")
    y = run_qgemv("q6_k", canon, np.ones(K, np.float32), N, K)
    assert np.all(y == np.float32(w * K)), (y[:4], w * K)
    y_ref, _ = O.gemv("q6_k", canon, np.ones(K, np.float32), N, K)
    assert np.all(y_ref == w * K)


KNOBS = ("QG_PERSIST", "QG_SPLIT_K", "QG_X_GLOBAL", "QG_WAVES_PER_WG", "QG_TILES_PER_GROUP", "QG_PREFETCH",
         "QG_STRIDE_GROUPS")


def _set(**kw):
    for k in KNOBS:
        os.environ.pop(k, None)
    for k, v in kw.items():
        os.environ[k] = str(v)
    qg.qg_reload_tuning()


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("N,K", [(203, 8192 + 256), (1000, 1024)])
def test_kquant_forced_launch_shapes(kind, N, K):
    rng = np.random.default_rng(N * K + 4)
    canon = W.matrix(kind, N, K, rng)
    packed = qg.pack_weights(kind, canon, N, K)
    x = W.activation(K, rng)
    xd = to_dev(x)
    y_ref, a_ref = O.gemv(kind, canon, x, N, K, threads=THREADS)
    nseg = -(-K // 1024)
    combos = [dict(QG_PERSIST=1, QG_X_GLOBAL=xg) for xg in (0, 1)]
    combos += [dict(QG_PERSIST=0, QG_STRIDE_GROUPS=3, QG_WAVES_PER_WG=1, QG_SPLIT_K=split)
               for split in (1, 2) if split <= nseg]
    for split, xg, wpw, tpg, pf in itertools.product((1, 2, 3, 4, 8), (0, 1), (1, 2, 4), (1, 3), (1, 2)):
        if split > nseg or (split > 1 and wpw != 4):
            continue
        combos.append(dict(QG_PERSIST=0, QG_SPLIT_K=split, QG_X_GLOBAL=xg, QG_WAVES_PER_WG=wpw,
                           QG_TILES_PER_GROUP=tpg, QG_PREFETCH=pf))
    try:
        for combo in combos:
            _set(**combo)
            ctx = f"{kind} {N}x{K} " + " ".join(f"{k[3:].lower()}={v}" for k, v in combo.items())
            announce(ctx)
            y = empty_f32(N)
            qg.qgemv(kind, packed, xd, y, N, K)
            sync()
            assert_linear(y.cpu().numpy(), y_ref, a_ref, ctx)
    finally:
        _set()


@pytest.mark.parametrize("kind", KINDS)
def test_kquant_run_to_run_bitwise_determinism(kind):
    for N, K in ((1024, 1024), (640, 17408)):
        rng = np.random.default_rng(98)
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
