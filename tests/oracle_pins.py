"""Pins of the fp64 oracle to facts other than itself.

Each pin is a function of a loaded oracle library ``L`` and raises
AssertionError when the oracle disagrees with:
  * IEEE binary16 decoding as numpy implements it (all 65536 patterns),
  * the byte sizes the pages print (1.06 and 0.56 bytes per weight),
  * hand-worked closed forms of single blocks (tests/golden/single_blocks.json),
  * exact rational brute force on tiny random shapes (fractions.Fraction),
  * textbook special cases that reduce to a float64 numpy matmul,
  * invariants (exact scaling, zero blocks, row permutation),
  * the composition rules of the fused and multi-row entry points,
  * closed forms of RMSNorm (a vector of ones with eps = 3; alternating +-c),
  * hand-worked Q4_K super-blocks (tests/golden/q4_k_blocks.json) and closed forms;
  * hand-worked Q6_K super-blocks (tests/golden/q6_k_blocks.json), closed forms and
    the integer-matrix special case.
``test_oracle_mutants.py`` plants plausible mistakes in a copy of oracle.c and
checks that every one of them trips at least one pin.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle as O
from block_dequant_gemv_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---- tiny canonical block builders (test side, written from the format) ----

def q8_block(scale_bits: int, quants) -> bytes:
    quants = list(quants)
    assert len(quants) == 32
    return bytes([scale_bits & 0xFF, scale_bits >> 8]) + bytes(q & 0xFF for q in quants)


def q4_block_from_bytes(scale_bits: int, qs) -> bytes:
    qs = list(qs)
    assert len(qs) == 16
    return bytes([scale_bits & 0xFF, scale_bits >> 8]) + bytes(qs)


def q4_block_from_values(scale_bits: int, vals) -> bytes:
    """Encode 32 values in [-8, 7]: byte j = (v[j]+8) | (v[j+16]+8) << 4."""
    vals = list(vals)
    assert len(vals) == 32 and all(-8 <= v <= 7 for v in vals)
    qs = [((vals[j] + 8) & 0xF) | (((vals[j + 16] + 8) & 0xF) << 4) for j in range(16)]
    return q4_block_from_bytes(scale_bits, qs)


def _u8(b: bytes) -> np.ndarray:
    return np.frombuffer(b, dtype=np.uint8).copy()


def _gemv(L, kind, w, x, N, K, threads=1):
    return O.gemv(kind, w, x, N, K, threads=threads, L=L)


# ---- independent exact decoding for brute force ----------------------------

def _exact_weights(kind: str, w: np.ndarray, N: int, K: int):
    """Fractions W[n][k] decoded with numpy's fp16 and the format definition."""
    rows = []
    if kind == "f16":
        vals = w.view(np.uint16).astype("<u2").view(np.float16).astype(np.float64).reshape(N, K)
        return [[Fraction(float(v)) for v in r] for r in vals]
    bb = W.Q8_0_BLOCK_BYTES if kind == "q8_0" else W.Q4_0_BLOCK_BYTES
    blocks = w.reshape(N, K // 32, bb)
    for n in range(N):
        row = []
        for b in range(K // 32):
            blk = blocks[n, b]
            d = Fraction(float(blk[0:2].copy().view("<u2").view(np.float16)[0]))
            if kind == "q8_0":
                q = blk[2:].view(np.int8).astype(int)
                row += [d * int(v) for v in q]
            else:
                qs = blk[2:].astype(int)
                lo = [int(v) & 0xF for v in qs]
                hi = [int(v) >> 4 for v in qs]
                row += [d * (v - 8) for v in lo + hi]
        rows.append(row)
    return rows


# ---- the pins --------------------------------------------------------------

def pin_half_decode_all_patterns(L):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([L.oracle_half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_format_sizes(L):
    g = _golden("format_sizes.json")
    assert round(g["q8_0"]["block_bytes"] / g["block_weights"], 2) == g["q8_0"]["printed_bytes_per_weight"]
    assert round(g["q4_0"]["block_bytes"] / g["block_weights"], 2) == g["q4_0"]["printed_bytes_per_weight"]
    # the oracle must step exactly one block size per 32 weights: a two-block
    # row whose blocks differ is read as two independent blocks
    for kind, bb in (("q8_0", 34), ("q4_0", 18)):
        if kind == "q8_0":
            blk0 = q8_block(0x3C00, [1] * 32)          # 1.0 * 1 * 32
            blk1 = q8_block(0x4000, [-3] * 32)         # 2.0 * -3 * 32
        else:
            blk0 = q4_block_from_values(0x3C00, [1] * 32)
            blk1 = q4_block_from_values(0x4000, [-3] * 32)
        assert len(blk0) == bb
        y, a = _gemv(L, kind, _u8(blk0 + blk1), np.ones(64, np.float32), 1, 64)
        assert y[0] == 32.0 - 192.0 and a[0] == 32.0 + 192.0


def pin_single_blocks(L):
    cases = {c["id"]: c for c in _golden("single_blocks.json")["cases"]}
    # E1
    c = cases["E1_q8_0_ramp"]
    assert 0.5 * sum(i - 16 for i in range(32)) == c["expected"]
    y, _ = _gemv(L, "q8_0", _u8(q8_block(0x3800, [i - 16 for i in range(32)])), np.ones(32, np.float32), 1, 32)
    assert y[0] == c["expected"]
    # E2: -128 is a legal Q8_0 quant
    c = cases["E2_q8_0_min_int8"]
    y, a = _gemv(L, "q8_0", _u8(q8_block(0x3C00, [127, -128] + [0] * 30)), np.ones(32, np.float32), 1, 32)
    assert y[0] == c["expected"] and a[0] == 255.0
    # E3: nibble order, with x_k = k so that the two orders differ
    c = cases["E3_q4_0_nibble_order"]
    xk = np.arange(32, dtype=np.float32)
    blk = _u8(q4_block_from_bytes(0x3400, range(16)))
    y, _ = _gemv(L, "q4_0", blk, xk, 1, 32)
    assert y[0] == c["expected"], (y[0], "interleaved order gives", c["interleaved_order_would_give"])
    y1, _ = _gemv(L, "q4_0", blk, np.ones(32, np.float32), 1, 32)
    assert y1[0] == c["x_all_ones_gives_for_both_orders"]
    # E4: all-equal quants, closed form c * d * K
    c = cases["E4a_q4_0_all_equal"]
    K = c["K"]
    w = _u8(q4_block_from_bytes(0x3800, [0xFF] * 16) * (K // 32))
    y, _ = _gemv(L, "q4_0", w, np.ones(K, np.float32), 1, K)
    assert y[0] == (15 - 8) * 0.5 * K == c["expected"]
    c = cases["E4b_q8_0_all_equal"]
    K = c["K"]
    w = _u8(q8_block(0x3400, [3] * 32) * (K // 32))
    y, _ = _gemv(L, "q8_0", w, np.ones(K, np.float32), 1, K)
    assert y[0] == 3 * 0.25 * K == c["expected"]
    # E4 with unequal scales and x: y = c * sum_b d_b * sum_{k in b} x_k
    rng = np.random.default_rng(11)
    K = 256
    scales = [0x3000 + 0x100 * b for b in range(K // 32)]
    x = rng.integers(-4, 5, K).astype(np.float32)
    w = _u8(b"".join(q8_block(s, [-5] * 32) for s in scales))
    y, _ = _gemv(L, "q8_0", w, x, 1, K)
    ds = np.array(scales, np.uint16).view(np.float16).astype(np.float64)
    assert y[0] == -5 * sum(ds[b] * float(x[32 * b:32 * b + 32].sum()) for b in range(K // 32))
    # E5: subnormal scale kept exactly
    c = cases["E5_subnormal_scale"]
    y, _ = _gemv(L, "q8_0", _u8(q8_block(0x0001, [127] * 32)), np.ones(32, np.float32), 1, 32)
    assert y[0] == c["expected"] == 32 * 127 * 2.0 ** -24


def pin_silu(L):
    c = {c["id"]: c for c in _golden("single_blocks.json")["cases"]}["E6_silu"]
    for g, u, expect in c["points"]:
        got = L.oracle_silu(g) * u
        assert math.isfinite(got)
        assert abs(got - expect) <= 1e-15 * max(1.0, abs(expect)), (g, got, expect)
    # odd part and limits: silu(g) - silu(-g) = g; silu(g) -> g for large g
    for g in (0.3, 2.5, 7.0):
        assert abs((L.oracle_silu(g) - L.oracle_silu(-g)) - g) <= 1e-15 * g
    assert L.oracle_silu(40.0) == 40.0


def pin_bruteforce_exact(L):
    rng = np.random.default_rng(1234)
    for kind in ("q8_0", "q4_0", "f16"):
        for N, K in ((1, 32), (3, 64), (4, 96), (2, 128), (4, 40 if kind == "f16" else 32)):
            w = W.matrix(kind, N, K, rng)
            x = rng.standard_normal(K).astype(np.float32)
            y, a = _gemv(L, kind, w, x, N, K)
            Wx = _exact_weights(kind, w, N, K)
            for n in range(N):
                prods = [Wx[n][k] * Fraction(float(x[k])) for k in range(K)]
                exact = sum(prods, Fraction(0))
                amag = sum((abs(p) for p in prods), Fraction(0))
                bound = K * 2.0 ** -53 * float(amag)
                assert abs(Fraction(y[n]) - exact) <= Fraction(bound), (kind, N, K, n)
                assert abs(Fraction(a[n]) - amag) <= Fraction(bound), (kind, N, K, n)


def pin_textbook(L):
    rng = np.random.default_rng(77)
    N, K = 16, 256
    x = rng.standard_normal(K).astype(np.float32)
    x64 = x.astype(np.float64)
    # Q8_0 with every scale 1.0: W is the int8 matrix itself
    q = rng.integers(-128, 128, size=(N * K // 32, 32), dtype=np.int8)
    blocks = b"".join(q8_block(0x3C00, row.astype(int)) for row in q)
    y, a = _gemv(L, "q8_0", _u8(blocks), x, N, K)
    Wm = q.astype(np.float64).reshape(N, K)
    ref = Wm @ x64
    assert np.all(np.abs(y - ref) <= 1e-12 * (np.abs(Wm) @ np.abs(x64)))
    # Q4_0 with every scale 1.0: W holds the integers v in [-8, 7]
    v = rng.integers(-8, 8, size=(N * K // 32, 32))
    blocks = b"".join(q4_block_from_values(0x3C00, row) for row in v)
    y, _ = _gemv(L, "q4_0", _u8(blocks), x, N, K)
    Wm = v.astype(np.float64).reshape(N, K)
    assert np.all(np.abs(y - Wm @ x64) <= 1e-12 * (np.abs(Wm) @ np.abs(x64)))
    # fp16 weights: numpy's own fp16 -> fp64 matmul
    w16 = rng.normal(0, 0.02, N * K).astype(np.float16)
    y, _ = _gemv(L, "f16", w16.view(np.uint16), x, N, K)
    Wm = w16.astype(np.float64).reshape(N, K)
    assert np.all(np.abs(y - Wm @ x64) <= 1e-12 * (np.abs(Wm) @ np.abs(x64)))


def pin_invariants(L):
    rng = np.random.default_rng(5)
    for kind in ("q8_0", "q4_0", "f16"):
        N, K = 12, 192
        w = W.matrix(kind, N, K, rng)
        x = rng.standard_normal(K).astype(np.float32)
        y, a = _gemv(L, kind, w, x, N, K)
        # exact power-of-two scaling
        y2, a2 = _gemv(L, kind, w, (2 * x).astype(np.float32), N, K)
        assert np.array_equal(y2, 2 * y) and np.array_equal(a2, 2 * a)
        # row permutation permutes y (rows are independent)
        perm = rng.permutation(N)
        if kind == "f16":
            wp = w.reshape(N, K)[perm].reshape(-1)
        else:
            bb = 34 if kind == "q8_0" else 18
            wp = w.reshape(N, -1)[perm].reshape(-1)
            assert w.size == N * (K // 32) * bb
        yp, _ = _gemv(L, kind, wp, x, N, K)
        assert np.array_equal(yp, y[perm])
        if kind == "f16":
            continue
        # a zero scale silences a block: same y as the block's x set to zero
        bb = 34 if kind == "q8_0" else 18
        wz = w.reshape(N, K // 32, bb).copy()
        wz[:, 2, 0:2] = 0
        yz, _ = _gemv(L, kind, wz.reshape(-1), x, N, K)
        xz = x.copy()
        xz[64:96] = 0
        yx, _ = _gemv(L, kind, w, xz, N, K)
        assert np.array_equal(yz, yx)


def pin_composites(L):
    rng = np.random.default_rng(9)
    for kind in ("q8_0", "q4_0"):
        N, K = 10, 128
        gate = W.matrix(kind, N, K, rng)
        up = W.matrix(kind, N, K, rng)
        x = rng.standard_normal(K).astype(np.float32)
        out, g, u, ag, au = O.gateup_silu(kind, gate, up, x, N, K, L=L)
        gy, ga = _gemv(L, kind, gate, x, N, K)
        uy, ua = _gemv(L, kind, up, x, N, K)
        assert np.array_equal(g, gy) and np.array_equal(u, uy)
        assert np.array_equal(ag, ga) and np.array_equal(au, ua)
        assert np.array_equal(out, np.array([L.oracle_silu(float(a)) for a in gy]) * uy)
        # verify rows are independent M=1 products
        X = rng.standard_normal((4, K)).astype(np.float32)
        Y, A = O.verify(kind, gate, X, N, K, L=L)
        for m in range(4):
            ym, am = _gemv(L, kind, gate, X[m], N, K)
            assert np.array_equal(Y[m], ym) and np.array_equal(A[m], am)
        # chosen rows, and threads, give the same bits as the plain loop
        rows = np.array([N - 1, 0, 3], np.int64)
        yr, ar = O.gemv_rows(kind, gate, x, rows, N, K, L=L)
        assert np.array_equal(yr, gy[rows]) and np.array_equal(ar, ga[rows])
        yt, at = _gemv(L, kind, gate, x, N, K, threads=3)
        assert np.array_equal(yt, gy) and np.array_equal(at, ga)


def pin_epilogue(L):
    # the epilogue adds bias and residual to the product: with every scale zero the
    # product is exactly 0 and the output is bias + residual (an exact double sum
    # of two fp32 values); on the worked single block E1 (product -8) a bias of
    # 0.5 and a residual of 0.25 give -7.25; with neither the plain product results
    rng = np.random.default_rng(31)
    for kind in ("q8_0", "q4_0"):
        N, K = 7, 96
        w = W.matrix(kind, N, K, rng)
        bb = W.Q8_0_BLOCK_BYTES if kind == "q8_0" else W.Q4_0_BLOCK_BYTES
        wz = w.reshape(N, K // 32, bb).copy()
        wz[:, :, 0:2] = 0                          # scale fields: fp16 +0
        wz = wz.reshape(-1)
        x = rng.standard_normal(K).astype(np.float32)
        b = rng.standard_normal(N).astype(np.float32)
        r = rng.standard_normal(N).astype(np.float32)
        out, a = O.gemv_epilogue(kind, wz, x, N, K, bias=b, residual=r, L=L)
        assert np.array_equal(out, b.astype(np.float64) + r.astype(np.float64)) and np.all(a == 0.0)
        out, _ = O.gemv_epilogue(kind, wz, x, N, K, bias=b, L=L)
        assert np.array_equal(out, b.astype(np.float64))
        out, _ = O.gemv_epilogue(kind, wz, x, N, K, residual=r, L=L)
        assert np.array_equal(out, r.astype(np.float64))
        y0, a0 = _gemv(L, kind, w, x, N, K)
        out, a = O.gemv_epilogue(kind, w, x, N, K, L=L)
        assert np.array_equal(out, y0) and np.array_equal(a, a0)
    e1 = _u8(q8_block(0x3800, [i - 16 for i in range(32)]))
    ones = np.ones(32, np.float32)
    out, _ = O.gemv_epilogue("q8_0", e1, ones, 1, 32, bias=np.array([0.5], np.float32),
                             residual=np.array([0.25], np.float32), L=L)
    assert out[0] == -7.25, out


def pin_rmsnorm(L):
    # closed forms of gamma * x / sqrt(mean(x^2) + eps):
    #  x = 1 everywhere, eps = 3, gamma = 2: 2 / sqrt(1 + 3) = 1 exactly, for any K
    #  (a sum instead of the mean, a dropped eps or sqrt, or a dropped gamma all move it)
    for K in (1, 5, 64, 1024):
        out = O.rmsnorm(np.ones(K, np.float32), np.full(K, 2.0, np.float32), 3.0, L=L)
        assert np.all(out == 1.0), (K, out[:4])
    #  x = +-c alternating (c a power of two), eps = 0: every |x| equals the rms, so
    #  out = +-gamma exactly, element by element (catches a shifted gamma or x index)
    K = 96
    sign = np.where(np.arange(K) % 2 == 0, 1.0, -1.0)
    gam = (np.arange(K) + 1).astype(np.float32) / 8
    for c in (0.25, 8.0, 2.0 ** -20):
        out = O.rmsnorm((c * sign).astype(np.float32), gam, 0.0, L=L)
        assert np.array_equal(out, sign * gam.astype(np.float64)), c
    #  eps = 0: scaling x by a power of two changes nothing, bit for bit
    rng = np.random.default_rng(41)
    x = rng.standard_normal(200).astype(np.float32)
    g = rng.standard_normal(200).astype(np.float32)
    assert np.array_equal(O.rmsnorm(x, g, 0.0, L=L), O.rmsnorm(x * np.float32(16), g, 0.0, L=L))
    #  x = (3, 4), eps = 0: mean(x^2) = 12.5, so out^2 sums to K = 2 (both components squared)
    out = O.rmsnorm(np.array([3, 4], np.float32), np.ones(2, np.float32), 0.0, L=L)
    assert abs(out[0] ** 2 + out[1] ** 2 - 2.0) < 1e-15 and abs(out[1] / out[0] - 4.0 / 3.0) < 1e-15
    # the product: with +-1 activations, eps = 0 and fp32 gamma the normalised vector
    # is exactly +-gamma, so W rmsnorm(x) equals the plain product on that vector, bit for bit
    for kind in ("q8_0", "q4_0", "f16"):
        N, K = 9, 128
        w = W.f16_matrix(N, K, rng) if kind == "f16" else W.matrix(kind, N, K, rng)
        sign = np.where(rng.random(K) < 0.5, 1.0, -1.0).astype(np.float32)
        gam = rng.standard_normal(K).astype(np.float32)
        y, a = O.gemv_rmsnorm(kind, w, sign, gam, 0.0, N, K, L=L)
        y0, a0 = _gemv(L, kind, w, sign * gam, N, K)
        assert np.array_equal(y, y0) and np.array_equal(a, a0), kind
    # gate|up on the normalised activation: silu(g) * u of the two products
    kind, N, K = "q8_0", 5, 64
    gate, up = W.matrix(kind, N, K, rng), W.matrix(kind, N, K, rng)
    x = rng.standard_normal(K).astype(np.float32)
    gam = rng.standard_normal(K).astype(np.float32)
    out, gg, uu, ag, au = O.gateup_silu_rmsnorm(kind, gate, up, x, gam, 1e-6, N, K, L=L)
    g1, a1 = O.gemv_rmsnorm(kind, gate, x, gam, 1e-6, N, K, L=L)
    u1, b1 = O.gemv_rmsnorm(kind, up, x, gam, 1e-6, N, K, L=L)
    assert np.array_equal(gg, g1) and np.array_equal(uu, u1) and np.array_equal(ag, a1) and np.array_equal(au, b1)
    assert np.array_equal(out, np.array([O.silu(v, L=L) for v in g1]) * u1)
    # the worked single block E1 (y = -8 for x = 1) with x = 1, eps = 3, gamma = 2:
    # the normalised activation is 1 everywhere, so the product is still -8
    e1 = _u8(q8_block(0x3800, [i - 16 for i in range(32)]))
    y, _ = O.gemv_rmsnorm("q8_0", e1, np.ones(32, np.float32), np.full(32, 2.0, np.float32), 3.0, 1, 32, L=L)
    assert y[0] == -8.0, y


def _q4_k_case(case) -> tuple[np.ndarray, np.ndarray]:
    """Build one golden Q4_K super-block and its activation from a case record."""
    blk = bytearray(144)
    blk[0:2] = int(case["d_bits"]).to_bytes(2, "little")
    blk[2:4] = int(case["dmin_bits"]).to_bytes(2, "little")
    blk[4:16] = bytes(case["scales"])
    if case["quant_byte"] in ("group0_low", "group0_high"):
        for l in range(32):
            blk[16 + l] = (l % 16) << (0 if case["quant_byte"] == "group0_low" else 4)
    else:
        blk[16:] = bytes([case["quant_byte"]] * 128)
    x = {"ones": np.ones(256), "index": np.arange(256.0),
         "subblock5": (np.arange(256) // 32 == 5) * 1.0, "subblock6": (np.arange(256) // 32 == 6) * 1.0}[case["x"]]
    return np.frombuffer(bytes(blk), np.uint8).copy(), x.astype(np.float32)


def pin_q4_k(L):
    # hand-worked single super-blocks (tests/golden/q4_k_blocks.json): the 6-bit
    # scale/min packing of the lower and upper sub-blocks, the min's sign, the
    # nibble order inside a 64-weight group, a subnormal d
    for case in _golden("q4_k_blocks.json")["cases"]:
        blk, x = _q4_k_case(case)
        y, a = _gemv(L, "q4_k", blk, x, 1, 256)
        assert y[0] == case["expect"], (case["name"], y[0], case["expect"])
    # closed form: every sub-block with scale s and min m, all quants c, two
    # super-blocks with different d / dmin: y = sum_b (d_b s c - dmin_b m) * sum x
    rng = np.random.default_rng(17)
    for s_, m_, c in ((5, 3, 9), (63, 63, 15), (0, 17, 4)):
        u = [(s_ & 63) | ((s_ >> 4) << 6) for _ in range(4)] + [(m_ & 63) | ((m_ >> 4) << 6) for _ in range(4)] + \
            [(s_ & 15) | ((m_ & 15) << 4) for _ in range(4)]
        blocks = []
        expect = 0.0
        x = rng.integers(-4, 5, size=512).astype(np.float32)
        for b, (db, mb) in enumerate(((0x3800, 0x3400), (0x2C00, 0x3C00))):   # (0.5, 0.25), (1/16, 1.0)
            blk = bytes([db & 255, db >> 8, mb & 255, mb >> 8]) + bytes(u) + bytes([c | (c << 4)] * 128)
            blocks.append(blk)
            dv, mv = float(np.array([db], np.uint16).view(np.float16)[0]), float(np.array([mb], np.uint16).view(np.float16)[0])
            expect += (dv * s_ * c - mv * m_) * float(x[256 * b:256 * (b + 1)].astype(np.float64).sum())
        w = np.frombuffer(b"".join(blocks), np.uint8).copy()
        y, _ = _gemv(L, "q4_k", w, x, 1, 512)
        assert y[0] == expect, (s_, m_, c, y[0], expect)
    # invariants on random matrices: exact power-of-two scaling of x, row permutation
    N, K = 5, 512
    w = W.matrix("q4_k", N, K, rng)
    x = rng.standard_normal(K).astype(np.float32)
    y, a = _gemv(L, "q4_k", w, x, N, K)
    y2, _ = _gemv(L, "q4_k", w, x * np.float32(4), N, K)
    assert np.array_equal(y2, 4 * y)
    perm = np.array([3, 0, 4, 1, 2])
    wp = w.reshape(N, -1)[perm].reshape(-1).copy()
    yp, _ = _gemv(L, "q4_k", wp, x, N, K)
    assert np.array_equal(yp, y[perm])
    # Q4_K rows must be whole super-blocks
    p = lambda arr: arr.ctypes.data_as(__import__("ctypes").c_void_p)  # noqa: E731
    ww, xx, yy, aa = np.zeros(144, np.uint8), np.zeros(288, np.float32), np.zeros(1), np.zeros(1)
    assert L.oracle_gemv(O.Q4_K, p(ww), p(xx), p(yy), p(aa), 1, 288, 1) != 0


def _q6_k_case(case) -> tuple[np.ndarray, np.ndarray]:
    """Build one golden Q6_K super-block and its activation from a case record."""
    blk = bytearray(210)
    for off, n, field in ((0, 128, case["ql"]), (128, 64, case["qh"])):
        blk[off:off + n] = bytes([field["fill"]] * n)
        for i, v in field["set"].items():
            blk[off + int(i)] = v
    blk[192:208] = np.array(case["scales"], np.int8).tobytes()
    blk[208:210] = int(case["d_bits"]).to_bytes(2, "little")
    x = {"ones": np.ones(256), "index": np.arange(256.0)}[case["x"]]
    return np.frombuffer(bytes(blk), np.uint8).copy(), x.astype(np.float32)


def q6_k_block_from_values(d_bits: int, scales, v) -> bytes:
    """Encode 256 values v in [-32, 31] as one Q6_K super-block (the inverse of
    the decode: q = v + 32 split into a low nibble and a high 2-bit part)."""
    ql, qh = bytearray(128), bytearray(64)
    for i in range(256):
        q = int(v[i]) + 32
        h, r = divmod(i, 128)
        g, l = divmod(r, 32)
        ql[64 * h + 32 * (g % 2) + l] |= (q & 15) << (4 * (g // 2))
        qh[32 * h + l] |= (q >> 4) << (2 * g)
    return bytes(ql) + bytes(qh) + np.array(scales, np.int8).tobytes() + int(d_bits).to_bytes(2, "little")


def pin_q6_k(L):
    # hand-worked single super-blocks (tests/golden/q6_k_blocks.json): the -32
    # offset, the nibble and 2-bit fields of each 32-weight group in both halves,
    # signed per-16 scales, scale -128 and a subnormal d stored last
    for case in _golden("q6_k_blocks.json")["cases"]:
        blk, x = _q6_k_case(case)
        y, _ = _gemv(L, "q6_k", blk, x, 1, 256)
        assert y[0] == case["expect"], (case["name"], y[0], case["expect"])
    # closed form: every quant c, random scales, two super-blocks with different
    # d: y = sum_b d_b (c - 32) sum_j sc_bj sum_{k in sub-block j} x_k
    rng = np.random.default_rng(23)
    for c in (0, 17, 32, 63):
        x = rng.integers(-4, 5, size=512).astype(np.float32)
        blocks, expect = [], 0.0
        for b, db in enumerate((0x3800, 0x2C00)):    # 0.5, 1/16
            sc = rng.integers(-128, 128, size=16)
            blocks.append(q6_k_block_from_values(db, sc, [c - 32] * 256))
            dv = float(np.array([db], np.uint16).view(np.float16)[0])
            xs = x[256 * b:256 * (b + 1)].astype(np.float64).reshape(16, 16).sum(axis=1)
            expect += dv * (c - 32) * float(np.dot(sc.astype(np.float64), xs))
        y, _ = _gemv(L, "q6_k", np.frombuffer(b"".join(blocks), np.uint8).copy(), x, 1, 512)
        assert y[0] == expect, (c, y[0], expect)
    # textbook case: d = 1 and every scale 1 make W the integer matrix v in [-32, 31]
    N, K = 8, 512
    v = rng.integers(-32, 32, size=(N * K // 256, 256))
    w = np.frombuffer(b"".join(q6_k_block_from_values(0x3C00, [1] * 16, row) for row in v), np.uint8).copy()
    x = rng.standard_normal(K).astype(np.float32)
    y, _ = _gemv(L, "q6_k", w, x, N, K)
    Wm = v.astype(np.float64).reshape(N, K)
    x64 = x.astype(np.float64)
    assert np.all(np.abs(y - Wm @ x64) <= 1e-12 * (np.abs(Wm) @ np.abs(x64)))
    # invariants on random matrices: exact power-of-two scaling of x, row permutation
    N, K = 5, 512
    w = W.matrix("q6_k", N, K, rng)
    x = rng.standard_normal(K).astype(np.float32)
    y, _ = _gemv(L, "q6_k", w, x, N, K)
    y2, _ = _gemv(L, "q6_k", w, x * np.float32(4), N, K)
    assert np.array_equal(y2, 4 * y)
    perm = np.array([3, 0, 4, 1, 2])
    wp = w.reshape(N, -1)[perm].reshape(-1).copy()
    yp, _ = _gemv(L, "q6_k", wp, x, N, K)
    assert np.array_equal(yp, y[perm])
    # Q6_K rows must be whole super-blocks
    p = lambda arr: arr.ctypes.data_as(__import__("ctypes").c_void_p)  # noqa: E731
    ww, xx, yy, aa = np.zeros(210, np.uint8), np.zeros(288, np.float32), np.zeros(1), np.zeros(1)
    assert L.oracle_gemv(O.Q6_K, p(ww), p(xx), p(yy), p(aa), 1, 288, 1) != 0


def pin_rejects_bad_shapes(L):
    w = np.zeros(34, np.uint8)
    x = np.zeros(33, np.float32)
    y = np.zeros(1)
    a = np.zeros(1)
    p = lambda arr: arr.ctypes.data_as(__import__("ctypes").c_void_p)  # noqa: E731
    assert L.oracle_gemv(O.Q8_0, p(w), p(x), p(y), p(a), 1, 33, 1) != 0
    assert L.oracle_gemv(O.Q4_0, p(w), p(x), p(y), p(a), 1, 48, 1) != 0
    assert L.oracle_gemv(7, p(w), p(x), p(y), p(a), 1, 32, 1) != 0


PINS = [
    pin_half_decode_all_patterns,
    pin_format_sizes,
    pin_single_blocks,
    pin_silu,
    pin_bruteforce_exact,
    pin_textbook,
    pin_invariants,
    pin_composites,
    pin_epilogue,
    pin_rmsnorm,
    pin_q4_k,
    pin_q6_k,
    pin_rejects_bad_shapes,
]


def failing_pins(lib_path: str) -> list[str]:
    """Names of the pins that fail against the oracle library at lib_path."""
    L = O.lib(lib_path)
    failed = []
    for pin in PINS:
        try:
            pin(L)
        except (AssertionError, ValueError, OverflowError, ZeroDivisionError):
            failed.append(pin.__name__)
    return failed


if __name__ == "__main__":
    # python tests/oracle_pins.py <liboracle variant.so>: print the failing pins as JSON
    import sys as _sys
    print(json.dumps(failing_pins(_sys.argv[1])))
