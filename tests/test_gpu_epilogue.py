"""GPU parity of qgemv_epilogue (bias / residual addends, fp16 output) against the
fp64 oracle, plus what its contract fixes exactly: with no addends it returns the
plain GEMV's bits, each addend is one fp32 addition on those bits (bias first),
and the fp16 output is the fp32 result rounded to nearest even.

Shapes cover both launch forms of the quantised GEMV: one wavefront group per
row tile (fused QKV 4096x1024 with its bias; the 1024x2048 O projection split
two ways along K, with the residual added in place; the 1024x3072 down projection
split three ways; a ragged 9x1056) and the
persistent form with K ranges combined in LDS (3300x5120, 640x17408) and with
one K range, whose half-tiles store their sums directly (20000x1024); the Q4_K
and Q6_K weights on two shapes each."""
import numpy as np
import pytest

import block_dequant_gemv_amd as qg
import oracle as O
from block_dequant_gemv_amd import workloads as W
from gpu_helpers import THREADS, announce, empty_f32, sync, to_dev, torch_dev

pytestmark = pytest.mark.gpu

SHAPES = [(4096, 1024), (1024, 2048), (1024, 3072), (9, 1056), (3300, 5120), (640, 17408), (20000, 1024)]
TAIL = 5


def _assert_epilogue(y, out, a, ctx, bias=None, residual=None, f16=False):
    y = np.asarray(y, np.float64)
    assert np.all(np.isfinite(y)), f"{ctx}: non-finite outputs"
    tol = O.epilogue_tol(a, bias=bias, residual=residual, out=out, f16=f16)
    err = np.abs(y - out)
    bad = np.flatnonzero(err > tol)
    if bad.size:
        i = bad[np.argmax(err[bad] / tol[bad])]
        raise AssertionError(f"{ctx}: {bad.size}/{out.size} outputs out of tolerance; worst {i}: "
                             f"gpu {y[i]!r} ref {out[i]!r} err {err[i]:.3e} tol {tol[i]:.3e}")


def _out(torch, n, f16, fill):
    t = torch.empty(n + TAIL, dtype=torch.float16 if f16 else torch.float32, device="cuda")
    t.fill_(fill)
    return t


@pytest.mark.parametrize("kind,N,K", [(k, n, kk) for k in ("q8_0", "q4_0") for n, kk in SHAPES] +
                         [("q4_k", 4096, 1024), ("q4_k", 1024, 2048), ("q6_k", 3300, 5120), ("q6_k", 640, 17408)])
def test_epilogue_matches_oracle_and_plain_bits(kind, N, K):
    torch = torch_dev()
    rng = np.random.default_rng(4242 + N + K)
    canon = W.matrix(kind, N, K, rng)
    x = W.activation(K, rng)
    bias = (0.5 * rng.standard_normal(N)).astype(np.float32)
    res = rng.standard_normal(N).astype(np.float32)
    packed = qg.pack_weights(kind, canon, N, K)
    xd, bd, rd = to_dev(x), to_dev(bias), to_dev(res)
    ctx = f"epilogue {kind} {N}x{K} plan={qg.qg_plan_info(kind, N, K)}"
    announce(ctx)

    y_plain = empty_f32(N)
    qg.qgemv(kind, packed, xd, y_plain, N, K)
    outs = {}
    for name, b, r, f16 in (("none", None, None, False), ("bias", bd, None, False), ("res", None, rd, False),
                            ("both", bd, rd, False), ("both16", bd, rd, True), ("bias16", bd, None, True)):
        y = _out(torch, N, f16, -3.0)
        qg.qgemv_epilogue(kind, packed, xd, y[:N], N, K, bias=b, residual=r)
        outs[name] = y
    # residual updated in place: y holds the residual on entry
    y_inp = torch.empty(N + TAIL, dtype=torch.float32, device="cuda")
    y_inp.fill_(-3.0)
    y_inp[:N].copy_(rd)
    qg.qgemv_epilogue(kind, packed, xd, y_inp[:N], N, K, bias=bd, residual=y_inp[:N])
    sync()

    p = y_plain.cpu().numpy()
    got = {k: v.cpu().numpy() for k, v in outs.items()}
    got["inplace"] = y_inp.cpu().numpy()
    for k, v in got.items():
        assert np.all(v[N:] == -3.0), f"{ctx} {k}: wrote past y[N-1]"
    got = {k: v[:N] for k, v in got.items()}

    # exact consequences of the contract, on the plain call's bits
    assert got["none"].tobytes() == p.tobytes(), f"{ctx}: no-addend epilogue != plain GEMV"
    pb = (p + bias).astype(np.float32)
    pbr = (pb + res).astype(np.float32)
    assert got["bias"].tobytes() == pb.tobytes(), f"{ctx}: bias is not one fp32 add"
    assert got["res"].tobytes() == (p + res).astype(np.float32).tobytes(), f"{ctx}: residual add"
    assert got["both"].tobytes() == pbr.tobytes(), f"{ctx}: (y + bias) + residual"
    assert got["inplace"].tobytes() == pbr.tobytes(), f"{ctx}: in-place residual"
    assert got["both16"].tobytes() == pbr.astype(np.float16).tobytes(), f"{ctx}: fp16 rounding"
    assert got["bias16"].tobytes() == pb.astype(np.float16).tobytes(), f"{ctx}: fp16 rounding (bias)"

    # the oracle, with the tolerance widened only by the addends and the fp16 rounding
    out_b, _ = O.gemv_epilogue(kind, canon, x, N, K, bias=bias, threads=THREADS)
    a = O.gemv_epilogue(kind, canon, x, N, K, threads=THREADS)[1]
    _assert_epilogue(got["bias"], out_b, a, ctx + " bias", bias=bias)
    out_r, _ = O.gemv_epilogue(kind, canon, x, N, K, residual=res, threads=THREADS)
    _assert_epilogue(got["res"], out_r, a, ctx + " residual", residual=res)
    out_br, _ = O.gemv_epilogue(kind, canon, x, N, K, bias=bias, residual=res, threads=THREADS)
    _assert_epilogue(got["both"], out_br, a, ctx + " both", bias=bias, residual=res)
    _assert_epilogue(got["inplace"], out_br, a, ctx + " in place", bias=bias, residual=res)
    _assert_epilogue(got["both16"].astype(np.float64), out_br, a, ctx + " fp16", bias=bias, residual=res, f16=True)
    out_n, _ = O.gemv_epilogue(kind, canon, x, N, K, threads=THREADS)
    _assert_epilogue(got["none"], out_n, a, ctx + " none")


@pytest.mark.parametrize("kind", ["q8_0", "q4_0"])
def test_epilogue_fp16_range_edges(kind):
    # zero scales make the product exactly 0, so the output is the fp16 rounding of
    # bias + residual: values past the fp16 range go to infinity, tiny ones land
    # in the fp16 subnormal range (not flushed), ties round to even
    torch = torch_dev()
    N, K = 64, 1024
    canon = W.matrix(kind, N, K, np.random.default_rng(3)).reshape(N * K // 32, -1)
    canon[:, 0:2] = 0
    canon = canon.reshape(-1)
    x = W.activation(K, np.random.default_rng(4))
    edge = [7e4, -7e4, 65504.0, 65519.0, 65520.0, 1e-6, -3e-7, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25,
            1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 0.0, -0.0, 6.1e-5, 5.9e-5]
    bias = np.zeros(N, np.float32)
    bias[:len(edge)] = np.array(edge, np.float32)
    bias[len(edge):] = np.random.default_rng(5).standard_normal(N - len(edge)).astype(np.float32) * 1e-4
    res = np.zeros(N, np.float32)
    packed = qg.pack_weights(kind, canon, N, K)
    y = _out(torch, N, True, 0.0)
    announce(f"epilogue fp16 edges {kind}")
    qg.qgemv_epilogue(kind, packed, to_dev(x), y[:N], N, K, bias=to_dev(bias), residual=to_dev(res))
    sync()
    got = y.cpu().numpy()[:N]
    expect = (bias + res).astype(np.float16)
    assert got.tobytes() == expect.tobytes()
    assert np.isinf(got[0]) and np.isinf(got[1]) and got[5] != 0
