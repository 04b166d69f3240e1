"""Every kernel variant, forced through the launch-shape overrides, against the
oracle; verify rows stay memcmp-equal to M=1 under the same split.

The planner picks one shape per (type, rows, K); the overrides
QG_PERSIST / QG_SPLIT_K / QG_X_GLOBAL / QG_WAVES_PER_WG / QG_TILES_PER_GROUP /
QG_PREFETCH / QG_STRIDE_GROUPS reach the others: the one-wavefront-per-tile form
with every split, activation source, workgroup size, tiles per group, grid-stride
tile order and prefetch depth (depth 2
exists for the single-row kernels; the verify kernels keep depth 1, and their
rows must still match), and the persistent form with activations in LDS or L2.
"""
import itertools
import os

import numpy as np
import pytest

import block_dequant_gemv_amd as qg
import oracle as O
from block_dequant_gemv_amd import workloads as W
from gpu_helpers import THREADS, announce, assert_linear, empty_f32, sync, to_dev

pytestmark = pytest.mark.gpu

KNOBS = ("QG_PERSIST", "QG_SPLIT_K", "QG_X_GLOBAL", "QG_WAVES_PER_WG", "QG_TILES_PER_GROUP", "QG_PREFETCH",
         "QG_STRIDE_GROUPS")


def _set(**kw):
    for k in KNOBS:
        os.environ.pop(k, None)
    for k, v in kw.items():
        os.environ[k] = str(v)
    qg.qg_reload_tuning()   # the library reads the overrides once, and on request


@pytest.mark.parametrize("kind,N,K", [("q4_0", 203, 8192 + 96), ("q8_0", 77, 3072), ("q4_0", 1000, 1024)])
def test_forced_launch_shapes(kind, N, K):
    rng = np.random.default_rng(N * K)
    canon = W.matrix(kind, N, K, rng)
    packed = qg.pack_weights(kind, canon, N, K)
    X = W.activation(K, rng, M=3)
    Xd = to_dev(X)
    Y_ref, A_ref = O.verify(kind, canon, X, N, K, threads=THREADS)
    nseg = -(-K // 1024)
    combos = [dict(QG_PERSIST=1, QG_X_GLOBAL=xg) for xg in (0, 1)]
    # grid-stride tile order: groups walk tiles g, g + groups, ... (3 groups leave a ragged last round)
    combos += [dict(QG_PERSIST=0, QG_STRIDE_GROUPS=sg, QG_WAVES_PER_WG=1, QG_SPLIT_K=split)
               for sg in (3, 8) for split in (1, 2) if split <= nseg]
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
            ys = []
            for m in range(3):
                y = empty_f32(N)
                qg.qgemv(kind, packed, Xd[m].contiguous(), y, N, K)
                ys.append(y)
            Y = empty_f32(3 * N)
            qg.qgemv_verify(kind, packed, Xd, Y, N, K, 3)
            sync()
            Yh = Y.cpu().numpy().reshape(3, N)
            for m in range(3):
                ym = ys[m].cpu().numpy()
                assert_linear(ym, Y_ref[m], A_ref[m], ctx + f" row {m}")
                assert Yh[m].tobytes() == ym.tobytes(), ctx + f" verify row {m} != M=1"
    finally:
        _set()


@pytest.mark.parametrize("N,K", [(300, 5120), (37, 1000), (2049, 64)])
def test_f16_forced_launch_shapes(N, K):
    # every rows-per-workgroup / wavefronts-per-workgroup shape of the fp16 split-K
    # form against the oracle, and the same bits run to run at a fixed shape
    rng = np.random.default_rng(N + K)
    w = W.f16_matrix(N, K, rng)
    x = W.activation(K, rng)
    wd, xd = to_dev(w), to_dev(x)
    y_ref, a_ref = O.gemv("f16", w, x, N, K, threads=THREADS)
    try:
        os.environ["QG_F16_FORM"] = "0"
        for r in (1, 2, 4):
            for wv in (1, 3, 8, 16):
                os.environ["QG_F16_ROWS"], os.environ["QG_F16_WAVES"] = str(r), str(wv)
                qg.qg_reload_tuning()
                ctx = f"f16 {N}x{K} rows={r} waves={wv}"
                announce(ctx)
                y0, y1 = empty_f32(N), empty_f32(N)
                qg.gemv_f16_splitk(wd, xd, y0, N, K)
                qg.gemv_f16_splitk(wd, xd, y1, N, K)
                sync()
                a0 = y0.cpu().numpy()
                assert_linear(a0, y_ref, a_ref, ctx)
                assert a0.tobytes() == y1.cpu().numpy().tobytes(), ctx + ": run-to-run bits differ"
    finally:
        for k in ("QG_F16_ROWS", "QG_F16_WAVES", "QG_F16_FORM"):
            os.environ.pop(k, None)
        qg.qg_reload_tuning()


# The row form (one wavefront per row, K = 512 L): L = 1 and L = 16, fewer rows
# than one workgroup holds, ragged last workgroups, every rows-per-workgroup
# choice, against the oracle; the same bits run to run; and the forced form on
# a K the row form cannot take falls back to the split-K form.
@pytest.mark.parametrize("N,K", [(1, 512), (3, 8192), (37, 1024), (1001, 5120), (2049, 512), (130, 8192)])
def test_f16_row_form(N, K):
    rng = np.random.default_rng(7 * N + K)
    w = W.f16_matrix(N, K, rng)
    x = W.activation(K, rng)
    wd, xd = to_dev(w), to_dev(x)
    y_ref, a_ref = O.gemv("f16", w, x, N, K, threads=THREADS)
    try:
        os.environ["QG_F16_FORM"] = "1"
        for wv in (2, 4, 8, 0):
            if wv:
                os.environ["QG_F16_WAVES"] = str(wv)
            else:
                os.environ.pop("QG_F16_WAVES", None)
            qg.qg_reload_tuning()
            ctx = f"f16 row form {N}x{K} rows/wg={wv or 'default'}"
            announce(ctx)
            y0, y1 = empty_f32(N + 1), empty_f32(N)
            y0[N:] = -7.0
            qg.gemv_f16_splitk(wd, xd, y0, N, K)
            qg.gemv_f16_splitk(wd, xd, y1, N, K)
            sync()
            a0 = y0.cpu().numpy()
            assert a0[N] == -7.0, ctx + ": wrote past y"
            assert_linear(a0[:N], y_ref, a_ref, ctx)
            assert a0[:N].tobytes() == y1.cpu().numpy().tobytes(), ctx + ": run-to-run bits differ"
    finally:
        for k in ("QG_F16_WAVES", "QG_F16_FORM"):
            os.environ.pop(k, None)
        qg.qg_reload_tuning()


# The split-K row form (one workgroup per row, K split into consecutive ranges
# over up to 16 wavefronts, 1, 2 or 4 16-byte chunks per lane, partials added
# in wavefront order): the configuration's short matrices, one chunk in all,
# ragged K (K / 8 not a multiple of 64), exactly 16 wavefronts (K = 16384 at 2
# chunks per lane, 32768 at 4) and a K that 2 chunks per lane cannot cover in
# 16 wavefronts (16392: that forced shape takes the lane-split form), against the oracle;
# the same bits run to run; and the default plan of a short matrix is this form.
@pytest.mark.parametrize("N,K", [(48, 5120), (256, 5120), (1, 8), (3, 1000), (37, 24), (5, 16384), (2, 16392),
                                 (7, 32768), (1023, 512)])
def test_f16_split_k_row_form(N, K):
    rng = np.random.default_rng(11 * N + K)
    w = W.f16_matrix(N, K, rng)
    x = W.activation(K, rng)
    wd, xd = to_dev(w), to_dev(x)
    y_ref, a_ref = O.gemv("f16", w, x, N, K, threads=THREADS)
    outs = {}
    try:
        for cpl in (0, 1, 2, 4):
            os.environ["QG_F16_FORM"] = "2"
            if cpl:
                os.environ["QG_F16_CPL"] = str(cpl)
            else:
                os.environ.pop("QG_F16_CPL", None)
            qg.qg_reload_tuning()
            ctx = f"f16 split-K row form {N}x{K} chunks/lane={cpl or 'default'}"
            announce(ctx)
            y0, y1 = empty_f32(N + 1), empty_f32(N)
            y0[N:] = -7.0
            qg.gemv_f16_splitk(wd, xd, y0, N, K)
            qg.gemv_f16_splitk(wd, xd, y1, N, K)
            sync()
            a0 = y0.cpu().numpy()
            assert a0[N] == -7.0, ctx + ": wrote past y"
            assert_linear(a0[:N], y_ref, a_ref, ctx)
            assert a0[:N].tobytes() == y1.cpu().numpy().tobytes(), ctx + ": run-to-run bits differ"
            outs[cpl] = a0[:N].tobytes()
    finally:
        for k in ("QG_F16_FORM", "QG_F16_CPL"):
            os.environ.pop(k, None)
        qg.qg_reload_tuning()
    announce(f"f16 default plan {N}x{K}")
    y = empty_f32(N)
    qg.gemv_f16_splitk(wd, xd, y, N, K)
    sync()
    assert y.cpu().numpy().tobytes() == outs[0], "the default plan of a short matrix is the split-K row form"
