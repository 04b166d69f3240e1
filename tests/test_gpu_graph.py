"""The GEMV calls recorded into a HIP graph (through torch.cuda.CUDAGraph on a
capture stream) replay to the same bits as the eager calls. Each replay is
checked, with eager work and a synchronisation between replays."""
import numpy as np
import pytest

import block_dequant_gemv_amd as qg
from block_dequant_gemv_amd import workloads as W
from gpu_helpers import announce, empty_f32, to_dev, torch_dev

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    torch = torch_dev()
    rng = np.random.default_rng(2024)
    side = torch.cuda.Stream()
    calls = []   # (name, fn(stream), output tensor)

    def add(name, fn, out):
        calls.append((name, fn, out))

    # one call of every entry point, both forms of the quantised GEMV
    for kind, N, K in (("q8_0", 4096, 1024), ("q4_0", 3300, 5120), ("q4_0", 1000, 2048)):
        w = qg.pack_weights(kind, W.matrix(kind, N, K, rng), N, K)
        x = to_dev(W.activation(K, rng))
        y = empty_f32(N)
        add(f"qgemv {kind} {N}x{K}", lambda s, w=w, x=x, y=y, kind=kind, N=N, K=K: qg.qgemv(kind, w, x, y, N, K, s), y)
        X = to_dev(W.activation(K, rng, M=3))
        Y = empty_f32(3 * N)
        add(f"verify {kind} {N}x{K}",
            lambda s, w=w, X=X, Y=Y, kind=kind, N=N, K=K: qg.qgemv_verify(kind, w, X, Y, N, K, 3, s), Y)
    N_ff, K = 1536, 1024
    wgu = qg.pack_gateup("q8_0", W.matrix("q8_0", N_ff, K, rng), W.matrix("q8_0", N_ff, K, rng), N_ff, K)
    xg = to_dev(W.activation(K, rng))
    yg = empty_f32(N_ff)
    add("gate|up", lambda s: qg.qgemv_fused_gateup_silu("q8_0", wgu, xg, yg, N_ff, K, s), yg)
    wf = to_dev(W.f16_matrix(256, 5120, rng))
    xf = to_dev(W.activation(5120, rng))
    yf = empty_f32(256)
    add("f16", lambda s: qg.gemv_f16_splitk(wf, xf, yf, 256, 5120, s), yf)

    # eager reference on the side stream
    with torch.cuda.stream(side):
        for name, fn, out in calls:
            announce(f"graph test eager {name}")
            fn(side)
    torch.cuda.synchronize()
    ref = [out.clone() for _, _, out in calls]

    g = torch.cuda.CUDAGraph()
    for _, _, out in calls:
        out.fill_(-1.0)
    torch.cuda.synchronize()
    announce("graph test capture")
    with torch.cuda.graph(g, stream=side, capture_error_mode="thread_local"):
        for name, fn, out in calls:
            fn(side)
    scratch = torch.ones(1 << 20, device="cuda")
    for rep in range(4):
        for _, _, out in calls:
            out.fill_(float("nan"))
        scratch.mul_(1.5)                    # eager work between replays
        torch.cuda.synchronize()
        announce(f"graph test replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for (name, _, out), r in zip(calls, ref):
            assert out.cpu().numpy().tobytes() == r.cpu().numpy().tobytes(), f"replay {rep}: {name} differs from eager"


def test_graph_capture_of_a_kernel_not_yet_launched():
    # A verify call whose activations exceed LDS at once (Q4_0 5120x17408, M = 5:
    # staged in phases, about 130 KiB of LDS) captured before the process has ever
    # launched that kernel: its first launch, with the dynamic-LDS limit it needs,
    # happens inside the capture. Every replay must equal an eager call made after.
    torch = torch_dev()
    rng = np.random.default_rng(2025)
    kind, N, K, M = "q4_0", 5120, 17408, 5
    w = qg.pack_weights(kind, W.matrix(kind, N, K, rng), N, K)
    X = to_dev(W.activation(K, rng, M=M))
    Y = empty_f32(M * N)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    announce("graph capture of a first launch (phased verify)")
    with torch.cuda.graph(g, stream=side, capture_error_mode="thread_local"):
        qg.qgemv_verify(kind, w, X, Y, N, K, M, side.cuda_stream)
    ref = empty_f32(M * N)
    qg.qgemv_verify(kind, w, X, ref, N, K, M)
    torch.cuda.synchronize()
    want = ref.cpu().numpy().tobytes()
    for rep in range(3):
        Y.fill_(float("nan"))
        torch.cuda.synchronize()
        announce(f"graph replay {rep} (phased verify)")
        g.replay()
        torch.cuda.synchronize()
        assert Y.cpu().numpy().tobytes() == want, f"replay {rep} differs from the eager call"
