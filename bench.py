"""Benchmark of the block-dequant GEMV path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline step (the decode weight set of a Qwen3-0.6B-shaped Q8_0 model, M=1):
  fused QKV 4096x1024 -> O 1024x2048 -> fused gate|up 2x3072x1024 + SiLU ->
  down 1024x3072 -> LM head 151936x1024.
Each step reads the next of several device copies of the whole weight set
(>= 1 GiB in total), so the weights are cold in the 256 MB Infinity Cache and
the 4 MB L2s when a step reads them. `value` is algorithmic bytes moved per
second over K timed steps (weights + scales + x + y, each read/written once).

Also measured in the same run:
  * every matrix of the five workload configurations, one call at a time, cold
    (each call's weight rotating through >= 1.2 GiB of device copies) and warm,
    as median us per call, GB/s and fraction of the 8 TB/s HBM3E peak;
  * the roofline entry of the step's dominant kernel: a second pass over the same
    steps binds HIP events to every launch, which receive each kernel's own start
    and end times;
  * the fp64 CPU oracle on the host cores (one thread and all threads) over one
    step of the same workload (the cpu_baseline leg; the only use of oracle/).
Prints one JSON line on stdout; a readable table goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0
METRIC = "Q8_0/Q4_0 GEMV achieved HBM GB/s (% of 8 TB/s, cold); µs per call"
COLD_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------

class Call:
    """One C-ABI call with its buffers and byte accounting. `weight` is its weight
    tensor and `make(ptr)` builds the same call on another copy of that weight."""

    def __init__(self, label, fn, nbytes, kernel, weight=None, make=None):
        self.label, self.fn, self.nbytes, self.kernel = label, fn, nbytes, kernel
        self.weight, self.make = weight, make


def qkernel_name(qg, kind, N, K, M=1, epi="plain"):
    p = qg.qg_plan_info(kind, N, K, M)
    form = "persist" if p["persistent"] else "tile"
    return f"qgemv<{kind},M{M},{epi},{form},R{p['split_k_ways']},{'lds' if p['x_in_lds'] else 'gx'}>"


def wbytes(kind, N, K):
    from block_dequant_gemv_amd.workloads import matrix_bytes
    return matrix_bytes(kind, N, K)


def make_qgemv(qg, kind, packed, x, y, N, K, stream, label):
    name = "qgemv_" + kind
    make = lambda wp: qg.bound_call(name, wp, x.data_ptr(), y.data_ptr(), N, K, stream)  # noqa: E731
    return Call(label, make(packed.data_ptr()), wbytes(kind, N, K) + 4 * K + 4 * N, qkernel_name(qg, kind, N, K),
                packed, make)


def make_gateup(qg, kind, packed, x, y, N_ff, K, stream, label):
    make = lambda wp: qg.bound_call("qgemv_fused_gateup_silu", qg.QTYPES[kind], wp, x.data_ptr(),  # noqa: E731
                                    y.data_ptr(), N_ff, K, stream)
    return Call(label, make(packed.data_ptr()), 2 * wbytes(kind, N_ff, K) + 4 * K + 4 * N_ff,
                qkernel_name(qg, kind, 2 * N_ff, K, epi="gateup"), packed, make)


def make_verify(qg, kind, packed, X, Y, N, K, M, stream, label):
    make = lambda wp: qg.bound_call("qgemv_verify", qg.QTYPES[kind], wp, X.data_ptr(), Y.data_ptr(),  # noqa: E731
                                    N, K, M, stream)
    return Call(label, make(packed.data_ptr()), wbytes(kind, N, K) + 4 * M * K + 4 * M * N,
                qkernel_name(qg, kind, N, K, M), packed, make)


def make_epilogue(qg, kind, packed, x, bias, res, y, N, K, stream, label):
    """qgemv_epilogue: y = ((W x) + bias) + residual, fp32 or fp16 (y's dtype)."""
    out16 = y.element_size() == 2
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    make = lambda wp: qg.bound_call("qgemv_epilogue", qg.QTYPES[kind], wp, x.data_ptr(), ptr(bias),  # noqa: E731
                                    ptr(res), y.data_ptr(), qg.QG_OUT_F16 if out16 else qg.QG_OUT_F32, N, K,
                                    stream)
    nbytes = wbytes(kind, N, K) + 4 * K + (2 if out16 else 4) * N + 4 * N * ((bias is not None) + (res is not None))
    return Call(label, make(packed.data_ptr()), nbytes, qkernel_name(qg, kind, N, K, epi="affine"), packed, make)


def make_f16(qg, w, x, y, N, K, stream, label):
    make = lambda wp: qg.bound_call("gemv_f16_splitk", wp, x.data_ptr(), y.data_ptr(), N, K, stream)  # noqa: E731
    return Call(label, make(w.data_ptr()), 2 * N * K + 4 * K + 4 * N, "gemv_f16", w, make)


# ---------------------------------------------------------------------------

def build_step(qg, torch, wl, stream, copies):
    """The headline decode set, packed once and cloned into `copies` device copies."""
    dev = "cuda"
    K = 1024
    base = {}
    base["qkv"] = qg.pack_concat("q8_0", [(wl.weight(n), wl.entry(n)[2]) for n in ("q_proj", "k_proj", "v_proj")],
                                 K)
    base["o"] = qg.pack_weights("q8_0", wl.weight("o_proj"), 1024, 2048)
    base["gateup"] = qg.pack_gateup("q8_0", wl.weight("gate"), wl.weight("up"), 3072, 1024)
    base["down"] = qg.pack_weights("q8_0", wl.weight("down"), 1024, 3072)
    base["lm_head"] = qg.pack_weights("q8_0", wl.weight("lm_head"), 151936, 1024)
    xs = {n: torch.from_numpy(wl.x(src)).to(dev) for n, src in
          (("qkv", "q_proj"), ("o", "o_proj"), ("gateup", "gate"), ("down", "down"), ("lm_head", "lm_head"))}
    ys = {"qkv": 4096, "o": 1024, "gateup": 3072, "down": 1024, "lm_head": 151936}
    ys = {n: torch.empty(v, dtype=torch.float32, device=dev) for n, v in ys.items()}
    sets = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(copies - 1)]
    torch.cuda.synchronize()
    steps = [step_calls(qg, s, xs, ys, stream) for s in sets]
    return steps, sets, xs, ys


def step_calls(qg, s, xs, ys, stream):
    """The five calls of one decode step on weight set `s`, launched on `stream`."""
    return [
        make_qgemv(qg, "q8_0", s["qkv"], xs["qkv"], ys["qkv"], 4096, 1024, stream, "qkv 4096x1024"),
        make_qgemv(qg, "q8_0", s["o"], xs["o"], ys["o"], 1024, 2048, stream, "o_proj 1024x2048"),
        make_gateup(qg, "q8_0", s["gateup"], xs["gateup"], ys["gateup"], 3072, 1024, stream,
                    "gate|up 2x3072x1024 silu"),
        make_qgemv(qg, "q8_0", s["down"], xs["down"], ys["down"], 1024, 3072, stream, "down 1024x3072"),
        make_qgemv(qg, "q8_0", s["lm_head"], xs["lm_head"], ys["lm_head"], 151936, 1024, stream,
                   "lm_head 151936x1024"),
    ]


def graph_headline(qg, torch, sets, xs, ys, K, warmup, copies, step_bytes):
    """Headline steps replayed from HIP graphs: one torch.cuda.CUDAGraph per weight
    copy capturing that step's five launches on a side stream (the GEMV calls record
    plain kernel launches and nothing else), then K replays cycling through the
    copies, between synchronisations."""
    side = torch.cuda.Stream()
    graphs = []
    for st in sets:
        calls = step_calls(qg, st, xs, ys, side.cuda_stream)
        with torch.cuda.stream(side):
            for c in calls:
                c.fn()
        side.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side, capture_error_mode="thread_local"):
            for c in calls:
                c.fn()
        graphs.append(g)
    with torch.cuda.stream(side):
        for s in range(warmup):
            graphs[s % copies].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(side)
        for s in range(K):
            graphs[s % copies].replay()
        e1.record(side)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    del graphs
    return {"ms_per_step": round(wall / K * 1e3, 5), "gpu_ms_per_step": round(e0.elapsed_time(e1) / K, 5),
            "value": round(step_bytes * K / wall / 1e9, 1)}


def timing_events(torch, n):
    """n timing events on the current stream, recorded once so that they exist
    (torch creates the underlying hipEvent_t lazily) and can be bound to launches."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()
    return evs


def time_call(qg, torch, fns, reps):
    """Kernel durations (us) of `reps` calls cycling through `fns`, each launch
    bound to an event pair that receives the kernel's start and end timestamps,
    and the mean us per call of a back-to-back batch bracketed by one event pair
    (kernel time plus the gap between dependent launches)."""
    evs = timing_events(torch, 2 * reps)
    torch.cuda.synchronize()
    for i in range(reps):
        qg.qg_time_next_launch(evs[2 * i], evs[2 * i + 1])
        fns[i % len(fns)]()
    nb = max(reps, len(fns))
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record()
    for i in range(nb):
        fns[i % len(fns)]()
    b1.record()
    torch.cuda.synchronize()
    us = np.array([evs[2 * i].elapsed_time(evs[2 * i + 1]) * 1e3 for i in range(reps)])
    return us, b0.elapsed_time(b1) * 1e3 / nb


def cold_copies(torch, weight, budget=COLD_BYTES * 6 // 5):
    """The weight plus clones totalling >= `budget` bytes (>= 3 copies), so that a
    call cycling through them finds its weight in neither the L2s nor the Infinity
    Cache -- the way other layers' weights evict it in a real decode step."""
    nbytes = weight.numel() * weight.element_size()
    n = max(3, min(8192, -(-budget // nbytes)))
    return [weight] + [weight.clone() for _ in range(n - 1)]


def per_config_calls(qg, torch, stream, step_calls):
    """All five configurations as lists of calls (the headline step's calls reused for config 1)."""
    from block_dequant_gemv_amd import workloads as W
    from block_dequant_gemv_amd.workloads import Workload
    dev = "cuda"
    keep = []
    res = {}

    def t(a):
        d = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        keep.append(d)
        return d

    def yb(n):
        d = torch.empty(n, dtype=torch.float32, device=dev)
        keep.append(d)
        return d

    wl = Workload(0)
    p = qg.pack_weights("q8_0", wl.weight("w"), 1024, 1024)
    keep.append(p)
    res[0] = [make_qgemv(qg, "q8_0", p, t(wl.x("w")), yb(1024), 1024, 1024, stream, "c0 q8_0 1024x1024")]

    res[1] = [Call("c1 " + c.label, c.fn, c.nbytes, c.kernel, c.weight, c.make) for c in step_calls]

    wl1 = Workload(1)
    wl = wl2 = Workload(2)
    pg = qg.pack_gateup("q4_0", wl.weight("gate"), wl.weight("up"), 17408, 5120)
    wl.drop("gate")
    wl.drop("up")
    pd = qg.pack_weights("q4_0", wl.weight("down"), 5120, 17408)
    wl.drop("down")
    pl = qg.pack_weights("q4_0", wl.weight("lm_head"), 248320, 5120)
    wl.drop("lm_head")
    keep += [pg, pd, pl]
    res[2] = [
        make_gateup(qg, "q4_0", pg, t(wl.x("gate")), yb(17408), 17408, 5120, stream, "c2 q4_0 gate|up 2x17408x5120"),
        make_qgemv(qg, "q4_0", pd, t(wl.x("down")), yb(5120), 5120, 17408, stream, "c2 q4_0 down 5120x17408"),
        make_qgemv(qg, "q4_0", pl, t(wl.x("lm_head")), yb(248320), 248320, 5120, stream,
                   "c2 q4_0 lm_head 248320x5120"),
    ]

    wl = Workload(3)
    res[3] = []
    for name in ("square", "thin", "small"):
        _, _, N, K, _ = wl.entry(name)
        res[3].append(make_f16(qg, t(wl.weight(name)), t(wl.x(name)), yb(N), N, K, stream, f"c3 f16 {N}x{K}"))

    wl = Workload(4)
    res[4] = []
    for name in ("q4_0_w", "q8_0_w"):
        _, kind, N, K, _ = wl.entry(name)
        pw = qg.pack_weights(kind, wl.weight(name), N, K)
        keep.append(pw)
        X = t(wl.x(name, M=6))
        res[4].append(make_qgemv(qg, kind, pw, X[0:1].reshape(-1), yb(N), N, K, stream,
                                 f"c4 {kind} {N}x{K} M=1"))
        for M in range(2, 7):
            res[4].append(make_verify(qg, kind, pw, X, yb(M * N), N, K, M, stream, f"c4 {kind} {N}x{K} M={M}"))
    # epilogue variants (qgemv_epilogue) on weights of the configurations above:
    # the fused QKV with its bias, the O projection added into the residual stream
    # in place, the Q4_0 down projection with a residual, the LM head writing fp16
    erng = np.random.default_rng(5)
    by = {c.label: c for c in step_calls}
    qkv, o, lm = by["qkv 4096x1024"], by["o_proj 1024x2048"], by["lm_head 151936x1024"]
    vec = lambda n: t((0.5 * erng.standard_normal(n)).astype(np.float32))  # noqa: E731
    y_o = t(erng.standard_normal(1024).astype(np.float32))
    y16 = torch.empty(151936, dtype=torch.float16, device=dev)
    keep.append(y16)
    res[5] = [
        make_epilogue(qg, "q8_0", qkv.weight, t(wl1.x("q_proj")), vec(4096), None, yb(4096), 4096, 1024, stream,
                      "e q8_0 qkv 4096x1024 +bias"),
        make_epilogue(qg, "q8_0", o.weight, t(wl1.x("o_proj")), None, y_o, y_o, 1024, 2048, stream,
                      "e q8_0 o_proj 1024x2048 +=residual"),
        make_epilogue(qg, "q4_0", pd, t(wl2.x("down")), None, vec(5120), yb(5120), 5120, 17408, stream,
                      "e q4_0 down 5120x17408 +residual"),
        make_epilogue(qg, "q8_0", lm.weight, t(wl1.x("lm_head")), None, None, y16, 151936, 1024, stream,
                      "e q8_0 lm_head 151936x1024 fp16 out"),
    ]
    # the super-block GEMVs (qgemv_q4_k, qgemv_q6_k) on the shapes of the Q4_0
    # configuration: 144 and 210 canonical bytes per 256 weights
    krng = np.random.default_rng(6)
    res[6] = []
    for kind in ("q4_k", "q6_k"):
        for label, N, K in (("down 5120x17408", 5120, 17408), ("gate 17408x5120", 17408, 5120),
                            ("lm_head 248320x5120", 248320, 5120)):
            canon = W.matrix(kind, N, K, krng)
            pk = qg.pack_weights(kind, canon, N, K)
            del canon
            keep.append(pk)
            res[6].append(make_qgemv(qg, kind, pk, t(W.activation(K, krng)), yb(N), N, K, stream,
                                     f"k {kind} {label}"))
            if label.startswith("gate"):
                # the verify call on the same weight: M = 2..6 activation rows in one weight stream
                X = t(W.activation(K, krng, M=6))
                for M in range(2, 7):
                    res[6].append(make_verify(qg, kind, pk, X, yb(M * N), N, K, M, stream,
                                              f"k {kind} {N}x{K} M={M}"))
    # the RMSNorm-prologue experiment: each case is (label, weight, bytes, fused(wp), norm(), gemv(wp)), the
    # unfused form being qg_rmsnorm into a separate buffer followed by the plain GEMV on it
    eps = 1e-6
    norm_cases = []

    def norm_case(label, kind, packed, N, K, gateup):
        x = t(erng.standard_normal(K).astype(np.float32))
        g = t((1.0 + 0.25 * erng.standard_normal(K)).astype(np.float32))
        xn = yb(K)
        y = yb(N)
        qt = qg.QTYPES[kind]
        if gateup:
            fused = lambda wp: qg.bound_call("qgemv_rmsnorm_gateup_silu", qt, wp, x.data_ptr(), g.data_ptr(),  # noqa
                                             eps, y.data_ptr(), N, K, stream)
            plain = lambda wp: qg.bound_call("qgemv_fused_gateup_silu", qt, wp, xn.data_ptr(), y.data_ptr(),  # noqa
                                             N, K, stream)
            nbytes = 2 * wbytes(kind, N, K) + 8 * K + 4 * N
        else:
            fused = lambda wp: qg.bound_call("qgemv_rmsnorm", qt, wp, x.data_ptr(), g.data_ptr(), eps,  # noqa
                                             y.data_ptr(), N, K, stream)
            plain = lambda wp: qg.bound_call("qgemv_q8_0" if kind == "q8_0" else "qgemv_q4_0", wp,  # noqa
                                             xn.data_ptr(), y.data_ptr(), N, K, stream)
            nbytes = wbytes(kind, N, K) + 8 * K + 4 * N
        norm = qg.bound_call("qg_rmsnorm", x.data_ptr(), g.data_ptr(), eps, xn.data_ptr(), K, stream)
        norm_cases.append((label, packed, nbytes, fused, norm, plain))

    norm_case("n q8_0 qkv 4096x1024", "q8_0", qkv.weight, 4096, 1024, False)
    norm_case("n q8_0 gate|up 2x3072x1024", "q8_0", by["gate|up 2x3072x1024 silu"].weight, 3072, 1024, True)
    norm_case("n q8_0 lm_head 151936x1024", "q8_0", lm.weight, 151936, 1024, False)
    norm_case("n q4_0 gate|up 2x17408x5120", "q4_0", pg, 17408, 5120, True)
    norm_case("n q4_0 lm_head 248320x5120", "q4_0", pl, 248320, 5120, False)
    res["norm"] = norm_cases

    # the small-M GEMM for prefill chunks (qgemm_prefill) on the same weights, M rows at once
    gemm_cases = []
    for label, kind, packed, N, K in (("q8_0 lm_head 151936x1024", "q8_0", lm.weight, 151936, 1024),
                                      ("q8_0 qkv 4096x1024", "q8_0", qkv.weight, 4096, 1024),
                                      ("q4_0 down 5120x17408", "q4_0", pd, 5120, 17408),
                                      ("q4_0 lm_head 248320x5120", "q4_0", pl, 248320, 5120)):
        for M in (16, 32, 128):
            X = t(erng.standard_normal((M, K)).astype(np.float32))
            Y = yb(M * N)
            ws = torch.empty(qg.qg_prefill_workspace_size(kind, N, K, M), dtype=torch.uint8, device=dev)
            keep.append(ws)
            make = (lambda wp, kind=kind, X=X, Y=Y, ws=ws, N=N, K=K, M=M:  # noqa: E731
                    qg.bound_call("qgemm_prefill", qg.QTYPES[kind], wp, X.data_ptr(), Y.data_ptr(), N, K, M,
                                  ws.data_ptr(), ws.numel(), stream))
            gemm_cases.append((f"g {label} M={M}", kind, packed, N, K, M, make))
    res["gemm"] = gemm_cases
    torch.cuda.synchronize()
    return res, keep


def rmsnorm_fusion(qg, torch, cases, reps):
    """The RMSNorm-prologue experiment, cold (weights rotating over >= 1.2 GiB of
    copies): the fused call (one dispatch) against qg_rmsnorm + the plain GEMV (two
    dispatches). Kernel times come from events bound to each launch; the batch
    times are back-to-back calls (pairs) with one event pair around the batch,
    i.e. what a decode loop pays, dispatch gaps included."""
    out = {}
    log("rmsnorm prologue: fused (1 dispatch) vs qg_rmsnorm + GEMV (2 dispatches), cold weights")
    for label, weight, nbytes, fused, norm, plain in cases:
        copies = cold_copies(torch, weight)
        f_fns = [fused(cp.data_ptr()) for cp in copies]
        p_fns = [plain(cp.data_ptr()) for cp in copies]
        for f in f_fns[:2] + p_fns[:2]:
            f()
        norm()
        uf, bf = time_call(qg, torch, f_fns, reps)
        un, _ = time_call(qg, torch, [norm], reps)
        up, _ = time_call(qg, torch, p_fns, reps)
        pairs = [(lambda p=p: (norm(), p())) for p in p_fns]
        nb = max(reps, len(pairs))
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        b0.record()
        for i in range(nb):
            pairs[i % len(pairs)]()
        b1.record()
        torch.cuda.synchronize()
        bu = b0.elapsed_time(b1) * 1e3 / nb
        del f_fns, p_fns, pairs, copies
        r = {"fused_us": round(float(np.median(uf)), 3), "norm_us": round(float(np.median(un)), 3),
             "gemv_us": round(float(np.median(up)), 3), "fused_batch_us": round(bf, 3),
             "unfused_batch_us": round(bu, 3), "bytes": nbytes}
        out[label] = r
        log(f"  {label:30s} fused {r['fused_us']:8.2f} us | norm {r['norm_us']:6.2f} + gemv {r['gemv_us']:8.2f} us"
            f"   batch: fused {bf:8.2f} us, unfused {bu:8.2f} us ({100 * (bu - bf) / bu:+.1f}% saved by fusing)")
        torch.cuda.empty_cache()
    return out


def prefill_gemm(qg, torch, cases, table):
    """The small-M GEMM (qgemm_prefill) for chunks of M activation rows, cold
    (weights rotating over >= 1.2 GiB of copies): mean us per call over a batch
    of back-to-back calls (the split, GEMM and K-sum kernels together), us per
    activation row against the M = 1 GEMV of the same weight, useful TFLOP/s
    (2 M N K per call) and the weight stream in GB/s."""
    out = {}
    log("prefill GEMM (qgemm_prefill, matrix cores): batch us per call, cold weights")
    m1 = {"q8_0 lm_head 151936x1024": "c1 lm_head 151936x1024", "q8_0 qkv 4096x1024": "c1 qkv 4096x1024",
          "q4_0 down 5120x17408": "c2 q4_0 down 5120x17408", "q4_0 lm_head 248320x5120": "c2 q4_0 lm_head 248320x5120"}
    for label, kind, weight, N, K, M, make in cases:
        copies = cold_copies(torch, weight)
        fns = [make(cp.data_ptr()) for cp in copies]
        for f in fns[:2]:
            f()
        nb = max(8, len(fns))
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        b0.record()
        for i in range(nb):
            fns[i % len(fns)]()
        b1.record()
        torch.cuda.synchronize()
        us = b0.elapsed_time(b1) * 1e3 / nb
        del fns, copies
        base = table.get(m1[label.split(" M=")[0][2:]], {}).get("batch_us")
        r = {"us": round(us, 2), "us_per_row": round(us / M, 3), "tflops": round(2.0 * M * N * K / us / 1e6, 1),
             "weight_GBps": round(wbytes(kind, N, K) / us / 1e3, 1),
             "m1_us_per_row": round(base, 3) if base else None}
        out[label] = r
        log(f"  {label:34s} {us:9.2f} us  {us / M:7.3f} us/row (M=1: {base or float('nan'):7.2f})  "
            f"{r['tflops']:6.1f} TFLOP/s  weights {r['weight_GBps']:7.1f} GB/s")
        torch.cuda.empty_cache()
    return out


def cpu_baseline(wl, threads_all):
    """The fp64 oracle over one headline step on the host: one thread, then all threads."""
    import oracle as O

    jobs = [
        ("q8_0", np.concatenate([wl.weight(n) for n in ("q_proj", "k_proj", "v_proj")]), wl.x("q_proj"), 4096, 1024),
        ("q8_0", wl.weight("o_proj"), wl.x("o_proj"), 1024, 2048),
        ("gateup", None, wl.x("gate"), 3072, 1024),
        ("q8_0", wl.weight("down"), wl.x("down"), 1024, 3072),
        ("q8_0", wl.weight("lm_head"), wl.x("lm_head"), 151936, 1024),
    ]
    nbytes = 4476928 + 2240512 + 6701056 + 3358720 + 165918208

    def one_step(threads):
        t0 = time.perf_counter()
        for kind, w, x, N, K in jobs:
            if kind == "gateup":
                O.gateup_silu("q8_0", wl.weight("gate"), wl.weight("up"), x, N, K, threads=threads)
            else:
                O.gemv(kind, w, x, N, K, threads=threads)
        return time.perf_counter() - t0

    t1 = one_step(1)
    tall = sorted(one_step(threads_all) for _ in range(3))[1]
    return {
        "value": nbytes / tall / 1e9, "unit": "GB/s", "cores": threads_all, "kind": "oracle",
        "sample": "one full headline step (qkv, o_proj, gate|up silu, down, lm_head; 182.7 MB), fp64, "
                  f"median of 3 with {threads_all} threads",
        "ms_per_step": tall * 1e3,
        "single_thread": {"value": nbytes / t1 / 1e9, "unit": "GB/s", "cores": 1, "ms_per_step": t1 * 1e3},
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def hbm_reference(torch):
    """Bandwidth of torch's own streaming kernels on 2 GiB buffers (well above the
    256 MB Infinity Cache): a read-only reduction and a device copy."""
    n = (2 << 30) // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    out = {}
    for name, fn, nbytes in (("sum_read", lambda: a.sum(), 4 * n),):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(nbytes * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    b = torch.empty(n // 2, dtype=torch.float32, device="cuda")
    src = a[: n // 2]
    for _ in range(2):
        b.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    out["copy"] = round(2 * 4 * (n // 2) * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    return out


def load_traffic(kernel: str):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    from block_dequant_gemv_amd.prof import kernel_source_hash
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    entry = t.get("calls", {}).get(kernel)
    return round(entry["bytes_per_launch"]) if entry else None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--reps", type=int, default=100, help="cold reps per call in the per-config table")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config table")
    ap.add_argument("--only", default=None,
                    help="comma-separated label prefixes: time only the per-config rows that start with one of "
                         "them, and skip the RMSNorm and prefill-GEMM legs (for profiler runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run torch.neg over 256 MiB, a plain copy-like kernel of known traffic "
                         "(counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--detail", default=None, help="write the full per-call results to this JSON file")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {max(args.gpus, world)} is not supported "
              "(the GEMV would shard by output rows with no communication)", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_dequant_gemv_amd as qg
    from block_dequant_gemv_amd.workloads import Workload

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream().cuda_stream
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), {props.multi_processor_count} CUs")

    wl1 = Workload(1)
    step_bytes_one = 4476928 + 2240512 + 6701056 + 3358720 + 165918208
    copies = max(3, -(-COLD_BYTES // step_bytes_one))
    steps, sets, xs, ys = build_step(qg, torch, wl1, stream, copies)
    step_bytes = sum(c.nbytes for c in steps[0])
    assert step_bytes == step_bytes_one

    if args.calib_copy:
        # counter calibration: an elementwise kernel that reads exactly 256 MiB and
        # writes exactly 256 MiB (torch.neg), identifiable by name in the counter CSV
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("calibration: 5 x torch.neg over 256 MiB (256 MiB read + 256 MiB written each)")
        del src, dst

    # ---- headline: K timed steps ------------------------------------------------
    # The timed region is K plain steps: one event pair brackets them on the
    # stream the kernels run on and nothing is recorded inside, so the region runs
    # exactly as a caller's decode loop would. (Binding timing events to a launch
    # costs the host ~20 us per launch, which would make the loop host-bound.)
    for s in range(args.warmup):
        for c in steps[s % copies]:
            c.fn()
    K = args.steps
    lm = len(steps[0]) - 1
    span = timing_events(torch, 2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    span[0].record()
    for s in range(K):
        for c in steps[s % copies]:
            c.fn()
    span[1].record()
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / K * 1e3
    value = step_bytes * K / wall / 1e9
    gpu_span_ms = span[0].elapsed_time(span[1])
    host_us = (t_enq - t0) / K * 1e6
    log(f"headline: {K} steps, {ms_per_step:.4f} ms/step wall, GPU span {gpu_span_ms / K:.4f} ms/step, host "
        f"enqueue {host_us:.1f} us/step, {value:.1f} GB/s ({100 * value / PEAK_GBPS:.1f}% of 8 TB/s), "
        f"{copies} weight copies")

    # ---- the same K steps replayed from HIP graphs --------------------------------
    # One graph per weight copy holds the step's five launches (captured on a side
    # stream); replaying them is what a decode loop that captures its step does.
    graph = graph_headline(qg, torch, sets, xs, ys, K, args.warmup, copies, step_bytes)
    log(f"graph replay: {graph['ms_per_step'] * 1e3:.1f} us/step, {graph['value']:.1f} GB/s "
        f"({100 * graph['value'] / PEAK_GBPS:.1f}% of 8 TB/s)")

    # ---- kernel pass: the same K steps with every launch timed -----------------
    # Each launch is bound to an event pair that receives the kernel's own start
    # and end timestamps (qg_time_next_launch; the dispatch times a rocprofv3
    # kernel trace reports), on the kernels' stream. Every launch is bound, so
    # each kernel starts after a timed one, the same way in every step. This
    # pass gives the roofline entry of the LM head (the dominant call) and each
    # kernel's share of the step.
    ncall = len(steps[0])
    evk = timing_events(torch, 2 * K * ncall)
    torch.cuda.synchronize()
    for s in range(K):
        for i, c in enumerate(steps[s % copies]):
            e = 2 * (s * ncall + i)
            qg.qg_time_next_launch(evk[e], evk[e + 1])
            c.fn()
    torch.cuda.synchronize()
    durs = np.array([[evk[2 * (s * ncall + i)].elapsed_time(evk[2 * (s * ncall + i) + 1]) * 1e3
                      for i in range(ncall)] for s in range(K)])  # us [K][ncall]
    lm_us = durs[:, lm]
    dom = steps[0][lm]
    avg_us = float(lm_us.mean())
    achieved = dom.nbytes / (avg_us * 1e-6) / 1e9
    traffic = load_traffic(dom.label)
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
        "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic,
        "kernel": dom.kernel, "call": dom.label,
        "avg_launch_us": round(avg_us, 3), "launches": K,
        "algorithmic_bytes_per_launch": dom.nbytes,
        "timing": "kernel start/end timestamps of the LM head launches of K decode steps with every launch bound "
                  "to HIP events (qg_time_next_launch), right after the timed region",
    }
    for i, c in enumerate(steps[0]):
        med = float(np.median(durs[:, i]))
        log(f"  kernel: {c.label:28s} {med:8.2f} us  {c.nbytes / med / 1e3:8.1f} GB/s  [{c.kernel}]")
    kern_sum = float(np.median(durs.sum(axis=1)))
    log(f"  {dom.label}: kernel {float(np.median(lm_us)):.2f} us median, {avg_us:.2f} us mean -> "
        f"{achieved:.1f} GB/s ({100 * achieved / PEAK_GBPS:.1f}%)  [{dom.kernel}]")
    log(f"  sum of the step's kernel times {kern_sum:.2f} us; the timed steps took {1e3 * gpu_span_ms / K:.2f} us of "
        f"GPU time each")

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {
            "workload": "qwen3-0.6b-shaped q8_0 decode gemv set, M=1: qkv 4096x1024, o_proj 1024x2048, "
                        "gate|up 2x3072x1024 + silu, down 1024x3072, lm_head 151936x1024",
            "step_bytes": step_bytes, "cold": f"{copies} rotating device copies of the weights "
                                             f"({copies * step_bytes / 1e9:.2f} GB)",
            "pct_of_peak": round(100 * value / PEAK_GBPS, 2),
            "gpu_ms_per_step": round(gpu_span_ms / K, 5),
            "host_enqueue_us_per_step": round(host_us, 2),
            "lm_head_kernel_us_median": round(float(np.median(lm_us)), 3),
            "kernel_us_per_step": round(kern_sum, 3),
            "device": props.name,
        },
        "roofline": roofline,
        "graph_replay": graph,
    }

    detail = {"kernel_us": {c.label: float(np.median(durs[:, i])) for i, c in enumerate(steps[0])},
              "lm_head_us": lm_us.tolist()}

    # ---- reference streams: what plain torch kernels reach on this device ----------------
    ref = hbm_reference(torch)
    result["config"]["hbm_reference_GBps"] = ref
    log(f"reference streams (torch, 2 GiB): read-only sum {ref['sum_read']:.0f} GB/s, "
        f"copy {ref['copy']:.0f} GB/s (read+write)")

    # ---- per-config cold / warm table ---------------------------------------------
    # Cold: each call's weight rotates through >= 1.2 GiB of device copies (no
    # flush kernel: a read+write flush leaves dirty Infinity Cache lines whose
    # write-back would slow the timed call). Kernel durations (events bound to
    # each launch) give the median and p10/p90; `batch_us` is the mean of
    # back-to-back calls through the same copies, launch gaps included.
    # Warm: the same copy again and again (served in part by the caches).
    if not args.no_configs:
        cfg_calls, keep = per_config_calls(qg, torch, stream, steps[0])
        table = {}
        log(f"per-call table: {args.reps} cold calls rotating over >= 1.2 GiB of weight copies, and warm calls")
        norm_cases = cfg_calls.pop("norm")
        gemm_cases = cfg_calls.pop("gemm")
        only = [o for o in args.only.split(",") if o] if args.only else None
        if only:
            norm_cases, gemm_cases = [], []
        for ci in sorted(cfg_calls):
            for c in cfg_calls[ci]:
                if only and not any(c.label.startswith(o) for o in only):
                    continue
                copies = cold_copies(torch, c.weight)
                fns = [c.fn] + [c.make(cp.data_ptr()) for cp in copies[1:]]
                torch.cuda.synchronize()
                for f in fns[:3]:
                    f()
                u, batch = time_call(qg, torch, fns, args.reps)
                uw, _ = time_call(qg, torch, [c.fn], max(10, args.reps // 2))
                ncopies = len(fns)
                del fns, copies
                med = float(np.median(u))
                gbps = c.nbytes / med / 1e3
                table[c.label] = {"us": round(med, 3), "us_p10": round(float(np.percentile(u, 10)), 3),
                                  "us_p90": round(float(np.percentile(u, 90)), 3), "GBps": round(gbps, 1),
                                  "pct": round(100 * gbps / PEAK_GBPS, 1), "batch_us": round(batch, 3),
                                  "batch_GBps": round(c.nbytes / batch / 1e3, 1), "bytes": c.nbytes,
                                  "warm_us": round(float(np.median(uw)), 3), "kernel": c.kernel,
                                  "copies": ncopies, "us_each": [round(float(v), 2) for v in u]}
                log(f"  {c.label:34s} cold {med:9.2f} us ({float(np.percentile(u, 10)):.2f}-"
                    f"{float(np.percentile(u, 90)):.2f})  {gbps:8.1f} GB/s {100 * gbps / PEAK_GBPS:5.1f}%   "
                    f"batch {batch:9.2f} us {c.nbytes / batch / 1e3:8.1f} GB/s   warm {float(np.median(uw)):8.2f} us")
            torch.cuda.empty_cache()
        result["configs"] = {k: {"us": v["us"], "GBps": v["GBps"], "pct": v["pct"], "batch_us": v["batch_us"],
                                 "warm_us": v["warm_us"]} for k, v in table.items()}
        detail["configs"] = table
        result["rmsnorm_fusion"] = rmsnorm_fusion(qg, torch, norm_cases, args.reps)
        del norm_cases
        result["prefill_gemm"] = prefill_gemm(qg, torch, gemm_cases, table)
        del gemm_cases
        del keep

    # ---- CPU oracle baseline ----------------------------------------------------------
    if not args.no_cpu:
        threads = max(1, min(16, os.cpu_count() or 1))
        cb = cpu_baseline(wl1, threads)
        result["cpu_baseline"] = cb
        log(f"cpu oracle: {cb['value']:.3f} GB/s on {threads} threads, {cb['single_thread']['value']:.3f} GB/s "
            f"on 1 thread ({cb['cpu_model']})")

    if args.detail:
        with open(args.detail, "w") as f:
            json.dump({"result": result, "detail": detail}, f, indent=1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
