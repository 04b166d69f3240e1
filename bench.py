"""Benchmark of the block-dequant GEMV path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline step: the decode GEMVs of the 27B-class Q4_0 configuration, M = 1,
one pass over its three matrices in order on one stream:
  fused gate|up 2x17408x5120 + SiLU -> down 5120x17408 -> LM head 248320x5120
(866.8 MB of weights, scales, activations and outputs per step). Each step
reads the next of three device copies of the whole weight set (2.6 GB), so
the weights are cold in the 256 MB Infinity Cache and the 4 MB L2s when a step
reads them. `value` is algorithmic bytes moved per second over K timed steps
(weights + scales + x + y, each read/written once), with the inputs already in
device memory.

Also measured in the same run:
  * the roofline entry of the step's dominant kernel, the Q4_0 LM head (83% of
    the step's bytes): after the timed region, K launches of it back to back on
    the rotating weight copies between two HIP events on the kernels' stream
    (the timed region itself runs plain launches: binding events to a launch
    costs the GPU a few us of marker work per launch);
  * the Qwen3-0.6B-shaped Q8_0 decode set (fused QKV, O, gate|up + SiLU, down,
    LM head 151936x1024) as a second step, with its LM head's roofline;
  * every matrix of the five workload configurations, one call at a time, cold
    (each call's weight rotating through >= 1.2 GiB of device copies) and warm,
    as median us per call, GB/s and fraction of the 8 TB/s HBM3E peak; the
    epilogue, Q4_K / Q6_K, RMSNorm-prologue and prefill-GEMM rows;
  * the three forms of the fp16 GEMV on the fp16 configuration's shapes;
  * reference streams: a plain streaming read at the GEMVs' sizes and an empty
    kernel (the library's measurement kernels), and torch's own copy and sum;
  * the fp64 CPU oracle on the host cores, one thread and all of them, over
    one headline step and every configuration's matrices (the cpu_baseline
    leg; the only use of oracle/).
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

# The two decode steps: (kind, label, weights, N, K) per call, in order. kind
# "gemv" is a plain product, "gateup" the fused gate|up with its SiLU epilogue,
# "qkv" the load-time concatenation of three projections.
STEPS = {
    "q4_0": {
        "cfg": 2, "qtype": "q4_0",
        "workload": "27b-class q4_0 decode gemv set, M=1: gate|up 2x17408x5120+silu, down 5120x17408, "
                    "lm_head 248320x5120",
        "calls": [("gateup", "gate|up 2x17408x5120 silu", ("gate", "up"), 17408, 5120),
                  ("gemv", "down 5120x17408", "down", 5120, 17408),
                  ("gemv", "lm_head 248320x5120", "lm_head", 248320, 5120)],
    },
    "q8_0": {
        "cfg": 1, "qtype": "q8_0",
        "workload": "qwen3-0.6b-shaped q8_0 decode gemv set, M=1: qkv 4096x1024, o 1024x2048, "
                    "gate|up 2x3072x1024+silu, down 1024x3072, lm_head 151936x1024",
        "calls": [("qkv", "qkv 4096x1024", ("q_proj", "k_proj", "v_proj"), 4096, 1024),
                  ("gemv", "o_proj 1024x2048", "o_proj", 1024, 2048),
                  ("gateup", "gate|up 2x3072x1024 silu", ("gate", "up"), 3072, 1024),
                  ("gemv", "down 1024x3072", "down", 1024, 3072),
                  ("gemv", "lm_head 151936x1024", "lm_head", 151936, 1024)],
    },
}


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
    form = qg.qg_f16_plan_info(N, K)["form"]
    return Call(label, make(w.data_ptr()), 2 * N * K + 4 * K + 4 * N, f"gemv_f16<{form}>", w, make)


# ---------------------------------------------------------------------------

def build_step(qg, torch, which, stream, copies):
    """One decode step's weights, packed once and cloned into `copies` device copies,
    and the step's calls on each copy."""
    from block_dequant_gemv_amd.workloads import Workload
    spec = STEPS[which]
    kind = spec["qtype"]
    wl = Workload(spec["cfg"])
    base, xs, ys = {}, {}, {}
    for role, label, src, N, K in spec["calls"]:
        if role == "qkv":
            base[label] = qg.pack_concat(kind, [(wl.weight(n), wl.entry(n)[2]) for n in src], K)
            xsrc, nout = src[0], N
        elif role == "gateup":
            base[label] = qg.pack_gateup(kind, wl.weight(src[0]), wl.weight(src[1]), N, K)
            xsrc, nout = src[0], N
        else:
            base[label] = qg.pack_weights(kind, wl.weight(src), N, K)
            xsrc, nout = src, N
        for n in (src if isinstance(src, tuple) else (src,)):
            wl.drop(n)
        xs[label] = torch.from_numpy(wl.x(xsrc)).to("cuda")
        ys[label] = torch.empty(nout, dtype=torch.float32, device="cuda")
    sets = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(copies - 1)]
    torch.cuda.synchronize()
    steps = [step_calls(qg, which, s, xs, ys, stream) for s in sets]
    return steps, sets, xs, ys


def step_calls(qg, which, s, xs, ys, stream):
    spec = STEPS[which]
    kind = spec["qtype"]
    out = []
    for role, label, _, N, K in spec["calls"]:
        if role == "gateup":
            out.append(make_gateup(qg, kind, s[label], xs[label], ys[label], N, K, stream, label))
        else:
            out.append(make_qgemv(qg, kind, s[label], xs[label], ys[label], N, K, stream, label))
    return out


def step_bytes(which):
    from block_dequant_gemv_amd.workloads import matrix_bytes
    total = 0
    for role, _, _, N, K in STEPS[which]["calls"]:
        kind = STEPS[which]["qtype"]
        if role == "gateup":
            total += 2 * matrix_bytes(kind, N, K) + 4 * K + 4 * N
        else:
            total += matrix_bytes(kind, N, K) + 4 * K + 4 * N
    return total


def timing_events(torch, n):
    """n timing events on the current stream, recorded once so that they exist
    (torch creates the underlying hipEvent_t lazily) and can be bound to launches."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()
    return evs


def settle(torch, fns, seconds):
    """Run `fns` in rounds until `seconds` of wall time have passed (untimed).
    After a weight set is built the first ~20 ms of sustained steps run about 15%
    slower than later ones (measured: 168 us per Q4_0 step over the first 100
    steps, 143-147 us afterwards), so every timed region starts after this."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            for f in fns:
                f()
        torch.cuda.synchronize()


def run_steps(qg, torch, which, stream, K, warmup, settle_s=0.1):
    """K timed steps of a decode set with plain launches, between synchronisations;
    then, outside the timed region:
      * a pass over the same K steps with every launch bound to an event pair that
        receives the kernel's start and end timestamps (the per-kernel breakdown;
        a bound launch costs the GPU a few us of marker work and reads a few us
        long, so these durations are upper bounds and are never used for `value`);
      * for each call of the step, K launches back to back on the rotating weight
        copies between two events on the kernels' stream: the call's mean time per
        launch with no marker inside the batch (launch gaps included), which gives
        the roofline entry."""
    nbytes = step_bytes(which)
    copies = max(3, -(-COLD_BYTES // nbytes))
    steps, sets, xs, ys = build_step(qg, torch, which, stream, copies)
    assert sum(c.nbytes for c in steps[0]) == nbytes
    ncall = len(steps[0])
    settle(torch, [c.fn for st in steps for c in st], settle_s)
    for s in range(warmup):
        for c in steps[s % copies]:
            c.fn()
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
    gpu_ms = span[0].elapsed_time(span[1])

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

    batch_us = []
    b0, b1 = timing_events(torch, 2)
    for i in range(ncall):
        for s in range(copies):
            steps[s % copies][i].fn()
        torch.cuda.synchronize()
        b0.record()
        for s in range(K):
            steps[s % copies][i].fn()
        b1.record()
        torch.cuda.synchronize()
        batch_us.append(b0.elapsed_time(b1) * 1e3 / K)
    out = {"steps": steps, "sets": sets, "xs": xs, "ys": ys, "copies": copies, "bytes": nbytes, "wall": wall,
           "gpu_ms": gpu_ms, "host_us": (t_enq - t0) / K * 1e6, "durs": durs, "batch_us": batch_us}
    return out


def roofline_of(run, K):
    """The roofline entry of a decode set's dominant call (its largest matrix):
    algorithmic bytes per launch over the mean time per launch of K back-to-back
    launches (cold, rotating weight copies) between two HIP events on the kernels'
    stream."""
    steps, durs = run["steps"], run["durs"]
    dom_i = max(range(len(steps[0])), key=lambda i: steps[0][i].nbytes)
    dom = steps[0][dom_i]
    avg_us = float(run["batch_us"][dom_i])
    bound = durs[:, dom_i]
    achieved = dom.nbytes / (avg_us * 1e-6) / 1e9
    return dom_i, {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
        "frac": round(achieved / PEAK_GBPS, 4), "traffic": load_traffic(dom.label),
        "kernel": dom.kernel, "call": dom.label,
        "avg_launch_us": round(avg_us, 3), "launches": K, "algorithmic_bytes_per_launch": dom.nbytes,
        "timing": ("mean time per launch of K back-to-back launches of the call on the rotating cold weight "
                   "copies, between two HIP events on the kernels' stream (launch gaps included, no marker "
                   "inside the batch)"),
        "bound_event_us": {"mean": round(float(bound.mean()), 3), "median": round(float(np.median(bound)), 3),
                           "p10_p90": [round(float(np.percentile(bound, 10)), 3),
                                       round(float(np.percentile(bound, 90)), 3)],
                           "note": "events bound to each launch of a second pass over the K steps; a bound "
                                   "launch reads a few us long (marker work around the dispatch)"},
    }


def graph_replay(torch, qg, which, run, K, warmup, stream_unused=None):
    """The headline steps replayed from HIP graphs: one torch.cuda.CUDAGraph capturing G
    consecutive steps on a side stream (cycling through the weight copies; the GEMV
    calls record plain kernel launches and nothing else), replayed until about K steps
    have run, so that one graph launch covers G steps of kernels."""
    side = torch.cuda.Stream()
    copies = run["copies"]
    per_graph = copies * max(1, 24 // copies)
    calls = [c for i in range(per_graph)
             for c in step_calls(qg, which, run["sets"][i % copies], run["xs"], run["ys"], side.cuda_stream)]
    with torch.cuda.stream(side):
        for c in calls:
            c.fn()
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side, capture_error_mode="thread_local"):
        for c in calls:
            c.fn()
    replays = max(1, round(K / per_graph))
    with torch.cuda.stream(side):
        for _ in range(max(1, warmup // per_graph)):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(replays):
            g.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    del g
    steps = replays * per_graph
    return {"ms_per_step": round(wall / steps * 1e3, 5), "value": round(run["bytes"] * steps / wall / 1e9, 1),
            "steps": steps, "steps_per_graph": per_graph}


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


def per_config_calls(qg, torch, stream, q4_step, q8_step):
    """All five configurations as lists of calls (the two decode steps' calls reused
    for configurations 1 and 2)."""
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
    res[1] = [Call("c1 " + c.label, c.fn, c.nbytes, c.kernel, c.weight, c.make) for c in q8_step]
    res[2] = [Call("c2 q4_0 " + c.label, c.fn, c.nbytes, c.kernel, c.weight, c.make) for c in q4_step]

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
    wl1, wl2 = Workload(1), Workload(2)
    by8 = {c.label: c for c in q8_step}
    by4 = {c.label: c for c in q4_step}
    qkv, o, lm = by8["qkv 4096x1024"], by8["o_proj 1024x2048"], by8["lm_head 151936x1024"]
    pd, pl, pg = by4["down 5120x17408"].weight, by4["lm_head 248320x5120"].weight, \
        by4["gate|up 2x17408x5120 silu"].weight
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
    norm_case("n q8_0 gate|up 2x3072x1024", "q8_0", by8["gate|up 2x3072x1024 silu"].weight, 3072, 1024, True)
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


def prefill_gemm(qg, torch, cases, table, settle_s):
    """The small-M GEMM (qgemm_prefill) for chunks of M activation rows, cold
    (weights rotating over >= 1.2 GiB of copies): mean us per call over a batch
    of back-to-back calls (the split, GEMM and K-sum kernels together) after
    `settle_s` seconds of untimed calls (the first calls after the weights are
    built run slower, as for the decode step: measured 803 against 715 us for
    the Q4_0 LM head at M = 128), us per activation row against the M = 1 GEMV
    of the same weight, useful TFLOP/s (2 M N K per call) and the weight stream
    in GB/s."""
    out = {}
    log("prefill GEMM (qgemm_prefill, matrix cores): batch us per call, cold weights")
    m1 = {"q8_0 lm_head 151936x1024": "c1 lm_head 151936x1024", "q8_0 qkv 4096x1024": "c1 qkv 4096x1024",
          "q4_0 down 5120x17408": "c2 q4_0 down 5120x17408", "q4_0 lm_head 248320x5120": "c2 q4_0 lm_head 248320x5120"}
    for label, kind, weight, N, K, M, make in cases:
        copies = cold_copies(torch, weight)
        fns = [make(cp.data_ptr()) for cp in copies]
        settle(torch, fns, settle_s)
        nb = max(16, len(fns))
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


F16_FORM_ENV = {"lane-split": {"QG_F16_FORM": "0"}, "row": {"QG_F16_FORM": "1"},
                "split-K row": {"QG_F16_FORM": "2"}}


def f16_forms(qg, torch, reps):
    """The three forms of gemv_f16_splitk (forced by QG_F16_FORM) on the fp16
    configuration's shapes and two between them, cold (weights rotating over
    >= 1.2 GiB of copies): kernel median (events bound to each launch) and the
    mean of back-to-back calls. The default form of each shape is marked."""
    from block_dequant_gemv_amd import workloads as W
    rng = np.random.default_rng(3)
    out = {}
    log("fp16 GEMV forms (cold): kernel median us / back-to-back us; * = the default form")
    try:
        for N, K in ((48, 5120), (256, 5120), (640, 5120), (1024, 5120), (5120, 5120)):
            w = torch.from_numpy(W.f16_matrix(N, K, rng)).cuda()
            x = torch.from_numpy(W.activation(K, rng)).cuda()
            y = torch.empty(N, dtype=torch.float32, device="cuda")
            for k in ("QG_F16_FORM", "QG_F16_CPL"):
                os.environ.pop(k, None)
            qg.qg_reload_tuning()
            default = qg.qg_f16_plan_info(N, K)["form"]
            copies = cold_copies(torch, w)
            row = {}
            for form, env in F16_FORM_ENV.items():
                os.environ.update(env)
                qg.qg_reload_tuning()
                assert qg.qg_f16_plan_info(N, K)["form"] == form
                fns = [qg.bound_call("gemv_f16_splitk", c.data_ptr(), x.data_ptr(), y.data_ptr(), N, K, 0)
                       for c in copies]
                for f in fns[:3]:
                    f()
                u, batch = time_call(qg, torch, fns, reps)
                row[form] = {"us": round(float(np.median(u)), 3), "batch_us": round(batch, 3)}
            out[f"{N}x{K}"] = {"default": default, **row}
            log(f"  f16 {N:5d}x{K}: " + "   ".join(
                f"{'*' if f == default else ' '}{f} {r['us']:6.2f} / {r['batch_us']:6.2f}" for f, r in row.items()))
            del copies, w
            torch.cuda.empty_cache()
    finally:
        for k in ("QG_F16_FORM", "QG_F16_CPL"):
            os.environ.pop(k, None)
        qg.qg_reload_tuning()
    return out


def reference_streams(qg, torch, reps):
    """What this device streams: the library's streaming-read kernel over the
    GEMVs' byte counts, cold (rotating over >= 1.2 GiB of buffers), and its empty
    kernel (the floor of any dispatch), each as the kernel median (events bound to
    the launch) and the mean of back-to-back launches; an empty kernel replayed
    from a HIP graph; and torch's own 2 GiB read-only sum and copy."""
    out = {"stream_read": {}}
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    log("reference streams (cold): streaming read, kernel median / back-to-back")
    for label, nbytes in (("4.5 MB (qkv 4096x1024)", 4476928), ("50.2 MB (q4_0 5120x17408)", 50225152),
                          ("100.4 MB (q4_0 gate|up)", 100360192), ("165.9 MB (q8_0 lm_head)", 165918208),
                          ("716.2 MB (q4_0 lm_head)", 716175360)):
        n = -(-nbytes // 1024) * 1024
        buf = torch.zeros(n // 4, dtype=torch.int32, device="cuda")
        copies = cold_copies(torch, buf)
        fns = [qg.bound_call("qg_probe_stream", c.data_ptr(), n, sink.data_ptr(), 0) for c in copies]
        for f in fns[:3]:
            f()
        u, batch = time_call(qg, torch, fns, reps)
        med = float(np.median(u))
        out["stream_read"][label] = {"bytes": n, "us": round(med, 3), "p10_us": round(float(np.percentile(u, 10)), 3),
                                     "GBps": round(n / med / 1e3, 1), "pct": round(100 * n / med / 1e3 / PEAK_GBPS, 1),
                                     "batch_us": round(batch, 3)}
        log(f"  stream read {label:28s} {med:8.2f} us ({n / med / 1e3:7.1f} GB/s, "
            f"{100 * n / med / 1e3 / PEAK_GBPS:4.1f}%)  batch {batch:8.2f} us")
        del copies, buf, fns
        torch.cuda.empty_cache()
    empty = qg.bound_call("qg_probe_empty", 0)
    empty()
    u, batch = time_call(qg, torch, [empty], reps)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side, capture_error_mode="thread_local"):
        for _ in range(20):
            qg.bound_call("qg_probe_empty", side.cuda_stream)()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(20):
        g.replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - t0) / 400 * 1e6
    out["empty_kernel"] = {"us": round(float(np.median(u)), 3), "batch_us": round(batch, 3),
                           "graph_node_us": round(graph_us, 3)}
    log(f"  empty kernel: {float(np.median(u)):.2f} us by kernel timestamps, {batch:.2f} us per launch back to back, "
        f"{graph_us:.2f} us per node replayed from a HIP graph")
    # torch's own 2 GiB kernels
    n = (2 << 30) // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    for _ in range(2):
        a.sum()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        a.sum()
    e1.record()
    torch.cuda.synchronize()
    out["torch_sum_read_GBps"] = round(4 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    b = torch.empty(n // 2, dtype=torch.float32, device="cuda")
    src = a[: n // 2]
    for _ in range(2):
        b.copy_(src)
    e0.record()
    for _ in range(5):
        b.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    out["torch_copy_GBps"] = round(2 * 4 * (n // 2) * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    log(f"  torch 2 GiB: read-only sum {out['torch_sum_read_GBps']:.0f} GB/s, copy {out['torch_copy_GBps']:.0f} GB/s")
    del a, b
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# The fp64 CPU oracle (the cpu_baseline leg)

def _host_cpus():
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = None
    quota = None
    try:
        q, per = open("/sys/fs/cgroup/cpu.max").read().split()
        if q != "max":
            quota = round(int(q) / int(per), 2)
    except (OSError, ValueError):
        pass
    return {"cpu_count": os.cpu_count(), "affinity": aff, "cgroup_quota_cpus": quota, "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(threads_all):
    """The fp64 oracle as it stands, on the host cores: one headline step (the
    27B-class Q4_0 set) with one thread and with all of them, and every matrix of
    the five configurations the same two ways (verify at M = 1 and M = 6)."""
    import oracle as O
    from block_dequant_gemv_amd.workloads import Workload

    jobs = []   # (config, label, bytes, rows, fn(threads))

    def gemv_job(cfg, label, wl, name, kind=None):
        _, k, N, K, _ = wl.entry(name)
        w, x = wl.weight(name), wl.x(name)
        jobs.append((cfg, label, wbytes(k, N, K) + 4 * K + 4 * N, N,
                     lambda th, w=w, x=x, k=k, N=N, K=K: O.gemv(k, w, x, N, K, threads=th)))

    def gateup_job(cfg, label, wl, kind, N_ff, K):
        g, u, x = wl.weight("gate"), wl.weight("up"), wl.x("gate")
        jobs.append((cfg, label, 2 * wbytes(kind, N_ff, K) + 4 * K + 4 * N_ff, N_ff,
                     lambda th: O.gateup_silu(kind, g, u, x, N_ff, K, threads=th)))

    wl = Workload(2)
    gateup_job(2, "c2 q4_0 gate|up 2x17408x5120 silu", wl, "q4_0", 17408, 5120)
    gemv_job(2, "c2 q4_0 down 5120x17408", wl, "down")
    gemv_job(2, "c2 q4_0 lm_head 248320x5120", wl, "lm_head")
    wl = Workload(0)
    gemv_job(0, "c0 q8_0 1024x1024", wl, "w")
    wl = Workload(1)
    qkv = np.concatenate([wl.weight(n) for n in ("q_proj", "k_proj", "v_proj")])
    xq = wl.x("q_proj")
    jobs.append((1, "c1 qkv 4096x1024", wbytes("q8_0", 4096, 1024) + 4 * 1024 + 4 * 4096, 4096,
                 lambda th: O.gemv("q8_0", qkv, xq, 4096, 1024, threads=th)))
    gemv_job(1, "c1 o_proj 1024x2048", wl, "o_proj")
    gateup_job(1, "c1 gate|up 2x3072x1024 silu", wl, "q8_0", 3072, 1024)
    gemv_job(1, "c1 down 1024x3072", wl, "down")
    gemv_job(1, "c1 lm_head 151936x1024", wl, "lm_head")
    wl = Workload(3)
    for name in ("square", "thin", "small"):
        _, _, N, K, _ = wl.entry(name)
        gemv_job(3, f"c3 f16 {N}x{K}", wl, name)
    wl = Workload(4)
    for name in ("q4_0_w", "q8_0_w"):
        _, kind, N, K, _ = wl.entry(name)
        w, X = wl.weight(name), wl.x(name, M=6)
        jobs.append((4, f"c4 {kind} {N}x{K} M=1", wbytes(kind, N, K) + 4 * K + 4 * N, N,
                     lambda th, w=w, X=X, kind=kind, N=N, K=K: O.gemv(kind, w, np.ascontiguousarray(X[0]), N, K,
                                                                      threads=th)))
        jobs.append((4, f"c4 {kind} {N}x{K} M=6", wbytes(kind, N, K) + 24 * K + 24 * N, N,
                     lambda th, w=w, X=X, kind=kind, N=N, K=K: O.verify(kind, w, X, N, K, threads=th)))

    per = {}
    for cfg, label, nbytes, rows, fn in jobs:
        t0 = time.perf_counter()
        fn(1)
        t1 = time.perf_counter() - t0
        reps = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn(threads_all)
            reps.append(time.perf_counter() - t0)
        ta = sorted(reps)[1]
        used = threads_all if rows >= threads_all else 1   # the oracle runs rows < threads on one thread
        per[label] = {"bytes": nbytes, "single_us": round(t1 * 1e6, 1), "all_us": round(ta * 1e6, 1),
                      "all_threads": used, "single_GBps": round(nbytes / t1 / 1e9, 3),
                      "all_GBps": round(nbytes / ta / 1e9, 3)}
        log(f"  cpu oracle {label:36s} 1 thread {t1 * 1e3:9.2f} ms   {used} threads {ta * 1e3:9.2f} ms")
    head = [lbl for cfg, lbl, *_ in jobs if cfg == 2]
    hb = sum(per[l]["bytes"] for l in head)
    t_all = sum(per[l]["all_us"] for l in head) * 1e-6
    t_one = sum(per[l]["single_us"] for l in head) * 1e-6
    return {
        "value": round(hb / t_all / 1e9, 3), "unit": "GB/s", "cores": threads_all, "kind": "oracle",
        "sample": "one full headline step (27b-class q4_0 gate|up+silu, down, lm_head; 866.8 MB), fp64, median of 3 "
                  f"with {threads_all} threads; per_config: every matrix of the five configurations (verify at M=1 "
                  "and M=6), one thread once and all threads median of 3",
        "ms_per_step": round(t_all * 1e3, 3),
        "single_thread": {"value": round(hb / t_one / 1e9, 3), "unit": "GB/s", "cores": 1,
                          "ms_per_step": round(t_one * 1e3, 3)},
        "host": _host_cpus(),
        "per_config": per,
    }


def load_traffic(label: str):
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
    entry = t.get("calls", {}).get(label)
    return round(entry["bytes_per_launch"]) if entry else None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed steps run for this long before the warm-up steps of each decode set")
    ap.add_argument("--reps", type=int, default=100, help="cold reps per call in the per-config table")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config table and the legs after it (fp16 forms, reference streams)")
    ap.add_argument("--no-q8-step", action="store_true", help="skip the Q8_0 decode step")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay of the headline steps")
    ap.add_argument("--only", default=None,
                    help="comma-separated label prefixes: time only the per-config, RMSNorm ('n ...') and "
                         "prefill-GEMM ('g ...') rows that start with one of them, and skip the fp16-form and "
                         "reference-stream legs")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-warm", action="store_true",
                    help="time only the cold calls of the per-config table (no warm column): every launch of a "
                         "row's kernel is then cold, for profiler runs")
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

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream().cuda_stream
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), {props.multi_processor_count} CUs")

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

    K = args.steps
    # ---- headline: the Q4_0 decode set ---------------------------------------------
    run4 = run_steps(qg, torch, "q4_0", stream, K, args.warmup, args.settle_ms / 1e3)
    value = run4["bytes"] * K / run4["wall"] / 1e9
    ms_per_step = run4["wall"] / K * 1e3
    log(f"headline (q4_0 set): {K} steps, {ms_per_step:.4f} ms/step wall, GPU span {run4['gpu_ms'] / K:.4f} "
        f"ms/step, host enqueue {run4['host_us']:.1f} us/step, {value:.1f} GB/s ({100 * value / PEAK_GBPS:.1f}% "
        f"of 8 TB/s), {run4['copies']} weight copies")
    dom_i, roofline = roofline_of(run4, K)
    for i, c in enumerate(run4["steps"][0]):
        b = run4["batch_us"][i]
        med = float(np.median(run4["durs"][:, i]))
        log(f"  kernel: {c.label:28s} {b:8.2f} us back to back ({c.nbytes / b / 1e3:7.1f} GB/s), "
            f"{med:8.2f} us bound-event median  [{c.kernel}]")
    log(f"  roofline: {roofline['call']} {roofline['avg_launch_us']:.2f} us per launch back to back -> "
        f"{roofline['achieved']:.1f} GB/s ({100 * roofline['frac']:.1f}% of 8 TB/s)")

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {
            "workload": STEPS["q4_0"]["workload"],
            "step_bytes": run4["bytes"],
            "cold": f"{run4['copies']} rotating device copies of the weights "
                    f"({run4['copies'] * run4['bytes'] / 1e9:.2f} GB)",
            "pct_of_peak": round(100 * value / PEAK_GBPS, 2),
            "gpu_ms_per_step": round(run4["gpu_ms"] / K, 5),
            "host_enqueue_us_per_step": round(run4["host_us"], 2),
            "kernel_us_back_to_back": {c.label: round(run4["batch_us"][i], 3)
                                       for i, c in enumerate(run4["steps"][0])},
            "kernel_us_bound_event_median": {c.label: round(float(np.median(run4["durs"][:, i])), 3)
                                             for i, c in enumerate(run4["steps"][0])},
            "device": props.name,
        },
        "roofline": roofline,
    }
    detail = {"q4_0_kernel_us": {c.label: run4["durs"][:, i].tolist() for i, c in enumerate(run4["steps"][0])}}
    if not args.no_graph:
        result["graph_replay"] = graph_replay(torch, qg, "q4_0", run4, K, args.warmup)
        gr = result["graph_replay"]
        log(f"graph replay (q4_0 set, {gr['steps_per_graph']} steps per graph): {gr['ms_per_step'] * 1e3:.1f} us/step, "
            f"{gr['value']:.1f} GB/s")
    q4_step = run4["steps"][0]

    # ---- the Q8_0 decode set ---------------------------------------------------------
    q8_step = None
    if not args.no_q8_step or not args.no_configs:
        run8 = run_steps(qg, torch, "q8_0", stream, K, args.warmup, args.settle_ms / 1e3)
        v8 = run8["bytes"] * K / run8["wall"] / 1e9
        _, roof8 = roofline_of(run8, K)
        result["q8_0_step"] = {"workload": STEPS["q8_0"]["workload"], "value": round(v8, 1), "unit": "GB/s",
                               "ms_per_step": round(run8["wall"] / K * 1e3, 5), "step_bytes": run8["bytes"],
                               "pct_of_peak": round(100 * v8 / PEAK_GBPS, 2), "roofline": roof8,
                               "kernel_us_back_to_back": {c.label: round(run8["batch_us"][i], 3)
                                                          for i, c in enumerate(run8["steps"][0])},
                               "kernel_us_bound_event_median": {
                                   c.label: round(float(np.median(run8["durs"][:, i])), 3)
                                   for i, c in enumerate(run8["steps"][0])}}
        log(f"q8_0 set: {run8['wall'] / K * 1e6:.2f} us/step, {v8:.1f} GB/s ({100 * v8 / PEAK_GBPS:.1f}%); "
            f"{roof8['call']} {roof8['avg_launch_us']:.2f} us per launch back to back ({100 * roof8['frac']:.1f}%)")
        q8_step = run8["steps"][0]
        keep8 = run8
    # the headline's extra weight copies are no longer needed
    del run4["steps"][1:], run4["sets"][1:]
    if q8_step is not None:
        del keep8["steps"][1:], keep8["sets"][1:]
    torch.cuda.empty_cache()

    # ---- per-config cold / warm table ---------------------------------------------
    # Cold: each call's weight rotates through >= 1.2 GiB of device copies (no
    # flush kernel: a read+write flush leaves dirty Infinity Cache lines whose
    # write-back would slow the timed call). Kernel durations (events bound to
    # each launch) give the median and p10/p90; `batch_us` is the mean of
    # back-to-back calls through the same copies, launch gaps included.
    # Warm: the same copy again and again (served in part by the caches).
    if not args.no_configs:
        cfg_calls, keep = per_config_calls(qg, torch, stream, q4_step, q8_step)
        table = {}
        log(f"per-call table: {args.reps} cold calls rotating over >= 1.2 GiB of weight copies, and warm calls")
        norm_cases = cfg_calls.pop("norm")
        gemm_cases = cfg_calls.pop("gemm")
        only = [o for o in args.only.split(",") if o] if args.only else None
        if only:   # the RMSNorm ("n ...") and GEMM ("g ...") rows take the same prefixes
            norm_cases = [c for c in norm_cases if any(c[0].startswith(o) for o in only)]
            gemm_cases = [c for c in gemm_cases if any(c[0].startswith(o) for o in only)]
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
                uw = np.array([np.nan]) if args.no_warm else time_call(qg, torch, [c.fn], max(10, args.reps // 2))[0]
                ncopies = len(fns)
                del fns, copies
                med = float(np.median(u))
                gbps = c.nbytes / med / 1e3
                table[c.label] = {"us": round(med, 3), "us_p10": round(float(np.percentile(u, 10)), 3),
                                  "us_p90": round(float(np.percentile(u, 90)), 3), "GBps": round(gbps, 1),
                                  "pct": round(100 * gbps / PEAK_GBPS, 1), "batch_us": round(batch, 3),
                                  "batch_GBps": round(c.nbytes / batch / 1e3, 1), "bytes": c.nbytes,
                                  "warm_us": None if args.no_warm else round(float(np.median(uw)), 3),
                                  "kernel": c.kernel,
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
        result["prefill_gemm"] = prefill_gemm(qg, torch, gemm_cases, table, args.settle_ms / 1e3)
        del gemm_cases
        del keep
        torch.cuda.empty_cache()
        if not only:
            result["f16_forms"] = f16_forms(qg, torch, args.reps)
            result["reference_streams"] = reference_streams(qg, torch, args.reps)

    # ---- CPU oracle baseline ----------------------------------------------------------
    if not args.no_cpu:
        threads = max(1, min(256, os.cpu_count() or 1))   # the oracle runs at most 256 threads
        log(f"cpu oracle (fp64): 1 thread and {threads} threads")
        cb = cpu_baseline(threads)
        result["cpu_baseline"] = cb
        log(f"cpu oracle: {cb['value']:.3f} GB/s on {threads} threads, {cb['single_thread']['value']:.3f} GB/s "
            f"on 1 thread over one headline step ({cb['host']})")

    if args.detail:
        with open(args.detail, "w") as f:
            json.dump({"result": result, "detail": detail}, f, indent=1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
