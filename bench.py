#!/usr/bin/env python3
"""Benchmark: a Qwen3-4B-shaped decode layer of quantized projections on one MI355X.

One step = one pass of the layer's projection calls over one batch of tokens:
  qgemv_triple  Q 4096x2560 Q4_K, K 1024x2560 Q4_K, V 1024x2560 Q6_K
  qgemv_add     Wo 2560x4096 Q4_K with the residual add
  qgemv_pair    gate, up 9728x2560 Q4_K
  qgemv_q6k / qgemm_rows   down 2560x9728 Q6_K
Weights are synthetic (seeded, the value distributions of the Q4_K_M workload),
resident in HBM before timing, repacked once into 16-row tiles (qg_pack_tiles: the
same superblocks in another order, the same bits of every product; --layout rows
keeps the row layout, and the row-layout N=1 layer is timed beside it); 36 distinct
copies of the layer (2.3 GB, beyond the 256 MB Infinity Cache) rotate so every step
streams its weights cold.  The
36-layer sequence is captured once in a HIP graph and replayed, so host launch
overhead is not part of the measurement.

Headline: achieved HBM GB/s (algorithmic bytes / time) at N=1, the figure the
decode-GEMV pages care about.  Beside it: a plain read of the same weight bytes
(the read-stream probe, same rotation and call order), the same layer at N=32,
the 512-token prefill GEMM in TFLOP/s (on the same tiled copies of its weights; the
row layout beside it), NVFP4 and block-scaled FP8 at 1/16/32
rows on 16384x8192 and the 151936x2560 head, and the CPU oracle on a bounded
sample.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
LAYERS = 36


def kernel_source_sha() -> str:
    """Hash of the sources the decode products and their launch choice are built
    from (the MFMA product kernels, their loads, device helpers and the C-ABI
    launch code); the prefill, dequant and probe kernels are left out."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gemm_q4_q5_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if not (name.startswith("qg_mma") or name in ("qg_loads.hpp", "qg_device.hpp", "qg_api.cpp")):
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def call_bytes(wtype, m, k, n, resid=False):
    import synth
    wb = m * synth.row_bytes(wtype, k)
    if wtype == synth.NVFP4:
        wb += m * (k // 16)                                  # one e4m3 scale per 16 weights
    elif wtype == synth.FP8:
        wb += 2 * (-(-m // synth.FP8_BLOCK)) * (k // synth.FP8_BLOCK)   # bf16 per 128x128 block
    return wb + 2 * n * k + 4 * n * m + (4 * n * m if resid else 0)


class Layer:
    """Device buffers of one decode layer (weights shared by reference when cloned)."""

    def __init__(self, W):
        self.W = W  # name -> QWeight


def build_layers(n_layers, seed=1, layout="tiles"):
    """n_layers distinct copies of the layer's weights, in the row layout as stored or
    repacked once into 16-row tiles (qg_pack_tiles: the same superblocks in another
    order, same bits of every product)."""
    import torch
    import gemm_q4_q5_amd as qg
    import synth
    base = {}
    for i, (name, wt, m, k) in enumerate(synth.QWEN3_4B_LAYER):
        data, scales = synth.weights(wt, m, k, synth.rng_for(seed, i))
        base[name] = qg.QWeight.from_host(wt, data, m, k, scales, device="cuda")
        if layout == "tiles":
            base[name] = qg.pack_tiles(base[name])
    layers = [Layer(base)]
    for _ in range(1, n_layers):
        layers.append(Layer({nm: qg.QWeight(w.type, w.data.clone(), w.m, w.k,
                                            None if w.scales is None else w.scales.clone(), w.layout)
                             for nm, w in base.items()}))
    torch.cuda.synchronize()
    return layers


class Buffers:
    def __init__(self, n, seed=1):
        import torch
        import synth
        rng = synth.rng_for(seed, 99)
        dev = "cuda"
        self.x_h = torch.from_numpy(synth.activations(n, 2560, rng)).to(dev)
        self.x_o = torch.from_numpy(synth.activations(n, 4096, rng)).to(dev)
        self.x_f = torch.from_numpy(synth.activations(n, 9728, rng)).to(dev)
        self.resid = torch.from_numpy(rng.standard_normal((n, 2560)).astype(np.float32)).to(dev)
        f = lambda m: torch.empty((n, m), dtype=torch.float32, device=dev)
        self.q, self.k, self.v = f(4096), f(1024), f(1024)
        self.o, self.g, self.u, self.d = f(2560), f(9728), f(9728), f(2560)


def layer_calls(L, B, n):
    """The layer's four projection calls, in order, as (name, thunk)."""
    import gemm_q4_q5_amd as qg
    W = L.W
    calls = [
        ("triple", lambda: qg.qgemv_triple(W["wq"], W["wk"], W["wv"], B.x_h, B.q, B.k, B.v)),
        ("add", lambda: qg.qgemv_add(W["wo"], B.x_o, B.resid, B.o)),
        ("pair", lambda: qg.qgemv_pair(W["gate"], W["up"], B.x_h, B.g, B.u)),
    ]
    if n == 1 and W["down"].layout == qg.LAYOUT_ROWS:
        calls.append(("down", lambda: qg.qgemv_q6k(W["down"], B.x_f[0], B.d[0])))
    else:   # the tiled layout goes through qgemm_rows (one token: the same kernel)
        calls.append(("down", lambda: qg.qgemm_rows(W["down"], B.x_f, B.d)))
    return calls


KERNELS = ("triple", "add", "pair", "down")


def layer_call_bytes(n):
    return {
        "triple": call_bytes(12, 4096, 2560, n) + call_bytes(12, 1024, 2560, n)
        + call_bytes(14, 1024, 2560, n) - 2 * 2 * n * 2560,  # x read once for the three
        "add": call_bytes(12, 2560, 4096, n, resid=True),
        "pair": call_bytes(12, 9728, 2560, n) * 2 - 2 * n * 2560,
        "down": call_bytes(14, 2560, 9728, n),
    }


def _capture(layers, B, n, only=None, nsteps=LAYERS):
    """A graph of `nsteps` layer steps over the 36-layer rotation (step i uses copy
    i % 36): all four calls per step, or only call `only`."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(nsteps):
            for name, fn in layer_calls(layers[i % len(layers)], B, n):
                if only is None or name == only:
                    fn()
    return g


def _time_graph(g, reps, wreps):
    """Total ms of `reps` back-to-back replays (after `wreps` untimed), synchronized
    on both sides."""
    import torch
    for _ in range(wreps):
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


MIN_REPLAYS = 5


def _replay_stats(g, per, reps=MIN_REPLAYS, wreps=1):
    """Time each of `reps` replays on its own (HIP events on the stream the graph
    runs on); `per` units of work per replay.  {median, min, max} ms per unit."""
    import torch
    for _ in range(wreps):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    ts = sorted(ev[i].elapsed_time(ev[i + 1]) / per for i in range(reps))
    return {"median": ts[len(ts) // 2], "min": ts[0], "max": ts[-1], "replays": reps}


def time_layer(layers, n, steps, warmup):
    """The contract's step timing, then statistics.

    Exactly `steps` layer steps (one graph of that many steps, the copies rotating)
    are timed between two synchronizations after `warmup` untimed steps; then the
    same graph is replayed MIN_REPLAYS more times, each replay timed on its own, for
    the median, minimum and maximum.  Each kernel's launch duration comes from a
    graph of that call alone over the 36 copies, replayed MIN_REPLAYS times (HIP
    events on the stream the graph runs on; HIP does not allow event nodes inside a
    captured graph, so per-kernel events cannot sit inside the step graph itself)."""
    import torch
    B = Buffers(n)
    s = torch.cuda.Stream()   # eager warm-up on a side stream: loads code objects
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _, fn in layer_calls(layers[0], B, n):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    if warmup > 0:
        gw = _capture(layers, B, n, nsteps=warmup)
        gw.replay()
        torch.cuda.synchronize()
        del gw
    g = _capture(layers, B, n, nsteps=steps)
    total_ms = _time_graph(g, 1, 0)
    out = {"steps": steps, "ms_per_step": total_ms / steps,
           "step_stats_ms": _replay_stats(g, steps)}
    del g
    kus = {}
    for name in KERNELS:
        gk = _capture(layers, B, n, only=name)
        st = _replay_stats(gk, LAYERS)
        kus[name] = {k: (1000.0 * v if k != "replays" else v) for k, v in st.items()}
        del gk
    out["kernel_us"] = kus
    return out


def _layer_regions(L):
    """The weight tensors each layer call streams, in the layer's call order."""
    W = L.W
    return (("triple", [W["wq"].data, W["wk"].data, W["wv"].data]), ("add", [W["wo"].data]),
            ("pair", [W["gate"].data, W["up"].data]), ("down", [W["down"].data]))


def time_read_ceiling(layers):
    """The read-stream probe (plain 16-byte loads, no arithmetic) over the same
    weight bytes, in the same 36-layer rotation and call order as the layer: the
    HBM read rate this memory system gives the step's byte pattern and launch
    count, against which the products are also reported (median of the replays)."""
    import torch
    import gemm_q4_q5_amd as qg
    out = torch.zeros(qg._lib.READ_PROBE_WORDS, dtype=torch.int32, device="cuda")
    for _, regs in _layer_regions(layers[0]):
        qg.qg_stream_read(regs, out)
    torch.cuda.synchronize()
    res = {}
    for only in (None,) + KERNELS:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(LAYERS):
                for name, regs in _layer_regions(layers[i % len(layers)]):
                    if only is None or name == only:
                        qg.qg_stream_read(regs, out)
        us = 1000.0 * _replay_stats(g, LAYERS)["median"]
        nbytes = sum(t.numel() for name, regs in _layer_regions(layers[0]) for t in regs
                     if only is None or name == only)
        res["layer" if only is None else only] = {"us": round(us, 3), "GB/s": round(nbytes / (us * 1e3), 1),
                                                  "bytes": nbytes}
        del g
    return res


def time_q4k_single(layers):
    """The Q4_K GEMV alone (one matrix per call, qgemm_rows with one token = the
    single-token kernel) on each Q4_K shape of the layer, rotated over the 36 copies,
    at 1 and 32 tokens: median / min / max us and GB/s of the replays."""
    import torch
    import gemm_q4_q5_amd as qg
    import synth
    out = {}
    for name in ("gate", "wq", "wo"):
        w0 = layers[0].W[name]
        for n in (1, 32):
            x = torch.from_numpy(synth.activations(n, w0.k, synth.rng_for(1, 97, n))).to("cuda")
            y = torch.empty((n, w0.m), dtype=torch.float32, device="cuda")
            qg.qgemm_rows(w0, x, y)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(LAYERS):
                    qg.qgemm_rows(layers[i % len(layers)].W[name], x, y)
            st = _replay_stats(g, LAYERS)
            b = call_bytes(12, w0.m, w0.k, n)
            out[f"{w0.m}x{w0.k}_n{n}"] = {"us": round(1000 * st["median"], 3), "us_min": round(1000 * st["min"], 3),
                                          "us_max": round(1000 * st["max"], 3),
                                          "GB/s": round(b / (1e6 * st["median"]), 1),
                                          "pct_of_peak": round(100 * b / (1e6 * st["median"]) / PEAK_HBM_GBS, 2)}
            del g
    return out


LARGE_SHAPES = (("16384x8192", 16384, 8192), ("151936x2560", 151936, 2560))


def time_scaled(wtype, reps=4):
    """A block-scaled format (NVFP4 W4A16 or FP8 W8A16) at 1, 16 and 32 rows on two
    large shapes (a 16384x8192 projection and the 151936x2560 output head), each
    rotated over enough distinct copies to exceed 1 GiB so every call streams cold;
    one graph per (shape, n)."""
    import torch
    import gemm_q4_q5_amd as qg
    import synth
    res = {}
    for i, (name, m, k) in enumerate(LARGE_SHAPES):
        data, scales = synth.weights(wtype, m, k, synth.rng_for(4, i) if wtype == synth.NVFP4
                                     else synth.rng_for(5, wtype, i))
        base = qg.QWeight.from_host(wtype, data, m, k, scales, device="cuda")
        wbytes = data.nbytes + scales.nbytes
        copies = max(2, -(-(1 << 30) // wbytes))
        ws = [base] + [qg.QWeight(wtype, base.data.clone(), m, k, base.scales.clone())
                       for _ in range(copies - 1)]
        res[name] = {"copies": copies}
        for n in (1, 16, 32):
            x = torch.from_numpy(synth.activations(n, k, synth.rng_for(4, i, n))).to("cuda")
            y = torch.empty((n, m), dtype=torch.float32, device="cuda")
            qg.qgemm_rows(ws[0], x, y)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for w in ws:
                    qg.qgemm_rows(w, x, y)
            us = 1000.0 * _time_graph(g, reps, 1) / (reps * copies)
            b = call_bytes(wtype, m, k, n)
            res[name][f"n{n}"] = {"us": round(us, 2), "GB/s": round(b / (us * 1e3), 1),
                                  "pct_of_peak": round(100 * b / (us * 1e3) / PEAK_HBM_GBS, 2)}
            del g
        del ws, base
        torch.cuda.empty_cache()
    return res


PREFILL = (("q4k_9728x2560", 12, 9728, 2560), ("q6k_2560x9728", 14, 2560, 9728), ("q5k_4096x2560", 13, 4096, 2560))
PREFILL_N = 512
PREFILL_COPIES = 4


def _prefill_calls(layout="tiles"):
    """calls(only=None): the prefill calls on the three shapes, each over its rotated copies
    (only = an index into PREFILL for one shape).  layout "tiles": the weights repacked once
    into 16-row tiles, the copy the decode calls read; "rows": as stored."""
    import torch
    import gemm_q4_q5_amd as qg
    import synth
    ws = []
    for i, (name, wt, m, k) in enumerate(PREFILL):
        data, scales = synth.weights(wt, m, k, synth.rng_for(3, i))
        base = qg.QWeight.from_host(wt, data, m, k, scales, device="cuda")
        if layout == "tiles":
            base = qg.pack_tiles(base)
        ws.append([base] + [qg.QWeight(wt, base.data.clone(), m, k, None, base.layout)
                            for _ in range(PREFILL_COPIES - 1)])
    rng = synth.rng_for(3, 99)
    xs = {k: torch.from_numpy(synth.activations(PREFILL_N, k, rng)).to("cuda") for k in (2560, 9728)}
    ys = [torch.empty((PREFILL_N, m), dtype=torch.float32, device="cuda") for _, _, m, _ in PREFILL]

    def calls(only=None):
        for c in range(PREFILL_COPIES):
            for i, (name, wt, m, k) in enumerate(PREFILL):
                if only is None or only == i:
                    qg.qgemm_prefill(ws[i][c], xs[k], ys[i])

    return calls


def replay_prefill(name, steps, warmup):
    """Profile mode: one prefill shape's graph (its rotated copies), `steps` launches after
    `warmup`; one JSON line."""
    import torch
    only = [p[0] for p in PREFILL].index(name)
    calls = _prefill_calls()
    calls(only)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(only)
    reps = max(1, steps // PREFILL_COPIES)
    ms = _time_graph(g, reps, max(1, warmup // PREFILL_COPIES))
    us = 1000.0 * ms / (reps * PREFILL_COPIES)
    _, _, m, k = PREFILL[only]
    print(json.dumps({"prefill_call": name, "tokens": PREFILL_N, "launches": reps * PREFILL_COPIES,
                      "us_per_launch": round(us, 2),
                      "TFLOP/s": round(2.0 * PREFILL_N * m * k / (us * 1e-6) / 1e12, 1)}))


def time_prefill(reps=10, layout="tiles"):
    """Prefill chunk of 512 tokens through the MFMA GEMM on the three config
    shapes (4 rotated copies of each weight), from a HIP graph."""
    import torch
    calls = _prefill_calls(layout)
    calls()
    torch.cuda.synchronize()
    out = {}
    flops_all = sum(2.0 * PREFILL_N * m * k for _, _, m, k in PREFILL)
    for only in (None, 0, 1, 2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls(only)
        ms = _time_graph(g, reps, 2) / (reps * PREFILL_COPIES)
        fl = flops_all if only is None else 2.0 * PREFILL_N * PREFILL[only][2] * PREFILL[only][3]
        key = "all" if only is None else PREFILL[only][0]
        out[key] = {"us": round(ms * 1000, 2), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1),
                    "pct_of_2.5PF": round(100 * fl / (ms * 1e-3) / 2.5e15, 2)}
        del g
    return out


def cpu_baseline(target_s=10.0):
    """The CPU oracle on the same layer at N=1, repeated to ~target_s of work."""
    import oracle
    import synth
    mats = []
    for i, (name, wt, m, k) in enumerate(synth.QWEN3_4B_LAYER):
        data, scales = synth.weights(wt, m, k, synth.rng_for(1, i))
        mats.append((wt, data, scales, m, k))
    xs = {k: synth.activations(1, k, synth.rng_for(1, 99, k)) for k in (2560, 4096, 9728)}
    layer_bytes = sum(layer_call_bytes(1).values())
    reps, t = 0, 0.0
    t0 = time.perf_counter()
    while t < target_s:
        for wt, data, scales, m, k in mats:
            oracle.gemm(wt, data, scales, m, k, xs[k])
        reps += 1
        t = time.perf_counter() - t0
    res = {"value": layer_bytes * reps / t / 1e9, "unit": "GB/s", "cores": oracle.last_threads(),
           "kind": "oracle", "cpu_model": _cpu_model(),
           "sample": f"the full decode layer (7 projections, N=1) {reps} times, {t:.1f} s; "
                     f"oracle = plain C dequant + fp64 dot, OpenMP over rows"}
    res["extras"] = cpu_extras(mats, xs)
    return res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed(fn, budget_s):
    """Median of up to 3 timed runs after one warm-up, stopping once budget_s is spent."""
    fn()
    ts = []
    t_end = time.perf_counter() + budget_s
    while len(ts) < 3 and (not ts or time.perf_counter() < t_end):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[len(ts) // 2]


def cpu_extras(mats, xs, budget_s=1.5):
    """The oracle on the other workloads, each bounded to about budget_s: the layer at
    N=1 on one thread and at N=32 on every core, the 1024x1024 Q4_K call, the 512-token
    prefill on a sample of 256 output rows, and NVFP4 16384x8192 at N=1."""
    import oracle
    import synth
    out = {}
    t1 = _timed(lambda: [oracle.gemm(wt, d, sc, m, k, xs[k], nthreads=1) for wt, d, sc, m, k in mats], budget_s)
    out["layer_n1_one_thread"] = {"ms": round(1e3 * t1, 2),
                                  "GB/s": round(sum(layer_call_bytes(1).values()) / t1 / 1e9, 3)}
    x32 = {k: synth.activations(32, k, synth.rng_for(1, 98, k)) for k in (2560, 4096, 9728)}
    t32 = _timed(lambda: [oracle.gemm(wt, d, sc, m, k, x32[k]) for wt, d, sc, m, k in mats], budget_s)
    out["layer_n32"] = {"ms": round(1e3 * t32, 2), "GB/s": round(sum(layer_call_bytes(32).values()) / t32 / 1e9, 3),
                        "threads": oracle.last_threads()}
    d0, _ = synth.weights(synth.Q4_K, 1024, 1024, synth.rng_for(0, 0))
    x0 = synth.activations(1, 1024, synth.rng_for(0, 1))
    t0 = _timed(lambda: oracle.gemm(synth.Q4_K, d0, None, 1024, 1024, x0), budget_s)
    out["q4k_1024x1024_n1"] = {"us": round(1e6 * t0, 1)}
    wt, d, sc, m, k = mats[4]   # the gate matrix, Q4_K 9728x2560
    xp = synth.activations(512, k, synth.rng_for(3, 10))
    rows = np.arange(0, m, m // 256)[:256]
    tp = _timed(lambda: oracle.gemm(wt, d, sc, m, k, xp, rows=rows), budget_s)
    out["prefill_512_q4k_9728x2560_256_rows"] = {"ms": round(1e3 * tp, 2),
                                                 "GFLOP/s": round(2 * 512 * len(rows) * k / tp / 1e9, 2)}
    dn, sn = synth.weights(synth.NVFP4, 16384, 8192, synth.rng_for(4, 0))
    xn = synth.activations(1, 8192, synth.rng_for(4, 10, 1))
    tn = _timed(lambda: oracle.gemm(synth.NVFP4, dn, sn, 16384, 8192, xn), budget_s)
    out["nvfp4_16384x8192_n1"] = {"ms": round(1e3 * tn, 2),
                                  "GB/s": round(call_bytes(synth.NVFP4, 16384, 8192, 1) / tn / 1e9, 3)}
    return out


CAL_BYTES = 1 << 30   # bytes read (and written) by one calibration copy


def calibration_copy(reps=3):
    """A plain elementwise copy of known size (torch.neg over 1 GiB of fp32, so
    1 GiB read and 1 GiB written, cold), run inside a counter-collection run
    beside the kernel: the ratio of what FETCH_SIZE / WRITE_SIZE report for it
    to its known byte counts scales the kernel's counters to bytes."""
    import torch
    bufs = [torch.ones(CAL_BYTES // 4, dtype=torch.float32, device="cuda") for _ in range(2 * reps)]
    torch.cuda.synchronize()
    for i in range(reps):
        torch.neg(bufs[2 * i], out=bufs[2 * i + 1])
    torch.cuda.synchronize()
    del bufs


def _counter_means(path, counter):
    """{kernel name: [per-dispatch values]} for one counter of a rocprofv3 counter CSV."""
    import csv
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def pmc_summary(kernel, fetch_csv, write_csv):
    """Turn two counter runs of `bench.py --kernel K` (FETCH_SIZE, then WRITE_SIZE)
    into HBM bytes per launch of K's kernel, scaled by the calibration copy, and
    store them in profiles/traffic_<K>.json keyed by the kernel sources' hash."""
    res = {"kernel_call": kernel, "kernel_source_sha": kernel_source_sha()}
    total = 0.0
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = _counter_means(path, counter)
        qg = {k: v for k, v in vals.items() if "qg::" in k}
        name = max(qg, key=lambda k: len(qg[k]))   # the kernel the graph replays
        cal = [v for k, vs in vals.items() if "neg" in k for v in vs]
        kib = float(np.median(qg[name]))
        cal_kib = float(np.median(cal))
        scale = (CAL_BYTES / 1024.0) / cal_kib
        res[counter] = {"kernel": name, "dispatches": len(qg[name]), "kib_per_dispatch": round(kib, 1),
                        "calibration_kib": round(cal_kib, 1), "scale": round(scale, 4),
                        "bytes_per_launch": round(kib * 1024.0 * scale)}
        total += kib * 1024.0 * scale
    res["bytes_per_launch"] = round(total)
    res["algorithmic_bytes"] = layer_call_bytes(1)[kernel]
    out = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res))


def load_traffic(sha):
    p = os.path.join(ROOT, "profiles", "traffic_pair.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != sha:
        return None
    return t.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=720)
    ap.add_argument("--warmup", type=int, default=72)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-n32", action="store_true", help="skip the N=32 pass")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-GEMM pass")
    ap.add_argument("--no-nvfp4", action="store_true", help="skip the NVFP4 large-shape pass")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 large-shape pass")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the read-stream ceiling")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--layout", choices=("tiles", "rows"), default="tiles",
                    help="weights in 16-row tiles (qg_pack_tiles) or in the row layout as stored")
    ap.add_argument("--no-rows", action="store_true", help="skip the row-layout N=1 comparison")
    ap.add_argument("--kernel", choices=KERNELS, default=None,
                    help="profile mode: replay only this call over the 36-layer rotation")
    ap.add_argument("--tokens", type=int, default=1, help="tokens per call in --kernel mode")
    ap.add_argument("--calibrate", action="store_true",
                    help="--kernel mode: also run the known-size copy that scales HBM counters")
    ap.add_argument("--prefill-call", choices=[p[0] for p in PREFILL], default=None,
                    help="profile mode: replay only this prefill call (its rotated copies)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two counter runs of --kernel K into profiles/traffic_K.json")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.kernel or "pair", *args.pmc_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the product is a single-GPU kernel library)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gemm_q4_q5_amd as qg
    qg.lib()   # fails loudly if the HIP library is not built
    torch.cuda.set_device(0)
    if args.prefill_call:
        replay_prefill(args.prefill_call, args.steps, args.warmup)
        return

    layers = build_layers(LAYERS, layout=args.layout)
    if args.kernel:
        n = args.tokens
        B = Buffers(n)
        for _, fn in layer_calls(layers[0], B, n):
            fn()
        gk = _capture(layers, B, n, only=args.kernel)
        reps = max(1, args.steps // LAYERS)
        ms = _time_graph(gk, reps, max(1, args.warmup // LAYERS))
        us = 1000.0 * ms / (reps * LAYERS)
        b = layer_call_bytes(n)[args.kernel]
        if args.calibrate:
            calibration_copy()
        print(json.dumps({"kernel": args.kernel, "tokens": n, "launches": reps * LAYERS,
                          "us_per_launch": round(us, 3), "GB/s": round(b / (us * 1e3), 1),
                          "algorithmic_bytes": b}))
        return
    r1 = time_layer(layers, 1, args.steps, args.warmup)
    bytes1 = layer_call_bytes(1)
    step_bytes = sum(bytes1.values())
    ms = r1["ms_per_step"]
    value = step_bytes / (ms * 1e-3) / 1e9
    gbs = lambda b, us: round(b / (us * 1e3), 1)

    res = {
        "metric": "achieved HBM GB/s (% of peak) for Q4_K GEMV, Qwen3-4B shapes, N=1 and N=32",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": r1["steps"],
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16 x 4/6-bit weights, f32 accumulate",
        "data": "synthetic (seeded; Q4_K_M value distributions)",
        "config": {"workload": "Qwen3-4B-shaped decode layer: QKV triple (Q4_K,Q4_K,Q6_K) + "
                               "Wo Q4_K with residual + gate/up Q4_K pair + down Q6_K; K=2560 "
                               "hidden, 36 distinct layers rotated (cold)", "tokens": 1,
                   "bytes_per_step": step_bytes,
                   "weight_layout": "16-row tiles (qg_pack_tiles, same superblocks and bits)"
                   if args.layout == "tiles" else "rows as stored"},
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "tok_s_equiv_projections": round(1000.0 / (LAYERS * ms), 1),
    }
    st = r1["step_stats_ms"]
    res["step_stats"] = {"replays": st["replays"], "steps_per_replay": r1["steps"],
                         **{f"{k}_GB/s": round(step_bytes / (st[k] * 1e-3) / 1e9, 1) for k in ("median", "min", "max")},
                         **{f"{k}_ms_per_step": round(st[k], 5) for k in ("median", "min", "max")}}
    ku = r1["kernel_us"]
    res["kernels_n1"] = {k: {"us": round(v["median"], 3), "us_min": round(v["min"], 3), "us_max": round(v["max"], 3),
                             "GB/s": gbs(bytes1[k], v["median"])} for k, v in ku.items()}
    sha = kernel_source_sha()
    pk = ku["pair"]
    ach = bytes1["pair"] / (pk["median"] * 1e3)
    res["roofline"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                       "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                       "traffic": load_traffic(sha),
                       "achieved_min": gbs(bytes1["pair"], pk["max"]), "achieved_max": gbs(bytes1["pair"], pk["min"]),
                       "replays": pk["replays"],
                       "kernel": f"qgemv_pair, two Q4_K 9728x2560, one token, {args.layout} layout "
                                 "(the MFMA product kernel, one launch per call)",
                       "algorithmic_bytes": bytes1["pair"], "kernel_source_sha": sha}
    res["q4k_gemv"] = time_q4k_single(layers)
    if not args.no_ceiling:
        ceil = time_read_ceiling(layers)
        res["read_ceiling"] = ceil
        res["pct_of_read_ceiling"] = round(100.0 * value / ceil["layer"]["GB/s"] * ceil["layer"]["bytes"]
                                           / step_bytes, 2)
    if not args.no_n32:
        r32 = time_layer(layers, 32, max(LAYERS, args.steps), LAYERS)
        b32 = layer_call_bytes(32)
        v32 = sum(b32.values()) / (r32["ms_per_step"] * 1e-3) / 1e9
        s32 = r32["step_stats_ms"]
        res["n32"] = {"value": round(v32, 2), "unit": "GB/s", "pct_of_peak": round(100 * v32 / PEAK_HBM_GBS, 2),
                      "ms_per_step": round(r32["ms_per_step"], 5),
                      "median_ms_per_step": round(s32["median"], 5), "min_ms_per_step": round(s32["min"], 5),
                      "max_ms_per_step": round(s32["max"], 5),
                      "kernels": {k: {"us": round(v["median"], 3), "us_min": round(v["min"], 3),
                                      "us_max": round(v["max"], 3), "GB/s": gbs(b32[k], v["median"])}
                                  for k, v in r32["kernel_us"].items()}}
    if args.layout == "tiles" and not args.no_rows:
        del layers
        torch.cuda.empty_cache()
        rows = build_layers(LAYERS, layout="rows")
        rr = time_layer(rows, 1, args.steps, args.warmup)
        res["rows_layout_n1"] = {"value": round(step_bytes / (rr["ms_per_step"] * 1e-3) / 1e9, 2), "unit": "GB/s",
                                 "ms_per_step": round(rr["ms_per_step"], 5),
                                 "median_ms_per_step": round(rr["step_stats_ms"]["median"], 5),
                                 "kernels": {k: round(v["median"], 3) for k, v in rr["kernel_us"].items()}}
        res["rows_layout_n1"]["q4k_gemv"] = time_q4k_single(rows)
        del rows
        torch.cuda.empty_cache()
    if not args.no_prefill:
        res["prefill_n512"] = time_prefill()
        res["prefill_n512_rows_layout"] = time_prefill(layout="rows")
    if not args.no_nvfp4:
        res["nvfp4_large"] = time_scaled(qg.NVFP4)
    if not args.no_fp8:
        res["fp8_large"] = time_scaled(qg.FP8)
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
