#!/usr/bin/env python3
"""Benchmark of the quantized-weight prefill matmul on one MI355X.

Workload (the timed step): one prefill forward's matmuls over a full 28-layer
7B weight set — per layer q, o (3584×3584), k, v (512×3584), gate, up
(18944×3584) in Q4_K and down (3584×18944) in Q6_K — at M = 2048 tokens with
f16 N(0,1) activations, Y = X·Wᵀ on the persistent f16 cache.  The weights
that share an input are stored and cached as one matrix each (q|k|v, N = 4608;
gate|up, N = 37888; Fucina "Eager GPU Offload Without A Compute Graph",
quantized linears: a shared-input batch), so a step is 112 GEMMs that compute
the 196 products; the same forward as 196 single GEMMs (row views of the same
caches) is timed beside it.  Before the steps, the load phase decodes all 196
weights into the cache (the method's one-time dequant; timed, reported as
GB/s).  After them, the fused dequant-in-GEMM is timed on the same forward,
and the fused-vs-cache crossover in M is swept on Llama-3.1-8B-like shapes.

Inputs are synthetic and seeded (the pages' real GGUF models are not
available): the 4.2 GB weight set is drawn on the device with torch's seeded
generator, same distributions as the numpy generator the tests use.

Prints human-readable tables on stderr and ONE JSON line on stdout.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

METRIC = "prefill GEMM TFLOP/s + matmul tok/s (7B Q4_K, M=2048); dequant GB/s"
PEAK_F16_TFLOPS = 2500.0     # MI355X dense f16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
# The dominant kernel of the step: the grouped gate|up GEMM (28 of the 112
# calls, ~58% of the matmul time): gemm_kernel<256, 256, f16> on 1184 whole
# tiles (one mq_gemm_f16cache call, no K split).
ROOFLINE_GROUP = "gu"
ROOFLINE_N, ROOFLINE_K = 37888, 3584
ROOFLINE_KERNEL = "gemm_kernel<256, 256, f16> (mq_gemm_f16cache, gate|up 37888x3584, 1184 whole tiles)"
# Measured HBM traffic of that call (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled
# by a plain copy of known size) with the hash of the GEMM source it was taken
# on; reported only while the source is unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_f16cache_gateup_7b_m2048_traffic.md")
# Shared-input groups of a layer: (group, member matrices in row order)
GROUPS = (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gu", ("gate", "up")), ("down", ("down",)))
GEMM_SOURCES = ("quantized_weight_prefill_q4_amd/csrc/gemm_kernel.h",
                "quantized_weight_prefill_q4_amd/csrc/gemm_fused_rb.h",
                "quantized_weight_prefill_q4_amd/csrc/gemm.hip",
                "quantized_weight_prefill_q4_amd/csrc/mq_device.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--M", type=int, default=2048)
    p.add_argument("--layers", type=int, default=synth.N_LAYERS_7B)
    p.add_argument("--load-reps", type=int, default=3)
    p.add_argument("--fused-steps", type=int, default=5)
    p.add_argument("--grouped-steps", type=int, default=5,
                   help="steps of the fused grouped forward (q|k|v, gate|up as one GEMM each); 0 = skip")
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-formats", action="store_true",
                   help="skip the per-format decode / fused table")
    p.add_argument("--no-xf32", action="store_true",
                   help="skip the f32-activation table")
    p.add_argument("--mmq-steps", type=int, default=3,
                   help="steps of the int8-path forward (0 = skip)")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=2048,
                   help="token rows of the oracle sample")
    p.add_argument("--cpu-layers", type=int, default=4,
                   help="layers (7 matrices each) of the oracle sample")
    p.add_argument("--only-shape", default=None,
                   help="profiling aid: run only this 7B matrix's (or group qkv, gate_up) cache GEMM --steps times")
    p.add_argument("--only-fused", default=None,
                   help="profiling aid: run only this 7B matrix's fused GEMM --steps times")
    p.add_argument("--only-mmq", default=None,
                   help="time only this 7B shape on the int8 path (for counter runs)")
    p.add_argument("--only-small-m", action="store_true",
                   help="profiling aid: M = 128 Q4_K GEMMs (cache and fused) on 4096x4096 with "
                        "K splits 0, 1, 2, 4, 8, 16 and on 14336x4096, 30 calls each")
    p.add_argument("--only-sweep", action="store_true",
                   help="only the fused-vs-cache sweep (for a kernel trace of its calls); "
                        "prints its JSON")
    p.add_argument("--only-load", action="store_true",
                   help="profiling aid: run only the batched decode of the 7B weight set --steps times")
    p.add_argument("--calib-copy", action="store_true",
                   help="profiling aid: run only a plain 1 GiB device copy --steps times "
                        "(the reference for the HBM byte counters)")
    return p.parse_args()


def gemm_source_hash() -> str:
    """Hash of the GEMM sources' code: comments and whitespace are dropped, so
    an edit of a comment keeps the stored counters valid and any edit of the
    code does not.  (The sources hold no string literal with a comment
    marker in it.)"""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """(bytes per call, note) from the committed counter summary, or (None, why)."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None, "no counter summary"
    vals = {}
    for line in text.splitlines():
        if line.startswith("traffic_bytes_per_call:") or line.startswith("source_sha256_16:"):
            k, v = line.split(":", 1)
            vals[k] = v.strip()
    if vals.get("source_sha256_16") != gemm_source_hash():
        return None, "GEMM source changed since the counters were taken"
    return int(vals["traffic_bytes_per_call"]), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"


def run_only_shape(torch, mq, name, steps, dev):
    shapes = {nm: (f, n, k) for nm, f, n, k in synth.LAYER_7B}
    shapes.update(qkv=(synth.Q4_K, 4608, 3584), gate_up=(synth.Q4_K, 37888, 3584))
    fmt, N, K = shapes[name]
    M = 2048
    q = synth.weights_device(fmt, 1, N, K, dev)
    cache = mq.dequant_to_f16(q, fmt, N, K)
    x = synth.activations_device(2, M, K, dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws_n = mq.workspace_bytes(0, M, N, K)
    ws = torch.empty(max(1, ws_n // 4), dtype=torch.float32, device=dev)
    mq.gemm_f16cache(x, cache, K, out=y, ws=ws)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        ev[i].record()
        mq.gemm_f16cache(x, cache, K, out=y, ws=ws)
    ev[steps].record()
    torch.cuda.synchronize()
    us = statistics.median(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps))
    print(json.dumps({"only_shape": name, "M": M, "N": N, "K": K, "calls": steps + 1,
                      "median_call_us": round(us, 2),
                      "tflops": round(2.0 * M * N * K / us / 1e6, 1),
                      "algorithmic_bytes_per_call": M * K * 2 + N * K * 2 + M * N * 4}), flush=True)


def run_only_fused(torch, mq, name, steps, dev):
    fmt, N, K = next((f, n, k) for nm, f, n, k in synth.LAYER_7B if nm == name)
    M = 2048
    q = synth.weights_device(fmt, 1, N, K, dev)
    x = synth.activations_device(2, M, K, dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, mq.workspace_bytes(fmt, M, N, K) // 4), dtype=torch.float32, device=dev)
    mq.gemm_fused(x, q, fmt, N, K, out=y, ws=ws)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        ev[i].record()
        mq.gemm_fused(x, q, fmt, N, K, out=y, ws=ws)
    ev[steps].record()
    torch.cuda.synchronize()
    us = statistics.median(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps))
    print(json.dumps({"only_fused": name, "format": fmt, "M": M, "N": N, "K": K,
                      "calls": steps + 1, "median_call_us": round(us, 2),
                      "tflops": round(2.0 * M * N * K / us / 1e6, 1)}), flush=True)


def run_only_mmq(torch, mq, name, steps, dev):
    """One 7B shape on the int8 path at M = 2048 (activations quantized once
    beforehand), for counter runs of the MMQ kernel alone."""
    fmt, N, K = next((f, n, k) for nm, f, n, k in synth.LAYER_7B if nm == name)
    M = 2048
    q = synth.weights_device(fmt, 1, N, K, dev)
    g = torch.Generator(device=dev)
    g.manual_seed(2)
    x = torch.randn((M, K), generator=g, device=dev, dtype=torch.float32)
    xq, ds = mq.quantize_q8_1(x)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws_n = mq.mmq_workspace_bytes(fmt, M, N, K)
    ws = torch.empty(max(1, ws_n // 4), dtype=torch.float32, device=dev)
    mq.gemm_mmq(xq, ds, q, fmt, N, K, out=y, ws=ws)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        ev[i].record()
        mq.gemm_mmq(xq, ds, q, fmt, N, K, out=y, ws=ws)
    ev[steps].record()
    torch.cuda.synchronize()
    us = statistics.median(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps))
    print(json.dumps({"only_mmq": name, "M": M, "N": N, "K": K, "calls": steps + 1,
                      "median_call_us": round(us, 2),
                      "tops": round(2.0 * M * N * K / us / 1e6, 1)}), flush=True)


def run_only_small_m(torch, mq, dev):
    """M = 128 GEMMs for counter runs: per (shape, path, split) 30 calls in a
    fixed order, so the dispatches of a trace can be attributed in order."""
    M, fmt = 128, synth.Q4_K
    order = []
    for N, K in ((4096, 4096), (14336, 4096)):
        q = synth.weights_device(fmt, 1, N, K, dev)
        c = mq.dequant_to_f16(q, fmt, N, K)
        x = synth.activations_device(2, M, K, dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        for path in ("fused", "cache"):
            for split in ((0, 1, 2, 4, 8, 16) if N == 4096 else (0,)):
                wsb = mq.workspace_bytes(fmt if path == "fused" else 0, M, N, K, split)
                ws = torch.empty(max(1, wsb // 4), dtype=torch.float32, device=dev)
                for _ in range(30):
                    if path == "fused":
                        mq.gemm_fused(x, q, fmt, N, K, split_k=split, out=y, ws=ws)
                    else:
                        mq.gemm_f16cache(x, c, K, split_k=split, out=y, ws=ws)
                torch.cuda.synchronize()
                order.append(f"{path} {N}x{K} split {split}")
    print(json.dumps({"only_small_m": order, "calls_each": 30}), flush=True)


def run_calib_copy(torch, steps, dev):
    n = 1 << 28   # 2^28 f32 = 1 GiB read + 1 GiB written per copy
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": 4 * n, "calib_copy_bytes_written": 4 * n,
                      "copies": steps}), flush=True)


# ---------------------------------------------------------------------------
# GPU phases
# ---------------------------------------------------------------------------

def make_weights(torch, mq, layers, dev):
    """Quantized weights on the device plus their (empty) f16 caches, per
    layer and shared-input group (GROUPS) one buffer each, the matrices row
    slices of it.  Returns (W, G): W[layer][matrix] = (fmt, N, K, q, cache)
    with views, G[layer][group] = (fmt, N, K, q, cache) with the buffers."""
    W, G = [], []
    spec = {name: (mi, fmt, N, K) for mi, (name, fmt, N, K) in enumerate(synth.LAYER_7B)}
    for L in range(layers):
        row, grp = {}, {}
        for gname, members in GROUPS:
            fmt, K = spec[members[0]][1], spec[members[0]][3]
            n_tot = sum(spec[m][2] for m in members)
            qbuf = torch.empty((n_tot, mq.row_bytes(fmt, K)), dtype=torch.uint8, device=dev)
            cbuf = torch.empty((n_tot, mq.cache_ld(K)), dtype=torch.float16, device=dev)
            r0 = 0
            for m in members:
                mi, f, N, _ = spec[m]
                qbuf[r0:r0 + N] = synth.weights_device(f, 1000 * L + mi, N, K, dev)
                row[m] = (f, N, K, qbuf[r0:r0 + N], cbuf[r0:r0 + N])
                r0 += N
            grp[gname] = (fmt, n_tot, K, qbuf, cbuf)
        W.append({m: row[m] for m, *_ in synth.LAYER_7B})
        G.append(grp)
    torch.cuda.synchronize()
    return W, G


def load_phase(torch, mq, W, reps):
    """Decode every weight into its cache as a model load does: one batched
    library call over all 196 weights (launches of 16 jobs).

    Returns (best GPU ms of the batched call over `reps` replays of a HIP
    graph holding it, best ms over `reps` eager calls, per-call records of one
    extra pass of single-matrix calls with HIP events around each call).  The
    eager figure also holds the binding's host-side check of the 196 jobs,
    during which the GPU idles after the first event (~0.5 ms)."""
    calls = [(name, fmt, N, K, q, cache) for row in W for name, (fmt, N, K, q, cache) in row.items()]
    jobs = [(q, fmt, N, K, cache) for name, fmt, N, K, q, cache in calls]

    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    eager = min(timed(lambda: mq.dequant_to_f16_batch(jobs)) for _ in range(reps))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mq.dequant_to_f16_batch(jobs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mq.dequant_to_f16_batch(jobs)
    g.replay()
    torch.cuda.synchronize()
    best = min(timed(g.replay) for _ in range(reps))
    del g
    evs = []
    for name, fmt, N, K, q, cache in calls:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        mq.dequant_to_f16(q, fmt, N, K, out=cache)
        b.record()
        evs.append((name, fmt, N, K, q.numel(), a, b))
    torch.cuda.synchronize()
    return best, eager, [(name, fmt, N, K, qb, a.elapsed_time(b)) for name, fmt, N, K, qb, a, b in evs]


def forward(mq, W, xa, xf, ys, ws, events=None, only=None):
    """One prefill forward: 196 cache GEMMs (events[i] recorded before call i);
    with `only`, just the calls of those matrices."""
    i = 0
    for row in W:
        for name, (fmt, N, K, q, cache) in row.items():
            if only is not None and name not in only:
                continue
            if events is not None:
                events[i].record()
            mq.gemm_f16cache(xf if name == "down" else xa, cache, K, out=ys[name], ws=ws)
            i += 1
    if events is not None:
        events[i].record()


def forward_grouped(mq, G, xa, xf, yg, ws, only=None):
    """One prefill forward as 4 GEMMs per layer (q|k|v, o, gate|up, down);
    with `only`, just the calls of those groups."""
    for grp in G:
        for gname, (fmt, N, K, q, cache) in grp.items():
            if only is not None and gname not in only:
                continue
            mq.gemm_f16cache(xf if gname == "down" else xa, cache, K, out=yg[gname], ws=ws)


def forward_fused(mq, W, xa, xf, ys, ws):
    for row in W:
        for name, (fmt, N, K, q, cache) in row.items():
            mq.gemm_fused(xf if name == "down" else xa, q, fmt, N, K, out=ys[name], ws=ws)


def sweep(torch, mq, dev, log_rows):
    """Fused vs cache GEMM time per (shape, M), GPU time from graph replays
    (graph_us) of 12 calls that rotate weight copies over > 512 MB; every M of
    the sweep and of its refinement list is measured."""
    out = {}
    for si, (name, fmt, N, K) in enumerate(synth.SWEEP_8B):
        q0 = synth.weights_device(fmt, 5000 + si, N, K, dev)
        cache0 = mq.dequant_to_f16(q0, fmt, N, K)
        nc = max(3, -(-512 * 2 ** 20 // (cache0.numel() * 2)))
        nq = max(3, -(-512 * 2 ** 20 // q0.numel()))
        caches = [cache0] + [cache0.clone() for _ in range(nc - 1)]
        qs = [q0] + [q0.clone() for _ in range(nq - 1)]
        x = synth.activations_device(6000 + si, max(synth.SWEEP_M), K, dev)
        res = {}

        def measure(M, record=True):
            xm = x[:M]
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            ws_c = torch.empty(max(1, mq.workspace_bytes(0, M, N, K) // 4), dtype=torch.float32, device=dev)
            ws_f = torch.empty(max(1, mq.workspace_bytes(fmt, M, N, K) // 4), dtype=torch.float32, device=dev)
            reps = 12
            t = {
                "cache": graph_us(torch, [lambda r=r: mq.gemm_f16cache(xm, caches[r % nc], K, out=y, ws=ws_c)
                                          for r in range(reps)], check=lambda: y.clone()),
                "fused": graph_us(torch, [lambda r=r: mq.gemm_fused(xm, qs[r % nq], fmt, N, K, out=y, ws=ws_f)
                                          for r in range(reps)], check=lambda: y.clone()),
            }
            if not record:
                return
            flops = 2.0 * M * N * K
            res[M] = {"cache_us": round(t["cache"], 2), "fused_us": round(t["fused"], 2),
                      "cache_tflops": round(flops / t["cache"] / 1e6, 1),
                      "fused_tflops": round(flops / t["fused"] / 1e6, 1)}
            log_rows.append(f"  {name:16s} M={M:5d}  cache {t['cache']:9.1f} us ({res[M]['cache_tflops']:7.1f} TF/s)"
                            f"  fused {t['fused']:9.1f} us ({res[M]['fused_tflops']:7.1f} TF/s)")

        def crossover():
            ms = sorted(res)
            wins = [M for M in ms if res[M]["cache_us"] < res[M]["fused_us"]]
            if not wins:
                return f">{max(ms)}"
            if wins[0] == ms[0]:
                return f"<={ms[0]}"
            return str(wins[0])

        ms = sorted(set(synth.SWEEP_M) | set(synth.SWEEP_REFINE))
        # a shape's first timed calls ran slow (freshly copied weights: up to
        # 7 us above the kernel sum at M = 128), so its first point is run
        # once untimed
        measure(ms[0], record=False)
        for M in ms:
            measure(M)
        cross = crossover()
        # points where the two paths are within 3% of each other: there the
        # order can flip from run to run (box, clock), and so can the crossover
        ties = [m for m in sorted(res)
                if abs(res[m]["cache_us"] - res[m]["fused_us"])
                <= 0.03 * min(res[m]["cache_us"], res[m]["fused_us"])]
        out[name] = {"crossover_M": cross, "within_3pct_M": ties,
                     "by_M": {m: res[m] for m in sorted(res)}}
        del caches, qs, cache0, q0
        torch.cuda.empty_cache()
    return out


def graph_us(torch, fns, replays=7, check=None):
    """GPU time per call (us) of the zero-argument calls `fns`, each of which
    enqueues library work on the current stream: all of them are captured into
    one HIP graph, which is replayed once untimed and then `replays` times
    between a pair of HIP events each.  Host launch gaps are not in the time,
    the GPU's own dispatch between kernels is.  Returns the median over replays
    of (replay time / len(fns)).  check(): called after an eager run of the
    calls and again after the timed replays, to confirm the graph computes what
    the eager calls did (the library records no memset nodes)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for fn in fns:
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = check() if check is not None else None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in fns:
            fn()
    g.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(replays)]
    for a, b in evs:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    if check is not None:
        got = check()
        if not torch.equal(got, ref):
            raise RuntimeError("graph replay computed other results than the eager calls")
    del g
    return statistics.median(a.elapsed_time(b) for a, b in evs) * 1e3 / len(fns)


def _median_us(torch, fn, reps, warm=2):
    """GPU time per call (us) of fn(r), r = 0 .. reps - 1, from graph replays
    (graph_us); `warm` is kept for the callers' signature (the graph's first
    replay is the warm-up)."""
    return graph_us(torch, [lambda r=r: fn(r) for r in range(reps)])


def hbm_fill_gbs(torch, dev, nbytes=4 << 30, reps=5):
    """A plain device fill of `nbytes` (torch zero_): the write-only rate,
    beside the copy, for a pass like the decode whose bytes are three
    quarters writes."""
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    us = graph_us(torch, [lambda: dst.zero_() for _ in range(reps)])
    del dst
    torch.cuda.empty_cache()
    return nbytes / us / 1e3


def hbm_copy_gbs(torch, dev, nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of `nbytes` (torch copy_), GB/s counting
    the bytes read plus the bytes written: the practical HBM ceiling the
    decode is judged against, measured in the same run."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.fill_(1)
    us = graph_us(torch, [lambda: dst.copy_(src) for _ in range(reps)])
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * nbytes / us / 1e3


def formats_table(torch, mq, dev, log_rows):
    """Every weight format on one shape (N = 14336, K = 4096, the Llama-3.1-8B
    gate/up projection): load-time decode GB/s (quantized bytes read + f16
    cache written), the fused GEMM and the int8 product at M = 128 and 2048
    (activations quantized beforehand; the quantize time is listed once),
    beside the cache GEMM on the same shape.  Weight copies rotate over
    > 512 MB."""
    N, K = 14336, 4096
    x = synth.activations_device(6100, 2048, K, dev)
    xq, xds = mq.quantize_q8_1(x.float())
    out = {}
    cache_us = {}
    quant_us = {}
    for fi, (fname, fmt) in enumerate(sorted(mq.FORMATS.items(), key=lambda kv: kv[1])):
        q0 = synth.weights_device(fmt, 6200 + fi, N, K, dev)
        nq = max(3, -(-512 * 2 ** 20 // q0.numel()))
        qs = [q0] + [q0.clone() for _ in range(nq - 1)]
        ld = mq.cache_ld(K)
        caches = [torch.empty((N, ld), dtype=torch.float16, device=dev) for _ in range(5)]
        t_deq = _median_us(torch, lambda r: mq.dequant_to_f16(qs[r % nq], fmt, N, K,
                                                              out=caches[r % 5]), 12)
        rec = {"quant_bytes": int(q0.numel()),
               "dequant_us": round(t_deq, 2),
               "dequant_gbs": round((q0.numel() + 2 * N * ld) / t_deq / 1e3, 1)}
        for M in (128, 2048):
            xm = x[:M]
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            ws = torch.empty(max(1, mq.workspace_bytes(fmt, M, N, K) // 4), dtype=torch.float32,
                             device=dev)
            t = _median_us(torch, lambda r: mq.gemm_fused(xm, qs[r % nq], fmt, N, K, out=y, ws=ws), 12)
            rec[f"fused_m{M}_us"] = round(t, 2)
            rec[f"fused_m{M}_tflops"] = round(2.0 * M * N * K / t / 1e6, 1)
            wsm = torch.empty(max(1, mq.mmq_workspace_bytes(fmt, M, N, K) // 4),
                              dtype=torch.float32, device=dev)
            qm, dm = xq[:M], xds[:M]
            t = _median_us(torch, lambda r: mq.gemm_mmq(qm, dm, qs[r % nq], fmt, N, K, out=y, ws=wsm), 12)
            rec[f"mmq_m{M}_us"] = round(t, 2)
            rec[f"mmq_m{M}_tops"] = round(2.0 * M * N * K / t / 1e6, 1)
            if M not in quant_us:
                xm32 = x[:M].float()
                quant_us[M] = _median_us(torch, lambda r: mq.quantize_q8_1(xm32, xq=qm, ds=dm), 12)
            if M not in cache_us:
                wsc = torch.empty(max(1, mq.workspace_bytes(0, M, N, K) // 4), dtype=torch.float32,
                                  device=dev)
                cache_us[M] = _median_us(torch, lambda r: mq.gemm_f16cache(
                    xm, caches[r % 5], K, out=y, ws=wsc), 12)
        out[fname] = rec
        log_rows.append(f"  {fname:5s} {rec['quant_bytes'] / 2 ** 20:6.1f} MiB  decode {t_deq:7.1f} us "
                        f"{rec['dequant_gbs']:6.0f} GB/s   fused M=128 {rec['fused_m128_us']:7.1f} us "
                        f"M=2048 {rec['fused_m2048_us']:7.1f} us ({rec['fused_m2048_tflops']:6.1f} TF/s)"
                        f"   int8 M=128 {rec['mmq_m128_us']:7.1f} us M=2048 {rec['mmq_m2048_us']:7.1f} us"
                        f" ({rec['mmq_m2048_tops']:6.1f} TOP/s)")
        del qs, q0, caches
        torch.cuda.empty_cache()
    out["cache_gemm"] = {f"m{M}_us": round(t, 2) for M, t in cache_us.items()}
    out["quantize_q8_1"] = {f"m{M}_us": round(t, 2) for M, t in quant_us.items()}
    log_rows.append("  cache GEMM on the same shape: " +
                    ", ".join(f"M={M} {t:.1f} us ({2.0 * M * N * K / t / 1e6:.1f} TF/s)"
                              for M, t in cache_us.items()) +
                    "; activation quantize (f32 -> int8 blocks): " +
                    ", ".join(f"M={M} {t:.1f} us" for M, t in quant_us.items()))
    return out


def xf32_table(torch, mq, dev, log_rows):
    """f32 activations on the Llama-3.1-8B gate/up shape (N = 14336, K = 4096),
    for the f16 cache and the fused Q4_K GEMM, per M: the f32-activation entry
    point (in-tile rounding up to M = 64, else one convert pass into the
    workspace and the f16 kernel), against the caller converting X itself and
    calling the f16-activation entry point; that entry point alone for
    reference.  Weight copies rotate over > 512 MB."""
    N, K = 14336, 4096
    fmt = mq.FORMATS["q4_k"]
    q0 = synth.weights_device(fmt, 6300, N, K, dev)
    nq = max(3, -(-512 * 2 ** 20 // q0.numel()))
    qs = [q0] + [q0.clone() for _ in range(nq - 1)]
    caches = [mq.dequant_to_f16(q0, fmt, N, K)] + [None] * 4
    for i in range(1, 5):
        caches[i] = caches[0].clone()
    g = torch.Generator(device=dev)
    g.manual_seed(6301)
    x32 = torch.randn((2048, K), generator=g, device=dev, dtype=torch.float32)
    x16 = torch.empty((2048, K), dtype=torch.float16, device=dev)
    out = {}
    for M in (64, 128, 512, 2048):
        xm32, xm16 = x32[:M], x16[:M]
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        rec = {"convert_us": round(_median_us(torch, lambda r: mq.convert_f32_to_f16(xm32, out=xm16), 12), 2)}
        for path in ("cache", "fused"):
            def gemm(x, r, path=path):
                ws = wss[(path, x.dtype)]
                if path == "cache":
                    mq.gemm_f16cache(x, caches[r % 5], K, out=y, ws=ws)
                else:
                    mq.gemm_fused(x, qs[r % nq], fmt, N, K, out=y, ws=ws)
            wss = {}
            for dt, xf in ((torch.float16, False), (torch.float32, True)):
                b = mq.workspace_bytes(0 if path == "cache" else fmt, M, N, K, 0, x_f32=xf)
                wss[(path, dt)] = (torch.empty(b // 4, dtype=torch.float32, device=dev)
                                   if b else None)
            t16 = _median_us(torch, lambda r: gemm(xm16, r), 12)
            t32 = _median_us(torch, lambda r: gemm(xm32, r), 12)
            tcv = _median_us(torch, lambda r: (mq.convert_f32_to_f16(xm32, out=xm16), gemm(xm16, r)), 12)
            rec[path] = {"x16_us": round(t16, 2), "xf32_us": round(t32, 2),
                         "convert_then_x16_us": round(tcv, 2),
                         "xf32_tflops": round(2.0 * M * N * K / t32 / 1e6, 1)}
            how = "in-tile" if M <= 64 else "convert-first"
            log_rows.append(f"  {path:5s} M={M:5d}  f16 X {t16:8.1f} us   f32 X ({how}) {t32:8.1f} us"
                            f"   caller convert + f16 X {tcv:8.1f} us   (convert alone {rec['convert_us']:.1f} us)")
        out[M] = rec
    ms = sorted(out)
    for path in ("cache", "fused"):
        wins = [M for M in ms if out[M][path]["convert_then_x16_us"] < out[M][path]["xf32_us"]]
        out[f"{path}_convert_first_from_M"] = wins[0] if wins else None
    del qs, caches, x32, x16
    torch.cuda.empty_cache()
    return out


def mmq_forward(torch, mq, W, M, steps, dev):
    """The 196 GEMMs of the forward on the int8 path: per layer the four
    distinct inputs (q|k|v, o, gate|up, down; f32) are quantized once each to
    Q8_1-style blocks, then the seven products read the quantized weights
    directly.  Returns (median ms per step, median ms of its quantize calls)."""
    g = torch.Generator(device=dev)
    g.manual_seed(7003)
    xa = torch.randn((M, 3584), generator=g, device=dev, dtype=torch.float32)
    xf = torch.randn((M, 18944), generator=g, device=dev, dtype=torch.float32)
    qa, da = mq.quantize_q8_1(xa)
    qf, df = mq.quantize_q8_1(xf)
    ys = {n: torch.empty((M, N), dtype=torch.float32, device=dev) for n, _, N, _ in synth.LAYER_7B}
    wsb = max(mq.mmq_workspace_bytes(f, M, N, K) for _, f, N, K in synth.LAYER_7B)
    ws = torch.empty(max(1, wsb // 4), dtype=torch.float32, device=dev)

    def step(evq=None):
        for row in W:
            for name in ("q", "k", "v", "o", "gate", "up", "down"):
                fmt, N, K, q, _ = row[name]
                if name in ("q", "o", "gate", "down"):      # a new layer input
                    x, xq, ds = (xf, qf, df) if name == "down" else (xa, qa, da)
                    mq.quantize_q8_1(x, xq=xq, ds=ds)
                xq, ds = (qf, df) if name == "down" else (qa, da)
                mq.gemm_mmq(xq, ds, q, fmt, N, K, out=ys[name], ws=ws)

    step()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        evs[i].record()
        step()
    evs[steps].record()
    torch.cuda.synchronize()
    d = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    # the quantize calls alone, as in one step (4 per layer)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(len(W)):
        mq.quantize_q8_1(xa, xq=qa, ds=da)
        mq.quantize_q8_1(xa, xq=qa, ds=da)
        mq.quantize_q8_1(xa, xq=qa, ds=da)
        mq.quantize_q8_1(xf, xq=qf, ds=df)
    b.record()
    torch.cuda.synchronize()
    qms = a.elapsed_time(b)
    del xa, xf, qa, qf, ys, ws
    return statistics.median(d), qms


def vendor_table(torch, W, xa, xf, shape_us, reps=20):
    """The same 7B products through the vendor library (torch.mm, hipBLASLt:
    f16 inputs, f16 output, f32 accumulation) on layer 0's decoded caches,
    median of `reps` calls, next to this library's per-call medians from the
    instrumented forward (f32 output).  Context only: the library writes half
    the output bytes."""
    out = {}
    for name in ("q", "k", "gate", "down"):
        fmt, N, K, q, cache = W[0][name]
        x = xf if name == "down" else xa
        wt = cache[:, :K].t().contiguous()          # [K, N]: a plain NN product
        torch.mm(x, wt)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        for i in range(reps):
            evs[i].record()
            torch.mm(x, wt)
        evs[reps].record()
        torch.cuda.synchronize()
        us = statistics.median(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(reps))
        M = x.shape[0]
        out[name] = {"N": N, "K": K, "vendor_us": round(us, 2),
                     "vendor_tflops": round(2.0 * M * N * K / us / 1e6, 1),
                     "ours_us": round(shape_us[name], 2),
                     "ours_tflops": round(2.0 * M * N * K / shape_us[name] / 1e6, 1)}
        del wt
    torch.cuda.empty_cache()
    return out


FWD_ROWS = 64     # token rows of the timed forward's output sample
FWD_COLS = 256    # output columns (weight rows) per matrix


def forward_sample(torch, G, xa, xf, yg, M):
    """Host copy of part of what the last timed forward computed: for each of
    the last layer's four grouped GEMMs (every call of a group writes the same
    output buffer, layer by layer, so the buffers hold layer 27's products),
    FWD_ROWS token rows x FWD_COLS output columns of Y, the same rows of X,
    and the quantized bytes and f16-cache rows of the FWD_COLS weight rows.
    Rows and columns are seeded draws that include the first and the last."""
    g = np.random.default_rng(7004)
    rows = np.sort(np.concatenate([[0, M - 1], 1 + g.choice(M - 2, FWD_ROWS - 2, replace=False)]))
    torch.cuda.synchronize()
    ridx = torch.from_numpy(rows).to(xa.device)

    def bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    out = {"rows": rows, "x": {"a": bits(xa[ridx]), "f": bits(xf[ridx])}, "mats": {}}
    for name, (fmt, N, K, q, cache) in G[-1].items():
        cols = np.sort(np.concatenate([[0, N - 1], 1 + g.choice(N - 2, FWD_COLS - 2, replace=False)]))
        cidx = torch.from_numpy(cols).to(xa.device)
        out["mats"][name] = {
            "fmt": fmt, "N": N, "K": K, "cols": cols,
            "y": yg[name][ridx][:, cidx].cpu().numpy(),
            "q": q[cidx].cpu().numpy(),
            "cache": bits(cache[cidx, :K]),
        }
    return out


def check_forward_sample(sample):
    """The CPU leg's check of the timed forward (untimed): the oracle decodes
    the sampled weight rows from their quantized bytes (the cache rows must be
    bit-identical) and computes the sampled outputs in f64 (|dY| <= 1e-3.S +
    1e-5 per element).  Returns a summary for the JSON line."""
    import oracle

    worst = max_rel = 0.0
    cache_ok = True
    n = 0
    for name, d in sample["mats"].items():
        fmt, K, cols = d["fmt"], d["K"], d["cols"]
        w = oracle.dequant_ref(fmt, d["q"].reshape(-1), len(cols), K)
        cache_ok &= bool(np.array_equal(w, d["cache"]))
        x = sample["x"]["f" if name == "down" else "a"]
        Yref, S = oracle.gemm_ref(x, w, K)
        ok, r, _, mr = oracle.within_tolerance(d["y"], Yref, S)
        worst = max(worst, float(r))
        max_rel = max(max_rel, float(mr))
        n += d["y"].size
    return {"gemms": len(sample["mats"]), "layer": "last", "rows": int(len(sample["rows"])),
            "cols_per_gemm": FWD_COLS, "outputs_checked": n, "cache_bit_exact": cache_ok,
            "worst_err_over_tolerance": worst, "max_abs_err_over_S": max_rel,
            "pass": bool(cache_ok and worst <= 1.0)}


def fused_grouped_forward(torch, mq, G, xa, xf, steps, dev):
    """The fused forward on the grouped quantized weights (q|k|v as one
    4608-row Q4_K weight, gate|up as one 37888-row weight: the rows of a group
    are contiguous blocks of one format), four fused GEMMs per layer.
    Returns (median ms per step, min ms per step)."""
    M = xa.shape[0]
    yg = {g: torch.empty((M, N), dtype=torch.float32, device=dev)
          for g, (f, N, K, q, c) in G[0].items()}
    wsb = max(mq.workspace_bytes(f, M, N, K) for f, N, K, q, c in G[0].values())
    ws = torch.empty(max(1, wsb // 4), dtype=torch.float32, device=dev)

    def step():
        for grp in G:
            for gname, (fmt, N, K, q, c) in grp.items():
                mq.gemm_fused(xf if gname == "down" else xa, q, fmt, N, K, out=yg[gname], ws=ws)

    step()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        evs[i].record()
        step()
    evs[steps].record()
    torch.cuda.synchronize()
    d = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    del yg, ws
    return statistics.median(d), min(d)


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample
# ---------------------------------------------------------------------------

def clock_sample(torch, fn, seconds=1.0):
    """Shader clock and socket power while fn() (one forward) runs back to back
    for about `seconds`: an untimed repeat of the timed step, sampled every
    ~25 ms by a host thread (amdsmi: per-XCD gfx clock, socket power and power
    cap; else the sysfs sclk line).  Returns None when neither is readable."""
    import re
    import threading

    smi = None
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        smi = (amdsmi, amdsmi.amdsmi_get_processor_handles()[0])
    except Exception:
        smi = None
    sysfs = None
    for d in sorted(os.listdir("/sys/class/drm")) if os.path.isdir("/sys/class/drm") else []:
        f = os.path.join("/sys/class/drm", d, "device", "pp_dpm_sclk")
        if d.startswith("card") and os.path.exists(f):
            sysfs = f
            break
    if smi is None and sysfs is None:
        return None
    clocks, power, stop = [], [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                if smi is not None:
                    m = smi[0].amdsmi_get_gpu_metrics_info(smi[1])
                    xcd = [c for c in m.get("current_gfxclks") or [] if isinstance(c, int)]
                    if xcd:
                        clocks.append(statistics.mean(xcd))
                    if isinstance(m.get("current_socket_power"), int):
                        power.append(m["current_socket_power"])
                else:
                    hit = re.search(r"(\d+)Mhz \*", open(sysfs).read())
                    if hit:
                        clocks.append(int(hit.group(1)))
            except Exception:
                pass
            stop.wait(0.025)

    fn()
    torch.cuda.synchronize()
    th = threading.Thread(target=sample, daemon=True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    th.start()
    a.record()
    n = 0
    while time.perf_counter() - t0 < seconds:
        fn()
        n += 1
        torch.cuda.synchronize()
    b.record()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    cap = None
    if smi is not None:
        try:
            cap = smi[0].amdsmi_get_power_cap_info(smi[1]).get("power_cap")
            cap = round(cap / 1e6) if isinstance(cap, int) and cap > 100000 else cap
        except Exception:
            cap = None
        try:
            smi[0].amdsmi_shut_down()
        except Exception:
            pass
    if not clocks:
        return None
    return {"sclk_mhz_median": round(statistics.median(clocks)), "sclk_mhz_min": round(min(clocks)),
            "sclk_mhz_max": round(max(clocks)), "samples": len(clocks),
            "socket_power_w_median": round(statistics.median(power)) if power else None,
            "power_cap_w": cap, "steps": n, "ms_per_step": round(a.elapsed_time(b) / n, 3),
            "source": "amdsmi gpu metrics" if smi is not None else sysfs}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _decode_shard(job):
    """Worker of the row-sharded oracle decode (a separate process): decode the
    given rows of one weight; returns (seconds, sum of the f16 bit patterns)."""
    import oracle

    fmt, qrows, n, K = job
    t0 = time.perf_counter()
    w = oracle.dequant_ref(fmt, qrows, n, K)
    return time.perf_counter() - t0, int(w.sum(dtype=np.int64))


def _noop(i):
    return i


def parallel_decode(mats, procs):
    """The oracle decode of `mats` [(fmt, q [N, row_bytes], N, K)], rows sharded
    over `procs` worker processes (started fresh, warmed before the clock
    starts).  Returns (wall seconds, per-matrix checksums)."""
    import concurrent.futures
    import multiprocessing

    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(max_workers=procs, mp_context=ctx) as pool:
        list(pool.map(_noop, range(4 * procs)))
        jobs, owner = [], []
        for mi, (fmt, q, N, K) in enumerate(mats):
            step = -(-N // procs)
            for r0 in range(0, N, step):
                r1 = min(N, r0 + step)
                jobs.append((fmt, np.ascontiguousarray(q[r0:r1]), r1 - r0, K))
                owner.append(mi)
        t0 = time.perf_counter()
        res = list(pool.map(_decode_shard, jobs))
        wall = time.perf_counter() - t0
    sums = [0] * len(mats)
    for (_, cs), mi in zip(res, owner):
        sums[mi] += cs
    return wall, sums


def cpu_baseline(rows: int, n_layers: int):
    import oracle

    try:
        import threadpoolctl
        threads = max(i["num_threads"] for i in threadpoolctl.threadpool_info()) \
            if threadpoolctl.threadpool_info() else 1
    except Exception:
        threads = len(os.sched_getaffinity(0))
    t_deq = t_gemm = t_blas = 0.0
    deq_bytes = 0
    flops = 0.0
    mats, sums = [], []
    for li, mi in ((li, mi) for li in range(n_layers) for mi in range(len(synth.LAYER_7B))):
        name, fmt, N, K = synth.LAYER_7B[mi]
        q = synth.weights(fmt, synth.rng(5, li, mi, 0), N, K)
        x = synth.activations(synth.rng(5, li, mi, 1), rows, K)
        t0 = time.perf_counter()
        w16 = oracle.dequant_ref(fmt, q, N, K)
        t1 = time.perf_counter()
        if li == 0:
            mats.append((fmt, q.reshape(N, -1), N, K))
            sums.append(int(w16.sum(dtype=np.int64)))
        oracle.gemm_ref(x, w16, K)
        t2 = time.perf_counter()
        # context only: the same product as an f32 BLAS call on the decoded weights
        xf32 = x.view(np.float16).astype(np.float32)
        wf32 = w16.view(np.float16).astype(np.float32)
        t3 = time.perf_counter()
        xf32 @ wf32.T
        t4 = time.perf_counter()
        t_deq += t1 - t0
        t_gemm += t2 - t1
        t_blas += t4 - t3
        deq_bytes += q.nbytes + 2 * N * K
        flops += 2.0 * rows * N * K
    layers = synth.N_LAYERS_7B
    t_gemm /= n_layers
    t_deq /= n_layers
    t_blas /= n_layers
    # the same decode of one layer's seven weights, rows sharded over the host
    # cores (at most 16 processes: the machine's CPU share)
    procs = max(1, min(16, len(os.sched_getaffinity(0))))
    par_wall, par_sums = parallel_decode(mats, procs)
    if par_sums != sums:
        raise RuntimeError("the row-sharded oracle decode disagrees with the single-process one")
    par_bytes = sum(q.nbytes + 2 * N * K for _, q, N, K in mats)
    return {
        "value": round(rows / (t_gemm * layers), 2),
        "unit": "tok/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{n_layers} of {layers} layers (7 matrices each), {rows} of 2048 token rows; "
                   f"f64 oracle gemm_ref (Y and S); tok/s = rows / (mean layer time x {layers})"),
        "cpu_model": cpu_model(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "gemm_layer_s": round(t_gemm, 3),
        "dequant_gbs": round(deq_bytes / (t_deq * n_layers) / 1e9, 3),
        "dequant_layer_s": round(t_deq, 3),
        "dequant_parallel_gbs": round(par_bytes / par_wall / 1e9, 3),
        "dequant_parallel_procs": procs,
        "dequant_parallel_layer_s": round(par_wall, 3),
        "f32_blas_tflops": round(flops / (t_blas * n_layers) / 1e12, 3),
        "f32_blas_tok_s": round(rows / (t_blas * layers), 2),
    }


# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the matmul path runs on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_weight_prefill_q4_amd as mq

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calib_copy:
        run_calib_copy(torch, args.steps, dev)
        return
    if args.only_shape:
        run_only_shape(torch, mq, args.only_shape, args.steps, dev)
        return
    if args.only_fused:
        run_only_fused(torch, mq, args.only_fused, args.steps, dev)
        return
    if args.only_mmq:
        run_only_mmq(torch, mq, args.only_mmq, args.steps, dev)
        return
    if args.only_small_m:
        run_only_small_m(torch, mq, dev)
        return
    if args.only_sweep:
        rows = []
        cross = sweep(torch, mq, dev, rows)
        for r in rows:
            log(r)
        print(json.dumps({"crossover": cross}), flush=True)
        return
    if args.only_load:
        W, _ = make_weights(torch, mq, args.layers, dev)
        jobs = [(q, fmt, N, K, cache) for row in W for fmt, N, K, q, cache in row.values()]
        for _ in range(args.steps):
            mq.dequant_to_f16_batch(jobs)
        torch.cuda.synchronize()
        qb = sum(j[0].numel() for j in jobs)
        cb = sum(j[2] * j[3] * 2 for j in jobs)
        print(json.dumps({"only_load": len(jobs), "loads": args.steps, "quant_bytes": qb,
                          "cache_bytes": cb}), flush=True)
        return
    M, layers = args.M, args.layers
    log(f"[bench] device {torch.cuda.get_device_name(0)}, library {mq.LIB_PATH}")

    # -- weights and the load phase (one-time dequant into the f16 cache) ------
    t0 = time.time()
    W, G = make_weights(torch, mq, layers, dev)
    qbytes = sum(r[n][3].numel() for r in W for n in r)
    cbytes = sum(r[n][1] * r[n][2] * 2 for r in W for n in r)
    log(f"[bench] {layers * 7} weights drawn on device in {time.time() - t0:.1f}s: "
        f"{qbytes / 1e9:.3f} GB quantized, {cbytes / 1e9:.3f} GB f16")
    copy_gbs = hbm_copy_gbs(torch, dev)
    fill_gbs = hbm_fill_gbs(torch, dev)
    log(f"[bench] plain device copy (1 GiB, read + write): {copy_gbs:.0f} GB/s; "
        f"fill (4 GiB, write only): {fill_gbs:.0f} GB/s")
    deq_ms, deq_eager_ms, rec = load_phase(torch, mq, W, args.load_reps)
    deq_gbs = (qbytes + cbytes) / (deq_ms / 1e3) / 1e9
    per_fmt = {}
    for name, fmt, N, K, qb, ms in rec:
        f = per_fmt.setdefault("Q6_K" if fmt == 14 else "Q4_K", [0, 0.0])
        f[0] += qb + 2 * N * K
        f[1] += ms
    log(f"[bench] load phase (one batched call, GPU time from graph replays): {deq_ms:.2f} ms for "
        f"{len(rec)} weights, {deq_gbs:.0f} GB/s ({100 * deq_gbs / PEAK_HBM_GBS:.1f}% of HBM peak); "
        f"eager call {deq_eager_ms:.2f} ms (with the binding's host-side job checks); " +
        "single calls: " + ", ".join(f"{k} {v[0] / v[1] / 1e6:.0f} GB/s" for k, v in per_fmt.items()))
    per_mat = {}
    for name, fmt, N, K, qb, ms in rec:
        m = per_mat.setdefault(name, [0, 0.0, 0])
        m[0] += qb + 2 * N * K
        m[1] += ms
        m[2] += 1
    log("    per matrix (instrumented pass): " + ", ".join(f"{n} {v[1] / v[2] * 1e3:.1f} us {v[0] / v[1] / 1e6:.0f} GB/s"
                                       for n, v in per_mat.items()))

    # -- the timed forward --------------------------------------------------------
    xa = synth.activations_device(7001, M, 3584, dev)
    xf = synth.activations_device(7002, M, 18944, dev)
    ys = {n: torch.empty((M, N), dtype=torch.float32, device=dev) for n, _, N, _ in synth.LAYER_7B}
    yg = {g: torch.empty((M, N), dtype=torch.float32, device=dev)
          for g, (f, N, K, q, c) in G[0].items()}
    ws_bytes = max([mq.workspace_bytes(0, M, N, K) for _, _, N, K in synth.LAYER_7B] +
                   [mq.workspace_bytes(0, M, N, K) for f, N, K, q, c in G[0].values()])
    ws = torch.empty(max(1, ws_bytes // 4), dtype=torch.float32, device=dev)
    calls = [(n, f, N, K) for row in W for n, (f, N, K, _, _) in row.items()]
    gcalls = [(g, f, N, K) for grp in G for g, (f, N, K, _, _) in grp.items()]
    flops_step = sum(2.0 * M * N * K for _, _, N, K in calls)
    assert abs(flops_step - sum(2.0 * M * N * K for _, _, N, K in gcalls)) < 1.0

    def timed_steps(step_fn):
        """(wall ms per step, median and min event ms per step) over args.steps
        steps after args.warmup untimed ones; one HIP event per step boundary."""
        for _ in range(args.warmup):
            step_fn()
        bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for st in range(args.steps):
            bounds[st].record()
            step_fn()
        bounds[args.steps].record()
        torch.cuda.synchronize()
        wall_ = time.perf_counter() - t0
        d = [bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps)]
        return wall_ * 1e3 / args.steps, statistics.median(d), min(d)

    # the headline: the grouped forward (112 GEMMs computing the 196 products)
    ms_per_step, ev_step_ms, min_step_ms = timed_steps(lambda: forward_grouped(mq, G, xa, xf, yg, ws))
    # What the timed forward computed: a sample of the last layer's four
    # grouped outputs with the rows of X and of the weights it needs, for the
    # oracle check of the CPU leg.  Untimed.
    fwd_sample = forward_sample(torch, G, xa, xf, yg, M)
    # the same forward as 196 single GEMMs on row views of the same caches
    f196_wall, f196_ev, f196_min = timed_steps(lambda: forward(mq, W, xa, xf, ys, ws))

    # Per-call GPU time per shape and of the roofline kernel: graph replays of
    # the forward's calls of that shape (28 per step), see graph_us.
    def shape_calls(names):
        return [lambda fmt=fmt, N=N, K=K, cache=cache, name=name:
                mq.gemm_f16cache(xf if name == "down" else xa, cache, K, out=ys[name], ws=ws)
                for row in W for name, (fmt, N, K, q, cache) in row.items() if name in names]

    def group_calls(gname):
        return [lambda N=N, K=K, cache=cache:
                mq.gemm_f16cache(xf if gname == "down" else xa, cache, K, out=yg[gname], ws=ws)
                for grp in G for g, (fmt, N, K, q, cache) in grp.items() if g == gname]

    shape_rows = []
    for n, f, N, K in synth.LAYER_7B:
        t_us = graph_us(torch, shape_calls((n,)), replays=5)
        shape_rows.append((n, N, K, t_us, 2.0 * M * N * K / t_us / 1e6))
    group_rows = []
    for g, (f, N, K, q, c) in G[0].items():
        t_us = graph_us(torch, group_calls(g), replays=7 if g == ROOFLINE_GROUP else 5)
        group_rows.append((g, N, K, t_us, 2.0 * M * N * K / t_us / 1e6))
    avg_launch_us = next(t for g, N, K, t, tf in group_rows if g == ROOFLINE_GROUP)
    ach = 2.0 * M * ROOFLINE_N * ROOFLINE_K / avg_launch_us / 1e6
    traffic, traffic_note = measured_traffic()
    gemm_tflops = flops_step / (ev_step_ms / 1e3) / 1e12
    tok_s = M / (ms_per_step / 1e3)
    log(f"[bench] forward (4 grouped GEMMs per layer, {len(gcalls)} calls): {ms_per_step:.3f} ms/step wall, "
        f"{ev_step_ms:.3f} ms in events, {tok_s:.0f} matmul tok/s, {gemm_tflops:.0f} TFLOP/s; "
        f"as 196 single GEMMs: {f196_ev:.3f} ms/step ({M / (f196_ev / 1e3):.0f} tok/s)")
    log("    per call (graph replays of each shape's 28 calls):")
    for n, N, K, t_us, tf in group_rows + shape_rows:
        log(f"    {n:5s} {N:6d}x{K:<6d} {t_us:9.1f} us  {tf:7.1f} TFLOP/s  "
            f"({100 * tf / PEAK_F16_TFLOPS:.1f}% of peak)")
    log(f"[bench] roofline kernel ({ROOFLINE_KERNEL}, {layers} calls/step): "
        f"{ach:.0f} TFLOP/s = {100 * ach / PEAK_F16_TFLOPS:.1f}% of {PEAK_F16_TFLOPS:.0f}, "
        f"avg call {avg_launch_us:.1f} us; traffic {traffic} B/call ({traffic_note})")

    # -- shader clock and power while the step runs (untimed repeat) -------------------
    # Once over the whole step, once over the roofline kernel's calls alone
    # (the gate/up GEMMs draw more power than the step's average).
    clock = None
    c_fwd = clock_sample(torch, lambda: forward_grouped(mq, G, xa, xf, yg, ws))
    c_dom = clock_sample(torch, lambda: forward_grouped(mq, G, xa, xf, yg, ws, only=(ROOFLINE_GROUP,)))
    if c_fwd is not None and c_dom is not None:
        at = PEAK_F16_TFLOPS * c_dom["sclk_mhz_median"] / 2400.0
        clock = {"forward": c_fwd, "roofline_kernel": c_dom,
                 "mfma_peak_at_kernel_sclk_tflops": round(at, 1),
                 "roofline_frac_at_kernel_sclk": round(ach / at, 4)}
        for what, c in (("the forward", c_fwd), ("gate|up calls only", c_dom)):
            log(f"[bench] clock during {what}: {c['sclk_mhz_median']} MHz median "
                f"({c['sclk_mhz_min']}-{c['sclk_mhz_max']}), socket power "
                f"{c['socket_power_w_median']} W of {c['power_cap_w']} W cap")
        log(f"[bench] dense f16 peak at the roofline kernel's clock {at:.0f} TFLOP/s; "
            f"the kernel reaches {100 * ach / at:.1f}% of it")

    # -- the vendor library on the same shapes (context) --------------------------------
    vendor = vendor_table(torch, W, xa, xf, {n: t for n, _, _, t, _ in shape_rows})
    log("[bench] vendor library (torch.mm / hipBLASLt, f16 out) vs this library (f32 out), M = 2048: " +
        ", ".join(f"{n} {v['vendor_us']:.1f} vs {v['ours_us']:.1f} us" for n, v in vendor.items()))

    # -- int8 (MMQ) forward ----------------------------------------------------------
    mmqf = None
    if args.mmq_steps > 0:
        m_ms, q_ms = mmq_forward(torch, mq, W, M, args.mmq_steps, dev)
        mmqf = {"ms_per_step": round(m_ms, 3), "tok_s": round(M / (m_ms / 1e3), 1),
                "tops": round(flops_step / (m_ms / 1e3) / 1e12, 1),
                "quantize_ms_per_step": round(q_ms, 3)}
        log(f"[bench] int8 (MMQ) forward: {m_ms:.3f} ms/step, {mmqf['tok_s']:.0f} tok/s, "
            f"{mmqf['tops']:.0f} TOP/s (of which {q_ms:.3f} ms quantizing activations)")
        torch.cuda.empty_cache()

    # -- fused forward (no cache) ---------------------------------------------------
    fused = None
    if args.fused_steps > 0:
        forward_fused(mq, W, xa, xf, ys, ws)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.fused_steps):
            forward_fused(mq, W, xa, xf, ys, ws)
        b.record()
        torch.cuda.synchronize()
        f_ms = a.elapsed_time(b) / args.fused_steps
        # element expansions: each weight element once per row tile of its plan
        expn = sum(-(-M // mq.gemm_plan(f, M, N, K)["bm"]) * N * K for _, f, N, K in calls)
        fused = {"ms_per_step": round(f_ms, 3), "tok_s": round(M / (f_ms / 1e3), 1),
                 "tflops": round(flops_step / (f_ms / 1e3) / 1e12, 1),
                 "expansions_per_step": int(expn),
                 "expansions_per_s": round(expn / (f_ms / 1e3), 1)}
        log(f"[bench] fused forward: {f_ms:.3f} ms/step, {fused['tok_s']:.0f} tok/s, "
            f"{expn / (f_ms / 1e3) / 1e12:.2f} T element expansions/s")
        if args.grouped_steps > 0:
            fg_med, fg_min = fused_grouped_forward(torch, mq, G, xa, xf, args.grouped_steps, dev)
            fused["grouped_ms_per_step_median"] = round(fg_med, 3)
            fused["grouped_tok_s"] = round(M / (fg_med / 1e3), 1)
            log(f"[bench] fused grouped forward (4 GEMMs per layer): {fg_med:.3f} ms/step median, "
                f"{fused['grouped_tok_s']:.0f} tok/s")
            torch.cuda.empty_cache()

    # -- crossover sweep -------------------------------------------------------------
    cross = None
    if not args.no_sweep:
        del W, G
        torch.cuda.empty_cache()
        rows = []
        cross = sweep(torch, mq, dev, rows)
        log("[bench] fused vs cache sweep (median of 12 calls, rotating copies > 512 MB):")
        for r in rows:
            log(r)
        log("  crossover M (smallest M where the cache GEMM is faster): " +
            ", ".join(f"{k}: {v['crossover_M']}" for k, v in cross.items()))
        log("  M where the two paths are within 3%: " +
            ", ".join(f"{k}: {v['within_3pct_M'] or '-'}" for k, v in cross.items()))

    # -- every weight format on one shape ------------------------------------------------
    fmts = None
    if not args.no_formats:
        rows = []
        fmts = formats_table(torch, mq, dev, rows)
        log("[bench] weight formats on 14336x4096 (decode; fused GEMM), median of 12 calls:")
        for r in rows:
            log(r)

    # -- f32 activations ----------------------------------------------------------------
    xf32 = None
    if not args.no_xf32:
        rows = []
        xf32 = xf32_table(torch, mq, dev, rows)
        log("[bench] f32 activations on 14336x4096 (cache and fused Q4_K), median of 12 calls:")
        for r in rows:
            log(r)

    # -- CPU oracle baseline -------------------------------------------------------------
    cpu = fwd_check = None
    if not args.no_cpu:
        t0 = time.time()
        fwd_check = check_forward_sample(fwd_sample)
        log(f"[bench] oracle check of the timed forward ({fwd_check['outputs_checked']} outputs of "
            f"{fwd_check['gemms']} GEMMs): cache bit-exact {fwd_check['cache_bit_exact']}, worst "
            f"error {fwd_check['worst_err_over_tolerance']:.2e} of the tolerance "
            f"({time.time() - t0:.1f}s)")
        t0 = time.time()
        cpu = cpu_baseline(args.cpu_rows, args.cpu_layers)
        log(f"[bench] cpu oracle: {cpu['value']} tok/s on {cpu['cores']} threads "
            f"({time.time() - t0:.1f}s)")

    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median_events": round(ev_step_ms, 4),
        "ms_per_step_min_events": round(min_step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": ("7B prefill matmuls: 28 layers x {q,o 3584x3584, k,v 512x3584, "
                         "gate,up 18944x3584 Q4_K; down 3584x18944 Q6_K}, f16 cache, M=2048; "
                         "shared-input weights grouped (q|k|v N=4608, gate|up N=37888): "
                         "112 GEMMs per step computing the 196 products"),
            "M": M, "layers": layers, "gemms_per_step": len(gcalls), "products_per_step": len(calls),
            "quant_gb": round(qbytes / 1e9, 3), "cache_gb": round(cbytes / 1e9, 3),
        },
        "gemm_tflops": round(gemm_tflops, 1),
        "dequant_gbs": round(deq_gbs, 1),
        "dequant_ms": round(deq_ms, 3),
        "dequant_ms_eager": round(deq_eager_ms, 3),
        "dequant_timing": "GPU time of one batched call (196 weights) from HIP graph replays; "
                          "dequant_ms_eager: events around one eager call, which also hold the "
                          "binding's host-side checks of the jobs",
        "redequant_tok_s": round(M / ((ev_step_ms + deq_ms) / 1e3), 1),
        "per_shape_tflops": {n: round(tf, 1) for n, _, _, _, tf in group_rows + shape_rows},
        "per_shape_us": {n: round(t, 2) for n, _, _, t, _ in group_rows + shape_rows},
        "forward_196": {"ms_per_step": round(f196_wall, 4), "ms_per_step_median_events": round(f196_ev, 4),
                        "ms_per_step_min_events": round(f196_min, 4),
                        "tok_s": round(M / (f196_ev / 1e3), 1),
                        "tflops": round(flops_step / (f196_ev / 1e3) / 1e12, 1), "gemms_per_step": len(calls)},
        "roofline": {
            "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / PEAK_F16_TFLOPS, 4), "traffic": traffic,
            "traffic_note": traffic_note,
            "kernel": ROOFLINE_KERNEL, "avg_launch_us": round(avg_launch_us, 2),
            "timing": "HIP events around graph replays of the 28 gate|up calls of a step "
                      "(host launch gaps excluded)",
            "launches_per_step": layers,
            "flops_per_call": 2 * M * ROOFLINE_N * ROOFLINE_K,
            "algorithmic_bytes_per_call": M * ROOFLINE_K * 2 + ROOFLINE_N * ROOFLINE_K * 2 + M * ROOFLINE_N * 4,
        },
        "clock": clock,
        "dequant_roofline": {
            "bound": "hbm", "achieved": round(deq_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(deq_gbs / PEAK_HBM_GBS, 4),
            "hbm_copy_gbs": round(copy_gbs, 1),
            "frac_of_copy": round(deq_gbs / copy_gbs, 4),
            "hbm_fill_gbs": round(fill_gbs, 1),
        },
        "forward_check": fwd_check,
        "fused": fused,
        "mmq_forward": mmqf,
        "vendor_gemm": vendor,
        "crossover": cross,
        "formats": fmts,
        "xf32": xf32,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
