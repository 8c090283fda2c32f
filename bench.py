"""Benchmark of the ternary g128 decode path on one MI355X.

A step is one decode pass (M = 1) over the 27B-class MLP projections
gate (K=5120, N=17408), up (K=5120, N=17408) and down (K=17408, N=5120):
two tl_linear launches, gate|up (rows concatenated: the input rotated once
with the signed 1024-block Hadamard transform, binary16 output) then down,
whose input is the gate part of that output (the SwiGLU between them in a
model is outside the library).  Each launch is the fused rotation + ternary
product kernel.  Inputs are seeded synthetic tensors with the workload's
distributions.  --fmt trit5 runs the same step with the dense trit
packing.

Timing.  Each step is captured once in a HIP graph; the weights are replicated
into --copies distinct buffers (one graph per copy) and the timed loop cycles
through them, so no step finds its weights in the 256 MB last-level cache.
W warm-up steps, then exactly K timed steps between two HIP events on the
launch stream, with a device synchronisation on both sides.

Dominant kernel (roofline): the fused rotate + GEMV kernel, two launches
per step; its average launch duration comes from HIP events recorded on the
launch stream between consecutive launches, enqueued behind a GPU sleep so
that host submission is not counted (the step-timed figure per launch is
reported beside it, and the rocprofv3 kernel-trace average from profiles/
when the summary matches the kernel source).  HBM
traffic comes from the rocprofv3 counter summary under profiles/ and is
reported only while the kernel source is the one those counters were taken
from.

Extras: each launch of the step, the step as one tl_linear_chain launch
(2-bit slots), the three projections as separate launches (and the GEMVs
alone), the step and the separate launches with the other packing, the 64-layer weight stream (one chain launch per token with
dependent and with independent inputs, and one launch per linear or per
input), the prefill GEMM sweep (and its bfloat16 variant at M = 4096),
batched decode over the attention projections, the rotation at prefill size,
the weight quantiser, the decode step with 1-bit weights, and the CPU oracle
on a bounded sample.

Prints one JSON line on stdout; progress goes to stderr.
    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--fmt slot2|trit5]
    python bench.py --profile-pass [--fmt slot2|trit5|bit1]
    python bench.py --profile-prefill | --profile-batched
    python bench.py --read-floor
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ternary GEMV GB/s (% HBM peak) + prefill GEMM TFLOP/s at 27B-class shapes"
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 matrix peak
STEP_LINEARS = ("gate", "up", "down")
FMT_NAMES = {"trit5": 0, "slot2": 1, "bit1": 2}
KERNEL_SRC = {0: "gemv_trit5.hip", 1: "gemv_m1.hip"}
PROFILE_NAME = {0: "linear_m1_trit5_decode_step", 1: "linear_m1_slot2_decode_step"}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def code_bytes(n: int, k: int, fmt: int) -> int:
    """Packed code bytes of an N x K weight: 26 per 128-group (dense trits),
    K/4 a row (2-bit slots) or K/8 a row (1-bit codes)."""
    return n * (k // 128) * 26 if fmt == 0 else n * k // 8 if fmt == 2 else n * k // 4


def linear_bytes(n: int, k: int, m: int, fmt: int) -> int:
    """Algorithmic bytes of one fused tl_linear launch: codes + scales +
    unrotated binary16 activations and int8 signs read, rotated activations
    (binary16) and fp32 outputs written."""
    return code_bytes(n, k, fmt) + n * (k // 128) * 2 + m * k * 2 + k + m * k * 2 + m * n * 4


def gemv_bytes(n: int, k: int, m: int, fmt: int) -> int:
    """Algorithmic bytes of one GEMV launch: packed codes + binary16 scales +
    binary16 activations read, fp32 outputs written."""
    return code_bytes(n, k, fmt) + n * (k // 128) * 2 + m * k * 2 + m * n * 4


def rotate_bytes(m: int, k: int) -> int:
    """Algorithmic bytes of one rotation: binary16 in and out, int8 signs."""
    return 2 * m * k * 2 + k


def source_sha(fmt: int) -> str:
    """First 16 hex digits of the SHA-256 of the kernel's source file followed
    by the kernel headers it includes, in the order of its #include lines
    (tl_internal.h and tl.h, the library's declarations, are left out)."""
    csrc = os.path.join(ROOT, "tl_hadamard_rotate_amd", "csrc")
    with open(os.path.join(csrc, KERNEL_SRC[fmt]), "rb") as f:
        data = f.read()
    h = hashlib.sha256(data)
    for name in re.findall(rb'^#include "([^"]+)"', data, re.M):
        path = os.path.join(csrc, name.decode())
        if name not in (b"tl_internal.h", b"../../include/tl.h") and os.path.exists(path):
            with open(path, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(fmt: int):
    """HBM bytes per GEMV launch from the committed counter summary, or None
    when there is none for the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{PROFILE_NAME[fmt]}_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"^kernel_source_sha256_16:\s*(\S+)", text, re.M)
    val = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not sha or not val or sha.group(1) != source_sha(fmt):
        return None
    return float(val.group(1))


def rocprof_launch_us(fmt: int):
    """Average duration (us) of the step's kernel in the committed rocprofv3
    kernel-trace summary, or None when there is none for the current kernel
    source."""
    path = os.path.join(ROOT, "profiles", f"{PROFILE_NAME[fmt]}_trace.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"^kernel_source_sha256_16:\s*(\S+)", text, re.M)
    val = re.search(r"^step_kernel_avg_ns:\s*([0-9.eE+]+)", text, re.M)
    if not sha or not val or sha.group(1) != source_sha(fmt):
        return None
    return round(float(val.group(1)) / 1e3, 3)


def build_step_inputs(torch, tl, synth, dev, fmt: int, copies: int):
    lins = []
    for name in STEP_LINEARS:
        k, n = synth.SHAPES[name]
        inp = synth.linear_inputs(n, k, 1, seed=0, cfg=2, layer=0, linear=synth.LINEAR_ID[name],
                                  binary=fmt == 2)
        codes = torch.from_numpy(inp.codes).to(dev)
        packed = tl.pack(codes, fmt)
        del codes
        scales = torch.from_numpy(inp.scales).to(dev)
        packs = [packed] + [packed.clone() for _ in range(copies - 1)]
        scs = [scales] + [scales.clone() for _ in range(copies - 1)]
        lins.append(dict(
            name=name, n=n, k=k, packs=packs, scales=scs,
            x=torch.from_numpy(inp.x).to(dev), signs=torch.from_numpy(inp.signs).to(dev),
            x_rot=torch.empty((1, k), dtype=torch.float16, device=dev),
            y=torch.empty((1, n), dtype=torch.float32, device=dev)))
    return lins


def step_fn(tl, lins, fmt, c):
    """One decode step: per projection, rotation + ternary product (tl_linear;
    a single fused kernel at M=1 with the 2-bit-slot and dense trit packings)."""
    for lin in lins:
        tl.linear(lin["packs"][c], lin["scales"][c], fmt, lin["x"], lin["signs"],
                  out=lin["y"], x_rot=lin["x_rot"])


def gemv_fn(tl, lins, fmt, c):
    """The products alone, on already rotated activations (tl_gemv)."""
    for lin in lins:
        tl.gemv(lin["packs"][c], lin["scales"][c], fmt, lin["x_rot"], out=lin["y"])


def capture(torch, fn, copies, stream):
    graphs = []
    for c in range(copies):
        fn(c)                                  # eager first call: one-time set-up
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn(c)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def timed_replays(torch, graphs, count, warmup, stream):
    """Replay graphs[i % len] for i in [0, count) between two HIP events on
    `stream`; returns the elapsed milliseconds."""
    with torch.cuda.stream(stream):
        for i in range(warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(count):
            graphs[(warmup + i) % len(graphs)].replay()
        end.record(stream)
        torch.cuda.synchronize()
    return start.elapsed_time(end)


def cpu_baseline(oracle, synth, fmt, budget_s=8.0, rows=512):
    """The oracle as it stands, timed on the host on a bounded sample: the
    rotation plus unpack, dequantisation and fp64 matrix-vector product of the
    first `rows` rows of gate, up and down (the step's projections), in GB/s
    of the same algorithmic bytes as the GPU figure; once with the BLAS
    thread pool as it is (the threads the oracle actually uses: `cores`) and
    once limited to one thread."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits, threads = None, os.cpu_count() or 1
    samples = []
    for name in STEP_LINEARS:
        k, n = synth.SHAPES[name]
        inp = synth.linear_inputs(rows, k, 1, seed=0, cfg=2, layer=0, linear=synth.LINEAR_ID[name])
        samples.append((inp, oracle.pack(inp.codes, fmt), k))

    def rate():
        done, t0, passes = 0, time.perf_counter(), 0
        while True:
            for inp, packed, k in samples:
                x_rot = oracle.rotate(inp.x, inp.signs)
                oracle.matvec_packed(packed, inp.scales, fmt, x_rot, k)
                done += gemv_bytes(rows, k, 1, fmt) + rotate_bytes(1, k)
            passes += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return done / dt / 1e9, passes, dt

    v_all, passes, dt = rate()
    v_one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            v_one = rate()[0]
    cpu = host_cpu()
    return {"value": round(v_all, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {rows} rows of gate, up and down at M=1 (rotation + unpack + fp64 "
                      f"dequantised matrix-vector product), {passes} passes in {dt:.1f} s with "
                      f"the BLAS pool of {threads} threads; the rate of the sample, not an "
                      f"extrapolation of a larger run",
            "value_one_thread": None if v_one is None else round(v_one, 4),
            "cpu_model": cpu["model"], "logical_cpus": cpu["logical_cpus"],
            "usable_cpus": cpu["usable_cpus"]}


def _event_time(torch, fn, reps):
    """Milliseconds per call of fn() over `reps` calls, between HIP events on
    torch's current stream (the stream the library launches on)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def bench_gemm(torch, tl, synth, dev, fmt, reps=5, bf16=False, ms_list=None):
    """Prefill GEMM TFLOP/s for M in {512, 2048, 4096} at the MLP shapes
    (gate: K=5120 N=17408, down: K=17408 N=5120); with bf16, tl_gemm_bf16 on
    bfloat16 activations (their conversion to binary16 included; bfloat16
    matrix peak = the fp16 one)."""
    out = []
    call = tl.gemm_bf16 if bf16 else tl.gemm
    xdt = torch.bfloat16 if bf16 else torch.float16
    for name in ("gate", "down"):
        k, n = synth.SHAPES[name]
        inp = synth.linear_inputs(n, k, 1, seed=0, cfg=4, linear=synth.LINEAR_ID[name])
        packed = tl.pack(torch.from_numpy(inp.codes).to(dev), fmt)
        scales = torch.from_numpy(inp.scales).to(dev)
        for m in ms_list or synth.PREFILL_M:
            gen = torch.Generator(device="cpu").manual_seed(4 + m)
            x = torch.randn((m, k), generator=gen).to(xdt).to(dev)
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            size = tl.gemm_bf16_workspace_bytes if bf16 else tl.gemm_workspace_bytes
            ws = torch.empty(max(1, size(m, n, k, fmt)), dtype=torch.uint8, device=dev)
            call(packed, scales, fmt, x, out=y, workspace=ws)
            torch.cuda.synchronize()
            ms = _event_time(torch, lambda i: call(packed, scales, fmt, x, out=y, workspace=ws),
                             reps)
            tflops = 2.0 * m * n * k / (ms * 1e-3) / 1e12
            out.append({"linear": name, "M": m, "K": k, "N": n, "ms": round(ms, 4),
                        "TFLOPs": round(tflops, 2),
                        "frac_of_fp16_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)})
            del x, y, ws
        del packed, scales
    torch.cuda.empty_cache()
    return out


def bench_batched(torch, tl, synth, dev, fmt, copies=20):
    """Batched decode GEMV over one layer's attention projections q, k, v, o
    at M in {1, 2, 4, 8, 16} (activations with 1% outliers x20); weights
    cycled over `copies` distinct buffers (> the last-level cache), the
    launches captured in one HIP graph (launch time per GEMV, gaps included);
    also q|k|v, the three projections that read one input with their rows
    concatenated, as one launch."""
    import dataclasses

    import numpy as np
    out = []
    ins = {}
    for name in ("q", "k", "v", "o"):
        k, n = synth.SHAPES[name]
        ins[name] = synth.linear_inputs(n, k, 16, seed=0, cfg=3, linear=synth.LINEAR_ID[name],
                                        outliers=True)
    # q, k and v read the same input: their rows concatenated along N run as
    # one launch (q's activations and signs)
    qkv = dataclasses.replace(ins["q"], codes=np.concatenate([ins[c].codes for c in "qkv"]),
                              scales=np.concatenate([ins[c].scales for c in "qkv"]))
    for name, inp in (("q", ins["q"]), ("k", ins["k"]), ("v", ins["v"]), ("o", ins["o"]),
                      ("q|k|v", qkv)):
        n, k = inp.codes.shape
        packed = tl.pack(torch.from_numpy(inp.codes).to(dev), fmt)
        scales = torch.from_numpy(inp.scales).to(dev)
        packs = [packed] + [packed.clone() for _ in range(copies - 1)]
        scs = [scales] + [scales.clone() for _ in range(copies - 1)]
        signs = torch.from_numpy(inp.signs).to(dev)
        x_rot = tl.hadamard_rotate(torch.from_numpy(inp.x).to(dev), signs)
        for m in synth.BATCHED_M:
            xm = x_rot[:m].contiguous()
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            for c in range(copies):
                tl.gemv(packs[c], scs[c], fmt, xm, out=y)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in range(copies):
                    tl.gemv(packs[c], scs[c], fmt, xm, out=y)
            g.replay()
            torch.cuda.synchronize()
            ms = _event_time(torch, lambda i: g.replay(), 3) / copies
            del g
            nbytes = gemv_bytes(n, k, m, fmt)
            out.append({"linear": name, "M": m, "us": round(ms * 1e3, 3),
                        "GBs": round(nbytes / (ms * 1e-3) / 1e9, 1)})
        del packs, scs
    torch.cuda.empty_cache()
    return out


def bench_rotate_prefill(torch, tl, dev, reps=10):
    """Activation rotation at prefill size M=4096, K in {5120, 17408}: GB/s of
    the binary16 read + write."""
    out = []
    for k in (5120, 17408):
        gen = torch.Generator(device="cpu").manual_seed(k)
        x = torch.randn((4096, k), generator=gen).to(torch.float16).to(dev)
        s = (torch.randint(0, 2, (k,), generator=gen) * 2 - 1).to(torch.int8).to(dev)
        o = torch.empty_like(x)
        tl.hadamard_rotate(x, s, out=o)
        torch.cuda.synchronize()
        ms = _event_time(torch, lambda i: tl.hadamard_rotate(x, s, out=o), reps)
        out.append({"M": 4096, "K": k, "us": round(ms * 1e3, 2),
                    "GBs": round(rotate_bytes(4096, k) / (ms * 1e-3) / 1e9, 1)})
        del x, o
    return out


def bench_stream(torch, tl, synth, dev, fmt, stream, reps=5):
    """The 27B-class weight stream at M=1: 64 layers x (q, k, v, o, gate, up,
    down), each a rotation + GEMV, captured in one HIP graph per token.  One
    layer is generated and replicated into 64 distinct device buffers (the
    values do not change the streaming cost; distinct addresses defeat the
    caches)."""
    layer = []
    for name in synth.LAYER_LINEARS:
        k, n = synth.SHAPES[name]
        inp = synth.linear_inputs(n, k, 1, seed=0, cfg=5, layer=0, linear=synth.LINEAR_ID[name],
                                  outliers=name in ("q", "k", "v", "o"))
        layer.append((name, k, n, tl.pack(torch.from_numpy(inp.codes).to(dev), fmt),
                      torch.from_numpy(inp.scales).to(dev), torch.from_numpy(inp.signs).to(dev),
                      torch.from_numpy(inp.x).to(dev)))
    lins = []
    for li in range(synth.N_LAYERS):
        for name, k, n, p, sc, sg, x in layer:
            lins.append(dict(k=k, n=n, packed=p if li == 0 else p.clone(),
                             scales=sc if li == 0 else sc.clone(), signs=sg, x=x,
                             x_rot=torch.empty((1, k), dtype=torch.float16, device=dev),
                             y=torch.empty((1, n), dtype=torch.float32, device=dev)))
    weight_bytes = sum(l["packed"].numel() + l["scales"].numel() * 2 for l in lins)
    act_bytes = sum(rotate_bytes(1, l["k"]) + 2 * l["k"] + 4 * l["n"] for l in lins)

    def token():
        for l in lins:
            tl.linear(l["packed"], l["scales"], fmt, l["x"], l["signs"], out=l["y"],
                      x_rot=l["x_rot"])

    with torch.cuda.stream(stream):
        token()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            token()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del g, lins, layer
    torch.cuda.empty_cache()
    return {"layers": synth.N_LAYERS, "linears_per_layer": len(synth.LAYER_LINEARS),
            "linear_calls_per_token": synth.N_LAYERS * len(synth.LAYER_LINEARS),
            "weight_bytes": int(weight_bytes), "activation_bytes": int(act_bytes),
            "ms_per_token": round(ms, 4), "weight_streams_per_s": round(1e3 / ms, 1),
            "GBs": round((weight_bytes + act_bytes) / (ms * 1e-3) / 1e9, 1)}


def bench_stream_shared(torch, tl, synth, dev, fmt, stream, reps=5):
    """The same 64-layer weight stream with one rotation per input instead of
    one per linear: q, k, v (which read the same input) concatenated along N
    into one linear, and gate, up likewise; 4 tl_linear calls per layer
    instead of 7.  Same weight bytes."""
    import numpy as np

    groups = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
    layer = []
    for grp in groups:
        k = synth.SHAPES[grp[0]][0]
        ins = [synth.linear_inputs(synth.SHAPES[g][1], k, 1, seed=0, cfg=5, layer=0,
                                   linear=synth.LINEAR_ID[g], outliers=g in ("q", "k", "v", "o"))
               for g in grp]
        codes = torch.from_numpy(np.concatenate([i.codes for i in ins])).to(dev)
        scales = torch.from_numpy(np.concatenate([i.scales for i in ins])).to(dev)
        layer.append((k, codes.shape[0], tl.pack(codes, fmt), scales,
                      torch.from_numpy(ins[0].signs).to(dev), torch.from_numpy(ins[0].x).to(dev)))
        del codes
    lins = []
    for li in range(synth.N_LAYERS):
        for k, n, p, sc, sg, x in layer:
            lins.append(dict(k=k, n=n, packed=p if li == 0 else p.clone(),
                             scales=sc if li == 0 else sc.clone(), signs=sg, x=x,
                             x_rot=torch.empty((1, k), dtype=torch.float16, device=dev),
                             y=torch.empty((1, n), dtype=torch.float32, device=dev)))
    weight_bytes = sum(l["packed"].numel() + l["scales"].numel() * 2 for l in lins)
    act_bytes = sum(rotate_bytes(1, l["k"]) + 2 * l["k"] + 4 * l["n"] for l in lins)

    def token():
        for l in lins:
            tl.linear(l["packed"], l["scales"], fmt, l["x"], l["signs"], out=l["y"],
                      x_rot=l["x_rot"])

    with torch.cuda.stream(stream):
        token()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            token()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del g, lins, layer
    torch.cuda.empty_cache()
    return {"layers": synth.N_LAYERS, "linear_calls_per_layer": len(groups),
            "linear_calls_per_token": synth.N_LAYERS * len(groups),
            "weight_bytes": int(weight_bytes), "activation_bytes": int(act_bytes),
            "ms_per_token": round(ms, 4), "weight_streams_per_s": round(1e3 / ms, 1),
            "GBs": round((weight_bytes + act_bytes) / (ms * 1e-3) / 1e9, 1)}


def bench_bit1(torch, tl, synth, dev, stream, copies, steps, warmup):
    """The decode step with 1-bit weights (codes -1/+1, g128 scales): per
    projection the rotation + the 1-bit GEMV (tl_linear, two launches), the
    GEMV alone on rotated activations, and the GEMV at M = 1, 4, 16 on gate
    (one graph of `copies` launches, one per weight copy); weights cycled
    over `copies` buffers, launches captured in HIP graphs."""
    fmt = 2
    lins = build_step_inputs(torch, tl, synth, dev, fmt, copies)
    with torch.cuda.stream(stream):
        sg = capture(torch, lambda c: step_fn(tl, lins, fmt, c), copies, stream)
        gg = capture(torch, lambda c: gemv_fn(tl, lins, fmt, c), copies, stream)
    ms = timed_replays(torch, sg, steps, warmup, stream) / steps
    reps = max(steps, 3 * copies)
    g_us = timed_replays(torch, gg, reps, warmup, stream) * 1e3 / (3 * reps)
    sbytes = sum(gemv_bytes(l["n"], l["k"], 1, fmt) + rotate_bytes(1, l["k"]) for l in lins)
    g_bytes = sum(gemv_bytes(l["n"], l["k"], 1, fmt) for l in lins) / 3.0
    out = {"step_GBs": round(sbytes / (ms * 1e-3) / 1e9, 1), "ms_per_step": round(ms, 5),
           "step_bytes": sbytes, "gemv_avg_launch_us": round(g_us, 3),
           "gemv_GBs": round(g_bytes / (g_us * 1e-6) / 1e9, 1), "gate_batched": []}
    del sg, gg
    gate = lins[0]
    k, n = gate["k"], gate["n"]
    for m in (1, 4, 16):
        xm = torch.randn((m, k), generator=torch.Generator(device="cpu").manual_seed(m)).to(
            torch.float16).to(dev)
        ym = torch.empty((m, n), dtype=torch.float32, device=dev)
        # all weight copies in one graph: launch time per GEMV, gaps included
        with torch.cuda.stream(stream):
            gm = capture(torch, lambda c: [tl.gemv(gate["packs"][i], gate["scales"][i], fmt, xm,
                                                   out=ym) for i in range(copies)], 1, stream)
        r = max(steps // copies, 3)
        us = timed_replays(torch, gm, r, warmup, stream) * 1e3 / (r * copies)
        out["gate_batched"].append({"M": m, "us": round(us, 3),
                                    "GBs": round(gemv_bytes(n, k, m, fmt) / (us * 1e-6) / 1e9, 1)})
        del gm
    del lins
    torch.cuda.empty_cache()
    return out


def quantize_bytes(n: int, k: int) -> int:
    """Algorithmic bytes of one tl_quantize launch: fp32 weights and int8
    signs read, int8 codes and binary16 scales written."""
    return n * k * 4 + k + n * k + n * (k // 128) * 2


def bench_quantize(torch, tl, synth, dev, reps=10):
    """The weight quantiser (rotation folded in, round to ternary g128) on the
    gate and down shapes: average launch time between HIP events, GB/s."""
    out = []
    for name in ("gate", "down"):
        k, n = synth.SHAPES[name]
        gen = torch.Generator(device="cpu").manual_seed(k)
        w = (0.02 * torch.randn((n, k), generator=gen)).to(dev)
        s = (torch.randint(0, 2, (k,), generator=gen) * 2 - 1).to(torch.int8).to(dev)
        tl.quantize(w, s)
        torch.cuda.synchronize()
        ms = _event_time(torch, lambda i: tl.quantize(w, s), reps)
        out.append({"linear": name, "N": n, "K": k, "us": round(ms * 1e3, 2),
                    "GBs": round(quantize_bytes(n, k) / (ms * 1e-3) / 1e9, 1)})
        del w
        torch.cuda.empty_cache()
    return out


def probe_lib():
    """The benchmark's read-only probe (libtl_probe.so, built beside libtl)."""
    import ctypes
    path = os.path.join(ROOT, "tl_hadamard_rotate_amd", "libtl_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m tl_hadamard_rotate_amd.build`")
    L = ctypes.CDLL(path)
    L.tlprobe_stream_read.restype = ctypes.c_int
    L.tlprobe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_int32, ctypes.c_void_p]
    return L


def read_floor(torch, tl, dev, reps=20) -> int:
    """What HBM delivers to a read-only kernel (tlprobe_stream_read) at transfer
    sizes from 4 MiB to 512 MiB, including the 23.8 MB one gate/up decode
    launch reads: buffers cycled through a 1 GiB pool, average time per
    launch between HIP events (the rocprofv3 trace of this mode gives the
    kernel durations).  Prints one JSON line."""
    probe = probe_lib()
    pool_bytes = 1 << 30
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device=dev).fill_(1)
    out = torch.full((65,), 0x5A5A5A5A, dtype=torch.int32, device=dev)   # out[0]: the key
    sizes = [4 << 20, 12 << 20, 23774208, 48 << 20, 96 << 20, 192 << 20, 512 << 20]
    res = []
    for b in sizes:
        blocks = max(1024, min(65536, b // (256 * 16 * 4)))
        slots = pool_bytes // b
        stream = torch.cuda.current_stream().cuda_stream

        def call(i):
            ptr = pool.data_ptr() + (i % slots) * b
            st = probe.tlprobe_stream_read(ptr, b, out.data_ptr(), blocks, stream)
            if st != 0:
                raise RuntimeError(f"tlprobe_stream_read failed: {st}")
        call(0)
        torch.cuda.synchronize()
        ms = _event_time(torch, call, reps)
        res.append({"bytes": b, "blocks": blocks, "us": round(ms * 1e3, 2),
                    "GBs": round(b / (ms * 1e-3) / 1e9, 1)})
        log(f"read {b / 2**20:7.1f} MiB: {ms * 1e3:8.2f} us, {b / (ms * 1e-3) / 1e9:7.1f} GB/s")
    print(json.dumps({"read_floor": res}), flush=True)
    return 0


def profile_pass(torch, tl, synth, dev, fmt) -> int:
    """Kernels for the HBM-counter runs: the calibration copy (256 MiB read and
    256 MiB written per launch), then, with 2-bit slots or dense trits, 10
    eager steps (the timed step: tl_linear on gate|up, then on down), then 10
    eager decode steps as separate launches per projection (tl_linear, and
    tl_gemv alone); weights cycled over 8 copies."""
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    if fmt in (0, 1):
        steps, _, _ = build_mlp_step(torch, tl, synth, dev, 8, fmt)
        for i in range(10):
            for fn in steps[i % 8]:
                fn()
        torch.cuda.synchronize()
        del steps
    lins = build_step_inputs(torch, tl, synth, dev, fmt, 8)
    for lin in lins:
        tl.hadamard_rotate(lin["x"], lin["signs"], out=lin["x_rot"])
    for i in range(10):
        step_fn(tl, lins, fmt, i % 8)
        gemv_fn(tl, lins, fmt, i % 8)
    torch.cuda.synchronize()
    log("profile pass done")
    return 0


def profile_prefill(torch, tl, synth, dev) -> int:
    """Kernels for the prefill counter runs: the calibration copy (3 launches
    of a 256 MiB device copy), then 3 launches each of the 2-bit-slot GEMM at
    M=4096 for gate (K=5120, N=17408) and down (K=17408, N=5120), then 3
    launches each of the rotation at M=4096 for K=5120 and K=17408."""
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    for name in ("gate", "down"):
        k, n = synth.SHAPES[name]
        inp = synth.linear_inputs(n, k, 1, seed=0, cfg=4, linear=synth.LINEAR_ID[name])
        packed = tl.pack(torch.from_numpy(inp.codes).to(dev), 1)
        scales = torch.from_numpy(inp.scales).to(dev)
        gen = torch.Generator(device="cpu").manual_seed(4 + 4096)
        x = torch.randn((4096, k), generator=gen).to(torch.float16).to(dev)
        y = torch.empty((4096, n), dtype=torch.float32, device=dev)
        for _ in range(3):
            tl.gemm(packed, scales, 1, x, out=y)
        torch.cuda.synchronize()
        del packed, scales, x, y
    for k in (5120, 17408):
        gen = torch.Generator(device="cpu").manual_seed(k)
        x = torch.randn((4096, k), generator=gen).to(torch.float16).to(dev)
        s = (torch.randint(0, 2, (k,), generator=gen) * 2 - 1).to(torch.int8).to(dev)
        o = torch.empty_like(x)
        for _ in range(3):
            tl.hadamard_rotate(x, s, out=o)
        torch.cuda.synchronize()
        del x, s, o
    log("prefill profile pass done")
    return 0


def profile_batched(torch, tl, synth, dev) -> int:
    """Kernels for the batched-decode, quantiser and bf16-GEMM counter runs:
    the calibration copy (3 launches of a 256 MiB device copy); then, for q
    (K=5120, N=6144) and o (K=6144, N=5120) with 2-bit slots, at M = 2, 4, 8
    and 16 in that order, 4 tl_gemv launches on rotated activations, one per
    weight copy; then 3 launches of tl_quantize at the gate shape (N=17408,
    K=5120); then 2 launches of tl_gemm_bf16 at M=4096 for gate."""
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    for name in ("q", "o"):
        k, n = synth.SHAPES[name]
        inp = synth.linear_inputs(n, k, 16, seed=0, cfg=3, linear=synth.LINEAR_ID[name],
                                  outliers=True)
        packed = tl.pack(torch.from_numpy(inp.codes).to(dev), 1)
        scales = torch.from_numpy(inp.scales).to(dev)
        packs = [packed] + [packed.clone() for _ in range(3)]
        scs = [scales] + [scales.clone() for _ in range(3)]
        x_rot = tl.hadamard_rotate(torch.from_numpy(inp.x).to(dev),
                                   torch.from_numpy(inp.signs).to(dev))
        for m in (2, 4, 8, 16):
            xm = x_rot[:m].contiguous()
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            for c in range(4):
                tl.gemv(packs[c], scs[c], 1, xm, out=y)
            torch.cuda.synchronize()
        del packs, scs, packed, scales, x_rot
    k, n = synth.SHAPES["gate"]
    gen = torch.Generator(device="cpu").manual_seed(77)
    w = (0.02 * torch.randn((n, k), generator=gen)).to(dev)
    signs = (torch.randint(0, 2, (k,), generator=gen) * 2 - 1).to(torch.int8).to(dev)
    for _ in range(3):
        tl.quantize(w, signs)
    torch.cuda.synchronize()
    del w, signs
    inp = synth.linear_inputs(n, k, 1, seed=0, cfg=4, linear=synth.LINEAR_ID["gate"])
    packed = tl.pack(torch.from_numpy(inp.codes).to(dev), 1)
    scales = torch.from_numpy(inp.scales).to(dev)
    x = torch.randn((4096, k), generator=gen).to(torch.bfloat16).to(dev)
    y = torch.empty((4096, n), dtype=torch.float32, device=dev)
    for _ in range(2):
        tl.gemm_bf16(packed, scales, 1, x, out=y)
    torch.cuda.synchronize()
    log("batched profile pass done")
    return 0


def chain_op_bytes(n: int, k: int, y_elem: int, fmt: int = 1, x_rot: bool = False) -> int:
    """Algorithmic bytes of one linear of a decode chain: codes + scales, the
    unrotated binary16 input and the int8 signs read, the output (y_elem
    bytes per element) written, and the rotated input when it is kept."""
    return (code_bytes(n, k, fmt) + n * (k // 128) * 2 + 2 * k + k + n * y_elem +
            (2 * k if x_rot else 0))


def build_chain_step(torch, tl, synth, dev, copies):
    """The decode step as one tl_linear_chain launch per weight copy: gate|up
    (the two projections that read the same input, rows concatenated: one
    rotation) then down, whose input is the gate part of gate|up's binary16
    output (the SwiGLU between them in a model is outside this library).
    Returns the chains and the step's algorithmic bytes."""
    import numpy as np

    ins = {}
    for name in STEP_LINEARS:
        k, n = synth.SHAPES[name]
        ins[name] = synth.linear_inputs(n, k, 1, seed=0, cfg=2, layer=0,
                                        linear=synth.LINEAR_ID[name])
    g, u, d = ins["gate"], ins["up"], ins["down"]
    kg, ng = synth.SHAPES["gate"]
    kd, nd = synth.SHAPES["down"]
    gu_packed = tl.pack(torch.from_numpy(np.concatenate([g.codes, u.codes])).to(dev), 1)
    gu_scales = torch.from_numpy(np.concatenate([g.scales, u.scales])).to(dev)
    dn_packed = tl.pack(torch.from_numpy(d.codes).to(dev), 1)
    dn_scales = torch.from_numpy(d.scales).to(dev)
    x = torch.from_numpy(g.x).to(dev).view(-1)
    s_gu, s_dn = torch.from_numpy(g.signs).to(dev), torch.from_numpy(d.signs).to(dev)
    y_gu = torch.empty(2 * ng, dtype=torch.float16, device=dev)
    y_dn = torch.empty(nd, dtype=torch.float32, device=dev)
    chains = []
    for c in range(copies):
        pg, sg = (gu_packed, gu_scales) if c == 0 else (gu_packed.clone(), gu_scales.clone())
        pd, sd = (dn_packed, dn_scales) if c == 0 else (dn_packed.clone(), dn_scales.clone())
        chains.append(tl.Chain([dict(packed=pg, scales=sg, fmt=1, x=x, signs=s_gu, y=y_gu),
                                dict(packed=pd, scales=sd, fmt=1, x=y_gu[:kd], signs=s_dn,
                                     y=y_dn)]))
    step_bytes = chain_op_bytes(2 * ng, kg, 2) + chain_op_bytes(nd, kd, 4)
    return chains, step_bytes


def build_mlp_step(torch, tl, synth, dev, copies, fmt=1):
    """The decode step as two tl_linear launches per weight copy: gate|up (the
    two projections that read the same input, rows concatenated: one rotation,
    binary16 output) then down on the gate part of that output (the SwiGLU
    between them in a model is outside this library; stream order makes down
    wait for gate|up), with packing fmt.  Returns per-copy lists of the two
    launches (callables), the step's algorithmic bytes and what the output
    checks read (the step's buffers and host inputs)."""
    import numpy as np

    ins = {}
    for name in STEP_LINEARS:
        k, n = synth.SHAPES[name]
        ins[name] = synth.linear_inputs(n, k, 1, seed=0, cfg=2, layer=0,
                                        linear=synth.LINEAR_ID[name])
    g, u, d = ins["gate"], ins["up"], ins["down"]
    kg, ng = synth.SHAPES["gate"]
    kd, nd = synth.SHAPES["down"]
    gu_packed = tl.pack(torch.from_numpy(np.concatenate([g.codes, u.codes])).to(dev), fmt)
    gu_scales = torch.from_numpy(np.concatenate([g.scales, u.scales])).to(dev)
    dn_packed = tl.pack(torch.from_numpy(d.codes).to(dev), fmt)
    dn_scales = torch.from_numpy(d.scales).to(dev)
    x = torch.from_numpy(g.x).to(dev)
    s_gu, s_dn = torch.from_numpy(g.signs).to(dev), torch.from_numpy(d.signs).to(dev)
    y_gu = torch.empty((1, 2 * ng), dtype=torch.float16, device=dev)
    y_dn = torch.empty((1, nd), dtype=torch.float32, device=dev)
    xr_gu = torch.empty((1, kg), dtype=torch.float16, device=dev)
    xr_dn = torch.empty((1, kd), dtype=torch.float16, device=dev)
    x_dn = y_gu[:, :kd]
    steps = []
    for c in range(copies):
        pg, sg = (gu_packed, gu_scales) if c == 0 else (gu_packed.clone(), gu_scales.clone())
        pd, sd = (dn_packed, dn_scales) if c == 0 else (dn_packed.clone(), dn_scales.clone())
        steps.append([
            (lambda pg=pg, sg=sg: tl.linear(pg, sg, fmt, x, s_gu, out_dtype=torch.float16,
                                            out=y_gu, x_rot=xr_gu)),
            (lambda pd=pd, sd=sd: tl.linear(pd, sd, fmt, x_dn, s_dn, out=y_dn, x_rot=xr_dn))])
    launch_bytes = [linear_bytes(2 * ng, kg, 1, fmt) - 2 * ng * 2,    # binary16 output
                    linear_bytes(nd, kd, 1, fmt)]
    io = dict(fmt=fmt, gu_packed=gu_packed, gu_scales=gu_scales, dn_packed=dn_packed,
              dn_scales=dn_scales, y_gu=y_gu, y_dn=y_dn, xr_gu=xr_gu, xr_dn=xr_dn, g=g, u=u, d=d,
              kd=kd)
    return steps, launch_bytes, io


def check_step_outputs(torch, tl, io):
    """After the timed steps: the step's outputs are finite and equal, bit for
    bit, the library's GEMV on the x_rot the fused launches wrote (one
    launch per linear, outside the timed region)."""
    y_gu = tl.gemv(io["gu_packed"], io["gu_scales"], io["fmt"], io["xr_gu"], out_dtype=torch.float16)
    y_dn = tl.gemv(io["dn_packed"], io["dn_scales"], io["fmt"], io["xr_dn"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    same = bool(torch.equal(y_gu.view(torch.int16), io["y_gu"].view(torch.int16)) and
                torch.equal(y_dn.view(torch.int32), io["y_dn"].view(torch.int32)))
    finite = bool(torch.isfinite(io["y_gu"].float()).all().item() and
                  torch.isfinite(io["y_dn"]).all().item())
    io["y_gu_host"] = io["y_gu"].cpu().numpy()
    io["y_dn_host"] = io["y_dn"].cpu().numpy()
    return {"finite": finite, "equal_to_gemv_on_x_rot": same}


def oracle_check_step(oracle, io, rows=32):
    """Sampled rows of the step's outputs against the oracle's layer (fp64
    rotation and product; down on the binary16 gate|up output the step
    produced): relative L2 errors, to compare with the 2e-3 bar."""
    import numpy as np
    rng = np.random.default_rng(7)
    g, u, d, kd = io["g"], io["u"], io["d"], io["kd"]
    codes_gu = np.concatenate([g.codes, u.codes])
    scales_gu = np.concatenate([g.scales, u.scales])
    y_gu, y_dn = io["y_gu_host"], io["y_dn_host"]
    r1 = rng.choice(codes_gu.shape[0], size=rows, replace=False)
    r2 = rng.choice(d.codes.shape[0], size=rows, replace=False)
    want_gu = oracle.linear(g.x, g.signs, codes_gu[r1], scales_gu[r1])
    want_dn = oracle.linear(y_gu[:, :kd], d.signs, d.codes[r2], d.scales[r2])
    return {"rows_per_linear": rows,
            "rel_l2_gate_up": float(oracle.rel_l2(y_gu[:, r1].astype(np.float64), want_gu)),
            "rel_l2_down": float(oracle.rel_l2(y_dn[:, r2].astype(np.float64), want_dn)),
            "bar": 2e-3}


def per_launch_times_us(torch, steps, reps, stream):
    """Duration of each launch of a step, measured with HIP events recorded on
    the launch stream between consecutive launches; everything is enqueued
    behind a GPU sleep, so that the time between two events is the launch's
    dispatch and execution, not the host's submission.  The median over the
    `reps` steps (at most 100, so that every launch and event fits in the
    queue before the sleep ends: a longer run made the host enqueue while the
    GPU waited, and single rows read tens of microseconds)."""
    reps = min(reps, 100)
    import statistics
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        torch.cuda._sleep(100_000_000)
        rows = []
        for r in range(reps):
            row = [torch.cuda.Event(enable_timing=True)]
            row[0].record(stream)
            for fn in steps[r % len(steps)]:
                fn()
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                row.append(e)
            rows.append(row)
        torch.cuda.synchronize()
    n = len(rows[0]) - 1
    return [statistics.median(row[j].elapsed_time(row[j + 1]) for row in rows) * 1e3 for j in range(n)]


def per_launch_us(torch, graphs, reps, stream):
    """Average duration of one launch, measured with an HIP event pair around
    each replay of one-kernel graphs on the launch stream (so the idle time
    between replays is not counted)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            graphs[i % len(graphs)].replay()
            b.record(stream)
        torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / reps * 1e3


def bench_stream_chain(torch, tl, synth, dev, stream, dependent=True, reps=5):
    """The 64-layer weight stream at M = 1 as one tl_linear_chain launch per
    token: per layer q|k|v, o, gate|up, down (the linears that read one input
    concatenated, one rotation each: 4 linears a layer), one layer generated
    and replicated into 64 distinct sets of buffers.  With `dependent`,
    every linear reads the binary16 output of the one before it (o the q part
    of q|k|v, gate|up the output of o, down the gate part of gate|up, the next
    layer's q|k|v the output of down), the data flow of a model whose
    attention, norms and SwiGLU are left out; the scales are multiplied by
    1/(0.02 sqrt(0.6 K)) so that the activations keep about unit variance
    along the 256 dependent linears.  Otherwise each linear reads its own
    synthetic input."""
    import numpy as np

    groups = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
    layer = []
    for grp in groups:
        k = synth.SHAPES[grp[0]][0]
        ins = [synth.linear_inputs(synth.SHAPES[g][1], k, 1, seed=0, cfg=5, layer=0,
                                   linear=synth.LINEAR_ID[g], outliers=g in ("q", "k", "v", "o"))
               for g in grp]
        sc = np.concatenate([i.scales for i in ins]).astype(np.float64)
        if dependent:
            sc = sc / (0.02 * np.sqrt(0.6 * k))
        codes = torch.from_numpy(np.concatenate([i.codes for i in ins])).to(dev)
        layer.append(dict(k=k, n=codes.shape[0], packed=tl.pack(codes, 1),
                          scales=torch.from_numpy(sc.astype(np.float16)).to(dev),
                          signs=torch.from_numpy(ins[0].signs).to(dev),
                          x=torch.from_numpy(ins[0].x).to(dev).view(-1)))
        del codes
    ops, prev = [], None
    weight_bytes = act_bytes = 0
    for li in range(synth.N_LAYERS):
        for spec in layer:
            y = torch.empty(spec["n"], dtype=torch.float16, device=dev)
            x = prev[:spec["k"]] if (dependent and prev is not None) else spec["x"]
            p = spec["packed"] if li == 0 else spec["packed"].clone()
            sc = spec["scales"] if li == 0 else spec["scales"].clone()
            ops.append(dict(packed=p, scales=sc, fmt=1, x=x, signs=spec["signs"], y=y))
            weight_bytes += p.numel() + sc.numel() * 2
            act_bytes += 2 * spec["k"] + spec["k"] + 2 * spec["n"]
            prev = y
    chain = tl.Chain(ops)
    with torch.cuda.stream(stream):
        chain()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            chain()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    err = chain.error()
    finite = bool(torch.isfinite(ops[-1]["y"].float()).all().item())
    del g, chain, ops, layer, prev
    torch.cuda.empty_cache()
    if err != 0:
        raise RuntimeError(f"tl_linear_chain reported error {err}")
    return {"layers": synth.N_LAYERS, "linears_per_layer": len(groups),
            "linears_per_launch": synth.N_LAYERS * len(groups), "launches_per_token": 1,
            "dependent": dependent, "last_output_finite": finite,
            "weight_bytes": int(weight_bytes), "activation_bytes": int(act_bytes),
            "ms_per_token": round(ms, 4), "weight_streams_per_s": round(1e3 / ms, 1),
            "GBs": round((weight_bytes + act_bytes) / (ms * 1e-3) / 1e9, 1)}


def host_cpu() -> dict:
    """The host's CPU: model name, logical CPUs, CPUs this process may use."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:   # pragma: no cover
        usable = os.cpu_count() or 1
    return {"model": model, "logical_cpus": os.cpu_count() or 1, "usable_cpus": usable}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--fmt", choices=tuple(FMT_NAMES), default="slot2")
    ap.add_argument("--copies", type=int, default=8,
                    help="distinct weight copies cycled through (defeats the last-level cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other-format and GEMM figures")
    ap.add_argument("--profile-pass", action="store_true",
                    help="for counter runs under rocprofv3: a 256 MiB device copy (the calibration "
                         "kernel, 3 launches) then 10 eager passes of the step's GEMVs; no timing")
    ap.add_argument("--read-floor", action="store_true",
                    help="time a read-only kernel at transfer sizes 4 MiB .. 512 MiB and exit")
    ap.add_argument("--profile-batched", action="store_true",
                    help="run only the batched-decode, quantiser and bf16 GEMM kernel set of "
                         "the counter runs")
    ap.add_argument("--profile-prefill", action="store_true",
                    help="for counter runs under rocprofv3: the calibration copy, then the prefill "
                         "GEMM (M=4096, gate and down) and the rotation at M=4096; no timing")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build has no "
              "multi-GPU path", file=sys.stderr)
        return 2

    import torch

    import synth
    import tl_hadamard_rotate_amd as tl

    dev = torch.device("cuda:0")
    fmt = FMT_NAMES[args.fmt]
    if fmt == 2 and not args.profile_pass:
        print("--fmt bit1 applies to --profile-pass; the 1-bit decode step is measured in the "
              "extras of the default run", file=sys.stderr)
        return 2
    stream = torch.cuda.Stream(dev)
    if args.profile_pass:
        return profile_pass(torch, tl, synth, dev, fmt)
    if args.profile_prefill:
        return profile_prefill(torch, tl, synth, dev)
    if args.profile_batched:
        return profile_batched(torch, tl, synth, dev)
    if args.read_floor:
        return read_floor(torch, tl, dev)

    extra = {}
    # the step: gate|up then down, two fused rotate + GEMV launches
    log(f"building the step (gate|up, down), fmt={args.fmt}, copies={args.copies}")
    steps, launch_bytes, step_io = build_mlp_step(torch, tl, synth, dev, args.copies, fmt)
    with torch.cuda.stream(stream):
        step_graphs = capture(torch, lambda c: [fn() for fn in steps[c]], args.copies, stream)
    log(f"timing {args.steps} steps after {args.warmup} warm-up steps")
    ms = timed_replays(torch, step_graphs, args.steps, args.warmup, stream) / args.steps
    sbytes = sum(launch_bytes)
    launches = 2
    per = per_launch_times_us(torch, steps, max(args.steps, 2 * args.copies), stream)
    extra["output_check"] = check_step_outputs(torch, tl, step_io)
    for key in ("gu_packed", "gu_scales", "dn_packed", "dn_scales", "y_gu", "y_dn", "xr_gu", "xr_dn"):
        del step_io[key]
    kern_us = sum(per) / len(per)
    per_launch = sbytes / len(per)
    kname = ("gemv_m1_slot2_kernel<FL, true> (tl_linear, rotation fused): gate|up and down"
             if fmt == 1 else
             "gemv_trit5_kernel<1, true, true> (tl_linear, rotation fused): gate|up and down")
    workload = ("decode step M=1 over the 27B-class MLP projections: gate|up (K=5120, "
                "N=2x17408, rows concatenated, one signed 1024-block Hadamard rotation of the "
                "input, binary16 output) then down (K=17408, N=5120) on the gate part of that "
                "output (the SwiGLU between them is outside the library), each one fused "
                "rotation + ternary g128 GEMV launch (tl_linear); binary16 activations, fp32 "
                "accumulation")
    extra["step_launches"] = [
        {"linear": "gate|up", "us": round(per[0], 3), "bytes": launch_bytes[0],
         "GBs": round(launch_bytes[0] / (per[0] * 1e-6) / 1e9, 1)},
        {"linear": "down", "us": round(per[1], 3), "bytes": launch_bytes[1],
         "GBs": round(launch_bytes[1] / (per[1] * 1e-6) / 1e9, 1)}]
    del step_graphs, steps
    torch.cuda.empty_cache()
    if fmt == 1:
        # the same step as one chain launch (down waits for gate|up on the device)
        log("the step as one tl_linear_chain launch")
        chains, cbytes = build_chain_step(torch, tl, synth, dev, args.copies)
        with torch.cuda.stream(stream):
            cg = capture(torch, lambda c: chains[c](), args.copies, stream)
        cms = timed_replays(torch, cg, args.steps, args.warmup, stream) / args.steps
        if any(c.error() for c in chains):
            raise RuntimeError(f"tl_linear_chain reported errors {[c.error() for c in chains]}")
        extra["step_as_chain"] = {"launches": 1, "ms_per_step": round(cms, 5),
                                  "step_bytes": cbytes,
                                  "step_GBs": round(cbytes / (cms * 1e-3) / 1e9, 1)}
        del cg, chains
        torch.cuda.empty_cache()
    # the three projections as separate launches (tl_linear per projection)
    log(f"separate launches per projection, fmt={args.fmt}")
    lins = build_step_inputs(torch, tl, synth, dev, fmt, args.copies)
    with torch.cuda.stream(stream):
        sep_graphs = capture(torch, lambda c: step_fn(tl, lins, fmt, c), args.copies, stream)
        gemv_graphs = capture(torch, lambda c: gemv_fn(tl, lins, fmt, c), args.copies, stream)
    sep_ms = timed_replays(torch, sep_graphs, args.steps, args.warmup, stream) / args.steps
    sep_bytes = sum(gemv_bytes(l["n"], l["k"], 1, fmt) + rotate_bytes(1, l["k"]) for l in lins)
    reps = max(args.steps, 3 * args.copies)
    g_ms = timed_replays(torch, gemv_graphs, reps, args.warmup, stream)
    g_us = g_ms * 1e3 / (3 * reps)
    g_bytes = sum(gemv_bytes(l["n"], l["k"], 1, fmt) for l in lins) / 3.0
    extra["separate_launches"] = {
        "fmt": args.fmt, "launches": 3, "ms_per_step": round(sep_ms, 5), "step_bytes": sep_bytes,
        "step_GBs": round(sep_bytes / (sep_ms * 1e-3) / 1e9, 1),
        "gemv_alone_avg_launch_us": round(g_us, 3),
        "gemv_alone_GBs": round(g_bytes / (g_us * 1e-6) / 1e9, 1)}
    del sep_graphs, gemv_graphs, lins
    torch.cuda.empty_cache()
    value = sbytes / (ms * 1e-3) / 1e9
    achieved = per_launch / (kern_us * 1e-6) / 1e9
    traffic = traffic_from_profiles(fmt)
    rp = rocprof_launch_us(fmt)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else round(traffic), "kernel": kname,
                "avg_launch_us": round(kern_us, 3),
                "avg_launch_us_step_timed": round(ms * 1e3 / launches, 3),
                "avg_launch_us_rocprof": rp,
                "frac_rocprof": None if rp is None else round(per_launch / (rp * 1e-6) / 1e9 /
                                                              HBM_PEAK_GBS, 4),
                "algorithmic_bytes_per_launch": round(per_launch)}
    log(f"step {ms * 1e3:.2f} us, {value:.1f} GB/s; dominant kernel {kern_us:.2f} us/launch, "
        f"{achieved:.1f} GB/s; separate launches {sep_ms * 1e3:.2f} us/step")

    if not args.no_extra:
        other = 1 - fmt
        oname = "slot2" if other == 1 else "trit5"
        log(f"the step (gate|up, down) with fmt={oname}")
        steps2, lb2, _ = build_mlp_step(torch, tl, synth, dev, args.copies, other)
        with torch.cuda.stream(stream):
            sg2 = capture(torch, lambda c: [fn() for fn in steps2[c]], args.copies, stream)
        ms3 = timed_replays(torch, sg2, args.steps, args.warmup, stream) / args.steps
        extra["other_format_step"] = {"fmt": oname, "launches": 2, "ms_per_step": round(ms3, 5),
                                      "step_bytes": sum(lb2),
                                      "step_GBs": round(sum(lb2) / (ms3 * 1e-3) / 1e9, 1)}
        del sg2, steps2
        torch.cuda.empty_cache()
        lins2 = build_step_inputs(torch, tl, synth, dev, other, args.copies)
        with torch.cuda.stream(stream):
            sg = capture(torch, lambda c: step_fn(tl, lins2, other, c), args.copies, stream)
            gg = capture(torch, lambda c: gemv_fn(tl, lins2, other, c), args.copies, stream)
        ms2 = timed_replays(torch, sg, args.steps, args.warmup, stream) / args.steps
        g2 = timed_replays(torch, gg, reps, args.warmup, stream)
        b2 = sum(gemv_bytes(l["n"], l["k"], 1, other) for l in lins2) / 3.0
        extra["other_format_separate_launches"] = {
            "fmt": "slot2" if other == 1 else "trit5",
            "step_GBs": round(sum(gemv_bytes(l["n"], l["k"], 1, other) + rotate_bytes(1, l["k"])
                                  for l in lins2) / (ms2 * 1e-3) / 1e9, 1),
            "ms_per_step": round(ms2, 5),
            "gemv_avg_launch_us": round(g2 * 1e3 / (3 * reps), 3),
            "gemv_GBs": round(b2 / (g2 * 1e-3 / (3 * reps)) / 1e9, 1)}
        del sg, gg, lins2
        torch.cuda.empty_cache()
        log("64-layer weight stream as one chain launch per token (dependent linears)")
        extra["weight_stream_chain"] = bench_stream_chain(torch, tl, synth, dev, stream, True)
        log("64-layer weight stream as one chain launch per token (independent inputs)")
        extra["weight_stream_chain_independent"] = bench_stream_chain(torch, tl, synth, dev, stream,
                                                                      False)
        log("64-layer weight stream, one tl_linear launch per linear")
        extra["weight_stream"] = bench_stream(torch, tl, synth, dev, fmt, stream)
        log("64-layer weight stream, one tl_linear launch per input (q|k|v and gate|up concatenated)")
        extra["weight_stream_shared_rotation"] = bench_stream_shared(torch, tl, synth, dev, fmt,
                                                                     stream)
        log("prefill GEMM (M = 512, 2048, 4096)")
        extra["gemm_prefill"] = bench_gemm(torch, tl, synth, dev, fmt)
        log("prefill GEMM with bfloat16 activations (M = 4096)")
        extra["gemm_prefill_bf16"] = bench_gemm(torch, tl, synth, dev, fmt, bf16=True,
                                                ms_list=(4096,))
        log("batched decode GEMV over q, k, v, o (M = 1..16)")
        extra["batched_decode"] = bench_batched(torch, tl, synth, dev, fmt)
        log("rotation at prefill size")
        extra["rotate_prefill"] = bench_rotate_prefill(torch, tl, dev)
        log("weight quantiser (rotation folded in), gate and down")
        extra["quantize"] = bench_quantize(torch, tl, synth, dev)
        log("decode step with 1-bit weights")
        extra["bit1_decode"] = bench_bit1(torch, tl, synth, dev, stream, args.copies, args.steps,
                                          args.warmup)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle   # the checker, timed as the CPU baseline; the GPU path never uses it
        log("timing the CPU oracle sample")
        cpu = cpu_baseline(oracle, synth, fmt)
        log("sampled rows of the step's outputs against the oracle")
        extra["output_check"].update(oracle_check_step(oracle, step_io))

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": workload, "format": args.fmt, "M": 1,
                   "weight_copies": args.copies, "step_bytes": sbytes,
                   "launches_per_step": launches},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
