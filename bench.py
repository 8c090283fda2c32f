"""Benchmark of the ternary g128 decode path on one MI355X.

A step is one decode pass (M = 1) over the 27B-class MLP projections
gate (K=5120, N=17408), up (K=5120, N=17408) and down (K=17408, N=5120): for
each projection the signed 1024-block Hadamard rotation of its input followed
by the ternary GEMV.  Inputs are seeded synthetic tensors with the workload's
distributions.  The weights are replicated into --copies distinct device
buffers and the steps cycle through them, so that no step finds its weights in
the 256 MB last-level cache.

Prints one JSON line on stdout; progress goes to stderr.
    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
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

METRIC = "ternary GEMV GB/s (% HBM peak) + prefill GEMM TFLOP/s at 27B-class shapes"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2516.6
STEP_LINEARS = ("gate", "up", "down")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemv_bytes(n: int, k: int, m: int, fmt: int) -> int:
    """Algorithmic bytes of one GEMV launch: packed codes + binary16 scales +
    binary16 activations read, fp32 outputs written."""
    code_bytes = n * (k // 128) * 26 if fmt == 0 else n * k // 4
    return code_bytes + n * (k // 128) * 2 + m * k * 2 + m * n * 4


def rotate_bytes(m: int, k: int) -> int:
    """Algorithmic bytes of one rotation: binary16 in and out, int8 signs."""
    return 2 * m * k * 2 + k


def build_step_inputs(torch, tl, synth, dev, fmt: int, copies: int):
    per_linear = []
    for name in STEP_LINEARS:
        k, n = synth.SHAPES[name]
        inp = synth.linear_inputs(n, k, 1, seed=0, cfg=2, layer=0, linear=synth.LINEAR_ID[name])
        codes = torch.from_numpy(inp.codes).to(dev)
        packed = tl.pack(codes, fmt)
        del codes
        scales = torch.from_numpy(inp.scales).to(dev)
        packs = [packed] + [packed.clone() for _ in range(copies - 1)]
        scs = [scales] + [scales.clone() for _ in range(copies - 1)]
        per_linear.append(dict(
            name=name, n=n, k=k, packs=packs, scales=scs,
            x=torch.from_numpy(inp.x).to(dev), signs=torch.from_numpy(inp.signs).to(dev),
            x_rot=torch.empty((1, k), dtype=torch.float16, device=dev),
            y=torch.empty((1, n), dtype=torch.float32, device=dev), inp=inp))
    return per_linear


def run_steps(torch, tl, lins, fmt, steps, warmup, copies, time_kernels=True):
    def step(i, evs=None):
        c = i % copies
        for lin in lins:
            tl.hadamard_rotate(lin["x"], lin["signs"], out=lin["x_rot"])
            if evs is not None:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                tl.gemv(lin["packs"][c], lin["scales"][c], fmt, lin["x_rot"], out=lin["y"])
                b.record()
                evs.append((lin["name"], a, b))
            else:
                tl.gemv(lin["packs"][c], lin["scales"][c], fmt, lin["x_rot"], out=lin["y"])

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [] if time_kernels else None
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        step(warmup + i, evs)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    kern = {}
    if evs:
        for name, a, b in evs:
            kern.setdefault(name, []).append(a.elapsed_time(b))
    return ms, wall, kern


def step_bytes(lins, fmt):
    return sum(gemv_bytes(l["n"], l["k"], 1, fmt) + rotate_bytes(1, l["k"]) for l in lins)


def cpu_baseline(oracle, lins, fmt, tl, budget_s=12.0):
    """The oracle as it stands, timed on the host on a bounded sample: the
    rotation plus unpack/dequant/fp64 matmul of the first rows of each
    projection.  Reported in the metric's unit (algorithmic GB/s)."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    rows = 512
    samples = []
    for lin in lins:
        inp = lin["inp"]
        packed = oracle.pack(inp.codes[:rows], fmt)
        samples.append((inp, packed, lin["k"]))
    done_bytes, t0, reps = 0, time.perf_counter(), 0
    while True:
        for inp, packed, k in samples:
            x_rot = oracle.rotate(inp.x, inp.signs)
            oracle.matvec_packed(packed, inp.scales[:rows], fmt, x_rot, k)
            done_bytes += gemv_bytes(rows, k, 1, fmt) + rotate_bytes(1, k)
        reps += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {rows} rows of gate, up and down at M=1 (rotate + unpack + "
                      f"fp64 dequant matmul), {reps} passes in {dt:.1f} s"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--fmt", choices=("trit5", "slot2"), default="trit5")
    ap.add_argument("--copies", type=int, default=16,
                    help="distinct weight copies cycled through (defeats the last-level cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the SLOT2 and GEMM side figures")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        return 2

    import torch

    import synth
    import tl_hadamard_rotate_amd as tl

    dev = torch.device("cuda:0")
    fmt = tl.FMT_TRIT5 if args.fmt == "trit5" else tl.FMT_SLOT2
    log(f"building inputs fmt={args.fmt} copies={args.copies}")
    lins = build_step_inputs(torch, tl, synth, dev, fmt, args.copies)
    log("timing")
    ms, wall, kern = run_steps(torch, tl, lins, fmt, args.steps, args.warmup, args.copies)
    sbytes = step_bytes(lins, fmt)
    value = sbytes / (ms * 1e-3) / 1e9

    # dominant kernel: the GEMV; algorithmic bytes over its average launch time
    g_bytes = sum(gemv_bytes(l["n"], l["k"], 1, fmt) for l in lins) * args.steps
    g_ms = sum(sum(v) for v in kern.values())
    g_launches = sum(len(v) for v in kern.values())
    achieved = g_bytes / (g_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "tl_gemv", "launches": g_launches,
                "avg_launch_us": round(g_ms * 1e3 / max(g_launches, 1), 3),
                "per_linear_us": {k: round(1e3 * float(np.mean(v)), 3) for k, v in kern.items()}}
    log(f"step {ms:.4f} ms, {value:.1f} GB/s; gemv {achieved:.1f} GB/s")

    extra = {}
    if not args.no_extra:
        other = tl.FMT_SLOT2 if fmt == tl.FMT_TRIT5 else tl.FMT_TRIT5
        del lins
        torch.cuda.empty_cache()
        lins2 = build_step_inputs(torch, tl, synth, dev, other, args.copies)
        ms2, _, kern2 = run_steps(torch, tl, lins2, other, args.steps, args.warmup, args.copies)
        g2 = sum(gemv_bytes(l["n"], l["k"], 1, other) for l in lins2) * args.steps
        extra["other_format"] = {
            "fmt": "slot2" if other == tl.FMT_SLOT2 else "trit5",
            "step_GBs": round(step_bytes(lins2, other) / (ms2 * 1e-3) / 1e9, 1),
            "ms_per_step": round(ms2, 5),
            "gemv_GBs": round(g2 / (sum(sum(v) for v in kern2.values()) * 1e-3) / 1e9, 1)}
        del lins2
        torch.cuda.empty_cache()
        extra["gemm"] = bench_gemm(torch, tl, synth, dev, fmt)
        lins = None

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("timing the CPU oracle sample")
        lins_cpu = [dict(n=synth.SHAPES[n][1], k=synth.SHAPES[n][0],
                         inp=synth.linear_inputs(512, synth.SHAPES[n][0], 1, seed=0, cfg=2,
                                                 layer=0, linear=synth.LINEAR_ID[n]))
                    for n in STEP_LINEARS]
        cpu = cpu_baseline(oracle, lins_cpu, fmt, tl)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "decode step M=1 over 27B-class MLP projections gate/up "
                               "(K=5120, N=17408) and down (K=17408, N=5120): signed "
                               "1024-block Hadamard rotation + ternary g128 GEMV per "
                               "projection; fp16 activations, fp32 accumulation",
                   "format": args.fmt, "M": 1, "weight_copies": args.copies,
                   "step_bytes": sbytes},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_gemm(torch, tl, synth, dev, fmt, m=2048, reps=5):
    """Prefill GEMM TFLOP/s at M=2048, K=5120, N=17408 (side figure)."""
    k, n = synth.SHAPES["gate"]
    inp = synth.linear_inputs(n, k, 1, seed=0, cfg=4, linear=4)
    packed = tl.pack(torch.from_numpy(inp.codes).to(dev), fmt)
    scales = torch.from_numpy(inp.scales).to(dev)
    x = torch.randn((m, k), device=dev, dtype=torch.float32).to(torch.float16)
    y = torch.empty((m, n), dtype=torch.float32, device=dev)
    tl.gemm(packed, scales, fmt, x, out=y)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        tl.gemm(packed, scales, fmt, x, out=y)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    tflops = 2.0 * m * n * k / (ms * 1e-3) / 1e12
    return {"M": m, "K": k, "N": n, "ms": round(ms, 4), "TFLOPs": round(tflops, 2),
            "frac_of_fp16_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)}


if __name__ == "__main__":
    sys.exit(main())
