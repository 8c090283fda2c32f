"""GPU parity of decode chains (tl_linear_chain): a list of M = 1 linears
run in one launch, inputs either ready at launch or read from an earlier
linear's binary16 output.  Every linear's output must equal, bit for bit,
tl_linear on the same input (the chain runs the same per-row arithmetic),
and match the oracle's layer on sampled rows (relative L2 < 2e-3); captured
graphs replay correctly; failures (a bad plan, an input wait that gives up)
are reported in the error word and leave the sync buffer usable."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tl_hadamard_rotate_amd as tl

pytestmark = pytest.mark.gpu

SLOT2 = tl.FMT_SLOT2


def dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def _weights(name, n, k, device, layer=0, scale=None):
    """Packed weights of a linear; `scale` multiplies the scales (in fp64,
    then rounded to binary16) to keep a long chain's activations in range."""
    inp = synth.linear_inputs(n, k, 1, cfg=5, layer=layer, linear=synth.LINEAR_ID.get(name, 9),
                              outliers=True)
    scales = inp.scales if scale is None else (inp.scales.astype(np.float64) * scale).astype(np.float16)
    return dict(codes=inp.codes, scales16=scales, signs_np=inp.signs, x_np=inp.x,
                packed=tl.pack(dev(inp.codes, device), SLOT2), scales=dev(scales, device),
                signs=dev(inp.signs, device))


def _check_op(o, x_vals, y, rows_per=200):
    """y of one chain linear: bit-identical to tl_linear on x_vals, and the
    oracle's layer on sampled rows."""
    xt = x_vals.reshape(1, -1).contiguous()
    ref = tl.linear(o["packed"], o["scales"], SLOT2, xt, o["signs"], out_dtype=y.dtype)
    got = host(y).reshape(-1)
    bits = np.uint32 if y.dtype == torch.float32 else np.uint16
    assert np.array_equal(got.view(bits), host(ref).reshape(-1).view(bits))
    n = got.size
    rows = np.unique(np.concatenate([np.random.default_rng(n).choice(n, size=min(n, rows_per),
                                                                      replace=False), [0, n - 1]]))
    want = oracle.linear(host(xt), o["signs_np"], o["codes"][rows], o["scales16"][rows])[0]
    assert oracle.rel_l2(got[rows].astype(np.float64), want) < 2e-3


def test_chain_independent_linears_match_tl_linear(gpu):
    """q|k|v, o, gate|up and down of one layer, each on its own input
    (no waits), fp32 and binary16 outputs, x_rot written for two of them."""
    ops, checks = [], []
    shapes = [("qkv", 8192, 5120), ("o", 5120, 6144), ("gateup", 34816, 5120), ("down", 5120, 17408)]
    for i, (name, n, k) in enumerate(shapes):
        w = _weights(name, n, k, gpu)
        x = dev(w["x_np"], gpu)
        y = torch.empty(n, dtype=torch.float32 if i % 2 == 0 else torch.float16, device=gpu)
        xr = torch.empty(k, dtype=torch.float16, device=gpu) if i < 2 else None
        ops.append(dict(packed=w["packed"], scales=w["scales"], fmt=SLOT2, x=x, signs=w["signs"],
                        y=y, x_rot=xr))
        checks.append((w, x, y, xr))
    chain = tl.Chain(ops)
    chain()
    torch.cuda.synchronize()
    assert chain.error() == 0
    assert int(chain.sync.abs().sum().item()) == 0       # counters reset for the next call
    for w, x, y, xr in checks:
        _check_op(w, x, y)
        if xr is not None:
            ref = torch.empty_like(xr).view(1, -1)
            tl.linear(w["packed"], w["scales"], SLOT2, x.view(1, -1), w["signs"], x_rot=ref)
            assert torch.equal(xr.view(torch.int16), ref.view(-1).view(torch.int16))


def test_chain_with_dependencies(gpu):
    """Two layers of q|k|v -> o -> gate|up -> down where each linear reads
    the previous one's binary16 output (o the q part of q|k|v, down the gate
    part of gate|up; the operations between linears in a model are left
    out), the scales shrunk so that the activations stay in range; every
    output checked after the chain against tl_linear on the values it read."""
    shapes = [("qkv", 8192, 5120), ("o", 5120, 6144), ("gateup", 34816, 5120), ("down", 5120, 17408)]
    ws = [_weights(name, n, k, gpu, scale=1.0 / (0.02 * np.sqrt(0.6 * k)))
          for name, n, k in shapes]
    x0 = dev(ws[0]["x_np"], gpu).view(-1)
    ops, outs = [], []
    prev = None
    for layer in range(2):
        for i, ((name, n, k), w) in enumerate(zip(shapes, ws)):
            if prev is None:
                x = x0
            else:
                x = prev[:k]            # q of q|k|v, gate of gate|up, or the whole output
            y = torch.empty(n, dtype=torch.float16, device=gpu)
            ops.append(dict(packed=w["packed"], scales=w["scales"], fmt=SLOT2, x=x,
                            signs=w["signs"], y=y))
            outs.append((w, x, y))
            prev = y
    chain = tl.Chain(ops)
    for rep in range(2):
        for _, _, y in outs:
            y.fill_(float("nan"))
        chain()
        torch.cuda.synchronize()
        assert chain.error() == 0, rep
        assert int(chain.sync.abs().sum().item()) == 0
        for w, x, y in outs:
            assert torch.isfinite(y.float()).all()
            _check_op(w, x, y)


def test_chain_graph_replays(gpu):
    """A dependent chain captured in a HIP graph, replayed three times with
    eager library work between the replays; every replay equals the eager
    chain bit for bit."""
    shapes = [("gateup", 34816, 5120), ("down", 5120, 17408), ("qkv", 8192, 5120)]
    ws = [_weights(name, n, k, gpu, scale=1.0 / (0.02 * np.sqrt(0.6 * k))) for name, n, k in shapes]
    x = dev(ws[0]["x_np"], gpu).view(-1)
    y0 = torch.empty(34816, dtype=torch.float16, device=gpu)
    y1 = torch.empty(5120, dtype=torch.float16, device=gpu)
    y2 = torch.empty(8192, dtype=torch.float32, device=gpu)
    ops = [dict(packed=ws[0]["packed"], scales=ws[0]["scales"], fmt=SLOT2, x=x, signs=ws[0]["signs"], y=y0),
           dict(packed=ws[1]["packed"], scales=ws[1]["scales"], fmt=SLOT2, x=y0[:17408],
                signs=ws[1]["signs"], y=y1),
           dict(packed=ws[2]["packed"], scales=ws[2]["scales"], fmt=SLOT2, x=y1, signs=ws[2]["signs"], y=y2)]
    chain = tl.Chain(ops)
    stream = torch.cuda.Stream(gpu)
    with torch.cuda.stream(stream):
        chain()
        torch.cuda.synchronize()
        eager = [host(y).copy() for y in (y0, y1, y2)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            chain()
    torch.cuda.synchronize()
    for rep in range(3):
        for y in (y0, y1, y2):
            y.fill_(float("nan"))
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert chain.error() == 0
        for a, b in zip(eager, (y0, y1, y2)):
            bits = np.uint32 if b.dtype == torch.float32 else np.uint16
            assert np.array_equal(host(b).view(bits), a.view(bits)), rep
        tl.linear(ws[rep]["packed"], ws[rep]["scales"], SLOT2, dev(ws[rep]["x_np"], gpu),
                  ws[rep]["signs"])
        torch.cuda.synchronize()


def test_chain_small_and_ragged(gpu):
    """Linears with fewer rows than CUs (workgroups without rows), ragged row
    counts and one block: results still equal tl_linear's."""
    specs = [(1, 1024), (67, 2048), (300, 1024), (4097, 3072)]
    ops, outs = [], []
    for n, k in specs:
        w = _weights("x", n, k, gpu)
        x = dev(w["x_np"], gpu).view(-1)
        y = torch.empty(n, dtype=torch.float32, device=gpu)
        ops.append(dict(packed=w["packed"], scales=w["scales"], fmt=SLOT2, x=x, signs=w["signs"], y=y))
        outs.append((w, x, y))
    chain = tl.Chain(ops)
    chain()
    torch.cuda.synchronize()
    assert chain.error() == 0
    for w, x, y in outs:
        _check_op(w, x, y)


def test_chain_bad_plan_reports_and_recovers(gpu):
    """A plan whose recorded count does not match the call's: the kernel
    writes nothing but the error word 1, leaves the counters at zero, and
    the chain runs normally once the error word is cleared and the plan is
    right again."""
    w = _weights("x", 2048, 2048, gpu)
    x = dev(w["x_np"], gpu).view(-1)
    y = torch.full((2048,), 7.0, dtype=torch.float32, device=gpu)
    chain = tl.Chain([dict(packed=w["packed"], scales=w["scales"], fmt=SLOT2, x=x, signs=w["signs"], y=y)])
    good = chain.plan.clone()
    chain.plan[4] = 5                      # bytes 4..7: the count
    chain()
    torch.cuda.synchronize()
    assert chain.error() == 1
    assert torch.all(y == 7.0)
    assert int(chain.sync[:chain.count + 1].abs().sum().item()) == 0
    chain.plan.copy_(good)
    chain.clear_error()
    chain()
    torch.cuda.synchronize()
    assert chain.error() == 0
    _check_op(w, x, y)


def test_chain_wait_limit(gpu):
    """The input waits are bounded: with a poll limit of 0 a linear whose
    input is not complete at its first look gives up.  Either every wait
    happened to find its input complete (then the outputs are right) or the
    error word names the linear that gave up; in both cases the counters
    are back at zero and, with the default limit restored, the chain runs
    correctly."""
    shapes = [("gateup", 34816, 5120), ("down", 5120, 17408)]
    ws = [_weights(name, n, k, gpu, scale=1.0 / (0.02 * np.sqrt(0.6 * k))) for name, n, k in shapes]
    x = dev(ws[0]["x_np"], gpu).view(-1)
    y0 = torch.empty(34816, dtype=torch.float16, device=gpu)
    y1 = torch.empty(5120, dtype=torch.float16, device=gpu)
    chain = tl.Chain([dict(packed=ws[0]["packed"], scales=ws[0]["scales"], fmt=SLOT2, x=x,
                           signs=ws[0]["signs"], y=y0),
                      dict(packed=ws[1]["packed"], scales=ws[1]["scales"], fmt=SLOT2, x=y0[:17408],
                           signs=ws[1]["signs"], y=y1)])
    good = chain.plan.clone()
    chain.plan[12:16] = 0                  # bytes 12..15: the poll limit
    chain()
    torch.cuda.synchronize()
    e = chain.error()
    assert e in (0, 3), e                   # 2 + index of the waiting linear
    assert int(chain.sync[:chain.count + 1].abs().sum().item()) == 0
    if e == 0:
        _check_op(ws[1], y0[:17408], y1)
    chain.plan.copy_(good)
    chain.clear_error()
    chain()
    torch.cuda.synchronize()
    assert chain.error() == 0
    _check_op(ws[0], x, y0)
    _check_op(ws[1], y0[:17408], y1)
