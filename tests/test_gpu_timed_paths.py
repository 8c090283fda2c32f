"""GPU parity on the launch plans the benchmark times, at the workloads' full
sizes: the prefill GEMM at M = 512, 2048, 4096 (whole tiles and K-split
tiles), the batched decode GEMV over the attention projections with
outliers, the fused M = 1 path on the o projection, the decode step as the
benchmark runs it (gate|up concatenated, then down), a captured graph of a
whole layer, and guard bands around every output of ragged shapes.

Full-size outputs are checked on samples the oracle computes one by one:
one token from every 256-row tile and one output column from every 256-wide
tile (plus the first and last of each), so every tile of the launch is
touched.  Two bars, as everywhere in these tests: against the oracle's
product on the binary16 rotated activations the kernel read (exact products,
fp32 sums: relative L2 < 1e-5), and against the fp64 layer on the unrotated
activations (relative L2 < 2e-3, the target's bar)."""
import functools

import numpy as np
import pytest
import torch

import oracle
import synth
import tl_hadamard_rotate_amd as tl

pytestmark = pytest.mark.gpu

FMTS = (tl.FMT_TRIT5, tl.FMT_SLOT2)
FMT_NAME = {tl.FMT_TRIT5: "trit5", tl.FMT_SLOT2: "slot2"}


def dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def tile_samples(size, tile, rng):
    """One random index per tile of `tile` along an axis of `size`, plus the
    first and last index of every tile."""
    out = set()
    for t0 in range(0, size, tile):
        t1 = min(size, t0 + tile)
        out.update((t0, t1 - 1, int(rng.integers(t0, t1))))
    return np.array(sorted(out))


@functools.lru_cache(maxsize=2)
def _inputs(name, m, cfg, outliers):
    k, n = synth.SHAPES[name]
    return synth.linear_inputs(n, k, m, cfg=cfg, linear=synth.LINEAR_ID[name], outliers=outliers)


def _check_sampled(y, inp, x_rot16, toks, rows, tight=1e-5):
    """y [M, N] (fp32 or binary16) on the sampled tokens x rows against the
    oracle's product on the kernel's x_rot and the fp64 layer."""
    ys = np.asarray(y, dtype=np.float64)[np.ix_(toks, rows)]
    want16 = oracle.matvec(inp.codes[rows], inp.scales[rows], x_rot16[toks])
    want = oracle.linear(inp.x[toks], inp.signs, inp.codes[rows], inp.scales[rows])
    return oracle.rel_l2(ys, want16), oracle.rel_l2(ys, want)


# ---------------------------------------------------------------------------
# prefill GEMM at the workload sizes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
@pytest.mark.parametrize("m", synth.PREFILL_M)
@pytest.mark.parametrize("shape", ["gate", "down"])
def test_gemm_prefill_full_size_every_tile(gpu, shape, m, fmt):
    """tl_gemm at M = 512, 2048, 4096 on the MLP shapes, fp32 and binary16
    output; one sampled output in every output tile, so the whole-tile
    epilogue and the K-split parts + reduction are both checked wherever
    the plan uses them."""
    k, n = synth.SHAPES[shape]
    inp = _inputs(shape, 4096, 4, False)
    x = inp.x[:m]
    packed = tl.pack(dev(inp.codes, gpu), fmt)
    scales = dev(inp.scales, gpu)
    x_rot = tl.hadamard_rotate(dev(x, gpu), dev(inp.signs, gpu))
    tiles, whole, splits = tl.gemm_plan(m, n, k)
    assert tiles == -(-m // 256) * -(-n // 256)
    y32 = host(tl.gemm(packed, scales, fmt, x_rot))
    y16 = host(tl.gemm(packed, scales, fmt, x_rot, out_dtype=torch.float16))
    rng = np.random.default_rng(m + n)
    toks, rows = tile_samples(m, 256, rng), tile_samples(n, 256, rng)
    xr = host(x_rot)
    sub = type(inp)(signs=inp.signs, codes=inp.codes, scales=inp.scales, x=x)
    e16, e = _check_sampled(y32, sub, xr, toks, rows)
    assert e16 < 1e-5 and e < 2e-3, (tiles, whole, splits, e16, e)
    # binary16 output = the fp32 result rounded to nearest even
    assert np.array_equal(y16.view(np.uint16), y32.astype(np.float16).view(np.uint16))
    _, e_h = _check_sampled(y16, sub, xr, toks, rows)
    assert e_h < 2e-3


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
@pytest.mark.parametrize("m,n,plan", [(1000, 16300, "whole"), (1000, 16600, "whole+split")])
def test_gemm_plans_element_by_element(gpu, m, n, plan, fmt):
    """Small K, many tiles, every output checked: 4 x 64 = 256 tiles (one
    whole round of workgroups: no split) and 4 x 65 = 260 tiles (256 whole,
    the last 4 split along K and reduced); ragged last tile row and column;
    fp32 output row by row, binary16 output = the fp32 one rounded."""
    k = 1024
    tiles, whole, splits = tl.gemm_plan(m, n, k)
    if torch.cuda.get_device_properties(gpu).multi_processor_count != 256:
        pytest.skip("plans asserted for a 256-CU device")
    if plan == "whole":
        assert (tiles, whole, splits) == (256, 256, 1)
    else:
        assert tiles == 260 and whole == 256 and splits > 1
    inp = synth.linear_inputs(n, k, m, cfg=4, linear=n)
    x_rot16 = oracle.rotate(inp.x, inp.signs).astype(np.float16)
    packed = tl.pack(dev(inp.codes, gpu), fmt)
    sc, xr = dev(inp.scales, gpu), dev(x_rot16, gpu)
    y = host(tl.gemm(packed, sc, fmt, xr))
    yh = host(tl.gemm(packed, sc, fmt, xr, out_dtype=torch.float16))
    want = oracle.matvec(inp.codes, inp.scales, x_rot16)
    assert oracle.rel_l2(y.astype(np.float64), want) < 1e-5
    # per output column and per token: no tile may hide behind the others
    d = y.astype(np.float64) - want
    assert (np.linalg.norm(d, axis=0) / np.linalg.norm(want, axis=0)).max() < 1e-5
    assert (np.linalg.norm(d, axis=1) / np.linalg.norm(want, axis=1)).max() < 1e-5
    assert np.array_equal(yh.view(np.uint16), y.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
def test_gemm_result_ignores_workspace_contents(gpu, fmt):
    """The workspace's contents on entry do not matter: a call on a
    workspace full of garbage gives the same bits as one on a fresh one."""
    m, n, k = 600, 1300, 3072
    inp = synth.linear_inputs(n, k, m, cfg=4, linear=3)
    packed = tl.pack(dev(inp.codes, gpu), fmt)
    sc = dev(inp.scales, gpu)
    x = dev(oracle.rotate(inp.x, inp.signs).astype(np.float16), gpu)
    need = tl.gemm_workspace_bytes(m, n, k, fmt)
    assert need > 0
    ws = torch.full((need,), 0xA7, dtype=torch.uint8, device=gpu)
    a = host(tl.gemm(packed, sc, fmt, x, workspace=ws))
    ws.fill_(0x7F)
    b = host(tl.gemm(packed, sc, fmt, x, workspace=ws))
    c = host(tl.gemm(packed, sc, fmt, x))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))
    with pytest.raises(tl.TLError, match="WORKSPACE"):
        tl.gemm(packed, sc, fmt, x, workspace=ws[:need - 256])


# ---------------------------------------------------------------------------
# batched decode GEMV over the attention projections
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
@pytest.mark.parametrize("shape", ["q", "k", "v", "o", "down"])
def test_batched_decode_full_size(gpu, shape, fmt):
    """tl_gemv at M = 2, 4, 8, 16 on q, k, v, o with 1 % outliers x 20 (the
    attention workload), and on down (K = 17408), whose activations at
    M = 4..8 do not fit in LDS beside the decode table; every token, one
    sampled row in every 16-row tile plus tile edges, binary16 output at
    M = 16."""
    k, n = synth.SHAPES[shape]
    inp = _inputs(shape, 16, 3, True)
    packed = tl.pack(dev(inp.codes, gpu), fmt)
    scales = dev(inp.scales, gpu)
    x_rot = tl.hadamard_rotate(dev(inp.x, gpu), dev(inp.signs, gpu))
    xr = host(x_rot)
    rng = np.random.default_rng(n + k)
    rows = tile_samples(n, 16, rng)
    for m in (2, 4, 8, 16):
        xm = x_rot[:m].contiguous()
        sub = type(inp)(signs=inp.signs, codes=inp.codes, scales=inp.scales, x=inp.x[:m])
        y = host(tl.gemv(packed, scales, fmt, xm))
        e16, e = _check_sampled(y, sub, xr[:m], np.arange(m), rows)
        assert e16 < 1e-5 and e < 2e-3, (m, e16, e)
        if m == 16:
            yh = host(tl.gemv(packed, scales, fmt, xm, out_dtype=torch.float16))
            assert np.array_equal(yh.view(np.uint16), y.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
def test_batched_decode_qkv_concatenated(gpu, fmt):
    """q, k and v read one input, so their rows concatenated along N run as
    one tl_linear (one rotation, one launch) at M = 1, 2, 4, 8, 16: every
    token on sampled rows of each part against the oracle, and each part
    equal to that projection's own call to fp32 rounding (a launch's plan
    follows its rows: with dense trits the K split, with 2-bit slots at
    M = 5..8 the token groups, one of 8 or two of 4, which sum the digit
    offsets in different orders), bit for bit for q with 2-bit slots, whose
    own launch has the plan of q|k|v."""
    ins = {c: _inputs(c, 16, 3, True) for c in "qkv"}
    codes = np.concatenate([ins[c].codes for c in "qkv"])
    scales = np.concatenate([ins[c].scales for c in "qkv"])
    bounds = np.cumsum([0] + [ins[c].codes.shape[0] for c in "qkv"])
    x, signs = ins["q"].x, ins["q"].signs
    packed = tl.pack(dev(codes, gpu), fmt)
    sc = dev(scales, gpu)
    parts = {c: (tl.pack(dev(ins[c].codes, gpu), fmt), dev(ins[c].scales, gpu)) for c in "qkv"}
    rng = np.random.default_rng(7)
    for m in synth.BATCHED_M:
        xm, sg = dev(x[:m], gpu), dev(signs, gpu)
        x_rot = torch.empty((m, x.shape[1]), dtype=torch.float16, device=gpu)
        y = host(tl.linear(packed, sc, fmt, xm, sg, x_rot=x_rot))
        xr = host(x_rot)
        for i, c in enumerate("qkv"):
            r0, r1 = bounds[i], bounds[i + 1]
            yc = y[:, r0:r1]
            own = host(tl.linear(parts[c][0], parts[c][1], fmt, xm, sg))
            if fmt == tl.FMT_SLOT2 and c == "q":
                assert np.array_equal(yc.view(np.uint32), own.view(np.uint32)), (m, c)
            assert oracle.rel_l2(yc, own) < 1e-6, (m, c)
            sub = type(ins[c])(signs=signs, codes=ins[c].codes, scales=ins[c].scales, x=x[:m])
            rows = tile_samples(r1 - r0, 64, rng)
            e16, e = _check_sampled(yc, sub, xr, np.arange(m), rows)
            assert e16 < 1e-5 and e < 2e-3, (m, c, e16, e)


# ---------------------------------------------------------------------------
# fused M = 1 path on the o projection, and a captured layer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16], ids=["f32", "f16"])
@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
def test_linear_o_projection(gpu, fmt, out_dtype):
    """tl_linear at M = 1 on o (K = 6144, N = 5120): its own launch plan
    of the fused kernels; every output row against the oracle."""
    k, n = synth.SHAPES["o"]
    inp = synth.linear_inputs(n, k, 1, cfg=5, linear=synth.LINEAR_ID["o"], outliers=True)
    packed = tl.pack(dev(inp.codes, gpu), fmt)
    x_rot = torch.empty((1, k), dtype=torch.float16, device=gpu)
    y = host(tl.linear(packed, dev(inp.scales, gpu), fmt, dev(inp.x, gpu), dev(inp.signs, gpu),
                       out_dtype=out_dtype, x_rot=x_rot)).astype(np.float64)
    xr = host(x_rot)
    assert oracle.rel_l2(y, oracle.matvec(inp.codes, inp.scales, xr)) < (
        1e-5 if out_dtype == torch.float32 else 2e-3)
    assert oracle.rel_l2(y, oracle.linear(inp.x, inp.signs, inp.codes, inp.scales)) < 2e-3


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
def test_decode_step_as_benchmarked(gpu, fmt):
    """The benchmark's decode step at M = 1: tl_linear on gate|up (rows
    concatenated, N = 34816, K = 5120, binary16 output), then tl_linear on
    down (K = 17408) reading the gate part of that output.  Every output of
    both launches against the oracle: on the binary16 rotated activations
    each launch read, and on the fp64 layer of its own input."""
    ins = {name: synth.linear_inputs(synth.SHAPES[name][1], synth.SHAPES[name][0], 1, cfg=2,
                                     linear=synth.LINEAR_ID[name])
           for name in ("gate", "up", "down")}
    g, u, d = ins["gate"], ins["up"], ins["down"]
    codes_gu = np.concatenate([g.codes, u.codes])
    scales_gu = np.concatenate([g.scales, u.scales])
    kg, kd = synth.SHAPES["gate"][0], synth.SHAPES["down"][0]
    y_gu = torch.empty((1, codes_gu.shape[0]), dtype=torch.float16, device=gpu)
    xr_gu = torch.empty((1, kg), dtype=torch.float16, device=gpu)
    xr_dn = torch.empty((1, kd), dtype=torch.float16, device=gpu)
    tl.linear(tl.pack(dev(codes_gu, gpu), fmt), dev(scales_gu, gpu), fmt, dev(g.x, gpu),
              dev(g.signs, gpu), out_dtype=torch.float16, out=y_gu, x_rot=xr_gu)
    y_dn = tl.linear(tl.pack(dev(d.codes, gpu), fmt), dev(d.scales, gpu), fmt, y_gu[:, :kd],
                     dev(d.signs, gpu), x_rot=xr_dn)
    got_gu = host(y_gu).astype(np.float64)
    # binary16 outputs: the fp32 sums rounded once more (half an ulp)
    assert oracle.rel_l2(got_gu, oracle.matvec(codes_gu, scales_gu, host(xr_gu))) < 1e-3
    assert oracle.rel_l2(got_gu, oracle.linear(g.x, g.signs, codes_gu, scales_gu)) < 2e-3
    x_dn = host(y_gu)[:, :kd]
    got_dn = host(y_dn).astype(np.float64)
    assert oracle.rel_l2(got_dn, oracle.matvec(d.codes, d.scales, host(xr_dn))) < 1e-5
    assert oracle.rel_l2(got_dn, oracle.linear(x_dn, d.signs, d.codes, d.scales)) < 2e-3


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
def test_captured_layer_graph(gpu, fmt):
    """One HIP graph of a layer's 7 tl_linear calls (q, k, v, o, gate, up,
    down at M = 1) over two copies of the weights (14 calls), replayed three
    times with eager library work and synchronisations between the replays;
    every output of every replay equals the eager result bit for bit and
    matches the oracle on sampled rows."""
    specs = []
    for name in synth.LAYER_LINEARS:
        k, n = synth.SHAPES[name]
        inp = synth.linear_inputs(n, k, 1, cfg=5, linear=synth.LINEAR_ID[name],
                                  outliers=name in ("q", "k", "v", "o"))
        packed = tl.pack(dev(inp.codes, gpu), fmt)
        specs.append(dict(name=name, inp=inp, packs=[packed, packed.clone()],
                          scales=dev(inp.scales, gpu), x=dev(inp.x, gpu),
                          signs=dev(inp.signs, gpu),
                          x_rot=[torch.empty((1, k), dtype=torch.float16, device=gpu)
                                 for _ in range(2)],
                          y=[torch.empty((1, n), dtype=torch.float32, device=gpu)
                             for _ in range(2)]))

    def layer():
        for c in range(2):
            for s in specs:
                tl.linear(s["packs"][c], s["scales"], fmt, s["x"], s["signs"], out=s["y"][c],
                          x_rot=s["x_rot"][c])

    stream = torch.cuda.Stream(gpu)
    with torch.cuda.stream(stream):
        layer()
        torch.cuda.synchronize()
        eager = [[host(s["y"][c]).copy() for s in specs] for c in range(2)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            layer()
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    wants = []
    for s in specs:
        inp = s["inp"]
        n = inp.codes.shape[0]
        rows = tile_samples(n, 256, rng)
        wants.append((rows, oracle.linear(inp.x, inp.signs, inp.codes[rows], inp.scales[rows])[0]))
    for rep in range(3):
        for s in specs:                       # clobber the outputs
            for c in range(2):
                s["y"][c].fill_(float("nan"))
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for c in range(2):
            for i, s in enumerate(specs):
                got = host(s["y"][c])
                assert np.array_equal(got.view(np.uint32), eager[c][i].view(np.uint32)), (rep, s["name"])
                rows, want = wants[i]
                assert oracle.rel_l2(got[0, rows].astype(np.float64), want) < 2e-3
        # eager work of the program between replays
        s = specs[rep]
        tl.linear(s["packs"][0], s["scales"], fmt, s["x"], s["signs"])
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# guard bands: no write outside an output
# ---------------------------------------------------------------------------

PAD = 4096     # bytes of guard band on each side


def guarded(numel, dtype, device):
    """(buffer, view): a view of `numel` elements in the middle of a buffer
    whose guard bands hold a canary byte pattern."""
    esz = torch.empty((), dtype=dtype).element_size()
    buf = torch.full((2 * PAD + numel * esz,), 0xA5, dtype=torch.uint8, device=device)
    return buf, buf[PAD:PAD + numel * esz].view(dtype)


def bands_intact(buf):
    b = host(buf)
    return bool(np.all(b[:PAD] == 0xA5) and np.all(b[-PAD:] == 0xA5))


@pytest.mark.parametrize("fmt", FMTS + (tl.FMT_BIT1,), ids=["trit5", "slot2", "bit1"])
@pytest.mark.parametrize("call,m,n,k", [
    ("gemv", 1, 67, 1024), ("gemv", 1, 4097, 2048), ("gemv", 3, 1000, 1024),
    ("gemv", 17, 333, 1024), ("gemv", 9, 333, 2048), ("gemv", 1, 1, 17408), ("gemm", 65, 67, 1024),
    ("gemm", 300, 1000, 2048), ("gemm", 257, 4099, 1024),
    ("linear", 1, 67, 1024), ("linear", 1, 5119, 6144), ("linear", 5, 300, 2048),
    ("linear", 70, 301, 1024)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16], ids=["f32", "f16"])
def test_outputs_guard_bands(gpu, call, m, n, k, fmt, out_dtype):
    """Ragged M and N: y (and x_rot for tl_linear) sit between canary guard
    bands, which must come back untouched; y itself is checked against the
    oracle so a write that lands in the wrong place inside y shows too."""
    binary = fmt == tl.FMT_BIT1
    inp = synth.linear_inputs(n, k, m, cfg=1, linear=m * n + k, binary=binary)
    packed = tl.pack(dev(inp.codes, gpu), fmt)
    scales = dev(inp.scales, gpu)
    ybuf, y = guarded(m * n, out_dtype, gpu)
    y = y.view(m, n)
    if call == "linear":
        xbuf, x_rot = guarded(m * k, torch.float16, gpu)
        x_rot = x_rot.view(m, k)
        tl.linear(packed, scales, fmt, dev(inp.x, gpu), dev(inp.signs, gpu), out_dtype=out_dtype,
                  out=y, x_rot=x_rot)
        assert bands_intact(xbuf)
        want = oracle.linear(inp.x, inp.signs, inp.codes, inp.scales)
    else:
        x_rot16 = oracle.rotate(inp.x, inp.signs).astype(np.float16)
        fn = tl.gemv if call == "gemv" else tl.gemm
        fn(packed, scales, fmt, dev(x_rot16, gpu), out_dtype=out_dtype, out=y)
        want = oracle.matvec(inp.codes, inp.scales, x_rot16)
    torch.cuda.synchronize()
    assert bands_intact(ybuf)
    assert oracle.rel_l2(host(y).astype(np.float64), want) < 2e-3


@pytest.mark.parametrize("m,k", [(1, 1024), (3, 5120), (33, 17408)])
def test_rotate_guard_bands(gpu, m, k):
    inp = synth.linear_inputs(1, k, m, cfg=3, linear=k, outliers=True)
    xbuf, x_rot = guarded(m * k, torch.float16, gpu)
    tl.hadamard_rotate(dev(inp.x, gpu), dev(inp.signs, gpu), out=x_rot.view(m, k))
    torch.cuda.synchronize()
    assert bands_intact(xbuf)
    got = host(x_rot).reshape(m, k).astype(np.float64)
    assert oracle.rel_l2(got, oracle.rotate(inp.x, inp.signs)) < 1e-3
