"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle
on identical seeded inputs.  Integer work must be bit-exact; floating-point
results must meet the relative-L2 bar of 2e-3 (and the tighter bounds derived
in each test from the arithmetic)."""
import math

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


def f16bits(a):
    return np.asarray(a, dtype=np.float16)


# ---------------------------------------------------------------------------
# pack / unpack
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
@pytest.mark.parametrize("n,k", [(1024, 1024), (3, 128), (7, 384), (33, 5120)])
def test_pack_bit_exact(gpu, fmt, n, k):
    inp = synth.linear_inputs(n, k, 1, cfg=1, linear=k)
    want = oracle.pack(inp.codes, fmt)
    bad = torch.zeros(1, dtype=torch.int32, device=gpu)
    got = tl.pack(dev(inp.codes, gpu), fmt, bad_count=bad)
    torch.cuda.synchronize()
    assert np.array_equal(host(got), want)
    assert int(bad.item()) == 0
    back = tl.unpack(got, k, fmt)
    assert np.array_equal(host(back), inp.codes)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
def test_pack_exhaustive_bytes(gpu, fmt):
    """Every valid code pattern of a byte, at every byte position of a group
    (TRIT5: the 25 full bytes and the 3-trit tail byte; SLOT2: 32 bytes)."""
    import itertools
    per, nbytes = (5, 25) if fmt == tl.FMT_TRIT5 else (4, 32)
    combos = np.array(list(itertools.product((-1, 0, 1), repeat=per)), dtype=np.int8)
    rows = []
    for pos in range(nbytes):
        block = np.zeros((len(combos), 128), dtype=np.int8)
        block[:, per * pos:per * pos + per] = combos
        rows.append(block)
    if fmt == tl.FMT_TRIT5:
        tail = np.array(list(itertools.product((-1, 0, 1), repeat=3)), dtype=np.int8)
        block = np.zeros((len(tail), 128), dtype=np.int8)
        block[:, 125:] = tail
        rows.append(block)
    codes = np.concatenate(rows)
    want = oracle.pack(codes, fmt)
    got = host(tl.pack(dev(codes, gpu), fmt))
    assert np.array_equal(got, want)
    assert np.array_equal(host(tl.unpack(dev(want, gpu), 128, fmt)), codes)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
def test_pack_counts_invalid_codes(gpu, fmt):
    inp = synth.linear_inputs(16, 1024, 1, cfg=1, linear=77)
    codes = inp.codes.copy()
    codes[3, 17] = 2
    codes[9, 1000] = -5
    codes[15, 127] = 100
    bad = torch.zeros(1, dtype=torch.int32, device=gpu)
    got = host(tl.pack(dev(codes, gpu), fmt, bad_count=bad))
    assert int(bad.item()) == 3
    fixed = codes.copy()
    fixed[(fixed < -1) | (fixed > 1)] = 0
    assert np.array_equal(got, oracle.pack(fixed, fmt))


# ---------------------------------------------------------------------------
# rotation
# ---------------------------------------------------------------------------

def _rotate_gpu(x16, signs, device, inplace=False):
    x = dev(x16, device)
    s = dev(signs, device)
    out = tl.hadamard_rotate(x, s, out=x if inplace else None)
    return host(out)


@pytest.mark.parametrize("m,k", [(1, 1024), (3, 5120), (17, 2048), (64, 17408)])
def test_rotate_random_within_derived_bound(gpu, m, k):
    inp = synth.linear_inputs(1, k, m, cfg=3, linear=m, outliers=True)
    got = _rotate_gpu(inp.x, inp.signs, gpu).astype(np.float64)
    want = oracle.rotate(inp.x, inp.signs)
    # Error bound of the kernel's arithmetic: each output is a 10-level tree of
    # fp32 additions of the 1024 terms +-x_j/32 (|error| <= 10 u sum_j |x_j|/32,
    # u = 2^-24), followed by one rounding to binary16 (half an ulp of the
    # larger of the two neighbouring binades).
    xa = np.abs(inp.x.astype(np.float64)).reshape(m, k // 1024, 1024).sum(-1) / 32.0
    fp32_err = np.repeat(10 * 2.0 ** -24 * xa, 1024, axis=1)
    half_ulp = 0.5 * np.maximum(oracle.fp16_ulp(got), oracle.fp16_ulp(want))
    excess = np.abs(got - want) - (half_ulp + fp32_err)
    assert np.all(excess <= 0), np.max(excess)
    # and nearly every entry is the correctly rounded binary16 value
    nearest = want.astype(np.float16).astype(np.float64)
    assert np.mean(got == nearest) > 0.99


def test_rotate_closed_forms_bit_exact(gpu):
    k = 2048
    rng = np.random.default_rng(1)
    s = rng.choice([-1, 1], size=k).astype(np.int8)
    js = [0, 1, 7, 8, 255, 256, 511, 1023, 1024, 1500, 2047]
    x = np.zeros((len(js), k), dtype=np.float16)
    for r, j in enumerate(js):
        x[r, j] = 1.0
    got = _rotate_gpu(x, s, gpu).astype(np.float64)
    h = oracle.hadamard(1024)
    for r, j in enumerate(js):
        b, jj = divmod(j, 1024)
        want = np.zeros(k)
        want[b * 1024:(b + 1) * 1024] = s[j] * h[:, jj] / 32.0
        assert np.array_equal(got[r], want), j
    # x = signs maps every block to 32 e_0
    got = _rotate_gpu(s[None, :].astype(np.float16), s, gpu)[0].astype(np.float64)
    want = np.zeros(k)
    want[0] = want[1024] = 32.0
    assert np.array_equal(got, want)


def test_rotate_in_place(gpu):
    inp = synth.linear_inputs(1, 3072, 5, cfg=3, linear=9)
    a = _rotate_gpu(inp.x, inp.signs, gpu)
    b = _rotate_gpu(inp.x, inp.signs, gpu, inplace=True)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_rotate_preserves_norm(gpu):
    inp = synth.linear_inputs(1, 5120, 8, cfg=3, linear=3, outliers=True)
    got = _rotate_gpu(inp.x, inp.signs, gpu).astype(np.float64)
    nx = np.linalg.norm(inp.x.astype(np.float64), axis=1)
    assert np.allclose(np.linalg.norm(got, axis=1), nx, rtol=1e-3)


# ---------------------------------------------------------------------------
# GEMV / GEMM
# ---------------------------------------------------------------------------

def _prep(n, k, m, fmt, device, cfg=1, linear=0, outliers=False):
    inp = synth.linear_inputs(n, k, m, cfg=cfg, linear=linear, outliers=outliers)
    packed = tl.pack(dev(inp.codes, device), fmt)
    scales = dev(inp.scales, device)
    return inp, packed, scales


LAYER_CALLS = {"gemv": tl.gemv, "gemm": tl.gemm}


@pytest.mark.parametrize("call", sorted(LAYER_CALLS))
@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
@pytest.mark.parametrize("m,n,k", [(1, 1024, 1024), (2, 1000, 2048), (5, 67, 1024),
                                   (16, 1024, 5120), (17, 130, 1024), (100, 200, 3072)])
def test_layer_matches_oracle(gpu, call, fmt, m, n, k):
    inp, packed, scales = _prep(n, k, m, fmt, gpu, cfg=1, linear=m + n)
    x_rot16 = oracle.rotate(inp.x, inp.signs).astype(np.float16)
    x_rot = dev(x_rot16, gpu)
    fn = LAYER_CALLS[call]
    y32 = host(fn(packed, scales, fmt, x_rot, out_dtype=torch.float32)).astype(np.float64)
    y16 = host(fn(packed, scales, fmt, x_rot, out_dtype=torch.float16)).astype(np.float64)
    want = oracle.matvec(inp.codes, inp.scales, x_rot16)
    # exact products, fp32 sums over K terms: relative error far below 1e-5
    assert oracle.rel_l2(y32, want) < 1e-5
    # the binary16 output is the fp32 result rounded to nearest even
    assert np.array_equal(y16.astype(np.float16).view(np.uint16),
                          y32.astype(np.float32).astype(np.float16).view(np.uint16))
    # end to end against the unrounded fp64 layer: the 2e-3 bar
    full = oracle.linear(inp.x, inp.signs, inp.codes, inp.scales)
    assert oracle.rel_l2(y32, full) < 2e-3
    assert oracle.rel_l2(y16, full) < 2e-3


@pytest.mark.parametrize("call", sorted(LAYER_CALLS))
@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
def test_layer_one_hot_bit_exact(gpu, call, fmt):
    """x_rot = e_k gives y[n] = code[n, k] * S[n, k/128] exactly; 16 one-hots
    per call over 64 calls cover all 1024 positions of a block."""
    n, k = 96, 1024
    inp, packed, scales = _prep(n, k, 1, fmt, gpu, linear=5)
    want_all = inp.codes.astype(np.float64) * np.repeat(inp.scales.astype(np.float64), 128, 1)
    fn = LAYER_CALLS[call]
    for start in range(0, k, 16):
        x = np.zeros((16, k), dtype=np.float16)
        for t in range(16):
            x[t, start + t] = 1.0
        y = host(fn(packed, scales, fmt, dev(x, gpu), out_dtype=torch.float32)).astype(np.float64)
        assert np.array_equal(y, want_all[:, start:start + 16].T), start


@pytest.mark.parametrize("call", sorted(LAYER_CALLS))
@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
@pytest.mark.parametrize("m", [1, 3, 8])
def test_layer_zero_codes(gpu, call, fmt, m):
    """All-zero codes give zero up to fp32 rounding.  Kernels that sum
    (code + 1) * x and subtract the group's sum of x (the 2-bit-slot decode
    kernels) cancel only to the rounding of two fp32 sums of the same terms,
    so the bar is a few fp32 ulps of sum |x| (S = 1), not exact zero."""
    n, k = 64, 2048
    codes = np.zeros((n, k), dtype=np.int8)
    scales = np.ones((n, k // 128), dtype=np.float16)
    x = np.random.default_rng(0).standard_normal((m, k)).astype(np.float16)
    packed = tl.pack(dev(codes, gpu), fmt)
    y = host(LAYER_CALLS[call](packed, dev(scales, gpu), fmt, dev(x, gpu))).astype(np.float64)
    bound = 2.0 ** -20 * np.abs(x.astype(np.float64)).sum(axis=1)
    assert np.all(np.abs(y) <= bound[:, None])


@pytest.mark.parametrize("call", sorted(LAYER_CALLS))
def test_formats_give_identical_results(gpu, call):
    n, k, m = 300, 2048, 4
    inp = synth.linear_inputs(n, k, m, cfg=1, linear=12)
    x = dev(oracle.rotate(inp.x, inp.signs).astype(np.float16), gpu)
    s = dev(inp.scales, gpu)
    c = dev(inp.codes, gpu)
    ys = [host(LAYER_CALLS[call](tl.pack(c, f), s, f, x)) for f in FMTS]
    want = oracle.matvec(inp.codes, inp.scales, host(x))
    for y in ys:
        assert oracle.rel_l2(y, want) < 1e-5


@pytest.mark.parametrize("call", sorted(LAYER_CALLS))
@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
def test_layer_deterministic(gpu, call, fmt):
    n, k, m = 2048, 5120, 4
    inp, packed, scales = _prep(n, k, m, fmt, gpu, linear=44)
    x = dev(oracle.rotate(inp.x, inp.signs).astype(np.float16), gpu)
    a = host(LAYER_CALLS[call](packed, scales, fmt, x))
    b = host(LAYER_CALLS[call](packed, scales, fmt, x))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_end_to_end_layer_and_missing_rotation(gpu):
    """rotate + gemv reproduces the fp64 layer; skipping the runtime rotation
    gives an unrelated result without any error (the pages' warning)."""
    n, k = 1024, 1024
    rng = np.random.default_rng(33)
    w = rng.standard_normal((n, k))
    s = rng.choice([-1, 1], size=k).astype(np.int8)
    wf = oracle.fold_weights(w, s)                # rotation folded into the weights
    scales = np.abs(wf).reshape(n, k // 128, 128).mean(-1)
    codes = np.clip(np.rint(wf / np.repeat(scales, 128, 1)), -1, 1).astype(np.int8)
    scales16 = scales.astype(np.float16)
    x = rng.standard_normal((1, k)).astype(np.float16)
    lin = tl.TernaryLinear(tl.pack(dev(codes, gpu), 0), dev(scales16, gpu), 0, dev(s, gpu))
    y = host(lin(dev(x, gpu))).astype(np.float64)
    want = oracle.linear(x, s, codes, scales16)
    assert oracle.rel_l2(y, want) < 2e-3
    y_wrong = host(tl.gemv(lin.packed, lin.scales, 0, dev(x, gpu))).astype(np.float64)
    assert oracle.rel_l2(y_wrong, want) > 0.5


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
@pytest.mark.parametrize("shape", ["gate", "down"])
def test_full_size_decode_sampled_rows(gpu, fmt, shape):
    """27B-class decode shapes at M = 1, full size; the oracle checks a sample
    of output rows one by one."""
    k, n = synth.SHAPES[shape]
    inp = synth.linear_inputs(n, k, 1, cfg=2, linear=synth.LINEAR_ID[shape])
    codes_d = dev(inp.codes, gpu)
    packed = tl.pack(codes_d, fmt)
    del codes_d
    x_rot = tl.hadamard_rotate(dev(inp.x, gpu), dev(inp.signs, gpu))
    y = host(tl.gemv(packed, dev(inp.scales, gpu), fmt, x_rot)).astype(np.float64)[0]
    rows = np.random.default_rng(0).choice(n, size=256, replace=False)
    rows = np.concatenate([rows, [0, n - 1]])
    x_rot_ref = oracle.rotate(inp.x, inp.signs)
    want = oracle.matvec(inp.codes[rows], inp.scales[rows], x_rot_ref)[0]
    assert oracle.rel_l2(y[rows], want) < 2e-3
    # against the binary16 rotated input the kernel actually read: tight
    want16 = oracle.matvec(inp.codes[rows], inp.scales[rows], host(x_rot))[0]
    assert oracle.rel_l2(y[rows], want16) < 1e-5


# ---------------------------------------------------------------------------
# tl_linear: rotation + product in one call
# ---------------------------------------------------------------------------

def _rotation_bound_ok(got, want, x16, roundings=10):
    """|got - want| within one binary16 rounding plus the fp32 error of
    `roundings` chained additions over the block's terms: 10 for the
    butterfly tree (as in the rotation tests); 37 for the 2-bit M = 1 kernels,
    whose first 32-point stage runs on the matrix cores (a 32-term fp32 sum,
    counted as up to 32 roundings in whatever order the hardware adds) and
    whose second is 5 butterfly levels."""
    m, k = x16.shape
    xa = np.abs(x16.astype(np.float64)).reshape(m, k // 1024, 1024).sum(-1) / 32.0
    fp32_err = np.repeat(roundings * 2.0 ** -24 * xa, 1024, axis=1)
    half_ulp = 0.5 * np.maximum(oracle.fp16_ulp(got), oracle.fp16_ulp(want))
    return np.all(np.abs(got - want) <= half_ulp + fp32_err)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
@pytest.mark.parametrize("m,n,k", [(1, 1024, 1024), (1, 333, 5120), (1, 2048, 17408),
                                   (1, 300, 24576), (3, 700, 2048), (70, 200, 3072)])
def test_linear_matches_oracle(gpu, fmt, m, n, k):
    """M = 1 runs the fused kernels (rotation in the GEMV's prologue, its first
    stage on the matrix cores); M > 1 the rotation and the product as two
    launches."""
    inp = synth.linear_inputs(n, k, m, cfg=3, linear=m + n + k, outliers=True)
    packed = tl.pack(dev(inp.codes, gpu), fmt)
    scales = dev(inp.scales, gpu)
    x_rot = torch.empty((m, k), dtype=torch.float16, device=gpu)
    y = host(tl.linear(packed, scales, fmt, dev(inp.x, gpu), dev(inp.signs, gpu),
                       x_rot=x_rot)).astype(np.float64)
    xr = host(x_rot)
    # the rotated activations it wrote: the rotation's own bound
    assert _rotation_bound_ok(xr.astype(np.float64), oracle.rotate(inp.x, inp.signs), inp.x,
                              roundings=37 if m == 1 else 10)
    # the product is exactly the library's product on those activations
    prod = tl.gemm if m >= 64 else tl.gemv
    y2 = host(prod(packed, scales, fmt, x_rot)).astype(np.float64)
    assert np.array_equal(y.astype(np.float32).view(np.uint32), y2.astype(np.float32).view(np.uint32))
    # end to end against the fp64 layer
    assert oracle.rel_l2(y, oracle.linear(inp.x, inp.signs, inp.codes, inp.scales)) < 2e-3


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
@pytest.mark.parametrize("n,k", [(1, 1024), (17, 2048), (1, 18432), (1, 46080), (4097, 1024)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16], ids=["f32", "f16"])
def test_linear_fused_plan_edges(gpu, fmt, n, k, out_dtype):
    """The fused M = 1 kernels at the edges of their launch plans: one row
    (one workgroup whose waves split K), a ragged row tile, 18 blocks, 45
    blocks (the largest K at which the dense-trit kernel's rotated
    activations fit in LDS beside its table: its waves rotate up to three
    blocks each; the 2-bit kernels take 32 blocks at most, so there the
    rotation and the product are two launches) and a ragged last row slice;
    fp32 and binary16 outputs.  The product equals the
    library's GEMV on the x_rot the call wrote, bit for bit, and the layer
    meets the 2e-3 bar against the oracle."""
    inp = synth.linear_inputs(n, k, 1, cfg=3, linear=n + k, outliers=True)
    packed = tl.pack(dev(inp.codes, gpu), fmt)
    scales = dev(inp.scales, gpu)
    x_rot = torch.empty((1, k), dtype=torch.float16, device=gpu)
    y = host(tl.linear(packed, scales, fmt, dev(inp.x, gpu), dev(inp.signs, gpu),
                       out_dtype=out_dtype, x_rot=x_rot))
    assert _rotation_bound_ok(host(x_rot).astype(np.float64), oracle.rotate(inp.x, inp.signs), inp.x,
                              roundings=37)
    y2 = host(tl.gemv(packed, scales, fmt, x_rot, out_dtype=out_dtype))
    assert np.array_equal(y.view(np.uint16 if out_dtype == torch.float16 else np.uint32),
                          y2.view(np.uint16 if out_dtype == torch.float16 else np.uint32))
    want = oracle.linear(inp.x, inp.signs, inp.codes, inp.scales)
    assert oracle.rel_l2(y.astype(np.float64), want) < 2e-3


@pytest.mark.parametrize("n,k", [(35071, 5120), (31234, 17408), (60000, 4096), (1031, 3072)])
def test_m1_row_layouts(gpu, n, k):
    """The 2-bit M = 1 kernels where a workgroup's rows are not a multiple of
    the four rows a wave takes per step (137 and 136 rows: the last unit of
    each block overlaps the one before), where they take two row chunks (122
    or 123 rows at K = 17408: the second chunk has fewer than four rows),
    where a wave's 15 steps run as a ring of three flights (234 or 235 rows
    at K = 4096), and a small ragged case.  Sampled rows in every
    64-row tile against the oracle on the binary16 x_rot the call wrote;
    tl_linear equals tl_gemv on that x_rot bit for bit."""
    fmt = tl.FMT_SLOT2
    inp = synth.linear_inputs(n, k, 1, cfg=3, linear=n + 3, outliers=True)
    packed = tl.pack(dev(inp.codes, gpu), fmt)
    scales = dev(inp.scales, gpu)
    x_rot = torch.empty((1, k), dtype=torch.float16, device=gpu)
    y = host(tl.linear(packed, scales, fmt, dev(inp.x, gpu), dev(inp.signs, gpu), x_rot=x_rot))
    y2 = host(tl.gemv(packed, scales, fmt, x_rot))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    rng = np.random.default_rng(n)
    rows = np.unique(np.concatenate([np.arange(0, n, 64), np.arange(63, n, 64), [n - 1],
                                     rng.integers(0, n, size=256)]))
    want = oracle.matvec(inp.codes[rows], inp.scales[rows], host(x_rot))
    assert oracle.rel_l2(y[:, rows].astype(np.float64), want) < 1e-5


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
@pytest.mark.parametrize("shape", ["gate", "down", "k"])
def test_linear_full_size_sampled_rows(gpu, fmt, shape):
    """The fused M = 1 path at the 27B-class shapes; sampled rows against the
    oracle's layer, with the rotation folded into the weights."""
    k, n = synth.SHAPES[shape]
    inp = synth.linear_inputs(n, k, 1, cfg=5, linear=synth.LINEAR_ID[shape])
    packed = tl.pack(dev(inp.codes, gpu), fmt)
    y = host(tl.linear(packed, dev(inp.scales, gpu), fmt, dev(inp.x, gpu),
                       dev(inp.signs, gpu))).astype(np.float64)[0]
    rows = np.concatenate([np.random.default_rng(1).choice(n, size=200, replace=False), [0, n - 1]])
    want = oracle.linear(inp.x, inp.signs, inp.codes[rows], inp.scales[rows])[0]
    assert oracle.rel_l2(y[rows], want) < 2e-3


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
@pytest.mark.parametrize("group", [("q", "k", "v"), ("gate", "up")])
def test_linear_shared_rotation_concatenated(gpu, fmt, group):
    """Linears that read the same input share one rotation: their packed rows
    and scales concatenated along N go through one tl_linear call.  Each row's
    result is the one its own call gives: bit for bit with 2-bit slots (the
    fused kernel adds a row's parts in an order that does not depend on the
    other rows), to fp32 rounding with dense trits (that GEMV splits K across
    waves by the size of a CU's slice of rows, which depends on N); sampled
    rows match the oracle's layer."""
    k = synth.SHAPES[group[0]][0]
    parts = [synth.linear_inputs(synth.SHAPES[g][1], k, 1, cfg=5, linear=synth.LINEAR_ID[g],
                                 outliers=g in ("q", "k", "v")) for g in group]
    x, signs = parts[0].x, parts[0].signs     # the shared input and its rotation
    codes = np.concatenate([p.codes for p in parts])
    scales = np.concatenate([p.scales for p in parts])
    xd, sd = dev(x, gpu), dev(signs, gpu)
    y_all = host(tl.linear(tl.pack(dev(codes, gpu), fmt), dev(scales, gpu), fmt, xd, sd))[0]
    off = 0
    for p in parts:
        n = p.codes.shape[0]
        y_one = host(tl.linear(tl.pack(dev(p.codes, gpu), fmt), dev(p.scales, gpu), fmt, xd, sd))[0]
        if fmt == tl.FMT_SLOT2:
            assert np.array_equal(y_all[off:off + n].view(np.uint32), y_one.view(np.uint32))
        else:
            assert np.allclose(y_all[off:off + n], y_one, rtol=1e-5, atol=1e-6 * np.abs(y_one).max())
        off += n
    n = codes.shape[0]
    rows = np.concatenate([np.random.default_rng(2).choice(n, size=160, replace=False), [0, n - 1]])
    want = oracle.linear(x, signs, codes[rows], scales[rows])[0]
    assert oracle.rel_l2(y_all.astype(np.float64)[rows], want) < 2e-3
