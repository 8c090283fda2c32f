"""GPU parity of the 1-bit packing (codes -1 and +1, one bit each, one
binary16 scale per 128 weights) against the fp64 CPU oracle on the same
seeded inputs: packing bit-exact, products to the bars of the ternary
formats (relative L2 1e-5 against the oracle on the binary16 rotated input,
2e-3 end to end), exact where every partial sum is exact."""
import itertools

import numpy as np
import pytest
import torch

import oracle
import synth
import tl_hadamard_rotate_amd as tl

pytestmark = pytest.mark.gpu

B = tl.FMT_BIT1
LAYER_CALLS = {"gemv": tl.gemv, "gemm": tl.gemm}


def dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def _inputs(n, k, m, linear, cfg=1, outliers=False):
    return synth.linear_inputs(n, k, m, cfg=cfg, linear=linear, outliers=outliers, binary=True)


def _abs_bound(codes, scales, x):
    """sum_k |code * S * x| per output: the scale of the fp32 rounding error."""
    return oracle.matvec(np.abs(codes), np.abs(scales.astype(np.float64)), np.abs(x.astype(np.float64)))


@pytest.mark.parametrize("n,k", [(1024, 1024), (3, 128), (7, 384), (33, 5120)])
def test_bit1_pack_bit_exact(gpu, n, k):
    inp = _inputs(n, k, 1, linear=k)
    want = oracle.pack(inp.codes, B)
    bad = torch.zeros(1, dtype=torch.int32, device=gpu)
    got = tl.pack(dev(inp.codes, gpu), B, bad_count=bad)
    torch.cuda.synchronize()
    assert np.array_equal(host(got), want)
    assert int(bad.item()) == 0
    assert np.array_equal(host(tl.unpack(got, k, B)), inp.codes)


def test_bit1_pack_exhaustive_bytes(gpu):
    """All 256 code patterns of a byte at each of the 16 byte positions of a group."""
    combos = np.array(list(itertools.product((-1, 1), repeat=8)), dtype=np.int8)
    rows = []
    for pos in range(16):
        block = np.ones((len(combos), 128), dtype=np.int8)
        block[:, 8 * pos:8 * pos + 8] = combos
        rows.append(block)
    codes = np.concatenate(rows)
    want = oracle.pack(codes, B)
    assert np.array_equal(host(tl.pack(dev(codes, gpu), B)), want)
    assert np.array_equal(host(tl.unpack(dev(want, gpu), 128, B)), codes)


def test_bit1_pack_counts_invalid_codes(gpu):
    """Codes other than -1 and +1 (0 included) are packed as +1 and counted."""
    inp = _inputs(16, 1024, 1, linear=77)
    codes = inp.codes.copy()
    codes[0, 0] = 0
    codes[3, 17] = 0
    codes[9, 1000] = -5
    codes[15, 127] = 2
    bad = torch.zeros(1, dtype=torch.int32, device=gpu)
    got = host(tl.pack(dev(codes, gpu), B, bad_count=bad))
    assert int(bad.item()) == 4
    fixed = codes.copy()
    fixed[fixed != -1] = 1
    assert np.array_equal(got, oracle.pack(fixed, B))


@pytest.mark.parametrize("call", sorted(LAYER_CALLS))
@pytest.mark.parametrize("m,n,k", [(1, 1024, 1024), (2, 1000, 2048), (3, 67, 1024),
                                   (5, 130, 3072), (16, 1024, 5120), (17, 130, 1024),
                                   (100, 200, 3072), (1, 64, 17408), (5, 64, 1 << 20)])
def test_bit1_layer_matches_oracle(gpu, call, m, n, k):
    """Ragged N, every token-count path of the GEMV (1, 2, passes of 4, more
    than 16, and K so long that the group sums of only two tokens fit in LDS)."""
    inp = _inputs(n, k, m, linear=m + n)
    packed = tl.pack(dev(inp.codes, gpu), B)
    scales = dev(inp.scales, gpu)
    x_rot16 = oracle.rotate(inp.x, inp.signs).astype(np.float16)
    x_rot = dev(x_rot16, gpu)
    fn = LAYER_CALLS[call]
    y32 = host(fn(packed, scales, B, x_rot, out_dtype=torch.float32)).astype(np.float64)
    y16 = host(fn(packed, scales, B, x_rot, out_dtype=torch.float16)).astype(np.float64)
    want = oracle.matvec(inp.codes, inp.scales, x_rot16)
    assert oracle.rel_l2(y32, want) < 1e-5
    # element by element: fp32 sums of exact products stay far inside 1e-5 of sum |terms|
    assert np.all(np.abs(y32 - want) <= 1e-5 * _abs_bound(inp.codes, inp.scales, x_rot16))
    assert np.array_equal(y16.astype(np.float16).view(np.uint16),
                          y32.astype(np.float32).astype(np.float16).view(np.uint16))
    if k <= 5120:
        full = oracle.linear(inp.x, inp.signs, inp.codes, inp.scales)
        assert oracle.rel_l2(y32, full) < 2e-3


@pytest.mark.parametrize("call", sorted(LAYER_CALLS))
def test_bit1_one_hot_bit_exact(gpu, call):
    """x = e_k gives y[n] = code[n, k] * S[n, k/128] exactly, for each of the
    1024 positions of a block (so each bit position of every weight dword)."""
    n, k = 96, 1024
    inp = _inputs(n, k, 1, linear=5)
    packed = tl.pack(dev(inp.codes, gpu), B)
    scales = dev(inp.scales, gpu)
    want_all = inp.codes.astype(np.float64) * np.repeat(inp.scales.astype(np.float64), 128, 1)
    fn = LAYER_CALLS[call]
    for start in range(0, k, 16):
        x = np.zeros((16, k), dtype=np.float16)
        for t in range(16):
            x[t, start + t] = 1.0
        y = host(fn(packed, scales, B, dev(x, gpu), out_dtype=torch.float32)).astype(np.float64)
        assert np.array_equal(y, want_all[:, start:start + 16].T), start


def test_bit1_subnormal_and_extreme_activations(gpu):
    """Binary16 subnormal and near-overflow activations: the bit masks are
    themselves tiny binary16 numbers, so these probe the products' range."""
    n, k = 128, 2048
    inp = _inputs(n, k, 1, linear=9)
    rng = np.random.default_rng(4)
    x = np.where(rng.random((1, k)) < 0.5, 2.0 ** -24 * rng.integers(1, 1024, (1, k)),
                 rng.choice([-1, 1], (1, k)) * 6e4 * rng.random((1, k)))
    x16 = x.astype(np.float16)
    scales = np.full_like(inp.scales, 2.0 ** -10)
    y = host(tl.gemv(tl.pack(dev(inp.codes, gpu), B), dev(scales, gpu), B,
                     dev(x16, gpu))).astype(np.float64)
    want = oracle.matvec(inp.codes, scales, x16)
    assert np.all(np.abs(y - want) <= 1e-5 * _abs_bound(inp.codes, scales, x16))


@pytest.mark.parametrize("m", [1, 4])
def test_bit1_same_result_as_slot2_packing(gpu, m):
    """The same +-1 weights in the 2-bit format give the same products."""
    n, k = 700, 5120
    inp = _inputs(n, k, m, linear=31)
    x = dev(oracle.rotate(inp.x, inp.signs).astype(np.float16), gpu)
    s, c = dev(inp.scales, gpu), dev(inp.codes, gpu)
    y1 = host(tl.gemv(tl.pack(c, B), s, B, x)).astype(np.float64)
    y2 = host(tl.gemv(tl.pack(c, tl.FMT_SLOT2), s, tl.FMT_SLOT2, x)).astype(np.float64)
    assert oracle.rel_l2(y1, y2) < 1e-5


@pytest.mark.parametrize("call", sorted(LAYER_CALLS))
def test_bit1_deterministic(gpu, call):
    n, k, m = 2048, 5120, 4
    inp = _inputs(n, k, m, linear=44)
    packed, scales = tl.pack(dev(inp.codes, gpu), B), dev(inp.scales, gpu)
    x = dev(oracle.rotate(inp.x, inp.signs).astype(np.float16), gpu)
    a = host(LAYER_CALLS[call](packed, scales, B, x))
    b = host(LAYER_CALLS[call](packed, scales, B, x))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("m", [1, 16])
@pytest.mark.parametrize("shape", ["gate", "down"])
def test_bit1_full_size_decode_sampled_rows(gpu, shape, m):
    """27B-class decode shapes, full size; the oracle checks sampled rows."""
    k, n = synth.SHAPES[shape]
    inp = synth.linear_inputs(n, k, m, cfg=2, linear=synth.LINEAR_ID[shape], binary=True)
    packed = tl.pack(dev(inp.codes, gpu), B)
    x_rot = tl.hadamard_rotate(dev(inp.x, gpu), dev(inp.signs, gpu))
    y = host(tl.gemv(packed, dev(inp.scales, gpu), B, x_rot)).astype(np.float64)
    rows = np.concatenate([np.random.default_rng(0).choice(n, size=256, replace=False), [0, n - 1]])
    want = oracle.matvec(inp.codes[rows], inp.scales[rows], oracle.rotate(inp.x, inp.signs))
    assert oracle.rel_l2(y[:, rows], want) < 2e-3
    want16 = oracle.matvec(inp.codes[rows], inp.scales[rows], host(x_rot))
    assert oracle.rel_l2(y[:, rows], want16) < 1e-5


@pytest.mark.parametrize("m,n,k", [(1, 1024, 1024), (1, 333, 5120), (3, 700, 2048),
                                   (70, 200, 3072)])
def test_bit1_linear_matches_oracle(gpu, m, n, k):
    inp = _inputs(n, k, m, cfg=3, linear=m + n + k, outliers=True)
    packed, scales = tl.pack(dev(inp.codes, gpu), B), dev(inp.scales, gpu)
    x_rot = torch.empty((m, k), dtype=torch.float16, device=gpu)
    y = host(tl.linear(packed, scales, B, dev(inp.x, gpu), dev(inp.signs, gpu),
                       x_rot=x_rot)).astype(np.float64)
    prod = tl.gemm if m >= 64 else tl.gemv
    y2 = host(prod(packed, scales, B, x_rot)).astype(np.float64)
    assert np.array_equal(y.astype(np.float32).view(np.uint32), y2.astype(np.float32).view(np.uint32))
    assert oracle.rel_l2(y, oracle.linear(inp.x, inp.signs, inp.codes, inp.scales)) < 2e-3
