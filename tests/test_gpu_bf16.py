"""GPU parity of the bfloat16 product (tl_gemm_bf16: each activation row
taken exactly to binary16 under a power-of-two factor, the binary16
register-decode product, the factor undone on the outputs) against the fp64
oracle.  The kernel and the oracle read the same bfloat16 activations (the
oracle's rotation rounded to bfloat16), so the products are exact and only
the fp32 sums round: relative L2 1e-5 and, element by element, 1e-5 of the
sum of |terms|.  End to end against the fp64 layer on the unrounded rotation,
the bfloat16 rounding of the activations (8 significant bits, relative error
<= 2^-9 per element) dominates; its derived size for random data is about
2^-9 / sqrt(3) = 1.1e-3, under the 2e-3 bar.  Rows far outside the binary16
range (factors 2^-100 .. 2^100) keep the same bars, and where the rows are
binary16 numbers the result equals tl_gemm's bit for bit (a power-of-two
factor commutes with the fp32 rounding)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tl_hadamard_rotate_amd as tl

pytestmark = pytest.mark.gpu

FMTS = (tl.FMT_TRIT5, tl.FMT_SLOT2, tl.FMT_BIT1)
FMT_NAME = {tl.FMT_TRIT5: "trit5", tl.FMT_SLOT2: "slot2", tl.FMT_BIT1: "bit1"}


def dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def bf16(a64, device):
    """fp64 values that are bfloat16 numbers, as a device bfloat16 tensor (exact)."""
    return torch.from_numpy(np.ascontiguousarray(a64, dtype=np.float32)).to(device).to(torch.bfloat16)


def _inputs(n, k, m, fmt, linear, cfg=1, outliers=False):
    return synth.linear_inputs(n, k, m, cfg=cfg, linear=linear, outliers=outliers,
                               binary=fmt == tl.FMT_BIT1)


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
@pytest.mark.parametrize("m,n,k", [(1, 64, 1024), (65, 300, 2048), (130, 1000, 3072),
                                   (257, 512, 5120), (64, 256, 17408)])
def test_bf16_gemm_matches_oracle(gpu, fmt, m, n, k):
    inp = _inputs(n, k, m, fmt, linear=m + n + k)
    xr = oracle.round_bf16(oracle.rotate(inp.x, inp.signs))
    packed = tl.pack(dev(inp.codes, gpu), fmt)
    scales = dev(inp.scales, gpu)
    y32 = host(tl.gemm_bf16(packed, scales, fmt, bf16(xr, gpu))).astype(np.float64)
    y16 = host(tl.gemm_bf16(packed, scales, fmt, bf16(xr, gpu), out_dtype=torch.float16))
    want = oracle.matvec(inp.codes, inp.scales, xr)
    assert oracle.rel_l2(y32, want) < 1e-5
    bound = oracle.matvec(np.abs(inp.codes), inp.scales.astype(np.float64), np.abs(xr))
    assert np.all(np.abs(y32 - want) <= 1e-5 * bound + 1e-30)
    assert np.array_equal(y16.view(np.uint16),
                          y32.astype(np.float32).astype(np.float16).view(np.uint16))
    if k <= 5120:
        full = oracle.linear(inp.x, inp.signs, inp.codes, inp.scales)
        assert oracle.rel_l2(y32, full) < 2e-3


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_NAME.get)
def test_bf16_gemm_one_hot_bit_exact(gpu, fmt):
    """x = e_k gives y[n] = code[n, k] * S[n, k/128] exactly (one product, an
    exact fp32 scale multiply)."""
    n, k = 96, 1024
    inp = _inputs(n, k, 1, fmt, linear=5)
    packed = tl.pack(dev(inp.codes, gpu), fmt)
    scales = dev(inp.scales, gpu)
    want_all = inp.codes.astype(np.float64) * np.repeat(inp.scales.astype(np.float64), 128, 1)
    for start in range(0, k, 64):
        x = np.zeros((64, k))
        for t in range(64):
            x[t, start + t] = 1.0
        y = host(tl.gemm_bf16(packed, scales, fmt, bf16(x, gpu))).astype(np.float64)
        assert np.array_equal(y, want_all[:, start:start + 64].T), start


def test_bf16_gemm_deterministic_and_scale_not_rounded(gpu):
    """Bitwise reproducible; and the scale is applied in fp32, not rounded to
    bfloat16: scales with 11 significant bits give the exact product for an
    x of ones in one group."""
    n, k, m = 512, 2048, 100
    inp = _inputs(n, k, m, tl.FMT_SLOT2, linear=3)
    xr = oracle.round_bf16(oracle.rotate(inp.x, inp.signs))
    packed, scales = tl.pack(dev(inp.codes, gpu), tl.FMT_SLOT2), dev(inp.scales, gpu)
    a = host(tl.gemm_bf16(packed, scales, tl.FMT_SLOT2, bf16(xr, gpu)))
    b = host(tl.gemm_bf16(packed, scales, tl.FMT_SLOT2, bf16(xr, gpu)))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    s = np.full((n, k // 128), np.float16(1.0 + 2.0 ** -10))          # not a bfloat16 number
    codes = np.ones((n, k), dtype=np.int8)
    x = np.zeros((1, k))
    x[0, :128] = 1.0
    y = host(tl.gemm_bf16(tl.pack(dev(codes, gpu), tl.FMT_SLOT2), dev(s, gpu), tl.FMT_SLOT2,
                          bf16(x, gpu))).astype(np.float64)
    assert np.all(y == 128 * (1.0 + 2.0 ** -10))


@pytest.mark.parametrize("shape", ["gate", "down"])
def test_bf16_gemm_prefill_size_sampled_rows(gpu, shape):
    """M = 4096 at the 27B-class shapes; the oracle checks sampled output rows."""
    k, n = synth.SHAPES[shape]
    m = 4096
    inp = synth.linear_inputs(n, k, m, cfg=4, linear=synth.LINEAR_ID[shape])
    xr = oracle.round_bf16(oracle.rotate(inp.x, inp.signs))
    packed, scales = tl.pack(dev(inp.codes, gpu), tl.FMT_SLOT2), dev(inp.scales, gpu)
    y = host(tl.gemm_bf16(packed, scales, tl.FMT_SLOT2, bf16(xr, gpu)))
    rng = np.random.default_rng(9)
    rows = np.concatenate([rng.choice(n, size=64, replace=False), [0, n - 1]])
    toks = np.concatenate([rng.choice(m, size=48, replace=False), [0, m - 1]])
    want = oracle.matvec(inp.codes[rows], inp.scales[rows], xr[toks])
    assert oracle.rel_l2(y[np.ix_(toks, rows)].astype(np.float64), want) < 1e-5


@pytest.mark.parametrize("fmt", (tl.FMT_SLOT2, tl.FMT_TRIT5), ids=["slot2", "trit5"])
def test_bf16_gemm_equals_binary16_product(gpu, fmt):
    """Activations that are both bfloat16 and binary16 numbers: tl_gemm_bf16
    gives tl_gemm's bits (fp32 outputs), whatever each row's factor."""
    n, k, m = 700, 3072, 300
    inp = _inputs(n, k, m, fmt, linear=21, cfg=3, outliers=True)
    xr = oracle.round_bf16(oracle.rotate(inp.x, inp.signs))
    xr[:20] *= 2.0 ** 6                    # rows whose factor differs
    xr[20:40] *= 2.0 ** -6
    xr[np.abs(xr) < 2.0 ** -14] = 0.0      # binary16 subnormals may not hold 8 bits
    assert np.array_equal(xr.astype(np.float16).astype(np.float64), xr)
    packed, scales = tl.pack(dev(inp.codes, gpu), fmt), dev(inp.scales, gpu)
    a = host(tl.gemm_bf16(packed, scales, fmt, bf16(xr, gpu)))
    b = host(tl.gemm(packed, scales, fmt, dev(xr.astype(np.float16), gpu)))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_bf16_gemm_rows_outside_binary16_range(gpu):
    """Rows scaled by 2^100, 2^-100, 2^40, 2^-40 (bfloat16 numbers far outside
    the binary16 range), an all-zero row and a row mixing 2^30 and 2^-30
    elements: every row keeps the fp32 bar of its own magnitude."""
    n, k, m = 512, 2048, 70
    inp = _inputs(n, k, m, tl.FMT_SLOT2, linear=8)
    xr = oracle.round_bf16(oracle.rotate(inp.x, inp.signs))
    for r, f in enumerate([2.0 ** 100, 2.0 ** -100, 2.0 ** 40, 2.0 ** -40]):
        xr[r] *= f
    xr[4] = 0.0
    xr[5, ::2] *= 2.0 ** 30
    xr[5, 1::2] *= 2.0 ** -30
    packed, scales = tl.pack(dev(inp.codes, gpu), tl.FMT_SLOT2), dev(inp.scales, gpu)
    y = host(tl.gemm_bf16(packed, scales, tl.FMT_SLOT2, bf16(xr, gpu))).astype(np.float64)
    want = oracle.matvec(inp.codes, inp.scales, xr)
    assert np.all(y[4] == 0.0)
    for r in [0, 1, 2, 3, 5, 6, m - 1]:
        assert oracle.rel_l2(y[r], want[r]) < 1e-5, r
