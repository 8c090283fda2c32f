"""GPU parity of the few-token decode GEMV with 2-bit slots (tl_gemv at
2 <= M <= 16): tokens ride on the matrix-core rows, 8 rows of weights per
unit, up to 8 tokens per workgroup (fewer when their activation images do
not fit in LDS); more tokens form a second group in the same launch, paired
workgroups taking the same rows.  Shapes cover a ragged last unit of rows,
fewer rows than a unit, one 1024-block, a partial group (M not a multiple of
the group), two groups (also with fewer row sets than a multiple of 8, so
that the paired grid has idle padding), groups of 2 at K = 17408, and a row
count that needs several row chunks per workgroup.  The 1-bit packing runs
the same kernel (each 16 bits of codes spread into a 2-bit-slot word) and
takes the same shapes.  Every output (or, at the largest N, a
sample of rows in every tile) is compared with the oracle's product on the
same binary16 activations (exact products, fp32 sums: relative L2 < 1e-5
per token) and with the fp64 layer (2e-3)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tl_hadamard_rotate_amd as tl

pytestmark = pytest.mark.gpu

SLOT2 = tl.FMT_SLOT2
BIT1 = tl.FMT_BIT1
FMTS = {"slot2": SLOT2, "bit1": BIT1}


def dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def _per_token_err(y, want):
    d = np.linalg.norm(y - want, axis=1)
    w = np.linalg.norm(want, axis=1)
    return float(np.max(d / np.maximum(w, 1e-300)))


@pytest.mark.parametrize("m,n,k", [
    (2, 1000, 2048), (3, 67, 1024), (5, 5, 1024), (7, 300, 3072), (8, 1000, 5120),
    (9, 130, 1024), (13, 777, 6144), (16, 4097, 2048), (2, 1024, 17408), (3, 333, 17408),
    (4, 515, 17408), (6, 2051, 4096)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16], ids=["f32", "f16"])
@pytest.mark.parametrize("fmt", sorted(FMTS))
def test_gemv_few_tokens_every_output(gpu, m, n, k, out_dtype, fmt):
    f = FMTS[fmt]
    inp = synth.linear_inputs(n, k, m, cfg=3, linear=7 * m + n, outliers=True, binary=f == BIT1)
    packed = tl.pack(dev(inp.codes, gpu), f)
    x_rot16 = oracle.rotate(inp.x, inp.signs).astype(np.float16)
    y = host(tl.gemv(packed, dev(inp.scales, gpu), f, dev(x_rot16, gpu),
                     out_dtype=out_dtype)).astype(np.float64)
    want16 = oracle.matvec(inp.codes, inp.scales, x_rot16)
    # binary16 outputs: the fp32 sum rounded once more (half an ulp, 2^-11)
    assert _per_token_err(y, want16) < (1e-5 if out_dtype == torch.float32 else 1e-3)
    assert oracle.rel_l2(y, oracle.linear(inp.x, inp.signs, inp.codes, inp.scales)) < 2e-3


@pytest.mark.parametrize("m", [8, 16])
@pytest.mark.parametrize("fmt", sorted(FMTS))
def test_gemv_few_tokens_row_chunks(gpu, fmt, m):
    """gate|up concatenated (N = 34816, K = 5120) at M = 8 and 16: a
    workgroup's 136 rows (272 with two token groups) take several row chunks
    of partial sums; sampled rows in every 64-row tile, all tokens."""
    f = FMTS[fmt]
    k, n = 5120, 34816
    inp = synth.linear_inputs(n, k, m, cfg=3, linear=11, outliers=True, binary=f == BIT1)
    packed = tl.pack(dev(inp.codes, gpu), f)
    x_rot16 = oracle.rotate(inp.x, inp.signs).astype(np.float16)
    y = host(tl.gemv(packed, dev(inp.scales, gpu), f, dev(x_rot16, gpu))).astype(np.float64)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(0, n, 64), np.arange(63, n, 64),
                                     rng.integers(0, n, size=400)]))
    want16 = oracle.matvec(inp.codes[rows], inp.scales[rows], x_rot16)
    assert _per_token_err(y[:, rows], want16) < 1e-5


def test_gemv_few_tokens_scale_per_token(gpu):
    """Tokens of very different magnitudes (factors 2^-12 .. 2^4, one all
    zero) in one launch: each token's activations are scaled on their own,
    so every token keeps the fp32 bar."""
    m, n, k = 8, 640, 4096
    inp = synth.linear_inputs(n, k, m, cfg=3, linear=3, outliers=False)
    x_rot = oracle.rotate(inp.x, inp.signs)
    f = np.array([1.0, 2.0 ** -12, 2.0 ** 4, 0.0, 2.0 ** -6, 1.0, 2.0 ** 3, 2.0 ** -9])
    x_rot16 = (x_rot * f[:, None]).astype(np.float16)
    packed = tl.pack(dev(inp.codes, gpu), SLOT2)
    y = host(tl.gemv(packed, dev(inp.scales, gpu), SLOT2, dev(x_rot16, gpu))).astype(np.float64)
    want16 = oracle.matvec(inp.codes, inp.scales, x_rot16)
    assert np.all(y[3] == 0.0)
    live = [i for i in range(m) if i != 3]
    assert _per_token_err(y[live], want16[live]) < 1e-5


def test_gemv_few_tokens_deterministic_and_token_independent(gpu):
    """Two calls give the same bits; a token's outputs do not depend on the
    other tokens of its group (token 0 next to zero partners equals token 0
    next to random ones, at M = 8 and at M = 2)."""
    m, n, k = 8, 2048, 5120
    inp = synth.linear_inputs(n, k, m, cfg=3, linear=5, outliers=True)
    packed = tl.pack(dev(inp.codes, gpu), SLOT2)
    scales = dev(inp.scales, gpu)
    x16 = oracle.rotate(inp.x, inp.signs).astype(np.float16)
    a = host(tl.gemv(packed, scales, SLOT2, dev(x16, gpu)))
    b = host(tl.gemv(packed, scales, SLOT2, dev(x16, gpu)))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    for mm in (8, 2):
        rand = host(tl.gemv(packed, scales, SLOT2, dev(x16[:mm], gpu)))
        lone = x16[:mm].copy()
        lone[1:] = 0
        c = host(tl.gemv(packed, scales, SLOT2, dev(lone, gpu)))
        assert np.array_equal(c[0].view(np.uint32), rand[0].view(np.uint32)), mm


@pytest.mark.parametrize("shape", ["q", "gate"])
def test_gemv_sixteen_tokens_are_two_groups_of_eight(gpu, shape):
    """At M = 16 on q and gate the few-token kernel runs two groups of 8 tokens
    in one launch, each with the arithmetic of an 8-token launch: tokens
    0..7 and 8..15 equal, bit for bit, the launches on those 8 tokens alone
    (a launch plan that sent M = 16 to another kernel would change the
    rounding of the sums).  Both shapes take one group of 8 at M = 8: their
    workgroups hold more than 8 M / 3 rows."""
    k, n = synth.SHAPES[shape]
    inp = synth.linear_inputs(n, k, 16, cfg=3, linear=synth.LINEAR_ID[shape], outliers=True)
    packed = tl.pack(dev(inp.codes, gpu), SLOT2)
    scales = dev(inp.scales, gpu)
    x16 = oracle.rotate(inp.x, inp.signs).astype(np.float16)
    y = host(tl.gemv(packed, scales, SLOT2, dev(x16, gpu)))
    for g in range(2):
        part = host(tl.gemv(packed, scales, SLOT2, dev(x16[8 * g:8 * g + 8], gpu)))
        assert np.array_equal(y[8 * g:8 * g + 8].view(np.uint32), part.view(np.uint32)), g
