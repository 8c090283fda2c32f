"""GPU parity of the weight quantiser (tl_quantize: the signed rotation folded
into fp32 weight rows, then round to nearest ternary g128 with a binary16
absmean scale) against the fp64 CPU oracle on the same seeded weights.

The codes are integers decided by floating point: the kernel rotates in fp32,
the oracle in fp64.  Where the two could round differently the test accepts
either result and checks it is valid; everywhere else it demands equality:
- a scale may differ only where the exact group mean lies within the fp32
  error bound of a binary16 rounding boundary;
- a code may differ only where |w'| lies within the rotation's fp32 error
  bound of S/2 (10 butterfly levels: 10 * 2^-24 * sum over the block |w| / 32).
Rows whose rotation is exact in fp32 (one-hot rows, 2 e_k + e_l) must match
bit for bit, the tie at S/2 included."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tl_hadamard_rotate_amd as tl

pytestmark = pytest.mark.gpu


def dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def _weights(n, k, seed, std=0.02):
    rng = np.random.default_rng(seed)
    return (std * rng.standard_normal((n, k))).astype(np.float32)


def _signs(k, seed):
    return synth.draw_signs(np.random.default_rng(seed), k)


def _check(w, signs, codes, scales):
    """codes/scales from the GPU against the oracle, to the bounds above;
    returns the number of positions that were allowed to differ."""
    n, k = w.shape
    wr = oracle.fold_weights(w.astype(np.float64), signs)
    c_o, s_o = oracle.quantize_ternary(wr)
    blk = np.abs(w.astype(np.float64)).reshape(n, k // 1024, 1024).sum(-1) / 32.0
    dw = np.repeat(10 * 2.0 ** -24 * blk, 1024, axis=1)           # |w'_gpu - w'| bound
    g_abs = np.abs(wr).reshape(n, k // 128, 128)
    mean = g_abs.mean(-1)
    dmean = dw.reshape(n, k // 128, 128).max(-1) + 130 * 2.0 ** -24 * mean
    lo = (mean - dmean).astype(np.float16).astype(np.float64)
    hi = (mean + dmean).astype(np.float16).astype(np.float64)
    sg = scales.astype(np.float64)
    assert np.all((sg >= lo) & (sg <= hi)), "a scale outside the rounding window"
    assert np.mean(sg == s_o.astype(np.float64)) > 0.999
    # codes against the scale the GPU chose: exact away from the S/2 boundary
    s_rep = np.repeat(sg, 128, axis=1)
    near = np.abs(np.abs(wr) - 0.5 * s_rep) <= dw
    want = np.where(s_rep == 0, 0, np.where(np.abs(wr) > 0.5 * s_rep, np.sign(wr), 0))
    sure = ~near
    assert np.array_equal(codes[sure], want[sure].astype(np.int8))
    # at the boundary either candidate is valid
    cand_ok = (codes[near] == 0) | (codes[near] == np.sign(wr[near]))
    assert np.all(cand_ok)
    same_s = np.repeat(sg == s_o.astype(np.float64), 128, axis=1)
    assert np.mean(codes[same_s] == c_o[same_s]) > 0.9999
    return int(near.sum())


@pytest.mark.parametrize("n,k", [(1, 1024), (4, 2048), (33, 5120), (7, 17408), (130, 3072)])
def test_quantize_matches_oracle(gpu, n, k):
    w = _weights(n, k, seed=n + k)
    s = _signs(k, seed=k)
    codes, scales = tl.quantize(dev(w, gpu), dev(s, gpu))
    _check(w, s, host(codes), host(scales))


def test_quantize_wide_dynamic_range(gpu):
    """Rows of very different magnitudes (1e-4 .. 1e2), and one all-zero row."""
    n, k = 6, 2048
    w = _weights(n, k, seed=3, std=1.0) * np.array([[1e-4], [1e-2], [1.0], [10.0], [100.0], [0.0]],
                                                   dtype=np.float32)
    s = _signs(k, seed=4)
    codes, scales = tl.quantize(dev(w, gpu), dev(s, gpu))
    c, sc = host(codes), host(scales)
    _check(w, s, c, sc)
    assert not c[5].any() and not sc[5].astype(np.float64).any()


def test_quantize_exact_rows_and_tie(gpu):
    """One-hot rows and rows 2 e_k + e_l rotate exactly in fp32; with k XOR l
    odd every group holds 64 entries of +-3/32 and 64 of +-1/32: S = 1/16 and
    the +-1/32 entries are ties at S/2, which round to 0."""
    k_total = 3072
    s = _signs(k_total, seed=21)
    rows = []
    for k in (0, 7, 1023, 1024 + 300, 2048 + 1023):
        r = np.zeros(k_total, np.float32)
        r[k] = 1.0
        rows.append(r)
    for k, l in ((4, 5), (1024 + 10, 1024 + 11 + 512), (2048 + 1, 2048 + 1022)):
        r = np.zeros(k_total, np.float32)
        r[k], r[l] = 2.0, 1.0
        rows.append(r)
    w = np.stack(rows)
    codes, scales = tl.quantize(dev(w, gpu), dev(s, gpu))
    c_o, s_o = oracle.quantize_weights(w.astype(np.float64), s)
    assert np.array_equal(host(scales), s_o)
    assert np.array_equal(host(codes), c_o)
    # the tie rows: S = 1/16 on their block, half of the codes zero
    for r in range(5, 8):
        sc = host(scales)[r].astype(np.float64)
        assert set(np.unique(sc)) == {0.0, 1.0 / 16}
        blk = np.nonzero(sc)[0][0] // 8
        cb = host(codes)[r, 1024 * blk:1024 * (blk + 1)]
        assert np.sum(cb == 0) == 512 and np.sum(np.abs(cb) == 1) == 512


def test_quantize_invariances_bit_exact(gpu):
    """The kernel's own arithmetic commutes with negation and power-of-two
    factors, so these hold bit for bit on the GPU."""
    n, k = 16, 5120
    w = _weights(n, k, seed=12)
    s = dev(_signs(k, seed=13), gpu)
    c, sc = (host(t) for t in tl.quantize(dev(w, gpu), s))
    c2, sc2 = (host(t) for t in tl.quantize(dev(-w, gpu), s))
    assert np.array_equal(c2, -c) and np.array_equal(sc2, sc)
    c3, sc3 = (host(t) for t in tl.quantize(dev(w * 8.0, gpu), s))
    assert np.array_equal(c3, c)
    assert np.array_equal(sc3.astype(np.float64), sc.astype(np.float64) * 8.0)


def test_quantize_deterministic(gpu):
    w = dev(_weights(64, 17408, seed=5), gpu)
    s = dev(_signs(17408, seed=6), gpu)
    a = [host(t) for t in tl.quantize(w, s)]
    b = [host(t) for t in tl.quantize(w, s)]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint16), b[1].view(np.uint16))


def test_quantize_full_size_sampled_rows(gpu):
    """The gate projection's shape (N = 17408, K = 5120) quantised whole; the
    oracle checks sampled rows."""
    k, n = synth.SHAPES["gate"]
    w = _weights(n, k, seed=77)
    s = _signs(k, seed=78)
    codes, scales = tl.quantize(dev(w, gpu), dev(s, gpu))
    rows = np.concatenate([np.random.default_rng(3).choice(n, size=192, replace=False), [0, n - 1]])
    _check(w[rows], s, host(codes)[rows], host(scales)[rows])


def test_quantize_then_linear_matches_oracle_layer(gpu):
    """quantise -> pack -> tl_linear on activations, against the oracle's own
    codes and scales through its fp64 layer: the whole weight-to-output path."""
    n, k, m = 700, 5120, 3
    w = _weights(n, k, seed=90)
    s = _signs(k, seed=91)
    x = synth.draw_x(np.random.default_rng(92), m, k)
    codes, scales = tl.quantize(dev(w, gpu), dev(s, gpu))
    sd = dev(s, gpu)
    y = host(tl.linear(tl.pack(codes, tl.FMT_SLOT2), scales, tl.FMT_SLOT2, dev(x, gpu), sd))
    c_o, s_o = oracle.quantize_weights(w.astype(np.float64), s)
    want = oracle.linear(x, s, c_o, s_o)
    assert oracle.rel_l2(y.astype(np.float64), want) < 2e-3
