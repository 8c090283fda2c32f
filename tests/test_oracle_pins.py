"""Pins for the CPU oracle: everything here checks the oracle against facts
that do not come from the oracle itself (a library routine, closed forms,
invariants, exhaustive enumeration, exact rational brute force, the pages'
printed figures, hand-worked packing examples)."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _popcount_hadamard(n):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    anded = i & j
    bits = np.zeros_like(anded)
    for b in range(int(math.log2(n)) + 1):
        bits += (anded >> b) & 1
    return np.where(bits % 2 == 0, 1.0, -1.0)


# ---------------------------------------------------------------------------
# Hadamard matrix
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024])
def test_hadamard_matches_scipy_and_popcount(n):
    h = oracle.hadamard(n)
    assert np.array_equal(h, scipy.linalg.hadamard(n).astype(np.float64))
    assert np.array_equal(h, _popcount_hadamard(n))


@pytest.mark.parametrize("n", [2, 8, 64, 1024])
def test_hadamard_orthogonal(n):
    h = oracle.hadamard(n)
    assert np.array_equal(h @ h.T, n * np.eye(n))
    q = h / math.sqrt(n)
    assert np.allclose(q @ q, np.eye(n), atol=1e-12)


def test_hadamard_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.hadamard(12)


# ---------------------------------------------------------------------------
# Rotation
# ---------------------------------------------------------------------------

def _rotate_bruteforce(x, s, n):
    """Per-element definition with the popcount form of H, pure Python."""
    m, k = len(x), len(x[0])
    out = [[0.0] * k for _ in range(m)]
    for r in range(m):
        for b in range(k // n):
            for i in range(n):
                acc = 0.0
                for j in range(n):
                    sign = -1.0 if bin(i & j).count("1") % 2 else 1.0
                    acc += sign * s[b * n + j] * x[r][b * n + j]
                out[r][b * n + i] = acc / math.sqrt(n)
    return out


def test_rotate_matches_elementwise_definition_multi_block():
    rng = np.random.default_rng(11)
    n, k, m = 8, 32, 3
    x = rng.standard_normal((m, k))
    s = rng.choice([-1, 1], size=k)
    ref = np.array(_rotate_bruteforce(x.tolist(), s.tolist(), n))
    got = oracle.rotate(x, s, block=n)
    assert np.allclose(got, ref, rtol=0, atol=1e-13)


def test_rotate_signs_applied_before_hadamard():
    # x = e_j: signs first gives s_j * H[:, j] / sqrt(n); signs last would
    # give s * H[:, j] / sqrt(n), which differs unless s is constant.
    n = 16
    s = np.array([1, -1] * 8)
    x = np.zeros((1, n))
    x[0, 3] = 1.0
    got = oracle.rotate(x, s, block=n)[0]
    want = s[3] * scipy.linalg.hadamard(n)[:, 3] / 4.0
    assert np.array_equal(got, want)


@pytest.mark.parametrize("block", [8, 1024])
def test_rotate_closed_forms(block):
    rng = np.random.default_rng(5)
    k = 2 * block
    s = rng.choice([-1, 1], size=k)
    # one-hot input: column j of H times s_j, divided by sqrt(n)
    for j in (0, 1, block - 1, block + 7):
        x = np.zeros((1, k))
        x[0, j] = 1.0
        got = oracle.rotate(x, s, block=block)[0]
        b, jj = divmod(j, block)
        want = np.zeros(k)
        want[b * block:(b + 1) * block] = s[j] * scipy.linalg.hadamard(block)[:, jj] / math.sqrt(block)
        assert np.array_equal(got, want)
    # x = s on a block: H . 1 = n e_0, so the block maps to sqrt(n) e_0
    x = s[None, :].astype(np.float64)
    got = oracle.rotate(x, s, block=block)[0]
    want = np.zeros(k)
    want[0] = want[block] = math.sqrt(block)
    # exact when sqrt(block) is a power of two (block 1024), else within 1 ulp
    assert np.allclose(got, want, rtol=2.3e-16, atol=0)
    if block == 1024:
        assert np.array_equal(got, want)


def test_rotate_is_orthogonal():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 3072))
    s = rng.choice([-1, 1], size=3072)
    r = oracle.rotate(x, s)
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    assert np.allclose(oracle.rotate_transpose(r, s), x, atol=1e-12)


def test_rotate_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.rotate(np.zeros((1, 1000)), np.ones(1000))


# ---------------------------------------------------------------------------
# Packings
# ---------------------------------------------------------------------------

def test_trit5_hand_worked_examples():
    g = _golden("packing_examples.json")
    for ex in g["trit5_full_bytes"]:
        codes = np.zeros((1, 128), dtype=np.int8)
        codes[0, :5] = ex["codes"]
        assert int(oracle.pack_trit5(codes)[0, 0]) == ex["byte"], ex
    for ex in g["trit5_tail_bytes"]:
        codes = np.zeros((1, 128), dtype=np.int8)
        codes[0, 125:] = ex["codes"]
        assert int(oracle.pack_trit5(codes)[0, 25]) == ex["byte"], ex


def test_slot2_hand_worked_examples():
    for ex in _golden("packing_examples.json")["slot2_bytes"]:
        codes = np.zeros((1, 128), dtype=np.int8)
        codes[0, :4] = ex["codes"]
        assert int(oracle.pack_slot2(codes)[0, 0]) == ex["byte"], ex


def test_trit5_exhaustive_full_bytes():
    # all 3^5 digit patterns in the first byte of a group, the rest zeros
    combos = np.array(list(itertools.product((-1, 0, 1), repeat=5)), dtype=np.int8)
    codes = np.zeros((len(combos), 128), dtype=np.int8)
    codes[:, :5] = combos
    packed = oracle.pack_trit5(codes)
    assert packed.shape == (243, 26)
    assert sorted(packed[:, 0].tolist()) == list(range(243))
    assert bytes(packed.tobytes()) == oracle.pack_trit5_loop(codes)
    assert np.array_equal(oracle.unpack_trit5(packed, 128), codes)


def test_trit5_exhaustive_tail_bytes():
    combos = np.array(list(itertools.product((-1, 0, 1), repeat=3)), dtype=np.int8)
    codes = np.zeros((len(combos), 128), dtype=np.int8)
    codes[:, 125:] = combos
    packed = oracle.pack_trit5(codes)
    assert sorted(packed[:, 25].tolist()) == list(range(108, 135))
    assert bytes(packed.tobytes()) == oracle.pack_trit5_loop(codes)
    assert np.array_equal(oracle.unpack_trit5(packed, 128), codes)


def test_trit5_pack_of_unpack_is_identity_on_every_valid_byte():
    zero_group = oracle.pack_trit5(np.zeros((1, 128), dtype=np.int8))[0]
    for pos in (0, 13, 24):
        for b in range(243):
            row = zero_group.copy()
            row[pos] = b
            c = oracle.unpack_trit5(row[None, :], 128)
            assert np.array_equal(oracle.pack_trit5(c)[0], row)
    for b in range(108, 135):
        row = zero_group.copy()
        row[25] = b
        c = oracle.unpack_trit5(row[None, :], 128)
        assert np.array_equal(oracle.pack_trit5(c)[0], row)


def test_trit5_rejects_every_invalid_byte():
    zero_group = oracle.pack_trit5(np.zeros((1, 128), dtype=np.int8))[0]
    for b in range(243, 256):
        row = zero_group.copy()
        row[3] = b
        with pytest.raises(ValueError):
            oracle.unpack_trit5(row[None, :], 128)
    for b in list(range(0, 108)) + list(range(135, 256)):
        row = zero_group.copy()
        row[25] = b
        with pytest.raises(ValueError):
            oracle.unpack_trit5(row[None, :], 128)


def test_slot2_exhaustive():
    combos = np.array(list(itertools.product((-1, 0, 1), repeat=4)), dtype=np.int8)
    codes = np.zeros((len(combos), 128), dtype=np.int8)
    codes[:, :4] = combos
    packed = oracle.pack_slot2(codes)
    assert bytes(packed.tobytes()) == oracle.pack_slot2_loop(codes)
    valid = sorted(packed[:, 0].tolist())
    assert len(set(valid)) == 81
    assert np.array_equal(oracle.unpack_slot2(packed, 128), codes)
    for b in range(256):
        row = packed[0].copy()
        row[0] = b
        has3 = any(((b >> (2 * i)) & 3) == 3 for i in range(4))
        if has3:
            with pytest.raises(ValueError):
                oracle.unpack_slot2(row[None, :], 128)
        else:
            c = oracle.unpack_slot2(row[None, :], 128)
            assert np.array_equal(oracle.pack_slot2(c)[0], row)


def test_bit1_hand_worked_examples():
    for ex in _golden("packing_examples.json")["bit1_bytes"]:
        codes = np.zeros((1, 128), dtype=np.int8) - 1
        codes[0, :8] = ex["codes"]
        assert int(oracle.pack_bit1(codes)[0, 0]) == ex["byte"], ex


def test_bit1_exhaustive():
    # all 256 bytes: unpack, repack, and the pure-Python packer agree
    packed = np.arange(256, dtype=np.uint8).reshape(1, 256)
    codes = oracle.unpack_bit1(packed, 2048)
    assert set(np.unique(codes).tolist()) == {-1, 1}
    assert np.array_equal(oracle.pack_bit1(codes), packed)
    assert bytes(packed.tobytes()) == oracle.pack_bit1_loop(codes)
    # bit i of byte j is weight 8j + i
    for b in range(256):
        want = [1 if (b >> i) & 1 else -1 for i in range(8)]
        assert codes[0, 8 * b:8 * b + 8].tolist() == want


def test_bit1_rejects_zero_and_bad_codes():
    for bad in (0, 2):
        c = np.ones((1, 128), dtype=np.int8)
        c[0, 5] = bad
        with pytest.raises(ValueError):
            oracle.pack_bit1(c)
        with pytest.raises(ValueError):
            oracle.pack_bit1_loop(c)


def test_bit1_holds_the_same_weights_as_the_ternary_packings():
    rng = np.random.default_rng(5)
    codes = (2 * rng.integers(0, 2, size=(5, 1024)) - 1).astype(np.int8)
    scales = rng.standard_normal((5, 8)).astype(np.float16)
    x = rng.standard_normal((2, 1024)).astype(np.float16)
    ys = [oracle.matvec_packed(oracle.pack(codes, f), scales, f, x.astype(np.float64), 1024)
          for f in (oracle.FMT_TRIT5, oracle.FMT_SLOT2, oracle.FMT_BIT1)]
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[1], ys[2])
    assert np.array_equal(oracle.unpack_bit1(oracle.pack_bit1(codes), 1024), codes)


def test_packings_hold_the_same_weights_random():
    rng = np.random.default_rng(3)
    codes = rng.integers(-1, 2, size=(7, 2048)).astype(np.int8)
    t = oracle.pack_trit5(codes)
    s = oracle.pack_slot2(codes)
    assert t.shape == (7, 16 * 26) and s.shape == (7, 512)
    assert bytes(t.tobytes()) == oracle.pack_trit5_loop(codes)
    assert bytes(s.tobytes()) == oracle.pack_slot2_loop(codes)
    assert np.array_equal(oracle.unpack_trit5(t, 2048), codes)
    assert np.array_equal(oracle.unpack_slot2(s, 2048), codes)


def test_pack_rejects_bad_codes():
    with pytest.raises(ValueError):
        oracle.pack_trit5(np.full((1, 128), 2, dtype=np.int8))
    with pytest.raises(ValueError):
        oracle.pack_slot2(np.zeros((1, 100), dtype=np.int8))


def test_packed_sizes_closed_form():
    for n, k in [(1, 128), (1024, 1024), (17408, 5120), (5120, 17408)]:
        assert oracle.packed_bytes(n, k, oracle.FMT_TRIT5) == n * 26 * k // 128
        assert oracle.packed_bytes(n, k, oracle.FMT_SLOT2) == n * k // 4
        assert oracle.packed_bytes(n, k, oracle.FMT_BIT1) == n * k // 8
    assert oracle.packed_bytes(1024, 1024, oracle.FMT_TRIT5) == 212_992
    assert oracle.packed_bytes(1024, 1024, oracle.FMT_SLOT2) == 262_144


def test_format_densities_against_page_figures():
    f = _golden("pages_figures.json")
    g = f["group_size"]["value"]
    # information of one trit and the effective cost with one FP16 scale per group
    assert abs(math.log2(3) - f["trit_information_bits"]["value"]) < 5e-4
    assert abs(math.log2(3) + 16 / g - f["ternary_effective_bpw"]["value"]) < 5e-3
    assert abs(1 + 16 / g - f["binary_effective_bpw"]["value"]) < 1e-12
    # this library's packings, bits per weight including the scale
    trit5_bpw = 8 * oracle.trit5_group_bytes(g) / g + 16 / g
    slot2_bpw = 8 * (g // 4) / g + 16 / g
    assert trit5_bpw == 1.75 and slot2_bpw == 2.125
    # the binary packing is exactly the page's 1.125 bits per weight
    bit1_bpw = 8 * oracle.packed_bytes(1, g, oracle.FMT_BIT1) / g + 16 / g
    assert bit1_bpw == f["binary_effective_bpw"]["value"]
    # both file sizes must describe the same number of weights (same weights,
    # different packing): 5.95 GB / 1.75 bpw vs 7.21 GB / 2.125 bpw
    w_dense = f["dense_trit_file_gb"]["value"] * 8 / trit5_bpw
    w_slot = f["slot2_file_gb"]["value"] * 8 / slot2_bpw
    assert abs(w_dense / w_slot - 1) < 0.005
    # and 16 bits vs 1.75 is the "about nine times smaller" of the pages
    assert abs(16 / trit5_bpw - f["size_ratio_vs_original"]["value"]) < 0.2
    # a packing of 5 trits per byte across group boundaries (1.6 code bits)
    # would not reconcile the two file sizes nearly as well
    w_cross = f["dense_trit_file_gb"]["value"] * 8 / (1.6 + 16 / g)
    assert abs(w_cross / w_slot - 1) > abs(w_dense / w_slot - 1)


# ---------------------------------------------------------------------------
# Dequantisation and the layer
# ---------------------------------------------------------------------------

def _exact_layer(x16, s, codes, scales16, block, group):
    """y[r, n] * sqrt(block) in exact rationals, H from the popcount form."""
    m, k = x16.shape
    xs = [[Fraction(float(v)) for v in row] for row in x16]
    sc = [[Fraction(float(v)) for v in row] for row in scales16]
    # rotated (times sqrt(block)) activations, exact
    xr = []
    for r in range(m):
        row = []
        for b in range(k // block):
            for i in range(block):
                acc = Fraction(0)
                for j in range(block):
                    sign = -1 if bin(i & j).count("1") % 2 else 1
                    acc += sign * int(s[b * block + j]) * xs[r][b * block + j]
                row.append(acc)
        xr.append(row)
    out = []
    for r in range(m):
        out.append([sum((int(codes[n, kk]) * sc[n][kk // group] * xr[r][kk]
                         for kk in range(k)), Fraction(0)) for n in range(codes.shape[0])])
    return out


def test_layer_bruteforce_exhaustive_code_rows():
    """All 3^8 code rows, K = 8, block 8, groups of 4, exact rationals."""
    rng = np.random.default_rng(2024)
    codes = np.array(list(itertools.product((-1, 0, 1), repeat=8)), dtype=np.int8)
    scales = np.abs(rng.standard_normal((codes.shape[0], 2))).astype(np.float16)
    x = rng.standard_normal((2, 8)).astype(np.float16)
    s = rng.choice([-1, 1], size=8).astype(np.int8)
    got = oracle.linear(x, s, codes, scales, block=8, group=4)
    exact = _exact_layer(x, s, codes, scales, 8, 4)
    want = np.array([[float(v) for v in row] for row in exact]) / math.sqrt(8)
    mag = np.abs(codes).astype(np.float64) @ np.ones(8)
    tol = 1e-14 * (1 + np.abs(want)) + 1e-14 * mag[None, :]
    assert np.all(np.abs(got - want) <= tol)


def test_layer_bruteforce_several_blocks_and_groups():
    rng = np.random.default_rng(99)
    n, k = 6, 24
    codes = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    scales = (rng.standard_normal((n, k // 4)) * 0.5).astype(np.float16)
    x = rng.standard_normal((3, k)).astype(np.float16)
    s = rng.choice([-1, 1], size=k).astype(np.int8)
    got = oracle.linear(x, s, codes, scales, block=8, group=4)
    want = np.array([[float(v) for v in row] for row in
                     _exact_layer(x, s, codes, scales, 8, 4)]) / math.sqrt(8)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


def test_dequant_group_index_along_k():
    codes = np.ones((2, 256), dtype=np.int8)
    scales = np.array([[1.0, 2.0], [3.0, 4.0]], dtype=np.float16)
    w = oracle.dequant(codes, scales)
    assert np.array_equal(w[0, :128], np.ones(128)) and np.array_equal(w[0, 128:], 2 * np.ones(128))
    assert np.array_equal(w[1, :128], 3 * np.ones(128)) and np.array_equal(w[1, 128:], 4 * np.ones(128))


def test_matvec_one_hot_closed_form():
    rng = np.random.default_rng(4)
    n, k = 16, 1024
    codes = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    scales = np.abs(rng.standard_normal((n, k // 128))).astype(np.float16)
    for kk in (0, 127, 128, 511, 1023):
        x = np.zeros((1, k))
        x[0, kk] = 1.0
        y = oracle.matvec(codes, scales, x)[0]
        want = codes[:, kk].astype(np.float64) * scales[:, kk // 128].astype(np.float64)
        assert np.array_equal(y, want)


def test_matvec_zero_codes_give_zero():
    rng = np.random.default_rng(8)
    codes = np.zeros((5, 1024), dtype=np.int8)
    scales = np.abs(rng.standard_normal((5, 8))).astype(np.float16)
    x = rng.standard_normal((3, 1024))
    assert np.array_equal(oracle.matvec(codes, scales, x), np.zeros((3, 5)))


def test_matvec_linear_in_scales():
    rng = np.random.default_rng(9)
    codes = rng.integers(-1, 2, size=(12, 2048)).astype(np.int8)
    s1 = np.abs(rng.standard_normal((12, 16)))
    s2 = np.abs(rng.standard_normal((12, 16)))
    x = rng.standard_normal((2, 2048))
    y1 = oracle.matvec(codes, s1, x)
    assert np.array_equal(oracle.matvec(codes, 4.0 * s1, x), 4.0 * y1)
    assert np.array_equal(oracle.matvec(codes, s1 / 8.0, x), y1 / 8.0)
    assert np.allclose(oracle.matvec(codes, s1 + s2, x), y1 + oracle.matvec(codes, s2, x),
                       rtol=1e-12, atol=1e-12)


def test_matvec_orientation_nonsymmetric():
    # y[m, n] = sum_k x[m, k] W[n, k]: a transposed operand fails this
    # square W (N = K = 128) so that a transposed operand still has the right shape
    codes = np.zeros((128, 128), dtype=np.int8)
    codes[0, 1] = 1
    codes[1, 0] = -1
    codes[0, 2] = 1
    scales = np.ones((128, 1), dtype=np.float16)
    scales[0, 0] = 2.0
    scales[1, 0] = 3.0
    x = np.zeros((1, 128))
    x[0, 0] = 5.0
    x[0, 1] = 7.0
    want = np.zeros((1, 128))
    want[0, 0] = 2.0 * 7.0
    want[0, 1] = -3.0 * 5.0
    assert np.array_equal(oracle.matvec(codes, scales, x), want)


def test_matvec_packed_same_result_both_formats():
    rng = np.random.default_rng(10)
    codes = rng.integers(-1, 2, size=(9, 3072)).astype(np.int8)
    scales = np.abs(rng.standard_normal((9, 24))).astype(np.float16)
    x = rng.standard_normal((2, 3072)).astype(np.float16)
    y_c = oracle.matvec(codes, scales, x)
    for fmt in (oracle.FMT_TRIT5, oracle.FMT_SLOT2):
        y_p = oracle.matvec_packed(oracle.pack(codes, fmt), scales, fmt, x, 3072)
        assert np.array_equal(y_p, y_c)


def test_fold_invariant_and_negative():
    """Folding the rotation into real weight rows and rotating the
    activations leaves the layer unchanged; forgetting the runtime rotation
    gives an unrelated result (the silent failure the pages warn about)."""
    rng = np.random.default_rng(12)
    k = 3072
    w = rng.standard_normal((64, k))
    x = rng.standard_normal((4, k))
    s = rng.choice([-1, 1], size=k)
    wf = oracle.fold_weights(w, s)
    y = x @ w.T
    assert oracle.rel_l2(oracle.rotate(x, s) @ wf.T, y) < 1e-12
    wrong = oracle.rel_l2(x @ wf.T, y)
    assert 1.2 < wrong < 1.6   # ~sqrt(2) for unrelated outputs of equal size


# ---------------------------------------------------------------------------
# Metrics
# ---------------------------------------------------------------------------

def test_rel_l2_hand_values():
    assert oracle.rel_l2([3.0, 4.0], [3.0, 4.0]) == 0.0
    assert oracle.rel_l2([3.0, 4.0 + 5.0], [3.0, 4.0]) == 1.0
    assert oracle.rel_l2([0.0], [0.0]) == 0.0


def test_fp16_ulp_matches_numpy_spacing():
    vals = np.array([0.0, 1e-7, 6e-5, 6.2e-5, 0.3, 1.0, 1.5, 2.0, 3.9, 1000.0, 60000.0])
    want = np.spacing(vals.astype(np.float16)).astype(np.float64)
    assert np.array_equal(oracle.fp16_ulp(vals.astype(np.float16)), want)


# ---------------------------------------------------------------------------
# Weight quantiser (fold the rotation into the rows, round to ternary g128)
# ---------------------------------------------------------------------------

def _runs(runs):
    return np.concatenate([np.full(c, v, dtype=np.float64) for v, c in runs])


def test_quantize_hand_worked_groups():
    """Groups worked by hand (tests/golden/quantize_examples.json), placed one
    after the other in a single row, so a scale taken over the wrong span
    shows too."""
    groups = _golden("quantize_examples.json")["groups"]
    row = np.concatenate([_runs(g["runs"]) for g in groups])[None, :]
    codes, scales = oracle.quantize_ternary(row)
    assert codes.dtype == np.int8 and scales.dtype == np.float16
    assert scales.shape == (1, len(groups))
    for i, g in enumerate(groups):
        assert float(scales[0, i]) == g["scale"], (i, g["work"])
        assert np.array_equal(codes[0, 128 * i:128 * (i + 1)], _runs(g["codes"])), (i, g["work"])


def _fp16_neighbours(v):
    h = np.float16(v)
    return [np.nextafter(h, np.float16(-np.inf)), h, np.nextafter(h, np.float16(np.inf))]


def test_quantize_scale_is_nearest_binary16_to_exact_mean_and_codes_nearest():
    """Exact rational brute force on small random rows: the scale is the
    binary16 number nearest the exact mean of |w| (ties to the even mantissa),
    and each code is the point of {-S, 0, S} nearest w (0 on a tie with S/2)."""
    rng = np.random.default_rng(11)
    w = rng.standard_normal((3, 256)) * np.array([[0.02], [1.0], [300.0]])
    w[1, :128] = np.round(w[1, :128] * 8) / 8      # many exact ties possible
    codes, scales = oracle.quantize_ternary(w)
    for n in range(w.shape[0]):
        for g in range(2):
            seg = w[n, 128 * g:128 * (g + 1)]
            mean = sum(Fraction(float(abs(v))) for v in seg) / 128
            s = scales[n, g]
            dist = abs(Fraction(float(s)) - mean)
            for nb in _fp16_neighbours(float(s)):
                d_nb = abs(Fraction(float(nb)) - mean)
                assert dist <= d_nb
                if dist == d_nb and nb != s:   # a tie between two binary16 numbers
                    assert int(np.float16(s).view(np.uint16)) % 2 == 0
            S = Fraction(float(s))
            for k in range(128):
                v = Fraction(float(seg[k]))
                c = int(codes[n, 128 * g + k])
                dists = {cc: abs(v - cc * S) for cc in (-1, 0, 1)}
                best = min(dists.values())
                assert dists[c] == best, (n, g, k)
                if list(dists.values()).count(best) > 1:
                    assert c == 0


def test_quantize_invariances():
    """Negating the weights negates the codes; a power-of-two factor scales S
    exactly; permuting a group permutes its codes; zero groups give S = 0."""
    rng = np.random.default_rng(5)
    w = rng.standard_normal((4, 512)) * 0.03
    c, s = oracle.quantize_ternary(w)
    c2, s2 = oracle.quantize_ternary(-w)
    assert np.array_equal(c2, -c) and np.array_equal(s2, s)
    for e in (3, -3):
        c3, s3 = oracle.quantize_ternary(w * 2.0 ** e)
        assert np.array_equal(c3, c)
        assert np.array_equal(s3.astype(np.float64), s.astype(np.float64) * 2.0 ** e)
    perm = rng.permutation(128)
    wp = w.copy()
    wp[:, 128:256] = w[:, 128:256][:, perm]
    c4, s4 = oracle.quantize_ternary(wp)
    assert np.array_equal(s4, s)
    assert np.array_equal(c4[:, 128:256], c[:, 128:256][:, perm])
    wz = w.copy()
    wz[2, 256:384] = 0.0
    c5, s5 = oracle.quantize_ternary(wz)
    assert s5[2, 2] == 0 and not c5[2, 256:384].any()


def test_quantize_weights_one_hot_closed_form():
    """A weight row e_k rotates to s_k * H[:, k mod 1024] / 32 on its block
    (Sylvester H[i, j] = (-1)^popcount(i AND j)): every group of that block has
    S = 1/32 and codes s_k * H[i, k mod 1024]; the other blocks are zero."""
    k_total = 3072
    rng = np.random.default_rng(8)
    signs = (rng.integers(0, 2, k_total) * 2 - 1).astype(np.int8)
    ks = [0, 5, 1023, 1024 + 77, 2048 + 600]
    w = np.zeros((len(ks), k_total))
    for r, k in enumerate(ks):
        w[r, k] = 1.0
    codes, scales = oracle.quantize_weights(w, signs)
    h = _popcount_hadamard(1024)
    for r, k in enumerate(ks):
        b, j = divmod(k, 1024)
        want = np.zeros(k_total, dtype=np.int8)
        want[1024 * b:1024 * (b + 1)] = (signs[k] * h[:, j]).astype(np.int8)
        assert np.array_equal(codes[r], want), k
        want_s = np.zeros(k_total // 128)
        want_s[8 * b:8 * (b + 1)] = 1.0 / 32
        assert np.array_equal(scales[r].astype(np.float64), want_s), k


# ---------------------------------------------------------------------------
# bfloat16 rounding of activations
# ---------------------------------------------------------------------------

def test_round_bf16_hand_worked():
    """bf16 keeps 8 significant bits: spacing 2^-7 in [1, 2)."""
    cases = [
        (1.0, 1.0),
        (1.0 + 2.0 ** -8, 1.0),                       # tie, even significand 1.0000000
        (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),       # tie between 1+2^-7 and 1+2^-6 -> even
        (1.0 + 2.0 ** -8 + 2.0 ** -20, 1.0 + 2.0 ** -7),   # just above the tie
        (-1.5, -1.5),
        (3.0 + 2.0 ** -7, 3.0),                       # spacing 2^-6 in [2, 4): a tie -> even
        (3.0 + 2.0 ** -6, 3.0 + 2.0 ** -6),           # representable
        (255.5, 256.0),                               # spacing 1 in [128, 256): tie -> 256
        (2.0 - 2.0 ** -9, 2.0),                       # rounds up into the next binade
        (0.1, 0.10009765625),                         # 0.1 * 2^4 = 1.6 -> 205/128 * 2^-4
    ]
    for x, want in cases:
        assert oracle.round_bf16(np.array([x]))[0] == want, x


def _bf16_bits_rne(x32):
    """Independent route: round the fp32 bit pattern to its top 16 bits,
    nearest with ties to even."""
    b = x32.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def test_round_bf16_matches_bit_rounding_of_fp32():
    rng = np.random.default_rng(17)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    # include exact ties of fp32 patterns: low 16 bits 0x8000
    t = (rng.integers(0, 2 ** 31, 20000, dtype=np.uint64) & ~np.uint64(0xFFFF)) | np.uint64(0x8000)
    x = np.concatenate([x, t.astype(np.uint32).view(np.float32)])
    x = x[np.isfinite(x) & (np.abs(x) >= 2.0 ** -120) & (np.abs(x) < 2.0 ** 120)]
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), _bf16_bits_rne(x))


def test_round_bf16_fixed_points_and_bound():
    rng = np.random.default_rng(18)
    x = rng.standard_normal(10000) * 10.0 ** rng.uniform(-6, 6, 10000)
    r = oracle.round_bf16(x)
    assert np.array_equal(oracle.round_bf16(r), r)                 # bf16 values stay put
    assert np.all(np.abs(r - x) <= 2.0 ** -8 * np.abs(x))          # half spacing bound
    assert np.all(np.diff(oracle.round_bf16(np.sort(x))) >= 0)     # monotone
