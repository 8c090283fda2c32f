"""Planted mistakes in the oracle (on the CPU only) must each make at least one
pin fail.  This shows the pins are strong enough to catch a dropped term, a
wrong sign or index, or a transposed operand anywhere in the oracle."""
import numpy as np
import pytest

import oracle
import oracle.ternary_ref as ref
from tests import test_oracle_pins as pins

_orig = {name: getattr(ref, name) for name in
         ("hadamard", "rotate", "dequant", "matvec", "pack_trit5", "unpack_trit5",
          "pack_slot2", "unpack_slot2", "pack_bit1", "unpack_bit1", "quantize_ternary",
          "fold_weights", "round_bf16")}


def _rotate_signs_last(x, signs, block=ref.BLOCK):
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[None, :]
    s = np.asarray(signs, dtype=np.float64)
    h = _orig["hadamard"](block)
    out = np.empty_like(x)
    for b in range(x.shape[1] // block):
        cols = slice(b * block, (b + 1) * block)
        out[:, cols] = (x[:, cols] @ h.T) / np.sqrt(block) * s[cols]
    return out


def _rotate_wrong_norm(x, signs, block=ref.BLOCK):
    return _orig["rotate"](x, signs, block) / np.sqrt(block)


def _rotate_one_sign_slice(x, signs, block=ref.BLOCK):
    # every block reuses the signs of block 0
    s = np.asarray(signs).reshape(-1)
    k = s.shape[0]
    return _orig["rotate"](x, np.tile(s[:block], k // block), block)


def _hadamard_bit_reversed(n):
    h = _orig["hadamard"](n)
    bits = max(n.bit_length() - 1, 0)
    perm = [int(format(i, f"0{bits}b")[::-1], 2) if bits else 0 for i in range(n)]
    return h[perm]


def _dequant_group_mod(codes, scales, group=ref.GROUP):
    c = np.asarray(codes, dtype=np.float64)
    s = np.asarray(scales, dtype=np.float64)
    n, k = c.shape
    idx = np.arange(k) % s.shape[1]
    return c * s[:, idx]


def _dequant_drop_scale(codes, scales, group=ref.GROUP):
    return np.asarray(codes, dtype=np.float64)


def _matvec_transposed(codes, scales, x_rot, group=ref.GROUP):
    xr = np.asarray(x_rot, dtype=np.float64)
    if xr.ndim == 1:
        xr = xr[None, :]
    w = _orig["dequant"](codes, scales, group)
    if w.shape[0] == w.shape[1]:
        return xr @ w
    return xr @ w.T


def _pack_trit5_big_endian(codes, group=ref.GROUP):
    c = np.asarray(codes, dtype=np.int64)
    flipped = c.copy()
    n, k = c.shape
    gb = ref.trit5_group_bytes(group)
    d = np.ones((n, k // group, gb * 5), dtype=np.int64)
    d[:, :, :group] = (c + 1).reshape(n, k // group, group)
    d = d.reshape(n, k // group, gb, 5)[..., ::-1]
    vals = (d * np.array([1, 3, 9, 27, 81])).sum(-1)
    del flipped
    return vals.reshape(n, -1).astype(np.uint8)


def _pack_slot2_signed(codes, group=ref.GROUP):
    c = np.asarray(codes, dtype=np.int64) & 3     # two's complement slots
    n, k = c.shape
    d = c.reshape(n, k // 4, 4)
    return (d << np.array([0, 2, 4, 6])).sum(-1).astype(np.uint8)


def _pack_bit1_msb_first(codes, group=ref.GROUP):
    c = np.asarray(codes, dtype=np.int64)
    n, k = c.shape
    b = ((c + 1) // 2).reshape(n, k // 8, 8)
    return (b << np.arange(7, -1, -1)).sum(-1).astype(np.uint8)


def _unpack_bit1_inverted(packed, k):
    return (-_orig["unpack_bit1"](packed, k)).astype(np.int8)


def _quantize_with(scale_fn, round_fn=np.rint, clip=True, to_half=True):
    def q(w_rot, group=ref.GROUP):
        w = np.asarray(w_rot, dtype=np.float64)
        n, k = w.shape
        g = w.reshape(n, k // group, group)
        s = scale_fn(np.abs(g), w)
        if to_half:
            s = s.astype(np.float16)
        sd = np.asarray(s, dtype=np.float64)[:, :, None]
        with np.errstate(divide="ignore", invalid="ignore"):
            r = round_fn(g / sd)
        if clip:
            r = np.clip(r, -1, 1)
        r = np.where(sd != 0, r, 0)
        return r.reshape(n, k).astype(np.int8), np.asarray(s).astype(np.float16)
    return q


_mean_scale = lambda a, w: a.mean(axis=2)
_max_scale = lambda a, w: a.max(axis=2)
_row_scale = lambda a, w: np.repeat(np.abs(w).mean(axis=1)[:, None], a.shape[1], axis=1)
_half_away = lambda v: np.trunc(v + 0.5 * np.sign(v))


def _quantize_weights_unrotated(w, signs, block=ref.BLOCK, group=ref.GROUP):
    return ref.quantize_ternary(np.asarray(w, dtype=np.float64), group)


def _round_bf16_truncate(x):
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.trunc(m * 256.0), e - 8)


def _round_bf16_half_up(x):
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.floor(m * 256.0 + 0.5), e - 8)


def _round_bf16_7_bits(x):
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.rint(m * 128.0), e - 7)


def _fold_weights_unsigned(w, signs, block=ref.BLOCK):
    return _orig["rotate"](w, np.ones_like(np.asarray(signs)), block)


MUTATIONS = {
    "rotate: signs after H": ("rotate", _rotate_signs_last),
    "rotate: 1/n instead of 1/sqrt(n)": ("rotate", _rotate_wrong_norm),
    "rotate: block 0 signs reused": ("rotate", _rotate_one_sign_slice),
    "hadamard: bit-reversed rows": ("hadamard", _hadamard_bit_reversed),
    "dequant: group index k % G": ("dequant", _dequant_group_mod),
    "dequant: scale dropped": ("dequant", _dequant_drop_scale),
    "matvec: transposed weight": ("matvec", _matvec_transposed),
    "pack_trit5: most significant trit first": ("pack_trit5", _pack_trit5_big_endian),
    "pack_slot2: two's complement slots": ("pack_slot2", _pack_slot2_signed),
    "pack_bit1: most significant bit first": ("pack_bit1", _pack_bit1_msb_first),
    "unpack_bit1: bit 1 read as -1": ("unpack_bit1", _unpack_bit1_inverted),
    "quantize: absmax scale": ("quantize_ternary", _quantize_with(_max_scale)),
    "quantize: one scale per row": ("quantize_ternary", _quantize_with(_row_scale)),
    "quantize: no clipping": ("quantize_ternary", _quantize_with(_mean_scale, clip=False)),
    "quantize: ties away from zero": ("quantize_ternary",
                                      _quantize_with(_mean_scale, round_fn=_half_away)),
    "quantize: scale kept in fp64": ("quantize_ternary",
                                     _quantize_with(_mean_scale, to_half=False)),
    "quantize_weights: rotation skipped": ("quantize_weights", _quantize_weights_unrotated),
    "fold_weights: signs dropped": ("fold_weights", _fold_weights_unsigned),
    "round_bf16: truncation": ("round_bf16", _round_bf16_truncate),
    "round_bf16: ties upward": ("round_bf16", _round_bf16_half_up),
    "round_bf16: one significant bit short": ("round_bf16", _round_bf16_7_bits),
}

PIN_TESTS = [
    (pins.test_hadamard_matches_scipy_and_popcount, {"n": 8}),
    (pins.test_hadamard_matches_scipy_and_popcount, {"n": 1024}),
    (pins.test_rotate_matches_elementwise_definition_multi_block, {}),
    (pins.test_rotate_signs_applied_before_hadamard, {}),
    (pins.test_rotate_closed_forms, {"block": 8}),
    (pins.test_rotate_is_orthogonal, {}),
    (pins.test_trit5_hand_worked_examples, {}),
    (pins.test_slot2_hand_worked_examples, {}),
    (pins.test_trit5_exhaustive_full_bytes, {}),
    (pins.test_slot2_exhaustive, {}),
    (pins.test_bit1_hand_worked_examples, {}),
    (pins.test_bit1_exhaustive, {}),
    (pins.test_layer_bruteforce_several_blocks_and_groups, {}),
    (pins.test_dequant_group_index_along_k, {}),
    (pins.test_matvec_one_hot_closed_form, {}),
    (pins.test_matvec_orientation_nonsymmetric, {}),
    (pins.test_fold_invariant_and_negative, {}),
    (pins.test_quantize_hand_worked_groups, {}),
    (pins.test_quantize_scale_is_nearest_binary16_to_exact_mean_and_codes_nearest, {}),
    (pins.test_quantize_invariances, {}),
    (pins.test_quantize_weights_one_hot_closed_form, {}),
    (pins.test_round_bf16_hand_worked, {}),
    (pins.test_round_bf16_matches_bit_rounding_of_fp32, {}),
    (pins.test_round_bf16_fixed_points_and_bound, {}),
]


def _any_pin_fails():
    for fn, kwargs in PIN_TESTS:
        try:
            fn(**kwargs)
        except (AssertionError, ValueError):
            return fn.__name__
    return None


def test_pins_pass_unmutated():
    assert _any_pin_fails() is None


@pytest.mark.parametrize("label", sorted(MUTATIONS))
def test_planted_mistake_is_caught(label, monkeypatch):
    name, fake = MUTATIONS[label]
    monkeypatch.setattr(ref, name, fake)
    monkeypatch.setattr(oracle, name, fake)
    failing = _any_pin_fails()
    assert failing is not None, f"no pin catches the planted mistake: {label}"
