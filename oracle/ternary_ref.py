"""Plain, slow fp64 CPU oracle for the ternary g128 linear layer with a signed
block-Hadamard rotation of the activations.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library; NumPy is its only dependency.

What it computes (every step is the plain definition, no fast algorithm):

* Weights are codes c in {-1, 0, +1} with one binary16 scale per 128
  consecutive weights of a row ("ternary g128").
  Sources: page "A 27-billion model that fits in 8.6 GB" (news.ditty.ir,
  Persian), paragraph 2; page "Ternary Bonsai 2 27B: 27B-модель в 5,9 ГБ"
  (ai4coding.ru), section "Что такое тернарная модель".
* Before quantisation every weight matrix went through an orthogonal block
  Hadamard transform on 1024-wide blocks, folded into the weights; at run
  time the activations must get the matching transform.  Sources: the same
  Persian page, paragraphs 2 and 3; page "OpenBonsai" (openbonsai.org),
  section "How it works", step 1 (the rotation is signed).
* Two byte packings of the same codes: a dense one with 5 trits per byte and
  one with a 2-bit slot per value.  Source: the Persian page, paragraph 5.
* A binary variant: every weight is -1 or +1 with one scale per 128 weights,
  about 1.125 bits per weight.  Source: page "How Prism ML Squeezed a 27B
  Model Into 3.9 GB" (dev.to), list "Two formats ship today".

Readings taken where the pages are silent:

* R(x)[1024 b + i] = (1/32) * sum_j H[i, j] * s[1024 b + j] * x[1024 b + j],
  H the Sylvester (natural order) Hadamard matrix, signs applied first.  The
  same map rotates a weight row, and then  R(w) . R(x) = w . x.
* digit d = c + 1.  TRIT5: per 128-group 26 bytes; byte j < 25 holds digits
  5j..5j+4 little-endian in base 3; byte 25 holds digits 125..127 plus two
  pad digits equal to 1 (code 0).  SLOT2: byte j holds digits 4j..4j+3,
  two bits each, least significant first.  BIT1 (codes -1 and +1 only):
  byte j holds bits b[8j..8j+7], least significant first, code = 2b - 1.
* Scales: binary16 array [N, K/128]; a weight is c * S.
* Weight-side quantisation (the pages' pipeline rotates, then rounds to
  -1/0/+1 with one scale per 128 by GPTQ on calibration data; without data
  the plain stand-in is round to nearest with an absmean scale):
  S = binary16(mean |w'| over the group), c = clip(rint(w' / S), -1, 1)
  (ties to even, so |w'| = S/2 gives 0), c = 0 where S = 0.

Every function here is pinned to something other than itself: hand-worked
values, closed forms, brute force on tiny cases and invariants in
tests/test_oracle_pins.py, and planted mistakes those pins must catch in
tests/test_oracle_mutations.py.  Parity unpinned: byte compatibility of the
packings with the published model files, whose layouts the pages do not give
(the formats above are this library's own and are pinned to their own
definition).
"""
from __future__ import annotations

import numpy as np

BLOCK = 1024          # Hadamard block width (Persian page, paragraph 2)
GROUP = 128           # weights per FP16 scale (Persian page, paragraph 2)

FMT_TRIT5 = 0
FMT_SLOT2 = 1
FMT_BIT1 = 2

TRIT5_GROUP_BYTES = 26   # 25 bytes of 5 trits + 1 byte of 3 trits and 2 pads
_POW3 = (1, 3, 9, 27, 81)


# ---------------------------------------------------------------------------
# Hadamard matrix and the activation rotation
# ---------------------------------------------------------------------------

def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), fp64, natural
    order: H_1 = [1],  H_2m = [[H_m, H_m], [H_m, -H_m]]."""
    if n < 1 or n & (n - 1):
        raise ValueError(f"Hadamard order must be a power of two, got {n}")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate(x: np.ndarray, signs: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Signed block-Hadamard rotation of the rows of x, in fp64.

    x: [M, K] (any float dtype, read as fp64); signs: [K] of +-1.
    For every row and every block b of ``block`` consecutive columns:
    out_b = H @ (s_b * x_b) / sqrt(block), H from ``hadamard``.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[None, :]
    m, k = x.shape
    s = np.asarray(signs, dtype=np.float64).reshape(-1)
    if k % block or s.shape[0] != k:
        raise ValueError("K must be a multiple of the block and match signs")
    h = hadamard(block)
    out = np.empty_like(x)
    for b in range(k // block):
        cols = slice(b * block, (b + 1) * block)
        v = x[:, cols] * s[cols][None, :]           # signs first
        out[:, cols] = (v @ h.T) / np.sqrt(block)    # then H, then 1/sqrt(n)
    return out


def rotate_transpose(y: np.ndarray, signs: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Transpose of ``rotate``: out_b = s_b * (H @ y_b) / sqrt(block).
    Since the rotation is orthogonal this is its inverse."""
    y = np.asarray(y, dtype=np.float64)
    if y.ndim == 1:
        y = y[None, :]
    s = np.asarray(signs, dtype=np.float64).reshape(-1)
    h = hadamard(block)
    out = np.empty_like(y)
    for b in range(y.shape[1] // block):
        cols = slice(b * block, (b + 1) * block)
        out[:, cols] = ((y[:, cols] @ h.T) / np.sqrt(block)) * s[cols][None, :]
    return out


# ---------------------------------------------------------------------------
# Packings
# ---------------------------------------------------------------------------

def _check_codes(codes: np.ndarray, group: int) -> np.ndarray:
    c = np.asarray(codes)
    if c.ndim != 2:
        raise ValueError("codes must be [N, K]")
    if c.shape[1] % group:
        raise ValueError("K must be a multiple of the group size")
    if not np.isin(c, (-1, 0, 1)).all():
        raise ValueError("codes must lie in {-1, 0, 1}")
    return c.astype(np.int64)


def packed_bytes(n: int, k: int, fmt: int, group: int = GROUP) -> int:
    """Bytes of the packed code array (scales not included)."""
    if fmt == FMT_TRIT5:
        return n * (k // group) * trit5_group_bytes(group)
    if fmt == FMT_SLOT2:
        return n * k // 4
    if fmt == FMT_BIT1:
        return n * k // 8
    raise ValueError("unknown format")


def trit5_group_bytes(group: int = GROUP) -> int:
    """ceil(group / 5) bytes: full bytes of 5 trits, then one partial byte."""
    return -(-group // 5)


def pack_trit5(codes: np.ndarray, group: int = GROUP) -> np.ndarray:
    """codes [N, K] in {-1,0,1} -> uint8 [N, (K/group) * ceil(group/5)].

    Within a group, byte j is sum_i d[5j+i] * 3**i (d = c + 1) over the
    digits that exist; missing digits of the last byte are pads equal to 1."""
    c = _check_codes(codes, group)
    n, k = c.shape
    gb = trit5_group_bytes(group)
    d = (c + 1).reshape(n, k // group, group)
    padded = np.ones((n, k // group, gb * 5), dtype=np.int64)
    padded[:, :, :group] = d
    digits = padded.reshape(n, k // group, gb, 5)
    vals = (digits * np.array(_POW3, dtype=np.int64)).sum(axis=-1)
    return vals.reshape(n, (k // group) * gb).astype(np.uint8)


def unpack_trit5(packed: np.ndarray, k: int, group: int = GROUP) -> np.ndarray:
    """Inverse of ``pack_trit5``; raises on any byte that is not a valid
    encoding (value >= 243, or pad digits different from 1)."""
    p = np.asarray(packed, dtype=np.int64)
    n = p.shape[0]
    gb = trit5_group_bytes(group)
    if p.shape[1] != (k // group) * gb:
        raise ValueError("packed width does not match K")
    if (p >= 243).any():
        raise ValueError("TRIT5 byte >= 243")
    v = p.reshape(n, k // group, gb)
    digits = np.empty((n, k // group, gb, 5), dtype=np.int64)
    rest = v.copy()
    for i in range(5):
        digits[..., i] = rest % 3
        rest //= 3
    flat = digits.reshape(n, k // group, gb * 5)
    if (flat[:, :, group:] != 1).any():
        raise ValueError("TRIT5 pad digit is not 1")
    return (flat[:, :, :group] - 1).reshape(n, k).astype(np.int8)


def pack_slot2(codes: np.ndarray, group: int = GROUP) -> np.ndarray:
    """codes [N, K] -> uint8 [N, K/4]; byte j bits 2i..2i+1 = d[4j+i]."""
    c = _check_codes(codes, group)
    n, k = c.shape
    d = (c + 1).reshape(n, k // 4, 4)
    vals = (d << np.array([0, 2, 4, 6], dtype=np.int64)).sum(axis=-1)
    return vals.astype(np.uint8)


def unpack_slot2(packed: np.ndarray, k: int) -> np.ndarray:
    """Inverse of ``pack_slot2``; raises on a slot holding 3."""
    p = np.asarray(packed, dtype=np.int64)
    if p.shape[1] * 4 != k:
        raise ValueError("packed width does not match K")
    d = (p[:, :, None] >> np.array([0, 2, 4, 6], dtype=np.int64)) & 3
    if (d == 3).any():
        raise ValueError("SLOT2 slot value 3")
    return (d.reshape(p.shape[0], k) - 1).astype(np.int8)


def pack_bit1(codes: np.ndarray, group: int = GROUP) -> np.ndarray:
    """codes [N, K] in {-1, +1} -> uint8 [N, K/8]; byte j bit i = b[8j+i],
    b = (c + 1) / 2."""
    c = _check_codes(codes, group)
    if (c == 0).any():
        raise ValueError("BIT1 codes must be -1 or +1")
    n, k = c.shape
    b = ((c + 1) // 2).reshape(n, k // 8, 8)
    vals = (b << np.arange(8, dtype=np.int64)).sum(axis=-1)
    return vals.astype(np.uint8)


def unpack_bit1(packed: np.ndarray, k: int) -> np.ndarray:
    """Inverse of ``pack_bit1``: every byte is valid."""
    p = np.asarray(packed, dtype=np.int64)
    if p.shape[1] * 8 != k:
        raise ValueError("packed width does not match K")
    b = (p[:, :, None] >> np.arange(8, dtype=np.int64)) & 1
    return (2 * b.reshape(p.shape[0], k) - 1).astype(np.int8)


def pack(codes: np.ndarray, fmt: int, group: int = GROUP) -> np.ndarray:
    if fmt == FMT_TRIT5:
        return pack_trit5(codes, group)
    if fmt == FMT_SLOT2:
        return pack_slot2(codes, group)
    if fmt == FMT_BIT1:
        return pack_bit1(codes, group)
    raise ValueError("unknown format")


def unpack(packed: np.ndarray, k: int, fmt: int, group: int = GROUP) -> np.ndarray:
    if fmt == FMT_TRIT5:
        return unpack_trit5(packed, k, group)
    if fmt == FMT_SLOT2:
        return unpack_slot2(packed, k)
    if fmt == FMT_BIT1:
        return unpack_bit1(packed, k)
    raise ValueError("unknown format")


def pack_trit5_loop(codes, group: int = GROUP) -> bytes:
    """Byte-by-byte pure-Python TRIT5 packer for tiny inputs."""
    out = bytearray()
    for row in codes:
        row = [int(v) for v in row]
        for g0 in range(0, len(row), group):
            grp = row[g0:g0 + group]
            for j in range(0, group, 5):
                val, w = 0, 1
                for i in range(5):
                    digit = grp[j + i] + 1 if j + i < group else 1
                    val += digit * w
                    w *= 3
                out.append(val)
    return bytes(out)


def pack_slot2_loop(codes) -> bytes:
    """Byte-by-byte pure-Python SLOT2 packer for tiny inputs."""
    out = bytearray()
    for row in codes:
        row = [int(v) for v in row]
        for j in range(0, len(row), 4):
            val = 0
            for i in range(4):
                val |= (row[j + i] + 1) << (2 * i)
            out.append(val)
    return bytes(out)


def pack_bit1_loop(codes) -> bytes:
    """Byte-by-byte pure-Python BIT1 packer for tiny inputs."""
    out = bytearray()
    for row in codes:
        row = [int(v) for v in row]
        for j in range(0, len(row), 8):
            val = 0
            for i in range(8):
                if row[j + i] == 1:
                    val |= 1 << i
                elif row[j + i] != -1:
                    raise ValueError("BIT1 codes must be -1 or +1")
            out.append(val)
    return bytes(out)


# ---------------------------------------------------------------------------
# Dequantisation and the linear layer
# ---------------------------------------------------------------------------

def dequant(codes: np.ndarray, scales: np.ndarray, group: int = GROUP) -> np.ndarray:
    """W[n, k] = c[n, k] * S[n, k // group], in fp64."""
    c = np.asarray(codes, dtype=np.float64)
    s = np.asarray(scales, dtype=np.float64)
    n, k = c.shape
    if s.shape != (n, k // group):
        raise ValueError("scales must be [N, K/group]")
    return c * np.repeat(s, group, axis=1)


def matvec(codes: np.ndarray, scales: np.ndarray, x_rot: np.ndarray,
           group: int = GROUP) -> np.ndarray:
    """y[m, n] = sum_k x_rot[m, k] * c[n, k] * S[n, k // group]  (fp64).

    This is what tl_gemv / tl_gemm compute from an already rotated input."""
    xr = np.asarray(x_rot, dtype=np.float64)
    if xr.ndim == 1:
        xr = xr[None, :]
    return xr @ dequant(codes, scales, group).T


def matvec_packed(packed: np.ndarray, scales: np.ndarray, fmt: int,
                  x_rot: np.ndarray, k: int, group: int = GROUP) -> np.ndarray:
    """``matvec`` from packed bytes: unpack, dequantise, fp64 matmul."""
    return matvec(unpack(packed, k, fmt, group), scales, x_rot, group)


def linear(x: np.ndarray, signs: np.ndarray, codes: np.ndarray, scales: np.ndarray,
           block: int = BLOCK, group: int = GROUP) -> np.ndarray:
    """The whole layer: y = R(x) . dequant(c, S)^T, fp64 end to end (the
    rotated activations are not rounded)."""
    return matvec(codes, scales, rotate(x, signs, block), group)


def fold_weights(w: np.ndarray, signs: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Fold the rotation into real-valued weight rows: every row gets the same
    map as the activations, so fold(w) . R(x) = w . x."""
    return rotate(w, signs, block)


# ---------------------------------------------------------------------------
# Weight-side quantisation: fold the rotation into the rows, round to ternary
# ---------------------------------------------------------------------------

def quantize_ternary(w_rot: np.ndarray, group: int = GROUP):
    """Round already rotated weight rows to ternary g128.

    Page "OpenBonsai", section "How it works", step 2: every large linear is
    rounded to -1, 0 or +1 with one scale per 128 weights (there by GPTQ on
    calibration data; here by rounding to nearest, the data-free reading).
    Page "A 27-billion model that fits in 8.6 GB", paragraph 2: the scale is
    an FP16 number shared by the 128 weights.

    Per group: S = mean of |w| in fp64, rounded to binary16 (nearest even);
    c = rint(w / S) (half to even) clipped to [-1, 1], and c = 0 where S is 0.
    Returns (codes int8 [N, K], scales float16 [N, K/group])."""
    w = np.asarray(w_rot, dtype=np.float64)
    n, k = w.shape
    if k % group:
        raise ValueError("K must be a multiple of the group")
    g = w.reshape(n, k // group, group)
    scales = np.abs(g).mean(axis=2).astype(np.float16)
    s = scales.astype(np.float64)[:, :, None]
    codes = np.zeros_like(g)
    nz = np.broadcast_to(s != 0.0, g.shape)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = np.clip(np.rint(g / s), -1.0, 1.0)
    codes[nz] = q[nz]
    return codes.reshape(n, k).astype(np.int8), scales


def quantize_weights(w: np.ndarray, signs: np.ndarray, block: int = BLOCK,
                     group: int = GROUP):
    """The weight side of the layer: rotate the real-valued rows with the
    activations' signed transform (page "OpenBonsai", section "How it works",
    step 1; Persian page, paragraph 2: the rotation is folded into the
    weights), then round them to ternary g128 (``quantize_ternary``)."""
    return quantize_ternary(fold_weights(w, signs, block), group)


# ---------------------------------------------------------------------------
# bfloat16 activations (the bf16 variant of the product)
# ---------------------------------------------------------------------------

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 number (8 significant bits, ties to the
    even significand), returned as fp64 values.  For the variant of the
    product whose activations are bfloat16; normal range only
    (|x| >= 2**-126), which activations never leave."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))   # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


# ---------------------------------------------------------------------------
# Error metrics
# ---------------------------------------------------------------------------

def rel_l2(y: np.ndarray, y_ref: np.ndarray) -> float:
    """||y - y_ref||_2 / ||y_ref||_2 over the whole array (0 if both are 0)."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(r)
    num = np.linalg.norm(y - r)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def fp16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of binary16 numbers at |v| (subnormal spacing below 2**-14)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)
