"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every function include/tl.h declares, and rejects bad arguments before any
launch.  Every call here fails validation, so nothing touches a device."""
import ctypes
import os
import re

import pytest

import tl_hadamard_rotate_amd as tl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tl.h")

A = 0x7F0000000000          # a 16-byte aligned fake device address (never dereferenced)
NULL = 0


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"TL_API\s+[\w\s\*]+?\b(tl_\w+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = _declared()
    for need in ("tl_pack", "tl_hadamard_rotate", "tl_gemv", "tl_gemm", "tl_linear", "tl_quantize"):
        assert need in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(tl.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_packed_bytes():
    L = tl.lib()
    assert L.tl_packed_bytes(1024, 1024, 0) == 212_992
    assert L.tl_packed_bytes(1024, 1024, 1) == 262_144
    assert L.tl_packed_bytes(17408, 5120, 0) == 17408 * 26 * 40
    assert L.tl_packed_bytes(5120, 17408, 1) == 5120 * 17408 // 4
    assert L.tl_packed_bytes(1, 128, 0) == 26
    assert L.tl_packed_bytes(0, 1024, 0) == -1
    assert L.tl_packed_bytes(4, 100, 0) == -1
    assert L.tl_packed_bytes(4, 1024, 2) == 512          # 1-bit codes: K/8 bytes a row
    assert L.tl_packed_bytes(17408, 5120, 2) == 17408 * 5120 // 8
    assert L.tl_packed_bytes(4, 1024, 3) == -1


def test_status_strings():
    L = tl.lib()
    for code, name in tl._STATUS.items():
        assert L.tl_status_str(code).decode() == name


def _gemv(fn, packed=A, scales=A + 0x1000000, fmt=0, x=A + 0x2000000, m=1, n=64, k=1024,
          y=A + 0x3000000, yd=0):
    return fn(packed, scales, fmt, x, m, n, k, y, yd, NULL)


@pytest.mark.parametrize("call", ["tl_gemv", "tl_gemm"])
def test_layer_validation(call):
    fn = getattr(tl.lib(), call)
    assert _gemv(fn, packed=NULL) == 1
    assert _gemv(fn, y=NULL) == 1
    assert _gemv(fn, k=1000) == 2
    assert _gemv(fn, k=512) == 2
    assert _gemv(fn, k=(1 << 20) + 1024) == 2
    assert _gemv(fn, m=0) == 2
    assert _gemv(fn, n=0) == 2
    assert _gemv(fn, m=1 << 25) == 2
    assert _gemv(fn, fmt=7) == 3
    assert _gemv(fn, yd=3) == 7
    assert _gemv(fn, x=A + 2) == 4
    assert _gemv(fn, y=A + 0x3000008) == 4
    # y overlapping x, the scales or the packed codes
    assert _gemv(fn, y=A + 0x2000000) == 5
    assert _gemv(fn, y=A + 0x1000000 - 16) == 5
    assert _gemv(fn, y=A + 16) == 5
    assert _gemv(fn, fmt=2, y=A + 64 * 1024 // 8 - 16) == 5   # 1-bit rows: K/8 bytes


def test_linear_validation():
    f = tl.lib().tl_linear
    P, S, X, G, XR, Y = A, A + 0x1000000, A + 0x2000000, A + 0x2800000, A + 0x3000000, A + 0x4000000

    def call(packed=P, scales=S, fmt=1, x=X, signs=G, m=1, n=1024, k=1024, x_rot=XR, y=Y, yd=0):
        return f(packed, scales, fmt, x, signs, m, n, k, x_rot, y, yd, NULL)

    assert call(signs=NULL) == 1
    assert call(x_rot=NULL) == 1
    assert call(x=NULL) == 1
    assert call(k=1000) == 2
    assert call(fmt=4) == 3
    assert call(signs=G + 4) == 4
    assert call(x_rot=XR + 2) == 4
    assert call(x_rot=X) == 5            # x_rot on top of x
    assert call(x_rot=G - 16) == 5       # over the signs
    assert call(x_rot=Y - 16) == 5       # into y
    assert call(y=G) == 5                # y over the signs
    assert call(yd=2) == 7


def test_rotate_validation():
    f = tl.lib().tl_hadamard_rotate
    assert f(NULL, A, 1, 1024, A + 0x100000, NULL) == 1
    assert f(A, A + 0x100000, 1, 1000, A + 0x200000, NULL) == 2
    assert f(A, A + 0x100000, 0, 1024, A + 0x200000, NULL) == 2
    assert f(A + 8, A + 0x100000, 1, 1024, A + 0x200000, NULL) == 4
    assert f(A, A + 0x100000, 2, 1024, A + 16, NULL) == 5          # partial overlap
    assert f(A, A + 0x100000, 1, 1024, A + 0x100000 - 16, NULL) == 5  # over the signs


def test_pack_validation():
    f = tl.lib().tl_pack
    assert f(NULL, 4, 1024, 0, A, NULL, NULL) == 1
    assert f(A, 4, 100, 0, A + 0x100000, NULL, NULL) == 2
    assert f(A, 0, 128, 0, A + 0x100000, NULL, NULL) == 2
    assert f(A, 4, 128, 5, A + 0x100000, NULL, NULL) == 3
    assert f(A, 4, 128, 0, A + 0x100001, NULL, NULL) == 4
    assert f(A, 4, 128, 0, A + 0x100000, A + 0x200002, NULL) == 4
    assert f(A, 4, 128, 0, A + 256, NULL, NULL) == 5
    assert f(A, 4, 128, 0, A + 0x100000, A + 0x100000, NULL) == 5
    g = tl.lib().tl_unpack
    assert g(A, 4, 128, 1, NULL, NULL) == 1
    assert g(A, 4, 128, 1, A + 16, NULL) == 5


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        tl.hadamard_rotate(torch.zeros((1, 1024), dtype=torch.float16),
                           torch.ones(1024, dtype=torch.int8))


def test_quantize_validation():
    f = tl.lib().tl_quantize
    W, G, C, S = A, A + 0x1000000, A + 0x2000000, A + 0x3000000

    def call(w=W, signs=G, n=4, k=1024, codes=C, scales=S):
        return f(w, signs, n, k, codes, scales, NULL)

    assert call(w=NULL) == 1
    assert call(scales=NULL) == 1
    assert call(k=1000) == 2
    assert call(k=512) == 2
    assert call(n=0) == 2
    assert call(w=W + 4) == 4
    assert call(codes=C + 8) == 4
    assert call(codes=W + 16) == 5                 # codes over the weights (16 KB)
    assert call(codes=G - 16) == 5                 # over the signs
    assert call(scales=C + 4096 - 16) == 5         # scales over the codes (4 KB)
    assert call(scales=W) == 5


def test_gemm_bf16_validation():
    fn = tl.lib().tl_gemm_bf16
    assert _gemv(fn, packed=NULL) == 1
    assert _gemv(fn, k=1000) == 2
    assert _gemv(fn, fmt=7) == 3
    assert _gemv(fn, x=A + 2) == 4
    assert _gemv(fn, y=A + 0x2000000) == 5
    assert _gemv(fn, yd=3) == 7


def test_stream_read_validation():
    f = tl.lib().tl_stream_read
    assert f(NULL, 1024, A, 4, NULL) == 1
    assert f(A, 1000, A + 0x100000, 4, NULL) == 2
    assert f(A, 1024, A + 0x100000, 0, NULL) == 2
    assert f(A + 8, 1024, A + 0x100000, 4, NULL) == 4
    assert f(A, 1024, A + 16, 4, NULL) == 5
