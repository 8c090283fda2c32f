"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every function include/tl.h declares, and rejects bad arguments before any
launch.  Every call here fails validation, so nothing touches a device."""
import ctypes
import os
import re
import struct

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
    for need in ("tl_pack", "tl_hadamard_rotate", "tl_gemv", "tl_gemm", "tl_linear", "tl_quantize",
                 "tl_gemm_workspace_bytes", "tl_gemm_bf16_workspace_bytes", "tl_gemm_plan"):
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


WS = A + 0x10000000        # a fake workspace far from every other buffer


def _gemv(fn, packed=A, scales=A + 0x1000000, fmt=0, x=A + 0x2000000, m=1, n=64, k=1024,
          y=A + 0x3000000, yd=0, ws=WS, ws_bytes=1 << 30):
    if fn.__name__ == "tl_gemv":
        return fn(packed, scales, fmt, x, m, n, k, y, yd, NULL)
    return fn(packed, scales, fmt, x, m, n, k, y, yd, ws, ws_bytes, NULL)


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

    def call(packed=P, scales=S, fmt=1, x=X, signs=G, m=1, n=1024, k=1024, x_rot=XR, y=Y, yd=0,
             ws=NULL, ws_bytes=0):
        return f(packed, scales, fmt, x, signs, m, n, k, x_rot, y, yd, ws, ws_bytes, NULL)

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
    # prefill (M >= 64) with dense trits needs the workspace of tl_gemm
    need = tl.lib().tl_gemm_workspace_bytes(64, 1024, 1024, 0)
    assert need >= 1024 * 1024 // 4
    assert call(fmt=0, m=64, n=1024) == 8
    assert call(fmt=0, m=64, n=1024, ws=WS, ws_bytes=need - 1) == 8
    assert call(fmt=0, m=64, n=1024, ws=WS + 8, ws_bytes=need) == 4
    assert call(fmt=0, m=64, n=1024, ws=XR, ws_bytes=need) == 5


def test_gemm_workspace_and_plan():
    L = tl.lib()
    # dense trits and 1-bit codes: the 2-bit-slot rewrite of the weights comes
    # first; the fp32 partial sums of K-split tiles (256 x 256 floats each)
    # after it, on a 256-byte boundary
    for m, n, k in [(64, 1024, 1024), (512, 17408, 5120), (512, 5120, 17408), (4096, 5120, 17408)]:
        out = (ctypes.c_int64 * 3)()
        assert L.tl_gemm_plan(m, n, k, out) == 0
        tiles, whole, splits = out[0], out[1], out[2]
        assert tiles == -(-m // 256) * -(-n // 256)
        assert 0 <= whole <= tiles and 1 <= splits <= 16
        assert (splits == 1) == (whole == tiles)
        partial = (tiles - whole) * splits * 256 * 256 * 4 if splits > 1 else 0
        assert partial <= 64 << 20
        assert L.tl_gemm_workspace_bytes(m, n, k, 1) == partial
        rewrite = -(-(n * k // 4) // 256) * 256
        assert L.tl_gemm_workspace_bytes(m, n, k, 0) == rewrite + partial
        assert L.tl_gemm_workspace_bytes(m, n, k, 2) == rewrite + partial
        # bfloat16 activations: their binary16 copy and the row factors
        # between the rewrite and the partial sums
        copy = -(-(m * k * 2) // 256) * 256 + -(-(m * 4) // 256) * 256
        assert L.tl_gemm_bf16_workspace_bytes(m, n, k, 1) == copy + partial
        assert L.tl_gemm_bf16_workspace_bytes(m, n, k, 0) == rewrite + copy + partial
    assert L.tl_gemm_workspace_bytes(64, 1024, 1000, 1) == -1
    assert L.tl_gemm_workspace_bytes(64, 1024, 1024, 9) == -1
    assert L.tl_gemm_bf16_workspace_bytes(64, 1024, 1000, 1) == -1
    assert L.tl_gemm_bf16_workspace_bytes(64, 1024, 1024, 9) == -1
    assert L.tl_gemm_plan(64, 1024, 1024, NULL) == 1
    out = (ctypes.c_int64 * 3)()
    assert L.tl_gemm_plan(0, 1024, 1024, out) == 2
    assert L.tl_gemm_plan(1 << 20, 1024, 4096, out) == 2      # M * K reaches 2^31


@pytest.mark.parametrize("call", ["tl_gemm", "tl_gemm_bf16"])
def test_gemm_workspace_validation(call):
    fn = getattr(tl.lib(), call)
    size = tl.lib().tl_gemm_bf16_workspace_bytes if call == "tl_gemm_bf16" else \
        tl.lib().tl_gemm_workspace_bytes
    need = size(64, 1024, 1024, 0)
    assert need >= 1024 * 1024 // 4
    assert _gemv(fn, m=64, n=1024, ws=NULL, ws_bytes=0) == 8            # missing
    assert _gemv(fn, m=64, n=1024, ws_bytes=need - 1) == 8               # too small
    assert _gemv(fn, m=64, n=1024, ws=WS + 4, ws_bytes=need) == 4        # misaligned
    assert _gemv(fn, m=64, n=1024, ws=A + 0x2000000, ws_bytes=need) == 5  # over x
    assert _gemv(fn, m=64, n=1024, ws=A + 0x3000000 - 16, ws_bytes=need) == 5   # into y


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


def test_gemm_noalloc_validation():
    """tl_gemm_noalloc: tl_gemm's argument checks, and shapes whose workspace
    exceeds its fixed scratch array are refused before any launch."""
    f = tl.lib().tl_gemm_noalloc
    P, S, X, Y = A, A + (1 << 32), A + (2 << 32), A + (3 << 32)

    def call(packed=P, scales=S, fmt=0, x=X, m=64, n=1024, k=1024, y=Y, yd=0):
        return f(packed, scales, fmt, x, m, n, k, y, yd, NULL)

    assert call(packed=NULL) == 1
    assert call(k=1000) == 2
    assert call(fmt=5) == 3
    assert call(x=X + 2) == 4
    assert call(y=X) == 5
    assert call(yd=4) == 7
    limit = 96 << 20
    n, k = 65536, 8192                  # 2-bit-slot rewrite of 128 MiB
    assert tl.lib().tl_gemm_workspace_bytes(64, n, k, 0) > limit
    assert call(fmt=0, n=n, k=k) == 8
    assert call(fmt=2, n=n, k=k) == 8


def test_layer_library_exports_no_probe():
    """The benchmark's read-only probe lives in its own library."""
    lib = ctypes.CDLL(tl.LIB_PATH)
    assert not hasattr(lib, "tl_stream_read")


def test_probe_library_validation():
    f = ctypes.CDLL(os.path.join(os.path.dirname(tl.LIB_PATH), "libtl_probe.so")).tlprobe_stream_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    assert f(NULL, 1024, A, 4, NULL) == 1
    assert f(A, 1000, A + 0x100000, 4, NULL) == 1
    assert f(A, 1024, A + 0x100000, 0, NULL) == 1
    assert f(A + 8, 1024, A + 0x100000, 4, NULL) == 1
    assert f(A, 1024, A + 16, 4, NULL) == 1


def _chain_encode(ops):
    L = tl.lib()
    arr = (tl.ChainOp * len(ops))(*ops)
    nbytes = L.tl_chain_plan_bytes(len(ops))
    host = (ctypes.c_uint8 * max(nbytes, 1))()
    return L.tl_chain_encode(arr, len(ops), host, nbytes), bytes(host)


def _op(base, n=1024, k=1024, y=None, x=None, yd=1, fmt=1, x_rot=0):
    """A chain linear on fake, far-apart addresses below `base`."""
    return tl.ChainOp(base, base + (1 << 28), x if x is not None else base + (2 << 28),
                      base + (3 << 28), x_rot, y if y is not None else base + (4 << 28), n, k, fmt, yd)


def test_chain_sizes():
    L = tl.lib()
    assert L.tl_chain_plan_bytes(1) == 128 and L.tl_chain_plan_bytes(448) == 64 * 449
    assert L.tl_chain_sync_bytes(1) == 16 and L.tl_chain_sync_bytes(448) == 1808   # 4 * 450, to 16
    for bad in (0, -1, 65537):
        assert L.tl_chain_plan_bytes(bad) == -1 and L.tl_chain_sync_bytes(bad) == -1


def test_chain_encode_validation():
    B0, B1, B2 = A, A + (8 << 28), A + (16 << 28)
    # a valid two-linear chain whose second input is the first output
    y0 = B0 + (4 << 28)
    st, plan = _chain_encode([_op(B0, n=1024, k=1024), _op(B1, n=512, k=1024, x=y0)])
    assert st == 0
    magic, count, grid, polls = struct.unpack_from("<IiiI", plan, 0)
    assert count == 2 and grid > 0 and polls > 0
    # per linear: 6 pointers, n, k, the producer of its input, binary16 output
    n1, k1, dep1, f16 = struct.unpack_from("<iiii", plan, 64 + 64 + 48)
    assert (n1, k1, dep1, f16) == (512, 1024, 0, 1)
    assert struct.unpack_from("<i", plan, 64 + 48 + 8)[0] == -1
    # x within a larger binary16 y (q inside q|k|v): a dependency too
    st, plan = _chain_encode([_op(B0, n=8192, k=5120), _op(B1, n=5120, k=6144, x=y0 + 2048)])
    assert st == 0 and struct.unpack_from("<i", plan, 64 + 64 + 56)[0] == 0
    # NULL, format, dtype, shape, alignment
    assert _chain_encode([_op(B0, y=0)])[0] == 1
    assert _chain_encode([_op(B0, fmt=0)])[0] == 3
    assert _chain_encode([_op(B0, yd=5)])[0] == 7
    assert _chain_encode([_op(B0, k=1000)])[0] == 2
    assert _chain_encode([_op(B0, k=33 * 1024)])[0] == 2
    assert _chain_encode([_op(B0, n=1 << 25)])[0] == 2
    assert _chain_encode([_op(B0, n=17408 * 8, k=17408)])[0] == 2   # one chunk per workgroup
    assert _chain_encode([_op(B0, x_rot=B2 + 8)])[0] == 4
    # a float32 y cannot feed a later linear; an input may not straddle a y;
    # a later output may not overwrite an earlier input; outputs may not overlap
    assert _chain_encode([_op(B0, yd=0), _op(B1, x=y0)])[0] == 5
    assert _chain_encode([_op(B0, n=1024), _op(B1, k=1024, x=y0 + 1024)])[0] == 5
    assert _chain_encode([_op(B0), _op(B1, y=B0 + (2 << 28))])[0] == 5
    assert _chain_encode([_op(B0), _op(B1, y=y0 + 16)])[0] == 5
    assert _chain_encode([_op(B0, x_rot=y0)])[0] == 5
    # a linear cannot read its own output
    assert _chain_encode([_op(B0, x=y0)])[0] == 5


def test_chain_launch_validation():
    f = tl.lib().tl_linear_chain
    assert f(NULL, 1, A, NULL) == 1
    assert f(A, 1, NULL, NULL) == 1
    assert f(A, 0, A + 0x100000, NULL) == 2
    assert f(A + 8, 1, A + 0x100000, NULL) == 4
    assert f(A, 1, A + 64, NULL) == 5          # sync inside the plan
