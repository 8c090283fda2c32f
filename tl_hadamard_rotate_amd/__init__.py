"""Python binding of libtl (ternary g128 linear layer with a signed
block-Hadamard rotation, MI355X / gfx950).

Argument marshalling only: every function checks dtype, shape, device and
contiguity of torch tensors, then passes raw device pointers and torch's
current HIP stream to the C ABI declared in include/tl.h.  All computation runs
in the library's HIP kernels; there is no fallback path.  A missing library
raises at first use.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtl.so")

FMT_TRIT5 = 0
FMT_SLOT2 = 1
FMT_BIT1 = 2
TL_F32 = 0
TL_F16 = 1
BLOCK = 1024
GROUP = 128

_STATUS = {0: "TL_OK", 1: "TL_ERR_NULL", 2: "TL_ERR_SHAPE", 3: "TL_ERR_FORMAT",
           4: "TL_ERR_ALIGN", 5: "TL_ERR_ALIAS", 6: "TL_ERR_LAUNCH", 7: "TL_ERR_DTYPE",
           8: "TL_ERR_WORKSPACE", 9: "TL_ERR_DATA"}

_lib = None


class TLError(RuntimeError):
    def __init__(self, call: str, status: int, detail: str = ""):
        self.status = status
        self.status_name = _STATUS.get(status, f"status {status}")
        msg = f"{call} failed: {self.status_name}"
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)


def lib() -> ctypes.CDLL:
    """Load libtl.so (built by ``python -m tl_hadamard_rotate_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m tl_hadamard_rotate_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        sig = {
            "tl_packed_bytes": (i64, [i64, i64, i32]),
            "tl_pack": (i32, [p, i64, i64, i32, p, p, p]),
            "tl_unpack": (i32, [p, i64, i64, i32, p, p]),
            "tl_hadamard_rotate": (i32, [p, p, i64, i64, p, p]),
            "tl_gemv": (i32, [p, p, i32, p, i64, i64, i64, p, i32, p]),
            "tl_gemm": (i32, [p, p, i32, p, i64, i64, i64, p, i32, p, i64, p]),
            "tl_gemm_noalloc": (i32, [p, p, i32, p, i64, i64, i64, p, i32, p]),
            "tl_gemm_workspace_bytes": (i64, [i64, i64, i64, i32]),
            "tl_gemm_bf16_workspace_bytes": (i64, [i64, i64, i64, i32]),
            "tl_gemm_plan": (i32, [i64, i64, i64, p]),
            "tl_linear": (i32, [p, p, i32, p, p, i64, i64, i64, p, p, i32, p, i64, p]),
            "tl_quantize": (i32, [p, p, i64, i64, p, p, p]),
            "tl_gemm_bf16": (i32, [p, p, i32, p, i64, i64, i64, p, i32, p, i64, p]),
            "tl_chain_plan_bytes": (i64, [i32]),
            "tl_chain_sync_bytes": (i64, [i32]),
            "tl_chain_encode": (i32, [p, i32, p, i64]),
            "tl_linear_chain": (i32, [p, i32, p, p]),
            "tl_status_str": (ctypes.c_char_p, [i32]),
            "tl_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(call: str, status: int) -> None:
    if status != 0:
        detail = lib().tl_last_error().decode() if status in (6, 9) else ""
        raise TLError(call, status, detail)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int | None = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def packed_bytes(n: int, k: int, fmt: int) -> int:
    return int(lib().tl_packed_bytes(n, k, fmt))


def pack(codes: torch.Tensor, fmt: int, bad_count: torch.Tensor | None = None) -> torch.Tensor:
    """int8 codes [N, K] -> uint8 packed [N, row_bytes] (see include/tl.h)."""
    _need(codes, "codes", torch.int8, 2)
    if bad_count is not None:
        _need(bad_count, "bad_count", torch.int32)
    n, k = codes.shape
    nbytes = packed_bytes(n, k, fmt)
    if nbytes < 0:
        raise TLError("tl_pack", 2)
    out = torch.empty((n, nbytes // n), dtype=torch.uint8, device=codes.device)
    _check("tl_pack", lib().tl_pack(_ptr(codes), n, k, fmt, _ptr(out), _ptr(bad_count),
                                    _stream(codes)))
    return out


def unpack(packed: torch.Tensor, k: int, fmt: int) -> torch.Tensor:
    _need(packed, "packed", torch.uint8, 2)
    n = packed.shape[0]
    out = torch.empty((n, k), dtype=torch.int8, device=packed.device)
    if packed.numel() != packed_bytes(n, k, fmt):
        raise ValueError("packed size does not match K and the format")
    _check("tl_unpack", lib().tl_unpack(_ptr(packed), n, k, fmt, _ptr(out), _stream(packed)))
    return out


def hadamard_rotate(x: torch.Tensor, signs: torch.Tensor,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """Signed 1024-block Hadamard rotation of the rows of fp16 x [M, K]."""
    _need(x, "x", torch.float16, 2)
    _need(signs, "signs", torch.int8, 1)
    m, k = x.shape
    if signs.shape[0] != k:
        raise ValueError("signs must have K entries")
    if out is None:
        out = torch.empty_like(x)
    else:
        _need(out, "out", torch.float16, 2)
        if out.shape != x.shape:
            raise ValueError("out must have the shape of x")
    _check("tl_hadamard_rotate",
           lib().tl_hadamard_rotate(_ptr(x), _ptr(signs), m, k, _ptr(out), _stream(x)))
    return out


def quantize(w: torch.Tensor, signs: torch.Tensor):
    """Rotate fp32 weight rows w [N, K] with the signed transform and round
    them to ternary g128: returns (codes int8 [N, K], scales float16 [N, K/128])."""
    _need(w, "w", torch.float32, 2)
    _need(signs, "signs", torch.int8, 1)
    n, k = w.shape
    if signs.shape[0] != k:
        raise ValueError("signs must have K entries")
    codes = torch.empty((n, k), dtype=torch.int8, device=w.device)
    scales = torch.empty((n, k // 128), dtype=torch.float16, device=w.device)
    _check("tl_quantize", lib().tl_quantize(_ptr(w), _ptr(signs), n, k, _ptr(codes), _ptr(scales),
                                            _stream(w)))
    return codes, scales


def gemm_workspace_bytes(m: int, n: int, k: int, fmt: int) -> int:
    """Device workspace bytes tl_gemm / tl_linear need (0: none)."""
    b = int(lib().tl_gemm_workspace_bytes(m, n, k, fmt))
    if b < 0:
        raise TLError("tl_gemm_workspace_bytes", 2)
    return b


def gemm_bf16_workspace_bytes(m: int, n: int, k: int, fmt: int) -> int:
    """Device workspace bytes tl_gemm_bf16 needs."""
    b = int(lib().tl_gemm_bf16_workspace_bytes(m, n, k, fmt))
    if b < 0:
        raise TLError("tl_gemm_bf16_workspace_bytes", 2)
    return b


def gemm_plan(m: int, n: int, k: int) -> tuple[int, int, int]:
    """tl_gemm's launch plan: (output tiles, tiles computed whole, K parts of
    each remaining tile)."""
    out = (ctypes.c_int64 * 3)()
    _check("tl_gemm_plan", lib().tl_gemm_plan(m, n, k, out))
    return int(out[0]), int(out[1]), int(out[2])


def _workspace(m, n, k, fmt, device, workspace, size=None):
    """(pointer, bytes) of the workspace a prefill call needs: the caller's
    uint8 tensor when given, else one from torch's allocator (None when the
    call needs none)."""
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
        return _ptr(workspace), workspace.numel(), workspace
    need = (size or gemm_workspace_bytes)(m, n, k, fmt)
    if need == 0:
        return _ptr(None), 0, None
    ws = torch.empty(need, dtype=torch.uint8, device=device)
    return _ptr(ws), need, ws


def _linear(call: str, packed, scales, fmt, x_rot, out_dtype, out, x_dtype=torch.float16,
            workspace=None):
    _need(packed, "packed", torch.uint8, 2)
    _need(scales, "scales", torch.float16, 2)
    _need(x_rot, "x_rot", x_dtype, 2)
    m, k = x_rot.shape
    n = packed.shape[0]
    if scales.shape != (n, k // GROUP):
        raise ValueError(f"scales must be [N, K/128] = {(n, k // GROUP)}, got {tuple(scales.shape)}")
    if packed.numel() != packed_bytes(n, k, fmt):
        raise ValueError("packed size does not match N, K and the format")
    if out_dtype not in (torch.float32, torch.float16):
        raise TypeError("out_dtype must be float32 or float16")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x_rot.device)
    else:
        _need(out, "out", out_dtype, 2)
        if out.shape != (m, n):
            raise ValueError("out must be [M, N]")
    yd = TL_F32 if out_dtype == torch.float32 else TL_F16
    fn = getattr(lib(), call)
    if call in ("tl_gemv", "tl_gemm_noalloc"):
        _check(call, fn(_ptr(packed), _ptr(scales), fmt, _ptr(x_rot), m, n, k, _ptr(out), yd,
                        _stream(x_rot)))
    else:
        size = gemm_bf16_workspace_bytes if call == "tl_gemm_bf16" else None
        wp, wb, _keep = _workspace(m, n, k, fmt, x_rot.device, workspace, size)
        _check(call, fn(_ptr(packed), _ptr(scales), fmt, _ptr(x_rot), m, n, k, _ptr(out), yd,
                        wp, wb, _stream(x_rot)))
    return out


def gemv(packed, scales, fmt, x_rot, out_dtype=torch.float32, out=None) -> torch.Tensor:
    """y[M, N] = x_rot . dequant(codes, scales)^T, decode-shaped (M <= 16)."""
    return _linear("tl_gemv", packed, scales, fmt, x_rot, out_dtype, out)


def gemm_noalloc(packed, scales, fmt, x_rot, out_dtype=torch.float32, out=None) -> torch.Tensor:
    """``gemm`` through tl_gemm_noalloc: no workspace argument and no
    allocation by the library (its workspace is a fixed device array of
    TL_GEMM_NOALLOC_MAX_WORKSPACE bytes shared by all calls on a GPU)."""
    return _linear("tl_gemm_noalloc", packed, scales, fmt, x_rot, out_dtype, out)


def gemm_bf16(packed, scales, fmt, x_rot, out_dtype=torch.float32, out=None,
              workspace=None) -> torch.Tensor:
    """The prefill product with bfloat16 rotated activations x_rot [M, K]: each
    row taken exactly to binary16 under a power-of-two factor, then the
    binary16 product (``workspace``: at least ``gemm_bf16_workspace_bytes``)."""
    return _linear("tl_gemm_bf16", packed, scales, fmt, x_rot, out_dtype, out,
                   x_dtype=torch.bfloat16, workspace=workspace)


def gemm(packed, scales, fmt, x_rot, out_dtype=torch.float32, out=None,
         workspace=None) -> torch.Tensor:
    """Same as ``gemv``, prefill-shaped (large M).  ``workspace`` (uint8, at
    least ``gemm_workspace_bytes``) is taken from torch's allocator when not
    given."""
    return _linear("tl_gemm", packed, scales, fmt, x_rot, out_dtype, out, workspace=workspace)


def linear(packed, scales, fmt, x, signs, out_dtype=torch.float32, out=None,
           x_rot=None, workspace=None) -> torch.Tensor:
    """y[M, N] = R(x) . dequant(codes, scales)^T on unrotated fp16 x [M, K];
    x_rot (allocated when None) receives R(x).  One fused launch at M = 1
    with the 2-bit-slot and dense trit packings (within their K limits)."""
    _need(packed, "packed", torch.uint8, 2)
    _need(scales, "scales", torch.float16, 2)
    _need(x, "x", torch.float16, 2)
    _need(signs, "signs", torch.int8, 1)
    m, k = x.shape
    n = packed.shape[0]
    if signs.shape[0] != k:
        raise ValueError("signs must have K entries")
    if scales.shape != (n, k // GROUP):
        raise ValueError(f"scales must be [N, K/128] = {(n, k // GROUP)}, got {tuple(scales.shape)}")
    if packed.numel() != packed_bytes(n, k, fmt):
        raise ValueError("packed size does not match N, K and the format")
    if out_dtype not in (torch.float32, torch.float16):
        raise TypeError("out_dtype must be float32 or float16")
    if x_rot is None:
        x_rot = torch.empty_like(x)
    else:
        _need(x_rot, "x_rot", torch.float16, 2)
        if x_rot.shape != x.shape:
            raise ValueError("x_rot must have the shape of x")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    else:
        _need(out, "out", out_dtype, 2)
        if out.shape != (m, n):
            raise ValueError("out must be [M, N]")
    yd = TL_F32 if out_dtype == torch.float32 else TL_F16
    if m >= 64:
        wp, wb, _keep = _workspace(m, n, k, fmt, x.device, workspace)
    else:
        wp, wb = _ptr(None), 0
    _check("tl_linear", lib().tl_linear(_ptr(packed), _ptr(scales), fmt, _ptr(x), _ptr(signs), m,
                                        n, k, _ptr(x_rot), _ptr(out), yd, wp, wb, _stream(x)))
    return out


class TernaryLinear:
    """A ternary g128 linear layer whose weights carry the folded rotation.

    ``forward`` always rotates its input first: skipping the runtime rotation
    gives wrong output without any error (page "A 27-billion model that fits
    in 8.6 GB", paragraph 3), so it is not optional here."""

    def __init__(self, packed, scales, fmt, signs, prefill_threshold: int = 64):
        self.packed, self.scales, self.fmt, self.signs = packed, scales, fmt, signs
        self.prefill_threshold = prefill_threshold

    def forward(self, x: torch.Tensor, out_dtype=torch.float32) -> torch.Tensor:
        if x.shape[0] >= self.prefill_threshold:
            return gemm(self.packed, self.scales, self.fmt, hadamard_rotate(x, self.signs),
                        out_dtype)
        return linear(self.packed, self.scales, self.fmt, x, self.signs, out_dtype)

    __call__ = forward


class ChainOp(ctypes.Structure):
    """tl_chain_op of include/tl.h."""
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("signs", ctypes.c_void_p), ("x_rot", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("fmt", ctypes.c_int32),
                ("y_dtype", ctypes.c_int32)]


class Chain:
    """A decode chain (tl_linear_chain): linears at M = 1 run in order in one
    launch, each the rotation of its input and the ternary product, with the
    next linear's weights requested before the current one ends.  ``ops``:
    dicts with packed, scales, fmt, x, signs, y and optionally x_rot (device
    tensors; x [1, K] or [K] binary16, y [1, N] or [N] float32/float16).  An
    x that is a view into the binary16 y of an earlier op makes that op wait
    for it.  The plan is encoded once (on the host, by the library) and kept
    on the device with the sync buffer; the tensors must stay alive."""

    def __init__(self, ops):
        if not ops:
            raise ValueError("a chain needs at least one linear")
        count = len(ops)
        arr = (ChainOp * count)()
        for i, o in enumerate(ops):
            _need(o["packed"], "packed", torch.uint8, 2)
            _need(o["scales"], "scales", torch.float16, 2)
            _need(o["x"], "x", torch.float16)
            _need(o["signs"], "signs", torch.int8, 1)
            n, k = o["packed"].shape[0], o["x"].numel()
            y = o["y"]
            if y.dtype not in (torch.float32, torch.float16) or y.numel() != n or not y.is_contiguous():
                raise ValueError("y must be a contiguous float32/float16 tensor of N elements")
            if o["signs"].numel() != k or o["scales"].shape != (n, k // GROUP):
                raise ValueError("signs must have K entries and scales be [N, K/128]")
            if o["packed"].numel() != packed_bytes(n, k, o["fmt"]):
                raise ValueError("packed size does not match N, K and the format")
            xr = o.get("x_rot")
            if xr is not None:
                _need(xr, "x_rot", torch.float16)
            arr[i] = ChainOp(o["packed"].data_ptr(), o["scales"].data_ptr(), o["x"].data_ptr(),
                             o["signs"].data_ptr(), 0 if xr is None else xr.data_ptr(),
                             y.data_ptr(), n, k, o["fmt"],
                             TL_F32 if y.dtype == torch.float32 else TL_F16)
        L = lib()
        nbytes = int(L.tl_chain_plan_bytes(count))
        host = (ctypes.c_uint8 * nbytes)()
        _check("tl_chain_encode", L.tl_chain_encode(arr, count, host, nbytes))
        device = ops[0]["x"].device
        self.count = count
        self.plan = torch.frombuffer(bytearray(host), dtype=torch.uint8).to(device)
        self.sync = torch.zeros(int(L.tl_chain_sync_bytes(count)) // 4, dtype=torch.int32,
                                device=device)
        self._ops = ops

    def __call__(self) -> None:
        _check("tl_linear_chain", lib().tl_linear_chain(_ptr(self.plan), self.count,
                                                        _ptr(self.sync), _stream(self.sync)))

    def error(self) -> int:
        """The chain's error word (0: none; see tl_linear_chain)."""
        return int(self.sync[self.count + 1].item())

    def clear_error(self) -> None:
        self.sync[self.count + 1].zero_()
