"""tl_gemm_noalloc, the prefill product that takes no workspace argument and
allocates nothing, against tl_gemm on the same inputs: two calls in a row on
the one shared scratch array, the second with a smaller input, through the C
ABI.  Both entry points run the same kernels and launch plan, so the outputs
must be identical bit for bit; they are also checked against the oracle."""
import ctypes

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


def _noalloc(packed, scales, fmt, x_rot, y):
    m, k = x_rot.shape
    n = packed.shape[0]
    stream = ctypes.c_void_p(torch.cuda.current_stream(x_rot.device).cuda_stream)
    yd = tl.TL_F32 if y.dtype == torch.float32 else tl.TL_F16
    return tl.lib().tl_gemm_noalloc(ctypes.c_void_p(packed.data_ptr()),
                                    ctypes.c_void_p(scales.data_ptr()), fmt,
                                    ctypes.c_void_p(x_rot.data_ptr()), m, n, k,
                                    ctypes.c_void_p(y.data_ptr()), yd, stream)


@pytest.mark.parametrize("fmt", [tl.FMT_TRIT5, tl.FMT_SLOT2, tl.FMT_BIT1],
                         ids=["trit5", "slot2", "bit1"])
def test_noalloc_matches_gemm_twice(gpu, fmt):
    # the first shape needs both parts of the scratch (the 2-bit-slot rewrite
    # of dense trits / 1-bit codes, and K-split partial sums: 3 x 34 tiles on
    # 256 CUs); the second is smaller and leaves stale bytes of the first
    # beyond its own extent
    cases = [(600, 8700, 5120, torch.float32), (130, 700, 2048, torch.float16)]
    for i, (m, n, k, out_dtype) in enumerate(cases):
        inp = synth.linear_inputs(n, k, m, cfg=4, linear=40 + i, binary=fmt == tl.FMT_BIT1)
        packed = tl.pack(dev(inp.codes, gpu), fmt)
        scales = dev(inp.scales, gpu)
        x_rot16 = oracle.rotate(inp.x, inp.signs).astype(np.float16)
        x_rot = dev(x_rot16, gpu)
        assert tl.gemm_workspace_bytes(m, n, k, fmt) > 0
        y = torch.full((m, n), float("nan"), dtype=out_dtype, device=gpu)
        assert _noalloc(packed, scales, fmt, x_rot, y) == 0
        want_gpu = tl.gemm(packed, scales, fmt, x_rot, out_dtype=out_dtype)
        got = host(y)
        bits = np.uint32 if out_dtype == torch.float32 else np.uint16
        assert np.array_equal(got.view(bits), host(want_gpu).view(bits)), (m, n, k)
        rows = np.arange(0, n, 7)
        want = oracle.matvec(inp.codes[rows], inp.scales[rows], x_rot16)
        assert oracle.rel_l2(got[:, rows].astype(np.float64), want) < (
            1e-5 if out_dtype == torch.float32 else 2e-3)
