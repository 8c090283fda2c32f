"""TL_DEBUG=1: calls that decode packed bytes first count the bytes that are
not valid encodings of their format and refuse with TL_ERR_DATA when there
is any (a 2-bit slot holding 3, a dense-trit byte above 242, a group's last
dense-trit byte whose pad digits are not 1).  Valid bytes pass and give the
same result as without the check; the 1-bit format has no invalid bytes."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tl_hadamard_rotate_amd as tl

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_env(monkeypatch):
    monkeypatch.setenv("TL_DEBUG", "1")


def dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def _layer(gpu, fmt, n=300, k=2048, m=3):
    inp = synth.linear_inputs(n, k, m, cfg=1, linear=fmt + 7, binary=fmt == tl.FMT_BIT1)
    packed = tl.pack(dev(inp.codes, gpu), fmt)
    x_rot = dev(oracle.rotate(inp.x, inp.signs).astype(np.float16), gpu)
    return inp, packed, dev(inp.scales, gpu), x_rot


@pytest.mark.parametrize("fmt", [tl.FMT_TRIT5, tl.FMT_SLOT2, tl.FMT_BIT1], ids=["trit5", "slot2", "bit1"])
def test_valid_bytes_pass(gpu, debug_env, fmt):
    inp, packed, scales, x_rot = _layer(gpu, fmt)
    y = tl.gemv(packed, scales, fmt, x_rot).cpu().numpy().astype(np.float64)
    assert oracle.rel_l2(y, oracle.matvec(inp.codes, inp.scales, x_rot.cpu().numpy())) < 1e-5
    assert np.array_equal(tl.unpack(packed, inp.codes.shape[1], fmt).cpu().numpy(), inp.codes)


@pytest.mark.parametrize("fmt,where,value", [
    (tl.FMT_SLOT2, 777, 0xFF), (tl.FMT_SLOT2, 12345, 0x0C),
    (tl.FMT_TRIT5, 100, 243), (tl.FMT_TRIT5, 25, 0), (tl.FMT_TRIT5, 26 * 9 + 25, 135)],
    ids=["slot2-ff", "slot2-one-slot", "trit5-243", "trit5-pad-low", "trit5-pad-high"])
def test_invalid_bytes_refused(gpu, debug_env, monkeypatch, fmt, where, value):
    inp, packed, scales, x_rot = _layer(gpu, fmt)
    bad = packed.clone()
    bad.view(-1)[where] = value
    y = torch.full((x_rot.shape[0], packed.shape[0]), 7.0, device=gpu)
    calls = [lambda: tl.gemv(bad, scales, fmt, x_rot, out=y),
             lambda: tl.gemm(bad, scales, fmt, x_rot, out=y),
             lambda: tl.unpack(bad, inp.codes.shape[1], fmt)]
    for call in calls:
        with pytest.raises(tl.TLError) as err:
            call()
        assert err.value.status == 9 and "1 packed bytes" in str(err.value)
    assert bool(torch.all(y == 7.0))          # nothing was launched
    # without the check the same call runs (its results are unspecified)
    monkeypatch.delenv("TL_DEBUG")
    tl.gemv(bad, scales, fmt, x_rot, out=y)
    torch.cuda.synchronize()
