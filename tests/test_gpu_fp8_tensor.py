"""FP8 on the device: the hardware fp32 -> E4M3FN conversion the pack uses,
and per-tensor scales across their accepted range, against the oracle.

The per-tensor path (fp8_quant_scale of the EnflameTechnology/DeepEP README
feature notes) accepts any scale in [2^-126, 2^126); every finite bf16 value is
dispatched at scales spread over that range, including tiny scales over
subnormal inputs, and the codes are compared bit for bit with the oracle's
E4M3FN(x / s)."""

import ctypes

import numpy as np
import pytest
import torch

from tests.gpu_common import assert_equal, device, make_buffer, np_

pytestmark = pytest.mark.gpu


def test_fp8_conversion_matches_encoder():
    """gfx950's packed conversion == e4m3_code for every |q| <= 448 + 1 ulp, both
    signs (the pack feeds it nothing larger: the quotient of a block's largest
    value by its rounded scale is at most one ulp above 448)."""
    device()
    from tests import device_check
    lib = device_check.load()
    bits448 = int(np.float32(448.0).view(np.uint32))
    bad, first = ctypes.c_uint32(), ctypes.c_uint32()
    rc = lib.fp8_cvt_check(bits448 + 2, ctypes.byref(bad), ctypes.byref(first))
    assert rc == 0, f"HIP error {rc}"
    assert bad.value == 0, f"{bad.value} mismatches, lowest at 0x{first.value:08x}"


def _all_bf16(T, H):
    """Every bf16 bit pattern once, as [T, H] (64 x 1024)."""
    assert T * H == 1 << 16
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(T, H)
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)


SCALES = [2.0 ** -126, 2.0 ** -120, 2.0 ** -100, 2.0 ** -90, 2.0 ** -20, 0.0123, 0.37, 1.0,
          1e3, 2.0 ** 100, 2.0 ** 120, float(np.nextafter(np.float32(2.0 ** 126), np.float32(0)))]


def _spread_scales(n, seed):
    """n scales with random significands and exponents spread over [-126, 125]."""
    rng = np.random.default_rng(seed)
    e = rng.integers(-126, 126, n)
    m = rng.integers(0, 1 << 23, n)
    bits = ((e + 127).astype(np.uint32) << 23) | m.astype(np.uint32)
    return [float(v) for v in bits.view(np.float32)]


@pytest.mark.parametrize("scales", ["listed", "spread"])
def test_fp8_tensor_scales_every_bf16(oracle, scales):
    dev = device()
    T, H, E, R = 64, 1024, 4, 4
    x_cpu = _all_bf16(T, H)
    idx_cpu = (torch.arange(T, dtype=torch.int64) % E).view(T, 1)  # one bucket per token
    lay = oracle.layout(idx_cpu.numpy(), E, R)
    pre = oracle.prefix(lay.is_token_in_rank, 1)
    x_u16 = x_cpu.view(torch.int16).numpy().view(np.uint16)
    buf = make_buffer(E, R, 1, T)
    x, idx = x_cpu.to(dev), idx_cpu.to(dev)
    todo = SCALES if scales == "listed" else _spread_scales(48, 5)
    h = None
    for s in todo:
        s = float(np.float32(s))
        print(f"[fp8 tensor] scale {s!r}", flush=True)
        if h is None:
            (codes, sc), _, _, _, h, _ = buf.dispatch(x, topk_idx=idx, fp8_quant_scale=s)
        else:
            (codes, sc), *_ = buf.dispatch(x, handle=h, fp8_quant_scale=s)
        assert sc is None
        want, _ = oracle.pack_fp8_mode(x_u16, pre, oracle.FP8_TENSOR, s)
        assert_equal(f"codes at scale {s!r}", np_(codes)[:pre.num_recv], want)
