"""Pins of the oracle's FP8 scale modes and pre-quantised pass-through.

The EnflameTechnology/DeepEP README (feature notes) lists power-of-two scales
(round_scale), UE8M0 exponent-byte scales (use_ue8m0), a single per-tensor
scale (fp8_quant_scale, exclusive with use_ue8m0) and the dispatch of an
already-quantised (codes, scales) pair.  Each check below reaches the result by
another route: exact rational arithmetic for the power-of-two scale, torch's
float8_e4m3fn cast for codes, numpy fancy indexing for the pass-through.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from combine_get_dispatch_layout_amd import workloads as wl
from tests.helpers import bf16_bits, bits_to_f32, f32_to_bf16_torch


def _bf16_values(n, seed, scale=3.0):
    g = torch.Generator().manual_seed(seed)
    return bf16_bits((torch.randn(n, generator=g) * scale).to(torch.bfloat16))


def _torch_e4m3(q: np.ndarray) -> np.ndarray:
    """E4M3FN codes of fp32 values |q| <= 448 by torch's cast (round to nearest even)."""
    assert (np.abs(q) <= 448).all()
    return torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def _is_pow2_ceiling(s: float, ap: float) -> bool:
    fs, q = Fraction(s), Fraction(ap) / 448
    m, _ = np.frexp(s)
    return m == 0.5 and fs >= q and fs / 2 < q


def test_pow2_scale_worked_values(oracle):
    # 3 / 448 lies in (2^-8, 2^-7]; 7 * 2^-5 / 448 = 2^-11 exactly; 448 / 448 = 1;
    # the 1e-4 floor: 1e-4 / 448 = 2.23e-7 in (2^-23, 2^-22].
    assert oracle.pow2_scale(3.0) == 2.0 ** -7
    assert oracle.pow2_scale(7 * 2.0 ** -5) == 2.0 ** -11
    assert oracle.pow2_scale(448.0) == 1.0
    assert oracle.pow2_scale(449.0) == 2.0
    assert oracle.pow2_scale(float(np.float32(1e-4))) == 2.0 ** -22
    assert np.isinf(oracle.pow2_scale(float("inf")))


def test_pow2_scale_is_the_power_of_two_ceiling(oracle):
    # every positive finite bf16 magnitude, and the fp32 floor value
    vals = bits_to_f32(np.arange(0x0001, 0x7F80, dtype=np.uint16))
    vals = np.concatenate([vals, np.float32([1e-4])])
    for ap in vals[::7]:
        s = oracle.pow2_scale(float(ap))
        assert _is_pow2_ceiling(s, float(ap)), (ap, s)
    for k in range(-30, 120):  # quotients that are exactly powers of two
        ap = float(np.float32(7 * 2.0 ** k))
        assert oracle.pow2_scale(ap) == Fraction(ap) / 448


@pytest.mark.parametrize("mode", ["pow2", "ue8m0"])
def test_pow2_block_codes_and_scale(oracle, mode):
    m = oracle.FP8_POW2 if mode == "pow2" else oracle.FP8_UE8M0
    x = _bf16_values(16 * 128, seed=5)
    x[:128] = 0                       # all-zero block: the 1e-4 floor
    x[128:256] = f32_to_bf16_torch(np.full(128, 7 * 2.0 ** -3, np.float32))  # exact quotient
    codes, scales = oracle.quant_row_fp8_mode(x, m)
    v = bits_to_f32(x).reshape(-1, 128)
    ap = np.maximum(np.abs(v).max(1), np.float32(1e-4))
    for j in range(v.shape[0]):
        if mode == "pow2":
            s = float(scales[j])
        else:
            s = 2.0 ** (int(scales[j]) - 127)
        assert _is_pow2_ceiling(s, float(ap[j])), j
        q = (v[j].astype(np.float64) / s).astype(np.float32)  # exact: s is a power of two
        assert np.array_equal(codes[j * 128:(j + 1) * 128], _torch_e4m3(q)), j
    assert scales[1] == (2.0 ** -9 if mode == "pow2" else 127 - 9)


def test_ue8m0_matches_pow2(oracle):
    x = _bf16_values(8 * 128, seed=6, scale=50.0)
    c1, s1 = oracle.quant_row_fp8_mode(x, oracle.FP8_POW2)
    c2, s2 = oracle.quant_row_fp8_mode(x, oracle.FP8_UE8M0)
    assert np.array_equal(c1, c2)
    assert np.array_equal(s2.astype(np.int32) - 127, np.log2(s1.astype(np.float64)).astype(np.int32))


def test_tensor_scale_codes_and_saturation(oracle):
    x = _bf16_values(4 * 128, seed=7, scale=2.0)
    for s in (0.001, 0.0078125, 0.37, 1.0):
        codes, scales = oracle.quant_row_fp8_mode(x, oracle.FP8_TENSOR, s)
        assert scales is None
        q = bits_to_f32(x) / np.float32(s)   # the fp32 quotient
        inr = np.abs(q) < 448
        assert np.array_equal(codes[inr], _torch_e4m3(q[inr]))
        big = np.abs(q) >= 464
        assert ((codes[big] & 0x7F) == 0x7E).all()
        assert np.array_equal(codes[big] >> 7, (q[big] < 0).astype(np.uint8))
        mid = (np.abs(q) >= 448) & ~big      # rounds to +/-448 anyway
        assert ((codes[mid] & 0x7F) == 0x7E).all()
        if s == 0.001:
            assert big.any()


def test_amax_mode_equals_plain_fp8(oracle):
    x = _bf16_values(6 * 128, seed=8)
    c1, s1 = oracle.quant_row_fp8(x)
    c2, s2 = oracle.quant_row_fp8_mode(x, oracle.FP8_AMAX)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("seed", [1, 2])
def test_pack_modes_and_rows_bytes_against_indexing(oracle, seed):
    rng = np.random.default_rng(seed)
    T, E, R, K, C, H = 37, 16, 4, 3, 5, 256
    idx = wl.random_routing(rng, T, E, K, 0.2)
    lay = oracle.layout(idx, E, R)
    pre = oracle.prefix(lay.is_token_in_rank, C)
    x = _bf16_values(T * H, seed=seed).reshape(T, H)
    src = pre.recv_src_idx
    for mode in (oracle.FP8_AMAX, oracle.FP8_POW2, oracle.FP8_UE8M0, oracle.FP8_TENSOR):
        codes, scales = oracle.pack_fp8_mode(x, pre, mode, 0.05)
        for n in range(pre.num_recv):
            c, s = oracle.quant_row_fp8_mode(x[src[n]], mode, 0.05)
            assert np.array_equal(codes[n], c)
            if s is not None:
                assert np.array_equal(scales[n], s)
    # pass-through of pre-quantised rows: a gather by recv_src_idx
    codes8 = rng.integers(0, 256, (T, H), dtype=np.uint8)
    sc = rng.standard_normal((T, H // 128)).astype(np.float32)
    assert np.array_equal(oracle.pack_rows_bytes(codes8, pre), codes8[src])
    assert np.array_equal(oracle.pack_rows_bytes(sc, pre).view(np.float32), sc[src])
