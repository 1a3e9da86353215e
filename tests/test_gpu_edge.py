"""GPU parity on edge cases: empty and ragged batches, more channels than
tokens, empty buckets, every expert of a token in one bucket, empty (-1) slots,
the size limits (R = 64, E = 1024, K = 16, H = 8) and FP8 blocks of zeros."""

import numpy as np
import pytest
import torch

import oracle as om
from combine_get_dispatch_layout_amd import workloads as wl
from tests.gpu_common import (assert_bf16_within_1ulp, assert_equal, check_handle, device,
                              make_buffer, np_)
from tests.helpers import bf16_bits

pytestmark = pytest.mark.gpu


def run_case(o, idx: np.ndarray, H: int, E: int, R: int, C: int, seed: int = 0,
             x_u16: np.ndarray = None, capacity: bool = False, fp8: bool = False,
             from_layout: bool = False):
    """get_dispatch_layout, then a first dispatch (that reuses the layout's
    outputs when from_layout), then the combine, all against the oracle."""
    dev = device()
    T, K = idx.shape
    print(f"[edge] T={T} K={K} H={H} E={E} R={R} C={C} cap={capacity} fp8={fp8} "
          f"from_layout={from_layout}", flush=True)
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    if x_u16 is not None:
        x = torch.from_numpy(x_u16.astype(np.int16)).view(torch.bfloat16).reshape(T, H)
    w = torch.softmax(torch.randn(T, K, generator=g, dtype=torch.float64), -1).to(torch.float32)
    ref = om.dispatch(o, bf16_bits(x), idx, w.numpy(), E, R, C)
    N = ref.prefix.num_recv
    buf = make_buffer(E, R, C, max(T, 1))
    ti = torch.from_numpy(idx).to(dev)
    ntr, _, nte, itr, _ = buf.get_dispatch_layout(ti, E)
    assert_equal("num_tokens_per_rank", np_(ntr), ref.layout.num_tokens_per_rank)
    assert_equal("num_tokens_per_expert", np_(nte), ref.layout.num_tokens_per_expert)
    assert_equal("is_token_in_rank", np_(itr).reshape(T, R), ref.layout.is_token_in_rank)
    cap = T * min(K, R) if capacity else 0
    reuse = dict(num_tokens_per_rank=ntr, is_token_in_rank=itr,
                 num_tokens_per_expert=nte) if from_layout else {}
    layouts = buf.stats()["layout_launches"]

    def no_second_layout():
        if from_layout:  # the handle was scanned from (or borrowed) the layout's outputs
            st = buf.stats()
            assert st["layout_launches"] == layouts, st

    if fp8:
        (codes, scales), _, _, _, h, _ = buf.dispatch(x.to(dev), topk_idx=ti, fp8=True,
                                                      num_worst_tokens=cap, **reuse)
        cref, sref = o.pack_fp8(bf16_bits(x), ref.prefix)
        assert_equal("codes", np_(codes)[:N], cref)
        assert_equal("scales", np_(scales)[:N].view(np.uint32), sref.view(np.uint32))
        check_handle(h, ref, N)
        no_second_layout()
        return
    recv, rti, rtw, _, h, _ = buf.dispatch(x.to(dev), topk_idx=ti, topk_weights=w.to(dev),
                                           num_worst_tokens=cap, **reuse)
    torch.cuda.synchronize()
    check_handle(h, ref, N)
    assert_equal("recv_x", np_(recv)[:N], ref.recv_x)
    assert_equal("recv_topk_idx", np_(rti)[:N], ref.recv_topk_idx)
    assert_equal("recv_topk_weights", np_(rtw)[:N].view(np.uint32), ref.recv_topk_weights.view(np.uint32))
    comb, cw, _ = buf.combine(recv, h, topk_weights=rtw, gate_weights=w.to(dev))
    want, want_cw = o.combine(ref.recv_x, idx, E, ref.prefix, gate_weights=w.numpy(),
                              recv_topk_weights=ref.recv_topk_weights)
    assert_bf16_within_1ulp("combine", np_(comb).reshape(T, H), want)
    assert_equal("combined_topk_weights", np_(cw).reshape(T, K).view(np.uint32), want_cw.view(np.uint32))
    no_second_layout()


def _rand(T, E, K, p_empty=0.0, seed=0):
    return wl.random_routing(np.random.default_rng(seed), T, E, K, p_empty)


def test_empty_batch(oracle):
    run_case(oracle, np.zeros((0, 4), np.int64), 64, 16, 4, 3)


def test_single_token(oracle):
    run_case(oracle, _rand(1, 16, 4), 256, 16, 4, 8)


@pytest.mark.parametrize("T", [255, 256, 257, 1000, 3001])
def test_ragged_tiles(oracle, T):
    run_case(oracle, _rand(T, 64, 6, seed=T), 128, 64, 16, 7)


# The combine takes its workgroups in runs of 16 per XCD, in spans of 128
# workgroups (a last partial span keeps the plain order): grids just below, at
# and past one and two spans, and spans whose last workgroup holds waves past
# the last token (H = 512: one wave per token; H = 7168: 14).
@pytest.mark.parametrize("T,H", [(508, 512), (512, 512), (516, 512), (1024, 512), (1030, 512),
                                 (36, 7168), (37, 7168), (73, 7168)])
def test_combine_workgroup_order_spans(oracle, T, H):
    run_case(oracle, _rand(T, 64, 6, seed=T + H), H, 64, 8, 4, capacity=True)


def test_more_channels_than_tokens(oracle):
    run_case(oracle, _rand(5, 16, 2, seed=3), 64, 16, 4, 24)


def test_all_slots_empty(oracle):
    run_case(oracle, np.full((40, 4), -1, np.int64), 64, 16, 4, 3)


def test_empty_slots_and_empty_bucket(oracle):
    idx = _rand(300, 12, 3, p_empty=0.4, seed=5)
    idx[(idx >= 4) & (idx < 8)] = -1  # bucket 1 of 3 gets nothing
    run_case(oracle, idx, 128, 12, 3, 5)


def test_token_with_all_experts_in_one_bucket(oracle):
    idx = _rand(200, 32, 4, seed=9)
    idx[::3] = np.array([8, 9, 10, 11])  # bucket 2 of 8 (P = 4) takes all four
    run_case(oracle, idx, 64, 32, 8, 4)


def test_single_bucket(oracle):
    run_case(oracle, _rand(300, 8, 8, seed=1), 64, 8, 1, 3)


def test_limits(oracle):
    run_case(oracle, _rand(700, 1024, 16, seed=2), 8, 1024, 64, 33)


def test_capacity_mode_small(oracle):
    run_case(oracle, _rand(333, 16, 3, p_empty=0.2, seed=4), 64, 16, 4, 3, capacity=True)


def test_fp8_zero_blocks_and_negative_zero(oracle):
    T, H = 64, 256
    x = np.asarray(np.random.default_rng(1).integers(0, 1 << 16, (T, H)), np.uint16)
    x[(x & 0x7F80) == 0x7F80] = 0x3F80  # no inf / nan inputs
    x[0, :128] = 0
    x[1, :128] = 0x8000
    x[2, 128:] = 0x0001  # denormal bf16 values
    run_case(oracle, _rand(T, 16, 2, seed=6), H, 16, 4, 2, x_u16=x, fp8=True)


def test_fp8_capacity(oracle):
    run_case(oracle, _rand(500, 64, 6, seed=8), 384, 64, 16, 5, fp8=True, capacity=True)


def _blocks_enumerating(limit_bits: int, amax_bits: int, rng) -> np.ndarray:
    """1x128 blocks that together hold every bf16 magnitude up to `limit_bits`
    (random signs); each block also holds `amax_bits` once, so its maximum and
    hence its scale are fixed."""
    vals = np.arange(limit_bits + 1, dtype=np.uint16)
    vals = vals | (rng.integers(0, 2, vals.size).astype(np.uint16) << 15)
    nb = -(-vals.size // 127)
    out = np.zeros((nb, 128), np.uint16)
    flat = np.concatenate([vals, np.zeros(nb * 127 - vals.size, np.uint16)]).reshape(nb, 127)
    for b in range(nb):
        pos = int(rng.integers(0, 128))
        out[b] = np.insert(flat[b], pos, np.uint16(amax_bits))
    return out


def test_fp8_every_bf16_magnitude(oracle):
    """Quotients at scale exactly 1 (block maximum 448) cover every bf16
    magnitude up to 448, every E4M3 midpoint among them; a block maximum of 3
    gives a scale that is not a power of two."""
    rng = np.random.default_rng(11)
    H = 1024
    blocks = np.concatenate([_blocks_enumerating(0x43E0, 0x43E0, rng),   # 448 -> s = 1
                             _blocks_enumerating(0x4040, 0x4040, rng),   # 3.0 -> s = 3 / 448
                             _blocks_enumerating(0x3C00, 0x3C00, rng),   # 2^-7: above the 1e-4 floor
                             _blocks_enumerating(0x38D0, 0x38D0, rng)])  # below it: s = 1e-4 / 448
    per_row = H // 128
    T = -(-blocks.shape[0] // per_row)
    pad = np.tile(blocks[:1], (T * per_row - blocks.shape[0], 1))
    x = np.concatenate([blocks, pad]).reshape(T, H)
    run_case(oracle, _rand(T, 16, 2, seed=12), H, 16, 4, 2, x_u16=x, fp8=True)


def test_fp8_inf_and_nan_blocks(oracle):
    """Blocks holding +inf, -inf or NaN: the scale becomes inf (or ignores the
    NaN), and codes follow the IEEE quotients (NaN -> 0x7F)."""
    T, H = 8, 512
    rng = np.random.default_rng(13)
    x = np.asarray(rng.integers(0, 1 << 16, (T, H)), np.uint16)
    x[(x & 0x7F80) == 0x7F80] = 0x3F80
    x[0, 5] = 0x7F80           # +inf
    x[1, 130] = 0xFF80         # -inf
    x[2, 300] = 0x7FC0         # NaN
    x[3, 0:128] = 0x7FC1       # a block of NaN only
    x[4, 256:384] = 0x8000     # -0.0 block next to
    x[4, 300] = 0xFFC0         # a negative NaN
    x[5, 400] = 0x7F80
    x[5, 401] = 0xFF80         # inf and -inf: inf / inf is NaN
    run_case(oracle, _rand(T, 16, 2, seed=14), H, 16, 4, 2, x_u16=x, fp8=True)


@pytest.mark.parametrize("H", [1000, 2056, 7176])
def test_ragged_hidden(oracle, H):
    """Row widths that leave a short last slice in the pack and the combine
    (H / 8 = 125, 257, 897 chunks of 16 bytes)."""
    run_case(oracle, _rand(150, 32, 4, p_empty=0.1, seed=H), H, 32, 8, 3)


@pytest.mark.parametrize("H", [1152, 2176])
def test_fp8_ragged_blocks(oracle, H):
    """FP8 rows whose 1x128 blocks do not split evenly over the waves of a row
    (9 and 17 blocks)."""
    run_case(oracle, _rand(90, 32, 4, seed=H), H, 32, 8, 3, fp8=True)


def test_large_batch_global_scan_paths(oracle):
    """200000 tokens, 16 buckets, 200 channels: the group prefixes (3125 groups
    x 16 buckets) and the channel partials (201 x 16) exceed the finishing
    workgroup's LDS staging, so both come from global memory, over several
    scan passes."""
    run_case(oracle, _rand(200_000, 64, 4, p_empty=0.05, seed=77), 64, 64, 16, 200)


# The layout's straight-line finishing step covers up to 256 groups (T <= 16384),
# 16 buckets, 32 tiles of expert partials per expert thread (256 / E threads per
# expert when E < 256) and 3 channel boundaries per thread (768); every shape
# below sits at one of those limits or one past it, so both finishing steps are
# checked against the oracle on either side of each bound (H = 8 keeps the
# rows small while every receive position is still compared).
@pytest.mark.parametrize("T,E,K,R,C", [
    (16384, 64, 6, 16, 47),   # 256 groups, 64 tiles over 4 threads per expert, 768 boundaries
    (16384, 64, 6, 16, 48),   # 784 boundaries: general step
    (16385, 64, 6, 16, 8),    # 257 groups: general step
    (8192, 256, 8, 16, 5),    # 32 tiles with one thread per expert
    (8193, 256, 8, 16, 5),    # 33 tiles: general step
    (1000, 68, 4, 17, 6),     # 17 buckets: general step
    (2000, 1024, 8, 16, 8),   # experts past the first 256 summed after the fast part
], ids=lambda v: str(v))
def test_layout_finishing_step_limits(oracle, T, E, K, R, C):
    run_case(oracle, _rand(T, E, K, p_empty=0.02, seed=T + R + C), 8, E, R, C, capacity=(T % 2 == 0))


# The first capacity-mode dispatch (bf16 or FP8) finishes the handle in its own
# launch when T <= 4096 and R is a multiple of 4 up to 16 (it reads its receive
# rows from the layout's partials); otherwise the layout writes every prefix at
# prepare.
# Shapes on both sides: the 64-group limit, ragged groups, R = 4, 8, 12, 16
# and R not a multiple of 4, and larger batches up to the layout's fast
# finishing limits.
@pytest.mark.parametrize("T,E,K,R,C", [
    (4096, 64, 8, 8, 8),      # 64 groups, one launch
    (4097, 64, 8, 8, 8),      # 65 groups: prefixes at prepare
    (8192, 64, 8, 8, 8),      # 128 groups: prefixes at prepare
    (8193, 64, 8, 8, 8),      # 129 groups
    (6000, 96, 8, 12, 6),     # ragged last group, R = 12
    (8192, 256, 8, 16, 20),   # R = 16 at 128 groups, 32 tiles per expert thread
    (333, 48, 6, 4, 3),       # ragged last group, R = 4
    (1500, 96, 8, 12, 6),     # R = 12 (16-bucket lookup, 4 buckets unused)
    (4096, 256, 8, 16, 20),   # R = 16 at 64 groups
    (777, 36, 5, 6, 4),       # R = 6: prefixes at prepare
    (64, 16, 4, 8, 2),        # one group
], ids=lambda v: str(v))
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_first_capacity_dispatch_one_launch(oracle, T, E, K, R, C, fp8):
    run_case(oracle, _rand(T, E, K, p_empty=0.05, seed=3 * T + R), 256 if fp8 else 16, E, R, C,
             capacity=True, fp8=fp8)


# A first dispatch given get_dispatch_layout's outputs (the normal-kernel
# example's call order): the handle is scanned from is_token_in_rank and the
# expert totals instead of running the layout again.  Shapes over every path:
# empty batch, one token, ragged tiles, R = 1, 3, 6 (byte loads of the mask
# rows) and 64, empty slots and buckets, exact and capacity mode (one-launch
# first dispatch, prefixes at prepare), FP8, and both finishing steps.
@pytest.mark.parametrize("T,E,K,R,C,p_empty,capacity,fp8", [
    (0, 16, 4, 4, 3, 0.0, False, False),
    (1, 16, 4, 4, 8, 0.0, True, False),
    (257, 64, 6, 16, 7, 0.0, False, False),
    (3001, 64, 6, 16, 7, 0.1, True, False),
    (300, 12, 3, 3, 5, 0.4, False, False),
    (300, 8, 8, 1, 3, 0.0, True, False),
    (777, 36, 5, 6, 4, 0.05, True, False),
    (700, 1024, 16, 64, 33, 0.0, False, False),
    (4096, 64, 8, 8, 8, 0.05, True, False),
    (4097, 64, 8, 8, 8, 0.05, True, False),
    (16385, 64, 6, 16, 8, 0.02, False, False),
    (500, 64, 6, 16, 5, 0.0, True, True),
    (1000, 256, 8, 8, 24, 0.0, False, True),
], ids=lambda v: str(v))
def test_dispatch_from_layout_outputs(oracle, T, E, K, R, C, p_empty, capacity, fp8):
    run_case(oracle, _rand(T, E, K, p_empty=p_empty, seed=T + 5 * R), 128 if fp8 else 16, E, R,
             C, capacity=capacity, fp8=fp8, from_layout=True)
