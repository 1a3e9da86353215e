"""Shared pieces of the GPU parity tests: buffers, transfers and comparisons."""

import numpy as np
import pytest
import torch

import oracle as om
from combine_get_dispatch_layout_amd import workloads as wl
from tests.helpers import bf16_bits, bf16_ulp_distance


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def make_buffer(E, R, C, max_tokens):
    from combine_get_dispatch_layout_amd import Buffer
    return Buffer(E, R, num_channels=C, max_tokens=max_tokens)


def np_(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    if t.dtype == torch.bool:
        return t.numpy().astype(np.uint8)
    return t.numpy()


def assert_equal(name, got, want):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{name}: shape {got.shape} != {want.shape}"
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} mismatches, first at {i}: got {got[i]} want {want[i]}")


def assert_bf16_within_1ulp(name, got_u16, want_u16):
    d = bf16_ulp_distance(got_u16, want_u16)
    assert d.shape == np.shape(want_u16)
    if (d > 1).any():
        i = tuple(np.argwhere(d > 1)[0])
        raise AssertionError(f"{name}: {int((d > 1).sum())} values beyond 1 bf16 ulp, first at {i}")


def check_handle(h, ref: "om.Dispatch", N: int):
    f = h.fields()
    assert_equal("is_token_in_rank", np_(f["is_token_in_rank"]), ref.layout.is_token_in_rank)
    assert_equal("num_tokens_per_rank", np_(f["num_tokens_per_rank"]), ref.layout.num_tokens_per_rank)
    assert_equal("num_tokens_per_expert", np_(f["num_tokens_per_expert"]), ref.layout.num_tokens_per_expert)
    assert_equal("rank_prefix_matrix", np_(f["rank_prefix_matrix"]), ref.prefix.rank_prefix_matrix)
    assert_equal("channel_prefix_matrix", np_(f["channel_prefix_matrix"]), ref.prefix.channel_prefix_matrix)
    assert_equal("recv_channel_prefix_matrix", np_(f["recv_channel_prefix_matrix"]),
                 ref.prefix.recv_channel_prefix_matrix)
    assert_equal("send_head", np_(f["send_head"]), ref.prefix.send_head)
    assert_equal("recv_src_idx", np_(f["recv_src_idx"])[:N], ref.prefix.recv_src_idx)
    assert int(np_(f["num_recv"])[0]) == ref.prefix.num_recv


def oracle_first_dispatch(o, inp: wl.Inputs, E, R, C, with_rows=True):
    return om.dispatch(o, bf16_bits(inp.x), inp.topk_idx.numpy(), inp.topk_weights.numpy(), E, R,
                       C, with_rows=with_rows)
