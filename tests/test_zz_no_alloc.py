"""The allocation-free get_dispatch_layout (moedx_get_dispatch_layout_static)
against the ctx-based moedx_get_dispatch_layout, bit for bit, through the C
ABI: two calls in a row on one stream (the second with a smaller batch and
other shapes), each compared with the ctx call on the same routing."""

import ctypes

import numpy as np
import pytest
import torch

from combine_get_dispatch_layout_amd import _capi as C
from combine_get_dispatch_layout_amd import workloads as wl
from tests.gpu_common import assert_equal, device, make_buffer, np_

pytestmark = pytest.mark.gpu


def _P(t):
    return ctypes.c_void_p(t.data_ptr() or t.untyped_storage().data_ptr() or None)


def _static_layout(idx, E, R, stream):
    """Enqueue the allocation-free layout; outputs start as sentinels."""
    T, K = idx.shape
    dev = idx.device
    ntr = torch.full((R,), -5, dtype=torch.int32, device=dev)
    nte = torch.full((E,), -5, dtype=torch.int32, device=dev)
    itr = torch.full((T, R), 7, dtype=torch.uint8, device=dev)
    C.check(C.moedx_get_dispatch_layout_static(_P(idx), T, K, E, R, _P(ntr), _P(nte), _P(itr),
                                               ctypes.c_void_p(stream.cuda_stream)))
    return ntr, nte, itr


CASES = [
    # (workload, tokens): each pair runs a larger call, then a smaller one
    [(wl.PREFILL, None), (wl.PREFILL, 1000)],
    [(wl.HANDLE_REUSE, None), (wl.TINY, None)],
    [(wl.FP8_SKEWED, None), (wl.LL_DECODE, None)],
]


@pytest.mark.parametrize("pair", CASES, ids=["prefill", "reuse-then-tiny", "fp8-then-ll"])
def test_static_layout_matches_ctx_layout(oracle, pair):
    dev = device()
    stream = torch.cuda.current_stream()
    runs = []
    for w, tokens in pair:  # both calls enqueued back to back, then compared
        inp = wl.make_inputs(w, tokens=tokens)
        idx = inp.topk_idx.to(dev)
        print(f"[no-alloc] {w.name} T={idx.shape[0]}", flush=True)
        runs.append((w, inp, idx, _static_layout(idx, w.experts, w.ranks, stream)))
    torch.cuda.synchronize()
    for w, inp, idx, (ntr, nte, itr) in runs:
        buf = make_buffer(w.experts, w.ranks, max(w.channels, 1), idx.shape[0])
        ntr_c, _, nte_c, itr_c, _ = buf.get_dispatch_layout(idx, w.experts)
        torch.cuda.synchronize()
        assert_equal("num_tokens_per_rank", np_(ntr), np_(ntr_c))
        assert_equal("num_tokens_per_expert", np_(nte), np_(nte_c))
        assert_equal("is_token_in_rank", np_(itr), np_(itr_c).astype(np.uint8))
        ref = oracle.layout(inp.topk_idx.numpy(), w.experts, w.ranks)
        assert_equal("num_tokens_per_expert vs oracle", np_(nte), ref.num_tokens_per_expert)


def test_static_layout_repeated_and_empty(oracle):
    """Many calls in a row (the ticket returns to zero after each) and an
    empty batch, which still writes zero counts."""
    dev = device()
    stream = torch.cuda.current_stream()
    w = wl.PREFILL
    inp = wl.make_inputs(w, tokens=3001)
    idx = inp.topk_idx.to(dev)
    outs = [_static_layout(idx, w.experts, w.ranks, stream) for _ in range(5)]
    empty = _static_layout(torch.empty(0, w.topk, dtype=torch.int64, device=dev), w.experts,
                           w.ranks, stream)
    torch.cuda.synchronize()
    ref = oracle.layout(inp.topk_idx.numpy(), w.experts, w.ranks)
    for ntr, nte, itr in outs:
        assert_equal("num_tokens_per_rank", np_(ntr), ref.num_tokens_per_rank)
        assert_equal("num_tokens_per_expert", np_(nte), ref.num_tokens_per_expert)
        assert_equal("is_token_in_rank", np_(itr), ref.is_token_in_rank)
    assert (np_(empty[0]) == 0).all() and (np_(empty[1]) == 0).all()
