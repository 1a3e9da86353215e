"""Events and streams: async completion, previous_event chaining, the ctx's
own stream, and capture() / current_stream_wait() ordering."""

import numpy as np
import pytest
import torch

import oracle as om
from combine_get_dispatch_layout_amd import workloads as wl
from tests.gpu_common import assert_equal, device, make_buffer, np_
from tests.helpers import bf16_bits

pytestmark = pytest.mark.gpu


def test_async_chain_on_ctx_stream(oracle):
    dev = device()
    w = wl.PREFILL
    inp = wl.make_inputs(w, tokens=2048)
    buf = make_buffer(w.experts, w.ranks, w.channels, 2048)
    x, idx, gw = inp.x.to(dev), inp.topk_idx.to(dev), inp.topk_weights.to(dev)
    ref = om.dispatch(oracle, bf16_bits(inp.x), inp.topk_idx.numpy(), inp.topk_weights.numpy(),
                      w.experts, w.ranks, w.channels)
    cap = 2048 * min(w.topk, w.ranks)
    ev0 = buf.capture()
    ntr, _, nte, itr, ev1 = buf.get_dispatch_layout(idx, w.experts, previous_event=ev0,
                                                    async_finish=True, allocate_on_comm_stream=True)
    assert ev1.event is not None
    recv, rti, rtw, _, h, ev2 = buf.dispatch(x, topk_idx=idx, topk_weights=gw, num_worst_tokens=cap,
                                             previous_event=ev1, async_finish=True,
                                             allocate_on_comm_stream=True)
    comb, _, ev3 = buf.combine(recv, h, gate_weights=gw, previous_event=ev2, async_finish=True,
                               allocate_on_comm_stream=True)
    with ev3:
        pass  # leaving the block makes the current stream wait for the combine
    got = comb.clone()  # ordered after ev3 on the current stream
    torch.cuda.synchronize()
    N = ref.prefix.num_recv
    assert_equal("layout", np_(itr), ref.layout.is_token_in_rank)
    assert_equal("recv_x", np_(recv)[:N], ref.recv_x)
    want, _ = oracle.combine(ref.recv_x, inp.topk_idx.numpy(), w.experts, ref.prefix,
                             gate_weights=inp.topk_weights.numpy())
    assert_equal("combine", np_(got), want)


def test_sync_call_returns_complete_event():
    dev = device()
    w = wl.TINY
    inp = wl.make_inputs(w)
    buf = make_buffer(w.experts, w.ranks, w.channels, w.tokens)
    *_, ev = buf.get_dispatch_layout(inp.topk_idx.to(dev), w.experts)
    assert ev.event is None
    ev.current_stream_wait()  # a no-op on a completed call


def test_on_ctx_stream_waits_for_caller_stream(oracle):
    """The ctx stream must not start before work already queued on the
    caller's stream (the input is written there just before the call)."""
    dev = device()
    w = wl.TINY
    inp = wl.make_inputs(w)
    buf = make_buffer(w.experts, w.ranks, w.channels, w.tokens)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        idx = torch.full((w.tokens, w.topk), -1, dtype=torch.int64, device=dev)
        torch.cuda._sleep(2_000_000)
        idx.copy_(inp.topk_idx.to(dev, non_blocking=False))
        ntr, _, nte, itr, ev = buf.get_dispatch_layout(idx, w.experts, async_finish=True,
                                                       allocate_on_comm_stream=True)
        ev.current_stream_wait()
    torch.cuda.synchronize()
    ref = oracle.layout(inp.topk_idx.numpy(), w.experts, w.ranks)
    assert_equal("num_tokens_per_expert", np_(nte), ref.num_tokens_per_expert)
