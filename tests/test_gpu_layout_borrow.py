"""A first dispatch prepared from exactly the outputs of the ctx's last
get_dispatch_layout borrows the partials that call left in the ctx's scratch
(no scan kernel), and its first pack builds the handle.  Every other way
the borrowed data can be needed is checked against the oracle: a new layout on
the ctx before the first dispatch, an FP8 first dispatch, an explicit finish, a
second handle borrowing the same layout, a destroyed borrower, a first pack on
another stream followed at once by a new layout, and a ctx destroyed first."""

import ctypes

import numpy as np
import pytest
import torch

from combine_get_dispatch_layout_amd import _capi as C
from combine_get_dispatch_layout_amd import workloads as wl
from tests.gpu_common import assert_equal, check_handle, device, make_buffer, np_, oracle_first_dispatch

pytestmark = pytest.mark.gpu

W = wl.PREFILL
T = 1000


def _setup(oracle, seed=None):
    dev = device()
    inp = wl.make_inputs(W, seed=seed, tokens=T)
    ref = oracle_first_dispatch(oracle, inp, W.experts, W.ranks, W.channels)
    return dev, inp, ref


def _layout(buf, inp, dev):
    idx = inp.topk_idx.to(dev)
    ntr, _, nte, itr, _ = buf.get_dispatch_layout(idx, W.experts)
    return idx, ntr, nte, itr


def _prepare(buf, idx, ntr, nte, itr):
    h, _ = buf.prepare(idx, T * min(W.topk, W.ranks), num_tokens_per_rank=ntr,
                       is_token_in_rank=itr, num_tokens_per_expert=nte)
    return h


def _check_first_dispatch(buf, h, inp, ref, dev):
    N = ref.prefix.num_recv
    recv, rti, _, _, h2, _ = buf.dispatch(inp.x.to(dev), handle=h)
    torch.cuda.synchronize()
    assert h2 is h
    check_handle(h, ref, N)
    assert_equal("recv_x", np_(recv)[:N], ref.recv_x)


def test_borrow_then_first_dispatch_runs_no_scan(oracle):
    dev, inp, ref = _setup(oracle)
    buf = make_buffer(W.experts, W.ranks, W.channels, T)
    idx, ntr, nte, itr = _layout(buf, inp, dev)
    before = buf.stats()
    recv, rti, rtw, _, h, _ = buf.dispatch(
        inp.x.to(dev), topk_idx=idx, topk_weights=inp.topk_weights.to(dev),
        num_tokens_per_rank=ntr, is_token_in_rank=itr, num_tokens_per_expert=nte,
        num_worst_tokens=T * min(W.topk, W.ranks))
    torch.cuda.synchronize()
    st = buf.stats()
    assert st["scan_launches"] == before["scan_launches"]
    assert st["layout_launches"] == before["layout_launches"]
    N = ref.prefix.num_recv
    check_handle(h, ref, N)
    assert_equal("recv_x", np_(recv)[:N], ref.recv_x)
    assert_equal("recv_topk_idx", np_(rti)[:N], ref.recv_topk_idx)
    # the handle's own copies of the routing (slot buckets, masks) serve the combine
    comb, _, _ = buf.combine(recv, h, gate_weights=inp.topk_weights.to(dev))
    want, _ = oracle.combine(ref.recv_x, inp.topk_idx.numpy(), W.experts, ref.prefix,
                             gate_weights=inp.topk_weights.numpy())
    assert_equal("combine", np_(comb), want)


def test_new_layout_before_first_dispatch(oracle):
    """The next layout copies the borrowed partials into the handle first."""
    dev, inp, ref = _setup(oracle)
    _, inp2, ref2 = _setup(oracle, seed=77)
    buf = make_buffer(W.experts, W.ranks, W.channels, T)
    idx, ntr, nte, itr = _layout(buf, inp, dev)
    h = _prepare(buf, idx, ntr, nte, itr)
    scans = buf.stats()["scan_launches"]
    _, ntr2, nte2, itr2 = _layout(buf, inp2, dev)  # overwrites the ctx's scratch
    assert buf.stats()["scan_launches"] == scans + 1
    assert_equal("second layout", np_(itr2), ref2.layout.is_token_in_rank)
    _check_first_dispatch(buf, h, inp, ref, dev)


def test_fp8_first_dispatch_of_a_borrower(oracle):
    dev, inp, ref = _setup(oracle)
    buf = make_buffer(W.experts, W.ranks, W.channels, T)
    idx, ntr, nte, itr = _layout(buf, inp, dev)
    h = _prepare(buf, idx, ntr, nte, itr)
    (codes, scales), *_ = buf.dispatch(inp.x.to(dev), handle=h, fp8=True)
    torch.cuda.synchronize()
    N = ref.prefix.num_recv
    check_handle(h, ref, N)
    cref, sref = oracle.pack_fp8(np_(inp.x), ref.prefix)
    assert_equal("codes", np_(codes)[:N], cref)
    assert_equal("scales", np_(scales)[:N].view(np.uint32), sref.view(np.uint32))


def test_finish_of_a_borrower_then_dispatch(oracle):
    dev, inp, ref = _setup(oracle)
    buf = make_buffer(W.experts, W.ranks, W.channels, T)
    idx, ntr, nte, itr = _layout(buf, inp, dev)
    h = _prepare(buf, idx, ntr, nte, itr)
    h.finish()
    f = h.fields()
    torch.cuda.synchronize()
    assert_equal("rank_prefix_matrix", np_(f["rank_prefix_matrix"]), ref.prefix.rank_prefix_matrix)
    assert_equal("num_tokens_per_expert", np_(f["num_tokens_per_expert"]),
                 ref.layout.num_tokens_per_expert)
    _check_first_dispatch(buf, h, inp, ref, dev)


def test_two_borrowers_of_one_layout(oracle):
    dev, inp, ref = _setup(oracle)
    buf = make_buffer(W.experts, W.ranks, W.channels, T)
    idx, ntr, nte, itr = _layout(buf, inp, dev)
    a = _prepare(buf, idx, ntr, nte, itr)
    b = _prepare(buf, idx, ntr, nte, itr)  # settles a's borrow first
    _check_first_dispatch(buf, b, inp, ref, dev)
    _check_first_dispatch(buf, a, inp, ref, dev)


def test_destroyed_borrower_then_new_layout(oracle):
    dev, inp, ref = _setup(oracle)
    buf = make_buffer(W.experts, W.ranks, W.channels, T)
    idx, ntr, nte, itr = _layout(buf, inp, dev)
    h = _prepare(buf, idx, ntr, nte, itr)
    del h
    idx, ntr, nte, itr = _layout(buf, inp, dev)
    h = _prepare(buf, idx, ntr, nte, itr)
    _check_first_dispatch(buf, h, inp, ref, dev)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_first_pack_on_another_stream_then_layout(oracle, fp8):
    """The layout after a borrowing first pack (bf16 or FP8) on another
    stream waits for that pack's reads of the scratch."""
    dev, inp, ref = _setup(oracle)
    _, inp2, ref2 = _setup(oracle, seed=78)
    buf = make_buffer(W.experts, W.ranks, W.channels, T)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    x = inp.x.to(dev)
    idx, idx2 = inp.topk_idx.to(dev), inp2.topk_idx.to(dev)
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"[borrow streams] rep {rep}", flush=True)
        with torch.cuda.stream(s1):
            ntr, _, nte, itr, ev = buf.get_dispatch_layout(idx, W.experts, async_finish=True)
        with torch.cuda.stream(s2):
            recv, _, _, _, h, _ = buf.dispatch(
                x, topk_idx=idx, num_tokens_per_rank=ntr, is_token_in_rank=itr,
                num_tokens_per_expert=nte, num_worst_tokens=T * min(W.topk, W.ranks),
                previous_event=ev, no_sync=True, fp8=fp8)
        with torch.cuda.stream(s1):
            ntr2, _, nte2, itr2, _ = buf.get_dispatch_layout(idx2, W.experts, async_finish=True)
        torch.cuda.synchronize()
        N = ref.prefix.num_recv
        check_handle(h, ref, N)
        if fp8:
            cref, sref = oracle.pack_fp8(np_(inp.x), ref.prefix)
            assert_equal("codes", np_(recv[0])[:N], cref)
            assert_equal("scales", np_(recv[1])[:N].view(np.uint32), sref.view(np.uint32))
        else:
            assert_equal("recv_x", np_(recv)[:N], ref.recv_x)
        assert_equal("second layout", np_(itr2), ref2.layout.is_token_in_rank)
        assert_equal("second experts", np_(nte2), ref2.layout.num_tokens_per_expert)


def test_ctx_destroyed_before_borrower_is_used(oracle):
    dev, inp, ref = _setup(oracle)
    buf = make_buffer(W.experts, W.ranks, W.channels, T)
    idx, ntr, nte, itr = _layout(buf, inp, dev)
    h = _prepare(buf, idx, ntr, nte, itr)
    other = make_buffer(W.experts, W.ranks, W.channels, T)
    C.check(C.moedx_destroy(buf.ctx))  # the ctx goes first (the Buffer object stays)
    buf.ctx = None
    recv = torch.empty(T * min(W.topk, W.ranks), W.hidden, dtype=torch.bfloat16, device=dev)
    ex = C.make_exec(torch.cuda.current_stream().cuda_stream)
    rc = C.moedx_dispatch(other.ctx, h.ptr, ctypes.c_void_p(inp.x.to(dev).data_ptr()), T,
                          W.hidden, C.MOEDX_QUANT_NONE, None, None,
                          ctypes.c_void_p(recv.data_ptr()), None, None, None, ctypes.byref(ex))
    assert rc == C.MOEDX_ESTATE
    assert "borrowed" in C.last_error()
