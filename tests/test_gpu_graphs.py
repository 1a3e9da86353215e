"""The normal path under HIP graphs and on concurrent streams.

A capacity-mode first dispatch (layout with every prefix, pack with the
handle rows and recv_topk_*, gate-weighted combine) needs no host
synchronisation and records no memset, so it can be captured once and
replayed with new routing and new rows each time; so can get_dispatch_layout
followed by a dispatch that borrows its partials, the allocation-free layout,
and a first and a cached FP8 dispatch.  Two contexts on two streams at once must not share any scratch memory.  Every result is compared
with the oracle: bit-exact for the handle and rows, within one bf16 ulp for
the combine.
"""

import numpy as np
import pytest
import torch

from combine_get_dispatch_layout_amd import workloads as wl
from tests.gpu_common import (assert_bf16_within_1ulp, assert_equal, check_handle, device,
                              make_buffer, np_, oracle_first_dispatch)
from tests.helpers import bf16_bits

pytestmark = pytest.mark.gpu

E, R, C, K = 64, 8, 8, 6


def _inputs(seed, T, H):
    rng = np.random.default_rng(seed)
    idx = wl.random_routing(rng, T, E, K, p_empty=0.05)
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    w = torch.softmax(torch.randn(T, K, generator=g), -1)
    return wl.Inputs(x=x, topk_idx=torch.from_numpy(idx), topk_weights=w)


def _check(oracle, inp, h, recv, rti, rtw, out):
    ref = oracle_first_dispatch(oracle, inp, E, R, C)
    N = ref.prefix.num_recv
    check_handle(h, ref, N)
    assert_equal("recv_x", np_(recv)[:N], ref.recv_x)
    assert_equal("recv_topk_idx", np_(rti)[:N], ref.recv_topk_idx)
    assert_equal("recv_topk_weights", np_(rtw)[:N].view(np.uint32),
                 ref.recv_topk_weights.view(np.uint32))
    want, _ = oracle.combine(ref.recv_x, inp.topk_idx.numpy(), E, ref.prefix,
                             gate_weights=inp.topk_weights.numpy())
    assert_bf16_within_1ulp("combine", np_(out), want)


def test_first_dispatch_hip_graph_replays(oracle):
    """Layout + pack + combine captured once; each replay sees new routing and
    new rows, with eager calls of another context between replays."""
    dev = device()
    T, H = 1000, 2048  # ragged: 3 full layout tiles and a short one; 16 row parts
    cap = T * min(K, R)
    buf = make_buffer(E, R, C, T)
    other = make_buffer(E, R, C, T)
    first = _inputs(11, T, H)
    x_s, idx_s, w_s = first.x.to(dev), first.topk_idx.to(dev), first.topk_weights.to(dev)
    # warm the allocator and the library outside the capture
    buf.dispatch(x_s, topk_idx=idx_s, topk_weights=w_s, num_worst_tokens=cap, no_sync=True)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            recv, rti, rtw, _, h, _ = buf.dispatch(x_s, topk_idx=idx_s, topk_weights=w_s,
                                                   num_worst_tokens=cap, no_sync=True)
            out, _, _ = buf.combine(recv, h, gate_weights=w_s, no_sync=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        inp = _inputs(200 + rep, T, H)
        x_s.copy_(inp.x.to(dev))
        idx_s.copy_(inp.topk_idx.to(dev))
        w_s.copy_(inp.topk_weights.to(dev))
        print(f"[graph] first dispatch replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        _check(oracle, inp, h, recv, rti, rtw, out)
        # eager work of another context between replays
        r2, i2, w2, _, h2, _ = other.dispatch(x_s, topk_idx=idx_s, topk_weights=w_s,
                                              num_worst_tokens=cap)
        o2, _, _ = other.combine(r2, h2, gate_weights=w_s)
        _check(oracle, inp, h2, r2, i2, w2, o2)


def test_cached_dispatch_hip_graph_replays(oracle):
    """A cached dispatch and its combine captured once and replayed on new rows."""
    dev = device()
    T, H = 777, 1024
    buf = make_buffer(E, R, C, T)
    inp = _inputs(21, T, H)
    idx, w = inp.topk_idx.to(dev), inp.topk_weights.to(dev)
    _, _, _, _, h, _ = buf.dispatch(inp.x.to(dev), topk_idx=idx, topk_weights=w)
    ref = oracle_first_dispatch(oracle, inp, E, R, C, with_rows=False)
    N = ref.prefix.num_recv
    x_s = inp.x.to(dev)
    buf.dispatch(x_s, handle=h, no_sync=True)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            recv, _, _, _, _, _ = buf.dispatch(x_s, handle=h, no_sync=True)
            out, _, _ = buf.combine(recv, h, gate_weights=w, no_sync=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    src = ref.prefix.recv_src_idx
    for rep in range(3):
        g = torch.Generator().manual_seed(300 + rep)
        x_new = torch.randn(T, H, generator=g).to(torch.bfloat16)
        x_s.copy_(x_new.to(dev))
        print(f"[graph] cached dispatch replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        xb = bf16_bits(x_new)
        assert recv.shape[0] == N
        assert_equal("recv_x", np_(recv), xb[src])
        want, _ = oracle.combine(xb[src], inp.topk_idx.numpy(), E, ref.prefix,
                                 gate_weights=inp.topk_weights.numpy())
        assert_bf16_within_1ulp("combine", np_(out), want)


def test_two_contexts_on_concurrent_streams(oracle):
    """Two contexts, each on its own stream, run whole steps at the same time."""
    dev = device()
    T, H = 2048, 1536
    cap = T * min(K, R)
    bufs = [make_buffer(E, R, C, T) for _ in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    inps = [_inputs(40 + i, T, H) for i in range(2)]
    dev_in = [(i.x.to(dev), i.topk_idx.to(dev), i.topk_weights.to(dev)) for i in inps]
    torch.cuda.synchronize()
    results = []
    for rep in range(3):
        outs = []
        for b, st, (x, idx, w) in zip(bufs, streams, dev_in):
            with torch.cuda.stream(st):
                recv, rti, rtw, _, h, _ = b.dispatch(x, topk_idx=idx, topk_weights=w,
                                                     num_worst_tokens=cap, no_sync=True)
                out, _, _ = b.combine(recv, h, gate_weights=w, no_sync=True)
                outs.append((h, recv, rti, rtw, out))
        results.append(outs)
    torch.cuda.synchronize()
    for rep, outs in enumerate(results):
        for inp, (h, recv, rti, rtw, out) in zip(inps, outs):
            print(f"[streams] rep {rep}", flush=True)
            _check(oracle, inp, h, recv, rti, rtw, out)


def test_release_inside_capture_is_deferred(oracle):
    """A context and an event released while a stream is capturing (here by
    the garbage collector, as happens when an old Buffer is collected during
    someone else's capture) are destroyed after the capture ends; the graph
    recorded meanwhile stays valid and replays correctly."""
    import gc

    from combine_get_dispatch_layout_amd import buffer as bm

    dev = device()
    T, H = 300, 512
    cap = T * min(K, R)
    buf = make_buffer(E, R, C, T)
    doomed = make_buffer(E, R, C, T)
    first = _inputs(21, T, H)
    x_s, idx_s, w_s = first.x.to(dev), first.topk_idx.to(dev), first.topk_weights.to(dev)
    _, _, _, _, _, ev = doomed.dispatch(x_s, topk_idx=idx_s, topk_weights=w_s,
                                        num_worst_tokens=cap, async_finish=True)
    ev.synchronize()
    buf.dispatch(x_s, topk_idx=idx_s, topk_weights=w_s, num_worst_tokens=cap, no_sync=True)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            recv, rti, rtw, _, h, _ = buf.dispatch(x_s, topk_idx=idx_s, topk_weights=w_s,
                                                   num_worst_tokens=cap, no_sync=True)
            del doomed, ev
            gc.collect()
            assert len(bm._deferred) >= 2, "ctx and event release not deferred"
            out, _, _ = buf.combine(recv, h, gate_weights=w_s, no_sync=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(2):
        inp = _inputs(22 + rep, T, H)
        x_s.copy_(inp.x.to(dev))
        idx_s.copy_(inp.topk_idx.to(dev))
        w_s.copy_(inp.topk_weights.to(dev))
        print(f"[graph] release-in-capture replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        _check(oracle, inp, h, recv, rti, rtw, out)
        # the next call outside a capture performs the queued releases
        buf.get_dispatch_layout(idx_s, E)
        assert not bm._deferred


def test_layout_then_dispatch_hip_graph_replays(oracle):
    """The normal-mode call order captured once: get_dispatch_layout, the first
    dispatch given its outputs (the handle borrows the layout's partials, so
    the captured pack reads what the captured layout writes), the combine;
    replayed on new routing and rows, with eager layouts of the same ctx
    between replays."""
    dev = device()
    T, H = 1000, 2048
    cap = T * min(K, R)
    buf = make_buffer(E, R, C, T)
    first = _inputs(12, T, H)
    x_s, idx_s, w_s = first.x.to(dev), first.topk_idx.to(dev), first.topk_weights.to(dev)

    def step():
        ntr, _, nte, itr, _ = buf.get_dispatch_layout(idx_s, E, no_sync=True)
        recv, rti, rtw, _, h, _ = buf.dispatch(
            x_s, topk_idx=idx_s, topk_weights=w_s, num_tokens_per_rank=ntr, is_token_in_rank=itr,
            num_tokens_per_expert=nte, num_worst_tokens=cap, no_sync=True)
        out, _, _ = buf.combine(recv, h, gate_weights=w_s, no_sync=True)
        return recv, rti, rtw, h, out

    step()  # warm the allocator and the library outside the capture
    torch.cuda.synchronize()
    scans = buf.stats()["scan_launches"]
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            recv, rti, rtw, h, out = step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert buf.stats()["scan_launches"] == scans  # the captured dispatch borrowed
    for rep in range(3):
        inp = _inputs(300 + rep, T, H)
        x_s.copy_(inp.x.to(dev))
        idx_s.copy_(inp.topk_idx.to(dev))
        w_s.copy_(inp.topk_weights.to(dev))
        print(f"[graph] layout -> dispatch replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        _check(oracle, inp, h, recv, rti, rtw, out)
        # an eager layout of the same ctx between replays (it rewrites the
        # scratch the captured pack reads; the next replay's layout rewrites it again)
        other = _inputs(400 + rep, T, H)
        ntr2, _, nte2, itr2, _ = buf.get_dispatch_layout(other.topk_idx.to(dev), E)
        ref2 = oracle.layout(other.topk_idx.numpy(), E, R)
        assert_equal("eager layout", np_(itr2), ref2.is_token_in_rank)


def test_static_layout_hip_graph_replays(oracle):
    """The allocation-free get_dispatch_layout captured in a graph (what it is
    for) and replayed on new routing, with eager calls between replays."""
    import ctypes

    from combine_get_dispatch_layout_amd import _capi as Cc

    dev = device()
    T = 3001
    ntr = torch.empty(R, dtype=torch.int32, device=dev)
    nte = torch.empty(E, dtype=torch.int32, device=dev)
    itr = torch.empty(T, R, dtype=torch.uint8, device=dev)
    idx_s = torch.from_numpy(wl.random_routing(np.random.default_rng(5), T, E, K)).to(dev)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def call(idx, a, b, c, stream):
        Cc.check(Cc.moedx_get_dispatch_layout_static(P(idx), T, K, E, R, P(a), P(b), P(c),
                                                     ctypes.c_void_p(stream.cuda_stream)))

    call(idx_s, ntr, nte, itr, torch.cuda.current_stream())  # first call on the device: eager
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            call(idx_s, ntr, nte, itr, s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        idx = wl.random_routing(np.random.default_rng(60 + rep), T, E, K, p_empty=0.05)
        idx_s.copy_(torch.from_numpy(idx).to(dev))
        print(f"[graph] static layout replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle.layout(idx, E, R)
        assert_equal("num_tokens_per_rank", np_(ntr), ref.num_tokens_per_rank)
        assert_equal("num_tokens_per_expert", np_(nte), ref.num_tokens_per_expert)
        assert_equal("is_token_in_rank", np_(itr), ref.is_token_in_rank)
        # an eager call between replays shares the static counters
        e_ntr = torch.empty_like(ntr)
        e_nte = torch.empty_like(nte)
        e_itr = torch.empty_like(itr)
        call(idx_s, e_ntr, e_nte, e_itr, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert_equal("eager experts", np_(e_nte), ref.num_tokens_per_expert)


def test_fp8_dispatch_hip_graph_replays(oracle):
    """A capacity-mode FP8 first dispatch (the layout with every prefix, then
    the FP8 pack, which runs with LDS reserved to cap its occupancy) and a
    cached FP8 dispatch of another batch of rows through the same handle,
    captured once and replayed on new routing and rows."""
    dev = device()
    T, H = 1000, 1024  # 8 blocks of 1x128 per row
    cap = T * min(K, R)
    buf = make_buffer(E, R, C, T)
    first = _inputs(31, T, H)
    x_s, idx_s = first.x.to(dev), first.topk_idx.to(dev)
    x2_s = first.x.to(dev)
    buf.dispatch(x_s, topk_idx=idx_s, fp8=True, num_worst_tokens=cap, no_sync=True)  # warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            (codes, scales), _, _, _, h, _ = buf.dispatch(x_s, topk_idx=idx_s, fp8=True,
                                                          num_worst_tokens=cap, no_sync=True)
            (codes2, scales2), _, _, _, _, _ = buf.dispatch(x2_s, handle=h, fp8=True, no_sync=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        inp = _inputs(500 + rep, T, H)
        g = torch.Generator().manual_seed(600 + rep)
        x2 = (torch.randn(T, H, generator=g) * 3).to(torch.bfloat16)
        x_s.copy_(inp.x.to(dev))
        idx_s.copy_(inp.topk_idx.to(dev))
        x2_s.copy_(x2.to(dev))
        print(f"[graph] FP8 dispatch replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle_first_dispatch(oracle, inp, E, R, C, with_rows=False)
        N = ref.prefix.num_recv
        check_handle(h, ref, N)
        for name, (c_, s_), xb in (("first", (codes, scales), bf16_bits(inp.x)),
                                   ("cached", (codes2, scales2), bf16_bits(x2))):
            cref, sref = oracle.pack_fp8(xb, ref.prefix)
            assert_equal(f"{name} codes", np_(c_)[:N], cref)
            assert_equal(f"{name} scales", np_(s_)[:N].view(np.uint32), sref.view(np.uint32))
