"""GPU parity of the low-latency pair: per-expert slot layout, counts, source
indices, slot-of map, packed slots and the weighted combine."""

import numpy as np
import pytest
import torch

from combine_get_dispatch_layout_amd import workloads as wl
from tests.gpu_common import assert_bf16_within_1ulp, assert_equal, device, make_buffer, np_
from tests.helpers import bf16_bits, bits_to_f32, f32_to_bf16_torch

pytestmark = pytest.mark.gpu


def run_ll(o, x: torch.Tensor, idx: np.ndarray, w: torch.Tensor, E: int, R: int, cap: int):
    dev = device()
    T, H = x.shape
    K = idx.shape[1]
    print(f"[ll] T={T} K={K} H={H} E={E} cap={cap}", flush=True)
    buf = make_buffer(E, R, 1, max(T, 1))
    rx_ref, cnt_ref, src_ref, slot_ref = o.ll_dispatch(bf16_bits(x), idx, E, cap)
    ti = torch.from_numpy(idx).to(dev)
    recv_x, cnt, h, ev, hook = buf.low_latency_dispatch(x.to(dev), ti, cap, E)
    assert hook is None
    torch.cuda.synchronize()
    assert_equal("recv_count", np_(cnt), cnt_ref)
    f = h.fields()
    src = np_(f["src_idx"])
    for e in range(E):
        n = cnt_ref[e]
        assert_equal(f"src_idx[{e}]", src[e, :n], src_ref[e, :n])
    assert_equal("slot_of", np_(f["slot_of"]), slot_ref)
    rx = np_(recv_x)
    for e in range(E):
        n = cnt_ref[e]
        if n:
            assert_equal(f"recv_x[{e}]", rx[e, :n], rx_ref[e, :n])
    # weighted combine of the slots as they came back
    comb, ev2, hook2 = buf.low_latency_combine(recv_x, ti, w.to(dev), h)
    assert hook2 is None
    want = o.ll_combine(rx, idx, w.numpy(), slot_ref)
    assert_bf16_within_1ulp("ll_combine", np_(comb), want)
    ones = torch.ones_like(w)
    comb1, _, _ = buf.low_latency_combine(recv_x, ti, ones.to(dev), h)
    kv = (idx >= 0).sum(1).astype(np.float32)[:, None]
    assert_equal("ll_combine(unit)", np_(comb1), f32_to_bf16_torch(bits_to_f32(bf16_bits(x)) * kv))
    return buf


def test_ll_decode_config(oracle):
    w = wl.LL_DECODE
    inp = wl.make_inputs(w)
    run_ll(oracle, inp.x, inp.topk_idx.numpy(), inp.topk_weights, w.experts, w.ranks, w.ll_capacity)


# Up to 4096 tokens: each token's slot counts every earlier entry (24 counting
# passes of 1024 entries at 4096 x 6), so the larger batches check the
# multi-pass count and the slot order far past the decode sizes.
@pytest.mark.parametrize("T,cap,p_empty", [(1, 4, 0.0), (64, 64, 0.0), (100, 256, 0.3), (37, 40, 0.0),
                                           (256, 256, 0.0), (1000, 1024, 0.1), (4096, 4096, 0.0)])
def test_ll_shapes(oracle, T, cap, p_empty):
    E, K, H = 32, 6, 512
    idx = wl.random_routing(np.random.default_rng(T), T, E, K, p_empty)
    g = torch.Generator().manual_seed(T)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    w = torch.softmax(torch.randn(T, K, generator=g, dtype=torch.float64), -1).to(torch.float32)
    run_ll(oracle, x, idx, w, E, 8, cap)


def test_ll_empty_batch(oracle):
    dev = device()
    buf = make_buffer(16, 4, 1, 8)
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    idx = torch.empty(0, 2, dtype=torch.int64, device=dev)
    recv_x, cnt, h, _, _ = buf.low_latency_dispatch(x, idx, 8, 16)
    assert np_(cnt).tolist() == [0] * 16


def test_ll_capacity_check():
    from combine_get_dispatch_layout_amd import _capi
    dev = device()
    buf = make_buffer(16, 4, 1, 64)
    x = torch.zeros(10, 64, dtype=torch.bfloat16, device=dev)
    idx = torch.zeros(10, 2, dtype=torch.int64, device=dev)
    with pytest.raises(_capi.MoedxError) as ei:
        buf.low_latency_dispatch(x, idx, 8, 16)  # T = 10 > cap = 8
    assert ei.value.code == _capi.MOEDX_ECAPACITY


def _ll_case(seed=5, T=96, E=64, K=6, H=1024, cap=128):
    idx = wl.random_routing(np.random.default_rng(seed), T, E, K, 0.1)
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    w = torch.softmax(torch.randn(T, K, generator=g), -1)
    return idx, x, w, E, cap


def _check_slots(o, recv_x, cnt, x, idx, E, cap):
    rx_ref, cnt_ref, _, _ = o.ll_dispatch(bf16_bits(x), idx, E, cap)
    assert_equal("recv_count", np_(cnt), cnt_ref)
    rx = np_(recv_x)
    for e in range(E):
        n = cnt_ref[e]
        if n:
            assert_equal(f"recv_x[{e}]", rx[e, :n], rx_ref[e, :n])
    return rx


def test_ll_receive_hooks(oracle):
    """return_recv_hook: the dispatch fills counts and the handle, the rows come
    with hook(); the combine's reduction runs in its hook."""
    dev = device()
    idx, x, w, E, cap = _ll_case()
    T, H = x.shape
    buf = make_buffer(E, 8, 1, T)
    ti = torch.from_numpy(idx).to(dev)
    recv_x, cnt, h, ev, hook = buf.low_latency_dispatch(x.to(dev), ti, cap, E,
                                                        return_recv_hook=True)
    assert callable(hook)
    torch.cuda.synchronize()
    _, cnt_ref, _, slot_ref = oracle.ll_dispatch(bf16_bits(x), idx, E, cap)
    assert_equal("recv_count before hook", np_(cnt), cnt_ref)
    assert_equal("slot_of before hook", np_(h.fields()["slot_of"]), slot_ref)
    recv_x.zero_()
    torch.cuda.synchronize()
    assert not np_(recv_x).any(), "rows arrived before the hook"
    hook()
    rx = _check_slots(oracle, recv_x, cnt, x, idx, E, cap)
    comb, ev2, hook2 = buf.low_latency_combine(recv_x, ti, w.to(dev), h, return_recv_hook=True)
    assert callable(hook2)
    hook2()
    assert_bf16_within_1ulp("ll_combine via hook", np_(comb),
                            oracle.ll_combine(rx, idx, w.numpy(), slot_ref))


def test_ll_hip_graph_replays(oracle):
    """The low-latency pair captured in a HIP graph (no host synchronisation, no
    memset nodes) and replayed three times on fresh inputs, with eager work of
    the same library between replays; every replay matches the oracle."""
    dev = device()
    idx, x, w, E, cap = _ll_case(seed=6)
    T, H = x.shape
    buf = make_buffer(E, 8, 1, T)
    other = make_buffer(E, 8, 1, T)
    ti = torch.from_numpy(idx).to(dev)
    x_static = x.to(dev)
    w_static = w.to(dev)
    # warm the allocator and the library outside the capture
    buf.low_latency_dispatch(x_static, ti, cap, E, no_sync=True)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            recv_x, cnt, h, _, _ = buf.low_latency_dispatch(x_static, ti, cap, E, no_sync=True)
            comb, _, _ = buf.low_latency_combine(recv_x, ti, w_static, h, no_sync=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    _, _, _, slot_ref = oracle.ll_dispatch(bf16_bits(x), idx, E, cap)
    for rep in range(3):
        g = torch.Generator().manual_seed(100 + rep)
        x_new = torch.randn(T, H, generator=g).to(torch.bfloat16)
        x_static.copy_(x_new.to(dev))
        print(f"[graph] replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        rx = _check_slots(oracle, recv_x, cnt, x_new, idx, E, cap)
        assert_bf16_within_1ulp(f"graph ll_combine {rep}", np_(comb),
                                oracle.ll_combine(rx, idx, w.numpy(), slot_ref))
        # eager work of the library between replays
        rx2, cnt2, _, _, _ = other.low_latency_dispatch(x_new.to(dev), ti, cap, E)
        _check_slots(oracle, rx2, cnt2, x_new, idx, E, cap)
