"""GPU parity: layout, handle, bf16 / FP8 pack and combine against the oracle.

Every configuration runs at its full size, in the launch configuration the
benchmark uses, and every output element is compared: bit-exact for counts,
prefixes, indices, packed bf16 rows and FP8 codes and scales; within one bf16
ulp for the combine.
"""

import numpy as np
import pytest
import torch

from combine_get_dispatch_layout_amd import workloads as wl
from tests.gpu_common import (assert_bf16_within_1ulp, assert_equal, check_handle, device,
                              make_buffer, np_, oracle_first_dispatch)
from tests.helpers import bf16_bits, bits_to_f32, f32_to_bf16_torch

pytestmark = pytest.mark.gpu

NORMAL = [wl.TINY, wl.PREFILL, wl.FP8_SKEWED, wl.HANDLE_REUSE]


def _channels(w):
    return max(w.channels, 1)


@pytest.mark.parametrize("w", NORMAL + [wl.LL_DECODE], ids=lambda w: w.name)
def test_get_dispatch_layout(oracle, w):
    dev = device()
    print(f"[layout] {w.name}", flush=True)
    inp = wl.make_inputs(w)
    buf = make_buffer(w.experts, w.ranks, _channels(w), w.tokens)
    ntr, none, nte, itr, ev = buf.get_dispatch_layout(inp.topk_idx.to(dev), w.experts)
    assert none is None
    ref = oracle.layout(inp.topk_idx.numpy(), w.experts, w.ranks)
    assert_equal("num_tokens_per_rank", np_(ntr), ref.num_tokens_per_rank)
    assert_equal("num_tokens_per_expert", np_(nte), ref.num_tokens_per_expert)
    assert_equal("is_token_in_rank", np_(itr), ref.is_token_in_rank)


@pytest.mark.parametrize("w", NORMAL, ids=lambda w: w.name)
@pytest.mark.parametrize("mode", ["exact", "capacity"])
def test_first_dispatch_and_combine(oracle, w, mode):
    dev = device()
    print(f"[dispatch] {w.name} {mode}", flush=True)
    inp = wl.make_inputs(w)
    E, R, C, T, H, K = w.experts, w.ranks, _channels(w), w.tokens, w.hidden, w.topk
    ref = oracle_first_dispatch(oracle, inp, E, R, C)
    N = ref.prefix.num_recv
    buf = make_buffer(E, R, C, T)
    x, idx, gw = inp.x.to(dev), inp.topk_idx.to(dev), inp.topk_weights.to(dev)
    cap = T * min(K, R) if mode == "capacity" else 0
    out = None
    if cap:
        out = torch.full((cap, H), -7.0, dtype=torch.bfloat16, device=dev)  # sentinel rows
    recv_x, rti, rtw, per_expert, h, _ = buf.dispatch(x, topk_idx=idx, topk_weights=gw,
                                                      num_worst_tokens=cap, out=out)
    torch.cuda.synchronize()
    check_handle(h, ref, N)
    rx = np_(recv_x)
    assert_equal("recv_x", rx[:N], ref.recv_x)
    assert_equal("recv_topk_idx", np_(rti)[:N], ref.recv_topk_idx)
    assert_equal("recv_topk_weights", np_(rtw)[:N].view(np.uint32), ref.recv_topk_weights.view(np.uint32))
    if cap:
        assert (rx[N:] == bf16_bits(torch.tensor([-7.0], dtype=torch.bfloat16))[0]).all()
        assert per_expert is None
    else:
        assert rx.shape[0] == N
        assert per_expert == ref.layout.num_tokens_per_expert.tolist()

    # Combine 1: identity expert, no gate weights -> |R(t)| * x, plus the weight payload.
    comb, cw, _ = buf.combine(recv_x, h, topk_weights=rtw)
    want, want_cw = oracle.combine(ref.recv_x, inp.topk_idx.numpy(), E, ref.prefix,
                                   recv_topk_weights=ref.recv_topk_weights)
    assert_bf16_within_1ulp("combine(unweighted)", np_(comb), want)
    assert_equal("combined_topk_weights", np_(cw).view(np.uint32), want_cw.view(np.uint32))
    # Combine 2: distinct expert outputs and gate weights.
    g = torch.Generator().manual_seed(w.seed + 100)
    scale = (torch.rand(N, H, generator=g) + 0.5).to(torch.bfloat16)
    y_cpu = (inp.x[torch.from_numpy(ref.prefix.recv_src_idx).long()] * scale).to(torch.bfloat16)
    y = torch.zeros(recv_x.shape[0], H, dtype=torch.bfloat16, device=dev)
    y[:N] = y_cpu.to(dev)
    comb_w, _, _ = buf.combine(y, h, gate_weights=gw)
    want_w, _ = oracle.combine(bf16_bits(y_cpu), inp.topk_idx.numpy(), E, ref.prefix, gate_weights=inp.topk_weights.numpy())
    assert_bf16_within_1ulp("combine(weighted)", np_(comb_w), want_w)
    torch.cuda.synchronize()


@pytest.mark.parametrize("w", [wl.FP8_SKEWED, wl.TINY, wl.PREFILL], ids=lambda w: w.name)
def test_fp8_dispatch(oracle, w):
    dev = device()
    print(f"[fp8] {w.name}", flush=True)
    inp = wl.make_inputs(w)
    E, R, C, T, H, K = w.experts, w.ranks, _channels(w), w.tokens, w.hidden, w.topk
    ref = oracle_first_dispatch(oracle, inp, E, R, C, with_rows=False)
    N = ref.prefix.num_recv
    codes_ref, scales_ref = oracle.pack_fp8(bf16_bits(inp.x), ref.prefix)
    buf = make_buffer(E, R, C, T)
    x, idx = inp.x.to(dev), inp.topk_idx.to(dev)
    (codes, scales), rti, rtw, _, h, _ = buf.dispatch(x, topk_idx=idx, fp8=True)
    torch.cuda.synchronize()
    assert rti is None and rtw is None
    check_handle(h, ref, N)
    assert_equal("fp8 scales", np_(scales).view(np.uint32), scales_ref.view(np.uint32))
    assert_equal("fp8 codes", np_(codes), codes_ref)
    # Combine of the dequantised rows (the expert sees bf16(decode(code) * s)).
    deq = (torch.from_numpy(codes_ref).view(torch.float8_e4m3fn).to(torch.float32).view(N, H // 128, 128)
           * torch.from_numpy(scales_ref)[:, :, None]).view(N, H).to(torch.bfloat16)
    comb, _, _ = buf.combine(deq.to(dev), h, gate_weights=inp.topk_weights.to(dev))
    want, _ = oracle.combine(bf16_bits(deq), inp.topk_idx.numpy(), E, ref.prefix,
                             gate_weights=inp.topk_weights.numpy())
    assert_bf16_within_1ulp("combine(fp8 rows)", np_(comb), want)


def test_handle_reuse(oracle):
    """First dispatch builds the handle; ten fresh batches reuse it with no
    layout or scan launch, each followed by a weighted combine."""
    w = wl.HANDLE_REUSE
    dev = device()
    inp = wl.make_inputs(w)
    E, R, C, T, H = w.experts, w.ranks, w.channels, w.tokens, w.hidden
    ref = oracle_first_dispatch(oracle, inp, E, R, C, with_rows=False)
    buf = make_buffer(E, R, C, T)
    gw = inp.topk_weights.to(dev)
    recv0, _, _, _, h, _ = buf.dispatch(inp.x.to(dev), topk_idx=inp.topk_idx.to(dev),
                                         topk_weights=gw)
    before = buf.stats()
    for i, seed in enumerate(w.reuse_seeds):
        print(f"[reuse] seed {seed}", flush=True)
        x2 = wl.fresh_x(w, seed)
        recv, rti, rtw, per_expert, h2, _ = buf.dispatch(x2.to(dev), handle=h)
        assert h2 is h and rti is None and rtw is None and per_expert is None
        want, _, _ = oracle.pack_bf16(bf16_bits(x2), inp.topk_idx.numpy(), None, E, ref.prefix,
                                      with_topk=False)
        assert_equal(f"reuse recv_x seed {seed}", np_(recv), want)
        comb, _, _ = buf.combine(recv, h, gate_weights=gw)
        if i < 2:  # the full fp32 combine oracle is the slow part; two reps suffice
            wc, _ = oracle.combine(want, inp.topk_idx.numpy(), E, ref.prefix,
                                   gate_weights=inp.topk_weights.numpy())
            assert_bf16_within_1ulp("reuse combine", np_(comb), wc)
        else:  # softmax gates on identity rows give x back bit for bit
            assert_equal("reuse combine == x", bits_to_f32(np_(comb)), bits_to_f32(bf16_bits(x2)))
    after = buf.stats()
    assert after["layout_launches"] == before["layout_launches"]
    assert after["host_syncs"] == before["host_syncs"]
    assert after["pack_launches"] == before["pack_launches"] + len(w.reuse_seeds)


def test_reuse_equals_first_dispatch(oracle):
    w = wl.PREFILL
    dev = device()
    inp = wl.make_inputs(w, tokens=1000)
    buf = make_buffer(w.experts, w.ranks, w.channels, 1000)
    x = inp.x.to(dev)
    first, _, _, _, h, _ = buf.dispatch(x, topk_idx=inp.topk_idx.to(dev))
    again, _, _, _, _, _ = buf.dispatch(x, handle=h)
    assert torch.equal(first.view(torch.int16), again.view(torch.int16))


def test_cached_dispatch_rejects_topk(oracle):
    from combine_get_dispatch_layout_amd import _capi
    dev = device()
    w = wl.TINY
    inp = wl.make_inputs(w)
    buf = make_buffer(w.experts, w.ranks, w.channels, w.tokens)
    _, _, _, _, h, _ = buf.dispatch(inp.x.to(dev), topk_idx=inp.topk_idx.to(dev))
    import ctypes
    recv = torch.empty(h.num_recv, w.hidden, dtype=torch.bfloat16, device=dev)
    rti = torch.empty(h.num_recv, w.topk, dtype=torch.int64, device=dev)
    rc = _capi.moedx_dispatch(buf.ctx, h.ptr, ctypes.c_void_p(inp.x.to(dev).data_ptr()), w.tokens,
                              w.hidden, 0, None, None, ctypes.c_void_p(recv.data_ptr()), None,
                              ctypes.c_void_p(rti.data_ptr()), None, None)
    assert rc == _capi.MOEDX_EINVAL
    # a handle for another T is refused
    rc = _capi.moedx_dispatch(buf.ctx, h.ptr, ctypes.c_void_p(recv.data_ptr()), w.tokens - 1,
                              w.hidden, 0, None, None, ctypes.c_void_p(recv.data_ptr()), None,
                              None, None, None)
    assert rc == _capi.MOEDX_ESTATE


@pytest.mark.parametrize("w,tokens", [(wl.TINY, None), (wl.PREFILL, 1000)],
                         ids=["tiny", "prefill-1000"])
def test_training_pairings(oracle, w, tokens):
    """The four functions of the normal-kernel example: dispatch_forward,
    combine_forward, and their backward pairings -- combine_backward is a cached
    dispatch of the output gradient, dispatch_backward a combine of the row
    gradients that also reduces the gradient of recv_topk_weights."""
    dev = device()
    inp = wl.make_inputs(w, tokens=tokens)
    T, H, K = inp.x.shape[0], w.hidden, w.topk
    E, R, C = w.experts, w.ranks, _channels(w)
    ref = oracle_first_dispatch(oracle, inp, E, R, C, with_rows=False)
    N = ref.prefix.num_recv
    buf = make_buffer(E, R, C, T)
    print(f"[pairings] {w.name} T={T}", flush=True)
    # dispatch_forward
    recv_x, rti, rtw, _, h, _ = buf.dispatch(inp.x.to(dev), topk_idx=inp.topk_idx.to(dev),
                                             topk_weights=inp.topk_weights.to(dev))
    rx_ref, rti_ref, rtw_ref = oracle.pack_bf16(bf16_bits(inp.x), inp.topk_idx.numpy(),
                                                inp.topk_weights.numpy(), E, ref.prefix)
    assert_equal("recv_x", np_(recv_x), rx_ref)
    assert_equal("recv_topk_idx", np_(rti), rti_ref)
    assert_equal("recv_topk_weights", np_(rtw).view(np.uint32), rtw_ref.view(np.uint32))
    g = torch.Generator().manual_seed(9)
    # combine_forward of expert outputs y (unweighted reduction of the rows)
    y = torch.randn(N, H, generator=g).to(torch.bfloat16)
    comb, cw, _ = buf.combine(y.to(dev), h)
    want, _ = oracle.combine(bf16_bits(y), inp.topk_idx.numpy(), E, ref.prefix)
    assert cw is None
    assert_bf16_within_1ulp("combine_forward", np_(comb), want)
    # combine_backward: the output gradient goes to every row like x did
    grad_out = torch.randn(T, H, generator=g).to(torch.bfloat16)
    grad_rows, g_rti, g_rtw, _, _, _ = buf.dispatch(grad_out.to(dev), handle=h)
    assert g_rti is None and g_rtw is None
    want_rows, _, _ = oracle.pack_bf16(bf16_bits(grad_out), inp.topk_idx.numpy(), None, E,
                                       ref.prefix, with_topk=False)
    assert_equal("combine_backward", np_(grad_rows), want_rows)
    # dispatch_backward: row gradients and the gradient of recv_topk_weights
    grad_recv = torch.randn(N, H, generator=g).to(torch.bfloat16)
    grad_rtw = torch.randn(N, K, generator=g)
    gx, gw, _ = buf.combine(grad_recv.to(dev), h, topk_weights=grad_rtw.to(dev))
    want_x, want_w = oracle.combine(bf16_bits(grad_recv), inp.topk_idx.numpy(), E, ref.prefix,
                                    recv_topk_weights=grad_rtw.numpy())
    assert_bf16_within_1ulp("dispatch_backward x", np_(gx), want_x)
    assert_equal("dispatch_backward weights", np_(gw).view(np.uint32), want_w.view(np.uint32))


@pytest.mark.parametrize("w", [wl.TINY, wl.PREFILL], ids=lambda w: w.name)
def test_capacity_handle_finished_before_first_use(oracle, w):
    """A capacity-mode handle read before any dispatch: the explicit finish
    writes its prefixes, totals and N (once; a second finish runs nothing),
    and the first dispatch that follows packs from those prefixes."""
    dev = device()
    print(f"[finish] {w.name}", flush=True)
    inp = wl.make_inputs(w)
    E, R, C, T, K = w.experts, w.ranks, _channels(w), w.tokens, w.topk
    ref = oracle_first_dispatch(oracle, inp, E, R, C)
    N = ref.prefix.num_recv
    buf = make_buffer(E, R, C, T)
    h, _ = buf.prepare(inp.topk_idx.to(dev), T * min(K, R))
    before = buf.stats()
    h.finish()
    h.finish()
    f = h.fields()
    torch.cuda.synchronize()
    assert buf.stats()["layout_launches"] == before["layout_launches"] + 1
    assert_equal("num_tokens_per_rank", np_(f["num_tokens_per_rank"]), ref.layout.num_tokens_per_rank)
    assert_equal("num_tokens_per_expert", np_(f["num_tokens_per_expert"]),
                 ref.layout.num_tokens_per_expert)
    assert_equal("rank_prefix_matrix", np_(f["rank_prefix_matrix"]), ref.prefix.rank_prefix_matrix)
    assert_equal("channel_prefix_matrix", np_(f["channel_prefix_matrix"]),
                 ref.prefix.channel_prefix_matrix)
    assert_equal("recv_channel_prefix_matrix", np_(f["recv_channel_prefix_matrix"]),
                 ref.prefix.recv_channel_prefix_matrix)
    assert int(np_(f["num_recv"])[0]) == N
    recv, _, _, _, h2, _ = buf.dispatch(inp.x.to(dev), handle=h)
    torch.cuda.synchronize()
    assert h2 is h
    assert buf.stats()["layout_launches"] == before["layout_launches"] + 1
    check_handle(h, ref, N)
    assert_equal("recv_x", np_(recv)[:N], ref.recv_x)


@pytest.mark.parametrize("w", NORMAL, ids=lambda w: w.name)
@pytest.mark.parametrize("mode", ["exact", "capacity"])
def test_layout_then_dispatch_and_combine(oracle, w, mode):
    """The normal-kernel example's call order at full size: get_dispatch_layout,
    then dispatch given its num_tokens_per_rank / is_token_in_rank /
    num_tokens_per_expert, then the gate-weighted combine.  The layout runs
    once: the dispatch scans its handle from the given outputs."""
    dev = device()
    print(f"[layout->dispatch] {w.name} {mode}", flush=True)
    inp = wl.make_inputs(w)
    E, R, C, T, H, K = w.experts, w.ranks, _channels(w), w.tokens, w.hidden, w.topk
    ref = oracle_first_dispatch(oracle, inp, E, R, C)
    N = ref.prefix.num_recv
    buf = make_buffer(E, R, C, T)
    x, idx, gw = inp.x.to(dev), inp.topk_idx.to(dev), inp.topk_weights.to(dev)
    ntr, _, nte, itr, _ = buf.get_dispatch_layout(idx, E)
    cap = T * min(K, R) if mode == "capacity" else 0
    recv_x, rti, rtw, per_expert, h, _ = buf.dispatch(
        x, topk_idx=idx, topk_weights=gw, num_tokens_per_rank=ntr, is_token_in_rank=itr,
        num_tokens_per_expert=nte, num_worst_tokens=cap)
    comb, _, _ = buf.combine(recv_x, h, gate_weights=gw)
    torch.cuda.synchronize()
    st = buf.stats()
    # capacity mode with a one-launch first pack (T <= 4096, R a multiple of 4
    # up to 16): the handle borrows the layout's partials and no scan runs
    borrowed = bool(cap) and T <= 4096 and R % 4 == 0 and R <= 16
    assert st["layout_launches"] == 1 and st["scan_launches"] == (0 if borrowed else 1), st
    assert st["pack_launches"] == 1 and st["combine_launches"] == 1, st
    check_handle(h, ref, N)
    assert_equal("recv_x", np_(recv_x)[:N], ref.recv_x)
    assert_equal("recv_topk_idx", np_(rti)[:N], ref.recv_topk_idx)
    assert_equal("recv_topk_weights", np_(rtw)[:N].view(np.uint32),
                 ref.recv_topk_weights.view(np.uint32))
    if not cap:
        assert per_expert == ref.layout.num_tokens_per_expert.tolist()
    # softmax gates over identity rows give x back bit for bit (a closed form
    # of the weighted combine; the oracle's combine is pinned to it)
    want, _ = oracle.combine(ref.recv_x, inp.topk_idx.numpy(), E, ref.prefix,
                             gate_weights=inp.topk_weights.numpy())
    assert_bf16_within_1ulp("combine", np_(comb), want)


def test_layout_concurrent_with_first_dispatch(oracle):
    """One ctx, two streams: get_dispatch_layout runs on one while a first
    capacity-mode dispatch (whose pack finishes its handle) and a combine of
    another handle run on the other; then a third layout.  Only the layout
    launches count tickets, so none of them is disturbed."""
    dev = device()
    w = wl.PREFILL
    inp = wl.make_inputs(w, tokens=4096)
    inp2 = wl.make_inputs(w, seed=31, tokens=4096)
    E, R, C, T, K = w.experts, w.ranks, w.channels, 4096, w.topk
    ref = oracle_first_dispatch(oracle, inp, E, R, C)
    ref2 = oracle.layout(inp2.topk_idx.numpy(), E, R)
    buf = make_buffer(E, R, C, T)
    x, idx, gw = inp.x.to(dev), inp.topk_idx.to(dev), inp.topk_weights.to(dev)
    idx2 = inp2.topk_idx.to(dev)
    cap = T * min(K, R)
    h, _ = buf.prepare(idx, cap)  # partials only: the first pack finishes it
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(3):
        print(f"[concurrent] rep {rep}", flush=True)
        with torch.cuda.stream(s1):
            ntr, _, nte, itr, _ = buf.get_dispatch_layout(idx2, E, async_finish=True)
        with torch.cuda.stream(s2):
            if rep == 0:
                recv, _, _, _, _, _ = buf.dispatch(x, handle=h, no_sync=True)
                comb, _, _ = buf.combine(recv, h, gate_weights=gw, no_sync=True)
        torch.cuda.synchronize()
        outs.append((np_(ntr), np_(nte), np_(itr)))
        if rep == 0:
            check_handle(h, ref, ref.prefix.num_recv)
            assert_equal("recv_x", np_(recv)[:ref.prefix.num_recv], ref.recv_x)
    for ntr_, nte_, itr_ in outs:
        assert_equal("num_tokens_per_rank", ntr_, ref2.num_tokens_per_rank)
        assert_equal("num_tokens_per_expert", nte_, ref2.num_tokens_per_expert)
        assert_equal("is_token_in_rank", itr_, ref2.is_token_in_rank)
