"""GPU parity of the FP8 scale modes and the pre-quantised pass-through
(moedx_dispatch_fp8) against the oracle, bit for bit: power-of-two scales
(round_scale), UE8M0 exponent bytes (use_ue8m0), one per-tensor scale
(fp8_quant_scale), and (codes, scales) input dispatched unchanged."""

import numpy as np
import pytest
import torch

from combine_get_dispatch_layout_amd import workloads as wl
from tests.gpu_common import assert_equal, check_handle, device, make_buffer, np_, oracle_first_dispatch
from tests.helpers import bf16_bits

pytestmark = pytest.mark.gpu

MODES = {"pow2": dict(round_scale=True), "ue8m0": dict(use_ue8m0=True),
         "tensor": dict(fp8_quant_scale=0.0123)}


def _mode(o, name):
    return {"pow2": o.FP8_POW2, "ue8m0": o.FP8_UE8M0, "tensor": o.FP8_TENSOR}[name]


def _check(o, name, x_cpu, pre, codes, scales):
    codes_ref, scales_ref = o.pack_fp8_mode(bf16_bits(x_cpu), pre, _mode(o, name),
                                            MODES["tensor"]["fp8_quant_scale"])
    N = pre.num_recv
    assert_equal(f"{name} codes", np_(codes)[:N], codes_ref)
    if name == "tensor":
        assert scales is None
    else:
        got = np_(scales)[:N]
        assert_equal(f"{name} scales", got.view(np.uint8) if name == "ue8m0" else got.view(np.uint32),
                     scales_ref.view(np.uint8) if name == "ue8m0" else scales_ref.view(np.uint32))


@pytest.mark.parametrize("name,tokens", [("pow2", None), ("pow2", 1000), ("ue8m0", 1000),
                                         ("tensor", 1000)])
def test_fp8_modes_skewed(oracle, name, tokens):
    """The FP8 workload (8192 x 7168, Zipf routing) in full for power-of-two
    scales, and a 1000-token cut of it for every mode."""
    w = wl.FP8_SKEWED
    dev = device()
    inp = wl.make_inputs(w, tokens=tokens)
    T = inp.x.shape[0]
    print(f"[fp8 {name}] T={T}", flush=True)
    ref = oracle_first_dispatch(oracle, inp, w.experts, w.ranks, w.channels, with_rows=False)
    buf = make_buffer(w.experts, w.ranks, w.channels, T)
    (codes, scales), rti, rtw, _, h, _ = buf.dispatch(inp.x.to(dev), topk_idx=inp.topk_idx.to(dev),
                                                       **MODES[name])
    torch.cuda.synchronize()
    assert rti is None and rtw is None
    check_handle(h, ref, ref.prefix.num_recv)
    _check(oracle, name, inp.x, ref.prefix, codes, scales)
    # cached dispatch of a fresh batch with the same handle
    x2 = wl.fresh_x(w, 77, tokens=T)
    (codes2, scales2), *_ = buf.dispatch(x2.to(dev), handle=h, **MODES[name])
    _check(oracle, name, x2, ref.prefix, codes2, scales2)


@pytest.mark.parametrize("borrow", [False, True], ids=["own_layout", "borrowed_layout"])
@pytest.mark.parametrize("name", ["amax"] + sorted(MODES))
def test_first_fp8_capacity_dispatch_one_launch(oracle, name, borrow):
    """A first FP8 dispatch on a capacity-mode handle of at most 4096 tokens
    (R a multiple of 4 up to 16) finishes the handle in its own launch, for
    every scale mode: no finishing or scan kernel runs before the pack, whether
    the dispatch prepared the handle (the layout's partials only) or the handle
    borrowed the partials of the get_dispatch_layout just before it."""
    w = wl.FP8_SKEWED
    dev = device()
    inp = wl.make_inputs(w, tokens=1000)
    T, K, E, R, C = inp.x.shape[0], w.topk, w.experts, w.ranks, w.channels
    print(f"[fp8 first one launch {name}] borrow={borrow}", flush=True)
    ref = oracle_first_dispatch(oracle, inp, E, R, C, with_rows=False)
    buf = make_buffer(E, R, C, T)
    ti = inp.topk_idx.to(dev)
    reuse = {}
    if borrow:
        ntr, _, nte, itr, _ = buf.get_dispatch_layout(ti, E)
        reuse = dict(num_tokens_per_rank=ntr, is_token_in_rank=itr, num_tokens_per_expert=nte)
    before = buf.stats()
    kw = dict(fp8=True) if name == "amax" else MODES[name]
    (codes, scales), rti, rtw, _, h, _ = buf.dispatch(inp.x.to(dev), topk_idx=ti,
                                                       num_worst_tokens=T * min(K, R), **kw, **reuse)
    torch.cuda.synchronize()
    st = buf.stats()
    assert st["layout_launches"] - before["layout_launches"] == (0 if borrow else 1), st
    assert st["scan_launches"] == before["scan_launches"], st
    assert st["pack_fp8_launches"] - before["pack_fp8_launches"] == 1, st
    assert rti is None and rtw is None
    N = ref.prefix.num_recv
    check_handle(h, ref, N)
    if name == "amax":
        cref, sref = oracle.pack_fp8(bf16_bits(inp.x), ref.prefix)
        assert_equal("codes", np_(codes)[:N], cref)
        assert_equal("scales", np_(scales)[:N].view(np.uint32), sref.view(np.uint32))
    else:
        _check(oracle, name, inp.x, ref.prefix, codes, scales)


@pytest.mark.parametrize("borrow", [False, True], ids=["own_layout", "borrowed_layout"])
@pytest.mark.parametrize("fmt", ["fp32", "ue8m0", "none", "ue8m0_5_blocks"])
def test_first_prequantized_capacity_dispatch_one_launch(oracle, fmt, borrow):
    """A first pre-quantised dispatch on a capacity-mode handle of at most
    4096 tokens copies the code and scale rows and finishes the handle in one
    launch (scale rows as 4-byte words, or byte by byte for 5 UE8M0 blocks)."""
    dev = device()
    T, E, R, C, K = 1000, 64, 8, 6, 6
    H = 640 if fmt == "ue8m0_5_blocks" else 1024
    G = H // 128
    rng = np.random.default_rng(47)
    idx = wl.random_routing(rng, T, E, K, p_empty=0.05)
    codes = rng.integers(0, 256, (T, H), dtype=np.uint8)
    if fmt == "fp32":
        sc, kw = rng.standard_normal((T, G)).astype(np.float32), {}
    elif fmt == "none":
        sc, kw = None, dict(fp8_quant_scale=0.5)
    else:
        sc, kw = rng.integers(0, 256, (T, G), dtype=np.uint8), dict(use_ue8m0=True)
    inp = wl.Inputs(torch.zeros(T, H, dtype=torch.bfloat16), torch.from_numpy(idx),
                    torch.full((T, K), 1.0 / K))
    print(f"[prequant first one launch {fmt}] borrow={borrow}", flush=True)
    ref = oracle_first_dispatch(oracle, inp, E, R, C, with_rows=False)
    buf = make_buffer(E, R, C, T)
    ti = inp.topk_idx.to(dev)
    reuse = {}
    if borrow:
        ntr, _, nte, itr, _ = buf.get_dispatch_layout(ti, E)
        reuse = dict(num_tokens_per_rank=ntr, is_token_in_rank=itr, num_tokens_per_expert=nte)
    before = buf.stats()
    pair = (torch.from_numpy(codes).to(dev), torch.from_numpy(sc).to(dev) if sc is not None else None)
    (rc, rs), _, _, _, h, _ = buf.dispatch(pair, topk_idx=ti, num_worst_tokens=T * min(K, R),
                                           **kw, **reuse)
    torch.cuda.synchronize()
    st = buf.stats()
    assert st["layout_launches"] - before["layout_launches"] == (0 if borrow else 1), st
    assert st["scan_launches"] == before["scan_launches"], st
    assert st["pack_fp8_launches"] - before["pack_fp8_launches"] == 1, st
    N = ref.prefix.num_recv
    check_handle(h, ref, N)
    assert_equal("codes", np_(rc)[:N], oracle.pack_rows_bytes(codes, ref.prefix))
    if sc is None:
        assert rs is None
    else:
        got = np_(rs)[:N].view(np.uint8).reshape(N, -1)
        assert_equal("scales", got, oracle.pack_rows_bytes(sc, ref.prefix))


def _edge_x(T, H, seed):
    rng = np.random.default_rng(seed)
    x = np.asarray(rng.integers(0, 1 << 16, (T, H)), np.uint16)
    x[(x & 0x7F80) == 0x7F80] = 0x3F80
    x[0, :128] = 0                 # zero block: the 1e-4 floor
    x[1, :128] = 0x8000            # -0.0
    x[2, 128:256] = 0x0001         # bf16 denormals
    x[3, 5] = 0x7F80               # +inf
    x[4, 130] = 0xFF80             # -inf
    x[5, 300] = 0x7FC0             # NaN
    x[6, 0:128] = 0x7FC1           # NaN only
    x[7, 256:384] = 0x3F60         # 0.875 = 7 * 2^-3: an exact power-of-two quotient
    x[7, 400] = 0x7F7F             # the largest finite bf16
    return x


@pytest.mark.parametrize("name", sorted(MODES))
@pytest.mark.parametrize("capacity", [False, True])
def test_fp8_modes_edge_values(oracle, name, capacity):
    dev = device()
    T, H, E, R, C = 8, 512, 16, 4, 2
    x_u16 = _edge_x(T, H, seed=21)
    x = torch.from_numpy(x_u16.astype(np.int16)).view(torch.bfloat16)
    idx = wl.random_routing(np.random.default_rng(22), T, E, 2)
    inp = wl.Inputs(x, torch.from_numpy(idx), torch.full((T, 2), 0.5))
    ref = oracle_first_dispatch(oracle, inp, E, R, C, with_rows=False)
    buf = make_buffer(E, R, C, T)
    cap = T * 2 if capacity else 0
    print(f"[fp8 edge {name}] capacity={capacity}", flush=True)
    (codes, scales), *_ = buf.dispatch(x.to(dev), topk_idx=inp.topk_idx.to(dev),
                                       num_worst_tokens=cap, **MODES[name])
    _check(oracle, name, x, ref.prefix, codes, scales)


@pytest.mark.parametrize("name", ["pow2", "tensor"])
def test_fp8_modes_every_bf16_magnitude(oracle, name):
    """Blocks enumerating every bf16 magnitude up to 448 (block maximum 448)."""
    from tests.test_gpu_edge import _blocks_enumerating
    dev = device()
    rng = np.random.default_rng(31)
    blocks = np.concatenate([_blocks_enumerating(0x43E0, 0x43E0, rng),
                             _blocks_enumerating(0x4040, 0x4040, rng)])
    H = 1024
    per_row = H // 128
    T = -(-blocks.shape[0] // per_row)
    pad = np.tile(blocks[:1], (T * per_row - blocks.shape[0], 1))
    x_u16 = np.concatenate([blocks, pad]).reshape(T, H)
    x = torch.from_numpy(x_u16.astype(np.int16)).view(torch.bfloat16)
    idx = wl.random_routing(np.random.default_rng(32), T, 16, 2)
    inp = wl.Inputs(x, torch.from_numpy(idx), torch.full((T, 2), 0.5))
    ref = oracle_first_dispatch(oracle, inp, 16, 4, 2, with_rows=False)
    buf = make_buffer(16, 4, 2, T)
    (codes, scales), *_ = buf.dispatch(x.to(dev), topk_idx=inp.topk_idx.to(dev), **MODES[name])
    _check(oracle, name, x, ref.prefix, codes, scales)


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0", "none"])
def test_prequantized_pass_through(oracle, fmt):
    """(codes, scales) input goes unchanged to the receive rows."""
    dev = device()
    w = wl.FP8_SKEWED
    inp = wl.make_inputs(w, tokens=600)
    T, H = inp.x.shape
    rng = np.random.default_rng(41)
    codes = rng.integers(0, 256, (T, H), dtype=np.uint8)
    if fmt == "fp32":
        sc = rng.standard_normal((T, H // 128)).astype(np.float32)
        kw = {}
    elif fmt == "ue8m0":
        sc = rng.integers(0, 256, (T, H // 128), dtype=np.uint8)
        kw = dict(use_ue8m0=True)
    else:
        sc = None
        kw = dict(fp8_quant_scale=0.5)
    ref = oracle_first_dispatch(oracle, inp, w.experts, w.ranks, w.channels, with_rows=False)
    buf = make_buffer(w.experts, w.ranks, w.channels, T)
    print(f"[prequant {fmt}]", flush=True)
    pair = (torch.from_numpy(codes).to(dev), torch.from_numpy(sc).to(dev) if sc is not None else None)
    (rc, rs), *_ = buf.dispatch(pair, topk_idx=inp.topk_idx.to(dev), **kw)
    N = ref.prefix.num_recv
    assert_equal("codes", np_(rc)[:N], oracle.pack_rows_bytes(codes, ref.prefix))
    if sc is None:
        assert rs is None
    else:
        got = np_(rs)[:N].view(np.uint8).reshape(N, -1)
        assert_equal("scales", got, oracle.pack_rows_bytes(sc, ref.prefix))


@pytest.mark.parametrize("case", ["5_blocks", "unaligned"])
def test_prequantized_scale_rows_copied_bytewise(oracle, case):
    """UE8M0 scale rows whose length is not a multiple of 4 bytes (H = 640: 5
    blocks), or whose array starts off a 4-byte boundary, take the byte-wise
    copy; the result is the same pass-through."""
    dev = device()
    T, E, R, C, K = 300, 32, 4, 3, 4
    H = 640 if case == "5_blocks" else 1024
    rng = np.random.default_rng(43)
    idx = wl.random_routing(rng, T, E, K, p_empty=0.1)
    codes = rng.integers(0, 256, (T, H), dtype=np.uint8)
    G = H // 128
    sc = rng.integers(0, 256, (T, G), dtype=np.uint8)
    inp = wl.Inputs(torch.zeros(T, H, dtype=torch.bfloat16), torch.from_numpy(idx),
                    torch.full((T, K), 0.25))
    ref = oracle_first_dispatch(oracle, inp, E, R, C, with_rows=False)
    buf = make_buffer(E, R, C, T)
    if case == "unaligned":  # a view one byte into a larger allocation
        big = torch.zeros(T * G + 1, dtype=torch.uint8, device=dev)
        big[1:] = torch.from_numpy(sc.reshape(-1)).to(dev)
        sc_dev = big[1:].view(T, G)
        assert sc_dev.data_ptr() % 4 != 0
    else:
        sc_dev = torch.from_numpy(sc).to(dev)
    print(f"[prequant bytes {case}]", flush=True)
    (rc, rs), *_ = buf.dispatch((torch.from_numpy(codes).to(dev), sc_dev),
                                topk_idx=inp.topk_idx.to(dev), use_ue8m0=True)
    N = ref.prefix.num_recv
    assert_equal("codes", np_(rc)[:N], oracle.pack_rows_bytes(codes, ref.prefix))
    assert_equal("scales", np_(rs)[:N].reshape(N, -1), oracle.pack_rows_bytes(sc, ref.prefix))


def test_prequantized_equals_quantising_dispatch(oracle):
    """Quantise on the GPU, then dispatch the (codes, scales) pair: the same rows."""
    dev = device()
    w = wl.FP8_SKEWED
    inp = wl.make_inputs(w, tokens=512)
    T, H = inp.x.shape
    buf = make_buffer(w.experts, w.ranks, w.channels, T)
    idx = inp.topk_idx.to(dev)
    # one row per token: quantise through a layout where every token goes to bucket 0 once
    (c1, s1), *_ = buf.dispatch(inp.x.to(dev), topk_idx=idx, fp8=True)
    ref = oracle_first_dispatch(oracle, inp, w.experts, w.ranks, w.channels, with_rows=False)
    src = ref.prefix.recv_src_idx
    # the codes of token t are in any of its rows; take its first
    first = np.full(T, -1)
    for n in range(len(src) - 1, -1, -1):
        first[src[n]] = n
    assert (first >= 0).all()
    xc = c1[torch.from_numpy(first).to(dev)].contiguous()
    xs = s1[torch.from_numpy(first).to(dev)].contiguous()
    (c2, s2), *_ = buf.dispatch((xc, xs), topk_idx=idx)
    N = ref.prefix.num_recv
    assert_equal("codes", np_(c2)[:N], np_(c1)[:N])
    assert_equal("scales", np_(s2)[:N].view(np.uint32), np_(s1)[:N].view(np.uint32))
