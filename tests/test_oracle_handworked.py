"""Oracle pin: a routing small enough to work out by hand.

The routing and every expected value live in the cited text fixture
tests/golden/handworked_t5_k2_e8_r4_c2.txt (T=5 tokens, K=2, E=8 experts in
R=4 buckets, C=2 channels), each with its derivation by counting.  The layout
outputs are the ones get_dispatch_layout returns in the GCU README's
normal-kernel example; the handle fields are those listed under "What the
Handle Contains" on the handle-reuse page.
"""

import numpy as np
import pytest

from tests.helpers import load_golden

G = load_golden("handworked_t5_k2_e8_r4_c2.txt")
TOPK = G["topk_idx"].astype(np.int64)
E, R, C = G["E"], G["R"], G["C"]


def test_layout_by_hand(oracle):
    lay = oracle.layout(TOPK, E, R)
    assert lay.num_tokens_per_expert.tolist() == G["num_tokens_per_expert"].tolist()
    assert lay.is_token_in_rank.tolist() == G["is_token_in_rank"].tolist()
    assert lay.num_tokens_per_rank.tolist() == G["num_tokens_per_rank"].tolist()


def test_handle_by_hand(oracle):
    lay = oracle.layout(TOPK, E, R)
    pre = oracle.prefix(lay.is_token_in_rank, C)
    assert pre.num_recv == G["num_recv"]
    assert pre.rank_prefix_matrix.tolist() == G["rank_prefix_matrix"].tolist()
    assert pre.channel_prefix_matrix.tolist() == G["channel_prefix_matrix"].tolist()
    assert pre.recv_channel_prefix_matrix.tolist() == G["recv_channel_prefix_matrix"].tolist()
    assert pre.recv_src_idx.tolist() == G["recv_src_idx"].tolist()
    assert pre.send_head.tolist() == G["send_head"].tolist()


def test_pack_by_hand(oracle):
    T, H = 5, 128
    x = (np.arange(T * H, dtype=np.uint32) * 7 + 0x3F00).astype(np.uint16).reshape(T, H)
    w = G["topk_weights"].astype(np.float32)
    lay = oracle.layout(TOPK, E, R)
    pre = oracle.prefix(lay.is_token_in_rank, C)
    rx, rti, rtw = oracle.pack_bf16(x, TOPK, w, E, pre)
    assert np.array_equal(rx, x[G["recv_src_idx"]])
    assert rti.tolist() == G["recv_topk_idx"].tolist()
    assert rtw.tolist() == G["recv_topk_weights"].tolist()


def test_combine_by_hand(oracle):
    T, H = 5, 128
    rng = np.random.default_rng(0)
    xf = rng.standard_normal((T, H)).astype(np.float32)
    x = (xf.view(np.uint32) >> 16).astype(np.uint16)  # any bf16 values will do
    lay = oracle.layout(TOPK, E, R)
    pre = oracle.prefix(lay.is_token_in_rank, C)
    y, _, _ = oracle.pack_bf16(x, TOPK, None, E, pre, with_topk=False)
    # Visit order: t0 rows (0,6), t1 (3), t2 (7,1), t3 (4), t4 (2,5).  With no
    # gate weights each distinct row counts once: out = |R(t)| * x[t].
    out, _ = oracle.combine(y, TOPK, E, pre)
    xv = (x.astype(np.uint32) << 16).view(np.float32)
    mult = np.array([2, 1, 2, 1, 2], np.float32)[:, None]
    expect = ((xv * mult).view(np.uint32) >> 16).astype(np.uint16)  # exact: no rounding
    assert np.array_equal(out, expect)
    # Dyadic gate weights summing to 1 per token: w(t,r) are (.75,.25), (1), (.625,.375),
    # (1), (.25,.75); every product and partial sum is exact, so out == x bit for bit.
    w = G["topk_weights"].astype(np.float32)
    out_w, _ = oracle.combine(y, TOPK, E, pre, gate_weights=w)
    assert np.array_equal(out_w, x)


def test_ll_by_hand(oracle):
    T, H, cap = 5, 128, G["ll_cap"]
    x = (np.arange(T * H, dtype=np.uint32) + 0x3000).astype(np.uint16).reshape(T, H)
    rx, cnt, src, slot = oracle.ll_dispatch(x, TOPK, E, cap)
    assert cnt.tolist() == G["ll_recv_count"].tolist()
    assert src.tolist() == G["ll_src_idx"].tolist()
    for e in range(E):
        for s_, t in enumerate(G["ll_src_idx"][e][: cnt[e]]):
            assert np.array_equal(rx[e, s_], x[t])
    assert slot.tolist() == G["ll_slot_of"].tolist()


def test_ll_capacity_overflow_raises(oracle):
    with pytest.raises(ValueError):
        oracle.ll_dispatch(None, TOPK, E, 1, hidden=0)
