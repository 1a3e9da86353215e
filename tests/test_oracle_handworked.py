"""Oracle pin: a routing small enough to work out by hand.

T=5 tokens, K=2, E=8 experts, R=4 buckets (P=2 experts each: bucket r holds
experts 2r and 2r+1), C=2 channels (per = ceil(5/2) = 3: channel 0 = tokens
0..2, channel 1 = tokens 3..4).

    topk_idx = [[1,6],[2,3],[7,0],[4,5],[0,4]]

Buckets per token (expert // 2): t0 {0,3}, t1 {1} (both experts in bucket 1),
t2 {3,0}, t3 {2}, t4 {0,2}.  Every expected value below is derived from that
line by counting, in the comments next to it.  The layout outputs are the ones
get_dispatch_layout returns in the GCU README's normal-kernel example; the
handle fields are those listed under "What the Handle Contains" on the
handle-reuse page.
"""

import numpy as np
import pytest

TOPK = np.array([[1, 6], [2, 3], [7, 0], [4, 5], [0, 4]], dtype=np.int64)
E, R, C = 8, 4, 2


def test_layout_by_hand(oracle):
    lay = oracle.layout(TOPK, E, R)
    # experts 0 (t2,t4) and 4 (t3,t4) are chosen twice, every other once
    assert lay.num_tokens_per_expert.tolist() == [2, 1, 1, 1, 2, 1, 1, 1]
    assert lay.is_token_in_rank.tolist() == [
        [1, 0, 0, 1],  # t0: buckets 0, 3
        [0, 1, 0, 0],  # t1: bucket 1
        [1, 0, 0, 1],  # t2: buckets 3, 0
        [0, 0, 1, 0],  # t3: bucket 2
        [1, 0, 1, 0],  # t4: buckets 0, 2
    ]
    # bucket 0: t0,t2,t4; bucket 1: t1; bucket 2: t3,t4; bucket 3: t0,t2
    assert lay.num_tokens_per_rank.tolist() == [3, 1, 2, 2]


def test_handle_by_hand(oracle):
    lay = oracle.layout(TOPK, E, R)
    pre = oracle.prefix(lay.is_token_in_rank, C)
    assert pre.num_recv == 8  # 3 + 1 + 2 + 2 receive rows
    assert pre.rank_prefix_matrix.tolist() == [3, 4, 6, 8]  # inclusive over buckets
    # per-channel counts n[r][c]: r0 (2,1) r1 (1,0) r2 (0,2) r3 (2,0); inclusive over c
    assert pre.channel_prefix_matrix.tolist() == [[2, 3], [1, 1], [0, 2], [2, 2]]
    # exclusive: where each channel's rows start inside its bucket
    assert pre.recv_channel_prefix_matrix.tolist() == [[0, 2], [0, 1], [0, 0], [0, 2]]
    # rows 0-2 bucket 0 (t0,t2,t4), row 3 bucket 1 (t1), rows 4-5 bucket 2 (t3,t4),
    # rows 6-7 bucket 3 (t0,t2)
    assert pre.recv_src_idx.tolist() == [0, 2, 4, 1, 3, 4, 0, 2]
    # position of each token inside each of its buckets
    assert pre.send_head.tolist() == [
        [0, -1, -1, 0],
        [-1, 0, -1, -1],
        [1, -1, -1, 1],
        [-1, -1, 0, -1],
        [2, -1, 1, -1],
    ]


def test_pack_by_hand(oracle):
    T, H = 5, 128
    x = (np.arange(T * H, dtype=np.uint32) * 7 + 0x3F00).astype(np.uint16).reshape(T, H)
    w = np.array([[.75, .25], [.5, .5], [.625, .375], [.875, .125], [.25, .75]], np.float32)
    lay = oracle.layout(TOPK, E, R)
    pre = oracle.prefix(lay.is_token_in_rank, C)
    rx, rti, rtw = oracle.pack_bf16(x, TOPK, w, E, pre)
    src = [0, 2, 4, 1, 3, 4, 0, 2]
    assert np.array_equal(rx, x[src])
    # local expert id (e - 2r) where the slot's expert lives in the row's bucket
    assert rti.tolist() == [[1, -1], [-1, 0], [0, -1], [0, 1], [0, 1], [-1, 0], [-1, 0], [1, -1]]
    assert rtw.tolist() == [[.75, 0], [0, .375], [.25, 0], [.5, .5], [.875, .125], [0, .75],
                            [0, .25], [.625, 0]]


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
    w = np.array([[.75, .25], [.5, .5], [.625, .375], [.875, .125], [.25, .75]], np.float32)
    out_w, _ = oracle.combine(y, TOPK, E, pre, gate_weights=w)
    assert np.array_equal(out_w, x)


def test_ll_by_hand(oracle):
    T, H, cap = 5, 128, 4
    x = (np.arange(T * H, dtype=np.uint32) + 0x3000).astype(np.uint16).reshape(T, H)
    rx, cnt, src, slot = oracle.ll_dispatch(x, TOPK, E, cap)
    assert cnt.tolist() == [2, 1, 1, 1, 2, 1, 1, 1]
    lists = {0: [2, 4], 1: [0], 2: [1], 3: [1], 4: [3, 4], 5: [3], 6: [0], 7: [2]}
    for e, lst in lists.items():
        assert src[e, : len(lst)].tolist() == lst
        assert (src[e, len(lst):] == -1).all()
        for s, t in enumerate(lst):
            assert np.array_equal(rx[e, s], x[t])
    # t4 is the second token of experts 0 and 4 (after t2 and t3)
    assert slot.tolist() == [[0, 0], [0, 0], [0, 0], [0, 0], [1, 1]]


def test_ll_capacity_overflow_raises(oracle):
    with pytest.raises(ValueError):
        oracle.ll_dispatch(None, TOPK, E, 1, hidden=0)
