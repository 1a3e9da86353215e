"""The HIP path on the hand-worked routing of the cited fixture
tests/golden/handworked_t5_k2_e8_r4_c2.txt: layout outputs, handle fields,
receive rows, recv_topk_* and low-latency slots compared directly with the
fixture's values (derived by hand, not by the oracle), in exact and capacity
mode and with the layout's outputs passed to the first dispatch."""

import numpy as np
import pytest
import torch

from tests.gpu_common import device, make_buffer, np_
from tests.helpers import load_golden

pytestmark = pytest.mark.gpu

G = load_golden("handworked_t5_k2_e8_r4_c2.txt")
T, K, E, R, C = G["T"], G["K"], G["E"], G["R"], G["C"]
H = 256


def _inputs(dev):
    idx = torch.from_numpy(G["topk_idx"].astype(np.int64)).to(dev)
    w = torch.from_numpy(G["topk_weights"].astype(np.float32)).to(dev)
    bits = (np.arange(T * H, dtype=np.uint32) * 5 + 0x3C00).astype(np.uint16).reshape(T, H)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    return idx, w, x, bits


@pytest.mark.parametrize("capacity", [False, True], ids=["exact", "capacity"])
@pytest.mark.parametrize("from_layout", [False, True], ids=["own-layout", "layout-outputs"])
def test_normal_path_matches_golden(capacity, from_layout):
    dev = device()
    idx, w, x, bits = _inputs(dev)
    buf = make_buffer(E, R, C, T)
    ntr, _, nte, itr, _ = buf.get_dispatch_layout(idx, E)
    assert np_(ntr).tolist() == G["num_tokens_per_rank"].tolist()
    assert np_(nte).tolist() == G["num_tokens_per_expert"].tolist()
    assert np_(itr).reshape(T, R).tolist() == G["is_token_in_rank"].tolist()
    reuse = dict(num_tokens_per_rank=ntr, is_token_in_rank=itr,
                 num_tokens_per_expert=nte) if from_layout else {}
    recv, rti, rtw, _, h, _ = buf.dispatch(x, topk_idx=idx, topk_weights=w,
                                           num_worst_tokens=T * min(K, R) if capacity else 0,
                                           **reuse)
    f = h.fields()
    N = G["num_recv"]
    assert int(np_(f["num_recv"]).reshape(-1)[0]) == N
    assert np_(f["rank_prefix_matrix"]).tolist() == G["rank_prefix_matrix"].tolist()
    assert np_(f["channel_prefix_matrix"]).tolist() == G["channel_prefix_matrix"].tolist()
    assert np_(f["recv_channel_prefix_matrix"]).tolist() == G["recv_channel_prefix_matrix"].tolist()
    assert np_(f["recv_src_idx"])[:N].tolist() == G["recv_src_idx"].tolist()
    assert np_(f["send_head"]).tolist() == G["send_head"].tolist()
    assert np_(f["num_tokens_per_expert"]).tolist() == G["num_tokens_per_expert"].tolist()
    assert np.array_equal(np_(recv)[:N], bits[G["recv_src_idx"]])
    assert np_(rti)[:N].tolist() == G["recv_topk_idx"].tolist()
    assert np_(rtw)[:N].tolist() == G["recv_topk_weights"].tolist()


def test_low_latency_matches_golden():
    dev = device()
    idx, _, x, bits = _inputs(dev)
    buf = make_buffer(E, R, 1, T)
    cap = 8  # the library takes at most cap tokens (T = 5); the slot lists do not depend on it
    recv_x, cnt, h, _, _ = buf.low_latency_dispatch(x, idx, cap, E)
    counts = np_(cnt).tolist()
    assert counts == G["ll_recv_count"].tolist()
    f = h.fields()
    src = np_(f["src_idx"])
    rx = np_(recv_x)
    for e in range(E):  # slots past an expert's count are not written
        n = counts[e]
        assert src[e, :n].tolist() == G["ll_src_idx"][e, :n].tolist()
        assert np.array_equal(rx[e, :n], bits[G["ll_src_idx"][e, :n]])
    assert np_(f["slot_of"]).tolist() == G["ll_slot_of"].tolist()
