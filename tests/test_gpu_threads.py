"""Contexts used from several host threads at once: each thread owns a Buffer
and a stream and runs whole capacity-mode steps (layout, first dispatch that
reuses the layout's outputs, cached dispatch, combine) on its own routing,
while the others do the same; every result is compared with the oracle, and
an error raised on one thread leaves the others' error messages alone."""

import threading

import numpy as np
import pytest
import torch

from combine_get_dispatch_layout_amd import workloads as wl
from tests.gpu_common import (assert_bf16_within_1ulp, assert_equal, check_handle, device,
                              make_buffer, np_, oracle_first_dispatch)

pytestmark = pytest.mark.gpu

E, R, C, K = 64, 8, 8, 6
THREADS = 4
STEPS = 3


def _inputs(seed, T, H):
    rng = np.random.default_rng(seed)
    idx = wl.random_routing(rng, T, E, K, p_empty=0.05)
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    w = torch.softmax(torch.randn(T, K, generator=g), -1)
    return wl.Inputs(x=x, topk_idx=torch.from_numpy(idx), topk_weights=w)


def test_contexts_on_concurrent_host_threads(oracle):
    dev = device()
    T, H = 1500, 1024
    cap = T * min(K, R)
    # inputs and references are made up front; the threads only run the library
    inputs = {(i, s): _inputs(1000 + 10 * i + s, T, H) for i in range(THREADS) for s in range(STEPS)}
    refs = {key: oracle_first_dispatch(oracle, inp, E, R, C) for key, inp in inputs.items()}
    bufs = [make_buffer(E, R, C, T) for _ in range(THREADS)]
    streams = [torch.cuda.Stream() for _ in range(THREADS)]
    results, errors = {}, []
    start = threading.Barrier(THREADS)

    def worker(i):
        try:
            buf, st = bufs[i], streams[i]
            with torch.cuda.stream(st):
                start.wait()
                for s in range(STEPS):
                    inp = inputs[(i, s)]
                    x = inp.x.to(dev, non_blocking=False)
                    idx = inp.topk_idx.to(dev)
                    w = inp.topk_weights.to(dev)
                    ntr, _, nte, itr, _ = buf.get_dispatch_layout(idx, E, no_sync=True)
                    recv, rti, rtw, _, h, _ = buf.dispatch(
                        x, topk_idx=idx, topk_weights=w, num_tokens_per_rank=ntr,
                        is_token_in_rank=itr, num_tokens_per_expert=nte, num_worst_tokens=cap,
                        no_sync=True)
                    again, _, _, _, _, _ = buf.dispatch(x, handle=h, no_sync=True)
                    out, _, _ = buf.combine(recv, h, gate_weights=w, no_sync=True)
                    # an invalid width on this thread: the message names this thread's
                    with pytest.raises(Exception) as exc:
                        buf.dispatch(x[:, :H - 4 - 8 * i].contiguous(), handle=h, no_sync=True)
                    st.synchronize()
                    results[(i, s)] = (h, recv, rti, rtw, again, out, str(exc.value))
        except Exception as e:  # reported on the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for (i, s), (h, recv, rti, rtw, again, out, msg) in sorted(results.items()):
        print(f"[threads] thread {i} step {s}", flush=True)
        inp, ref = inputs[(i, s)], refs[(i, s)]
        N = ref.prefix.num_recv
        check_handle(h, ref, N)
        assert_equal("recv_x", np_(recv)[:N], ref.recv_x)
        assert_equal("cached recv_x", np_(again)[:N], ref.recv_x)
        assert_equal("recv_topk_idx", np_(rti)[:N], ref.recv_topk_idx)
        assert_equal("recv_topk_weights", np_(rtw)[:N].view(np.uint32),
                     ref.recv_topk_weights.view(np.uint32))
        want, _ = oracle.combine(ref.recv_x, inp.topk_idx.numpy(), E, ref.prefix,
                                 gate_weights=inp.topk_weights.numpy())
        assert_bf16_within_1ulp("combine", np_(out), want)
        assert f"H={H - 4 - 8 * i} " in msg, msg
    assert len(results) == THREADS * STEPS
