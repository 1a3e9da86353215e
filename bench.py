#!/usr/bin/env python3
"""Throughput of the MoE dispatch + combine hot path on one MI355X.

Workload: 4096 tokens x 7168 hidden bf16, 256 experts top-8 with group-limited
routing (8 groups of 32 experts, 4 groups kept), 8 logical rank buckets, 24
channels; seeded synthetic inputs (x ~ N(0,1) in bf16, softmax gate weights).

One step = layout + scan + bf16 pack (with recv_topk_idx / recv_topk_weights)
+ gate-weighted combine of the identity expert's rows, in capacity mode (no
host synchronisation inside the step).  Each step's dispatch and combine are
timed with HIP events on the stream the kernels run on, each after a 1 GiB read
that evicts the caches, so the figure is HBM-resident work.  The value is
algorithmic bytes / time (GB/s); tokens/s and the fraction of the 8 TB/s HBM
peak are reported beside it, with the CPU oracle timed on a sample of the same
workload as a baseline.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch+combine HBM GB/s & tokens/s, 4096x7168 bf16 top-8, % of roofline"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(T, H, K, E, R, C, N):
    """Bytes each step must move (caching re-reads not credited).

    layout : read topk_idx (8TK), write is_token_in_rank (TR) and the R + E + RC counts
    scan   : read the mask (TR), write send_head (4TR), recv_src_idx (4N),
             two [R, C] prefix matrices and the [R] rank prefix
    pack   : read x (2TH) + topk_idx and weights (12TK); write N rows (2NH) and
             recv_topk_idx / recv_topk_weights (12NK)
    combine: read N rows (2NH), send_head (4TR), topk ids and gate weights
             (8TK + 4TK); write T rows (2TH)
    """
    layout = 8 * T * K + T * R + 4 * (R + E + R * C)
    scan = T * R + 4 * (T * R + N + 2 * R * C + R)
    pack = 2 * T * H + 2 * N * H + 12 * T * K + 12 * N * K
    combine = 2 * N * H + 2 * T * H + 4 * T * R + 8 * T * K + 4 * T * K
    return {"layout": layout, "scan": scan, "pack": pack, "combine": combine}


def cpu_baseline(inp, w, budget_s):
    """The CPU oracle (single thread, as it stands) on the same inputs."""
    import numpy as np
    import oracle as om

    o = om.Oracle()
    x = inp.x.view(__import__("torch").int16).numpy().view(np.uint16)
    idx = inp.topk_idx.numpy()
    gw = inp.topk_weights.numpy()
    times = []
    N = 0
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        lay = o.layout(idx, w.experts, w.ranks)
        pre = o.prefix(lay.is_token_in_rank, w.channels)
        rx, _, _ = o.pack_bf16(x, idx, gw, w.experts, pre)
        o.combine(rx, idx, w.experts, pre, gate_weights=gw)
        times.append(time.perf_counter() - t0)
        N = pre.num_recv
        if time.perf_counter() - t_start >= budget_s or len(times) >= 20:
            break
    return statistics.median(times), len(times), N


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget-s", type=float, default=10.0,
                    help="seconds of CPU time for the oracle baseline (0 skips it)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the exchange (logical ranks are buckets "
              "in one HBM); runs on more than one GPU are not part of this build.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from combine_get_dispatch_layout_amd import Buffer
    from combine_get_dispatch_layout_amd import _capi as C
    from combine_get_dispatch_layout_amd import workloads as wl

    w = wl.PREFILL
    T, H, K, E, R, Ch = w.tokens, w.hidden, w.topk, w.experts, w.ranks, w.channels
    log(f"[bench] generating {w.name}")
    inp = wl.make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = inp.x.to(dev)
    idx = inp.topk_idx.to(dev)
    gw = inp.topk_weights.to(dev)
    cap = T * min(K, R)
    buf = Buffer(E, R, num_channels=Ch, max_tokens=T)
    ctx = buf.ctx
    nbytes = ctypes.c_size_t()
    C.check(C.moedx_handle_workspace_bytes(ctx, T, K, cap, ctypes.byref(nbytes)))
    ws = torch.empty(nbytes.value, dtype=torch.uint8, device=dev)
    recv_x = torch.empty(cap, H, dtype=torch.bfloat16, device=dev)
    rti = torch.empty(cap, K, dtype=torch.int64, device=dev)
    rtw = torch.empty(cap, K, dtype=torch.float32, device=dev)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    sink = torch.empty((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    p_idx, p_x, p_gw, p_ws = P(idx), P(x), P(gw), P(ws)
    p_recv, p_rti, p_rtw, p_out = P(recv_x), P(rti), P(rtw), P(out)

    def new_event():
        ev = ctypes.c_void_p()
        C.check(C.moedx_event_create(ctypes.byref(ev)))
        return ev.value

    def make_ex(ev_pair=None):
        a, b = ev_pair if ev_pair else (None, None)
        return C.make_exec(stream.cuda_stream, None, None, C.MOEDX_ASYNC, a, b)

    def elapsed(pair):
        ms = ctypes.c_float()
        C.check(C.moedx_event_elapsed_ms(pair[0], pair[1], ctypes.byref(ms)))
        return ms.value

    def flush():
        torch.sum(flush_buf, dim=(0,), out=sink)

    def prepare(ex):
        h = ctypes.c_void_p()
        C.check(C.moedx_dispatch_prepare(ctx, p_idx, T, K, p_ws, nbytes.value, cap,
                                         ctypes.byref(h), ctypes.byref(ex)))
        return h

    def pack(h, ex):
        C.check(C.moedx_dispatch(ctx, h, p_x, T, H, C.MOEDX_QUANT_NONE, p_idx, p_gw, p_recv, None,
                                 p_rti, p_rtw, ctypes.byref(ex)))

    def combine(h, ex):
        C.check(C.moedx_combine(ctx, h, p_recv, H, p_gw, None, p_out, None, ctypes.byref(ex)))

    plain = make_ex()

    # Kernel-accurate per-op timing: each op is one kernel, stamped at its own
    # start and end; a 1 GiB read before the dispatch and before the combine
    # evicts the caches, so every op starts from HBM.
    def flushed_steps(n):
        recs = []
        for _ in range(n):
            evs = {k: (new_event(), new_event()) for k in ("layout", "pack", "combine")}
            flush()
            h = prepare(make_ex(evs["layout"]))
            pack(h, make_ex(evs["pack"]))
            flush()
            combine(h, make_ex(evs["combine"]))
            C.moedx_handle_destroy(h)
            recs.append(evs)
        return recs

    def finish(recs):
        torch.cuda.synchronize()
        out_ = {k: [elapsed(r[k]) for r in recs] for k in ("layout", "pack", "combine")}
        for r in recs:
            for a, b in r.values():
                C.moedx_event_destroy(a)
                C.moedx_event_destroy(b)
        return out_

    log(f"[bench] warmup {args.warmup} steps")
    finish(flushed_steps(args.warmup))
    h = prepare(plain)
    dev_n = ctypes.c_void_p()
    shape = (ctypes.c_int64 * 2)()
    C.check(C.moedx_handle_tensor(h, C.MOEDX_T_NUM_RECV, ctypes.byref(dev_n), shape))
    torch.cuda.synchronize()
    off = dev_n.value - ws.data_ptr()
    N = int(ws[off:off + 4].view(torch.int32).item())
    C.moedx_handle_destroy(h)
    bytes_ = algorithmic_bytes(T, H, K, E, R, Ch, N)
    step_bytes = sum(bytes_.values())
    log(f"[bench] N={N} receive rows; {step_bytes / 1e6:.1f} MB per step")

    log(f"[bench] {args.steps} steps, each op timed at its kernel, caches flushed")
    torch.cuda.synchronize()
    times = finish(flushed_steps(args.steps))
    torch.cuda.synchronize()
    step_ms = [a + b + c for a, b, c in zip(times["layout"], times["pack"], times["combine"])]
    ms_flushed = statistics.mean(step_ms)
    t_lay = statistics.mean(times["layout"])
    t_pack = statistics.mean(times["pack"])
    t_comb = statistics.mean(times["combine"])

    log(f"[bench] {args.steps} steps back to back, bracketed by two events")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ea = ctypes.c_void_p()
    C.check(C.moedx_event_record(ctypes.byref(ea), stream.cuda_stream))
    for _ in range(args.steps):
        hh = prepare(plain)
        pack(hh, plain)
        combine(hh, plain)
        C.moedx_handle_destroy(hh)
    eb = ctypes.c_void_p()
    C.check(C.moedx_event_record(ctypes.byref(eb), stream.cuda_stream))
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_b2b = elapsed((ea.value, eb.value)) / args.steps
    for ev in (ea.value, eb.value):
        C.moedx_event_destroy(ev)

    # Headline: the slower (more conservative) of the two measurements.
    ms = max(ms_flushed, ms_b2b)
    gbs = step_bytes / (ms * 1e-3) / 1e9

    log("[bench] plain device copy of one receive buffer (context: practical ceiling)")
    nb = 2 * N * H
    src_c = torch.empty(nb // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst_c = torch.empty_like(src_c)
    t_copy = []
    for _ in range(10):
        flush()
        ea_, eb_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea_.record(stream)
        dst_c.copy_(src_c)
        eb_.record(stream)
        t_copy.append((ea_, eb_))
    torch.cuda.synchronize()
    copy_ms = statistics.median(a.elapsed_time(b) for a, b in t_copy)
    copy_gbs = 2 * nb / (copy_ms * 1e-3) / 1e9
    del src_c, dst_c

    kern = {"pack": (t_pack, bytes_["pack"]), "combine": (t_comb, bytes_["combine"])}
    dom = max(kern, key=lambda k: kern[k][0])
    dom_ms, dom_bytes = kern[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9

    cpu = None
    if args.cpu_budget_s > 0:
        log(f"[bench] CPU oracle baseline (~{args.cpu_budget_s:.0f} s)")
        t_cpu, reps, n_cpu = cpu_baseline(inp, w, args.cpu_budget_s)
        assert n_cpu == N
        cpu = {"value": round(step_bytes / t_cpu / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "tokens_per_s": round(T / t_cpu, 1),
               "sample": f"median of {reps} full {T}x{H} steps (layout+scan+pack+weighted "
                         f"combine), single-threaded C oracle"}

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded x ~ N(0,1) bf16, group-limited top-8 routing, softmax gates",
        "config": {"workload": w.name, "tokens": T, "hidden": H, "experts": E, "topk": K,
                   "ranks": R, "channels": Ch, "routing": w.routing, "recv_rows": N,
                   "mode": "capacity (no host sync)",
                   "timing": "max of (kernel-stamped ops, caches flushed) and (back-to-back steps)"},
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "step_roofline_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
        "kernels_us": {"layout": round(t_lay * 1e3, 2), "pack": round(t_pack * 1e3, 2),
                       "combine": round(t_comb * 1e3, 2)},
        "kernel_GBps": {"pack": round(bytes_["pack"] / (t_pack * 1e-3) / 1e9, 1),
                        "combine": round(bytes_["combine"] / (t_comb * 1e-3) / 1e9, 1)},
        "ms_per_step_flushed_kernels": round(ms_flushed, 5),
        "ms_per_step_back_to_back": round(ms_b2b, 5),
        "step_ms_p10_p50_p90_flushed": [round(v, 5) for v in statistics.quantiles(step_ms, n=10)[::4]]
        if len(step_ms) >= 10 else None,
        "copy_ceiling_GBps": round(copy_gbs, 1),
        "algorithmic_bytes": bytes_,
        "wall_s_back_to_back": round(wall, 4),
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
