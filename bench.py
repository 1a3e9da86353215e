#!/usr/bin/env python3
"""Throughput of the MoE dispatch + combine hot path on one MI355X.

Workload: 4096 tokens x 7168 hidden bf16, 256 experts top-8 with group-limited
routing (8 groups of 32 experts, 4 groups kept), 8 logical rank buckets, 24
channels; seeded synthetic inputs (x ~ N(0,1) in bf16, softmax gate weights).

One step = the dispatch — the layout's counts and masks at prepare, then the
bf16 first pack on that handle, which also finishes every prefix (with
recv_topk_idx / recv_topk_weights and the handle's send_head / recv_src_idx) —
+ the gate-weighted combine of the identity expert's rows, in capacity mode (no
host synchronisation inside the step); three kernel launches.

Timing: each op (dispatch on a fresh handle, combine) runs back to back
`--steps` times between two HIP events on its stream, rotating over enough
buffer sets that every launch reads its input from HBM: at least twice the
256 MB Infinity Cache is read between two reads of one set (the cache otherwise
serves a good part of a just-written receive buffer, and keeps up to four
copies of x while the pack's streaming stores pass); a step's time is the sum
of the two per-op means.  Each kernel's own duration (events stamped at its
start and end) is reported beside it.  The value is algorithmic bytes / step
time (GB/s); tokens/s and
the fraction of the 8 TB/s HBM peak are reported beside it, with whole steps
back to back (cache-assisted, labelled as such) and the CPU oracle timed on the
same workload as a baseline.

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
INFINITY_CACHE_BYTES = 256 << 20  # MI355X last-level (memory-side) cache


# Seconds of back-to-back launches before each row of measure_rows is timed.
ROW_SETTLE_S = 0.05


def input_copies(nbytes):
    """Copies of an op's input to rotate over so that at least twice the
    Infinity Cache is read between two reads of one copy: every launch then
    reads its input from HBM (with 3 copies of a 58.7 MB x the bf16 pack read
    x from the cache and looked 16% faster than it is)."""
    return max(3, -(-2 * INFINITY_CACHE_BYTES // max(int(nbytes), 1)) + 1)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(T, H, K, E, R, C, N):
    """Bytes each step must move (caching re-reads not credited).

    layout : read topk_idx (8TK); write is_token_in_rank (TR), the R + E counts,
             the [R] rank prefix and the two [R, C] channel prefix matrices
    pack   : read x (2TH) + topk_idx and weights (12TK); write N rows (2NH),
             recv_topk_idx / recv_topk_weights (12NK), and the handle's
             send_head (4TR) and recv_src_idx (4N)
    combine: read N rows (2NH), send_head (4TR), topk ids and gate weights
             (8TK + 4TK); write T rows (2TH)
    """
    layout = 8 * T * K + T * R + 4 * (R + E + R + 2 * R * C)
    pack = 2 * T * H + 2 * N * H + 12 * T * K + 12 * N * K + 4 * T * R + 4 * N
    combine = 2 * N * H + 2 * T * H + 4 * T * R + 8 * T * K + 4 * T * K
    return {"layout": layout, "pack": pack, "combine": combine}


TRAFFIC_SOURCES = {"layout": "layout.hip", "get_layout": "layout.hip", "pack": "pack.hip",
                   "get_layout_fp8_skewed": "layout.hip",
                   "pack_fp8": "pack.hip", "pack_fp8_ue8m0": "pack.hip",
                   "pack_fp8_tensor": "pack.hip", "pack_fp8_prequant": "pack.hip",
                   "cached_dispatch": "pack.hip", "combine": "combine.hip",
                   "combine_fp8_skewed": "combine.hip", "combine_reuse": "combine.hip",
                   "ll_dispatch": "ll.hip", "ll_combine": "ll.hip", "launch_floor": "ll.hip",
                   "pack_ltd": "pack.hip"}
# headers every kernel source includes: a change there changes the kernels too
SHARED_HEADERS = ("launch.h", "rows.h", "fastdiv.h", "layout_core.h", "fp8_codec.h", "xcd.h")


def source_digest(src):
    """First 16 hex digits of the sha256 over a kernel source and the shared headers."""
    import hashlib

    h = hashlib.sha256()
    for name in (src,) + SHARED_HEADERS:
        with open(os.path.join(ROOT, "combine_get_dispatch_layout_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def input_digests(inp) -> dict:
    """First 16 hex digits of the sha256 of each generated input tensor's bytes
    (x as bf16, topk_idx as int64, topk_weights as fp32), so that a rerun can
    check it measured the same inputs."""
    import hashlib

    import torch

    def digest(t):
        return hashlib.sha256(t.contiguous().view(-1).view(torch.uint8).numpy().tobytes()).hexdigest()[:16]

    return {"x": digest(inp.x), "topk_idx": digest(inp.topk_idx),
            "topk_weights": digest(inp.topk_weights)}


def measured_traffic(op):
    """HBM bytes per launch of `op` from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy of known size), or
    None once the kernel source differs from the one profiled."""
    if op not in TRAFFIC_SOURCES:
        return None
    digest = source_digest(TRAFFIC_SOURCES[op])
    summary = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(summary):
        return None
    rec = json.load(open(summary)).get("ops", {}).get(op)
    if not rec or rec.get("source_sha256_16") != digest:
        return None
    return rec["traffic_bytes_per_launch"]


def cpu_model():
    """The host CPU as /proc/cpuinfo names it: model name, family / model /
    stepping, and the number of logical CPUs it lists."""
    fields, cpus = {}, 0
    try:
        for line in open("/proc/cpuinfo"):
            key = line.split(":", 1)[0].strip()
            if key == "processor":
                cpus += 1
            elif key in ("model name", "cpu family", "model", "stepping") and key not in fields:
                fields[key] = line.split(":", 1)[1].strip()
    except OSError:
        return "unknown"
    return (f"{fields.get('model name', 'unknown')} (family {fields.get('cpu family', '?')}, "
            f"model {fields.get('model', '?')}, stepping {fields.get('stepping', '?')}; "
            f"{cpus} logical CPUs listed)")


def cpu_threads():
    """Host threads for the oracle's all-cores leg: the CPUs this process may
    run on, capped by OMP_NUM_THREADS where it is set (a GPU machine gives one GPU
    a share of its cores and says so there)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(n, 1)


def hbm_ceilings(nbytes, n, flush):
    """What plain PyTorch kernels reach on this machine over buffers of `nbytes`:
    a write-only fill and a copy, each launched n times back to back over
    enough buffers that every launch reads from (and writes to) HBM rather than
    the Infinity Cache; GB/s of bytes read plus written."""
    import torch

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    k = input_copies(nbytes)
    words = nbytes // 4
    bufs = [torch.ones(words, dtype=torch.float32, device=dev) for _ in range(k)]
    outs = [torch.empty(words, dtype=torch.float32, device=dev) for _ in range(k)]
    ops = {"write_GBps": (lambda i: outs[i].fill_(0.5), nbytes),
           "copy_GBps": (lambda i: outs[i].copy_(bufs[i]), 2 * nbytes)}
    res = {"bytes": int(nbytes), "buffers": k}
    for name, (op, moved) in ops.items():
        for i in range(k):  # warm up, fill the rotation
            op(i)
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            op(i % k)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / n
        res[name] = round(moved / (ms * 1e-3) / 1e9, 1)
    res["note"] = ("torch's fill_ (write) and copy_ kernels, back to back over "
                   f"{k} rotating buffers of {nbytes / 1e6:.0f} MB")
    del bufs, outs
    torch.cuda.empty_cache()
    return res


def kernel_us_distribution(C, stream, launch, n, flush):
    """Per-launch kernel durations of n back-to-back launches: HIP events
    stamped at each kernel's own start and end.  launch(i, exec_ptr) enqueues
    launch i (one kernel) with that exec.  Returns p10 / median / p90 in us."""
    evs = []
    for _ in range(n):
        a_, b_ = ctypes.c_void_p(), ctypes.c_void_p()
        C.check(C.moedx_event_create(ctypes.byref(a_)))
        C.check(C.moedx_event_create(ctypes.byref(b_)))
        evs.append((a_.value, b_.value))
    flush()
    for i, (ka, kb) in enumerate(evs):
        launch(i, ctypes.byref(C.make_exec(stream.cuda_stream, None, None, C.MOEDX_ASYNC, ka, kb)))
    stream.synchronize()
    d = []
    for ka, kb in evs:
        ms = ctypes.c_float()
        C.check(C.moedx_event_elapsed_ms(ka, kb, ctypes.byref(ms)))
        C.moedx_event_destroy(ka)
        C.moedx_event_destroy(kb)
        d.append(ms.value * 1e3)
    d.sort()
    q = lambda f: d[min(len(d) - 1, int(round(f * (len(d) - 1))))]  # noqa: E731
    return {"p10": round(q(0.1), 2), "median": round(q(0.5), 2), "p90": round(q(0.9), 2),
            "mean": round(statistics.mean(d), 2)}


def oracle_step(o, x, idx, gw, E, R, C, threads=1, pool=None):
    """One step of the CPU oracle: layout, prefixes, bf16 pack with recv_topk_*,
    gate-weighted combine.  With threads > 1 the per-token parts (layout, pack,
    combine) run over `threads` contiguous token ranges at once (the oracle's
    C functions release the GIL); each range calls the oracle unchanged on its
    rows, the range counts of the layout are added up, and the prefixes, a
    sequential scan, run once.  Returns (N, receive rows, combined rows)."""
    import dataclasses

    import numpy as np

    T, K = idx.shape
    H = x.shape[1]
    if threads <= 1:
        lay = o.layout(idx, E, R)
        pre = o.prefix(lay.is_token_in_rank, C)
        rx, _, _ = o.pack_bf16(x, idx, gw, E, pre)
        out, _ = o.combine(rx, idx, E, pre, gate_weights=gw)
        return pre.num_recv, rx, out
    bounds = [(T * i // threads, T * (i + 1) // threads) for i in range(threads)]
    itr = np.empty((T, R), np.uint8)
    lays = list(pool.map(lambda b: o.layout(idx[b[0]:b[1]], E, R, out_itr=itr[b[0]:b[1]]),
                         bounds))
    ntr = sum(lay.num_tokens_per_rank for lay in lays)
    pre = o.prefix(itr, C)
    assert int(ntr.sum()) == pre.num_recv
    N = pre.num_recv
    rx = np.zeros((N, H), np.uint16)
    rti = np.empty((N, K), np.int64)
    rtw = np.empty((N, K), np.float32)
    rows = lambda b: dataclasses.replace(pre, send_head=pre.send_head[b[0]:b[1]])  # noqa: E731
    list(pool.map(lambda b: o.pack_bf16(x[b[0]:b[1]], idx[b[0]:b[1]], gw[b[0]:b[1]], E, rows(b),
                                        out=(rx, rti, rtw)), bounds))
    out = np.empty((T, H), np.uint16)
    list(pool.map(lambda b: o.combine(rx, idx[b[0]:b[1]], E, rows(b), gate_weights=gw[b[0]:b[1]],
                                      out=out[b[0]:b[1]]), bounds))
    return N, rx, out


def cpu_baseline(inp, w, budget_s, threads=1):
    """The CPU oracle (as it stands) on the same inputs, on `threads` host
    threads: median step time, steps run, N."""
    import concurrent.futures as cf

    import numpy as np
    import oracle as om

    o = om.Oracle()
    x = inp.x.view(__import__("torch").int16).numpy().view(np.uint16)
    idx = inp.topk_idx.numpy()
    gw = inp.topk_weights.numpy()
    times = []
    N = 0
    with cf.ThreadPoolExecutor(max_workers=threads) as pool:
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            N = oracle_step(o, x, idx, gw, w.experts, w.ranks, w.channels, threads, pool)[0]
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start >= budget_s or len(times) >= 20:
                break
    return statistics.median(times), len(times), N


def row_bytes(kind, T, H, K, E, N=0, V=0, R=0):
    """Algorithmic bytes of one launch of a further step of the path.

    pack_fp8       : read x (2TH); write N rows of codes (NH) and their 1x128
                     scales (4N*H/128); with UE8M0 scales 1 byte each, with
                     one per-tensor scale none
    pack_fp8_prequant: read codes (TH) and fp32 scales (4T*H/128); write them
                     to N rows
    combine        : read N rows (2NH), send_head (4TR), topk ids and gate
                     weights (12TK); write T rows (2TH)
    cached_dispatch: read x (2TH); write N rows (2NH)
    get_layout     : read topk_idx (8TK); write is_token_in_rank (TR) and the
                     R + E counts
    ll_dispatch    : read x (2TH) and topk_idx (8TK); write the V filled slots
                     (2VH), their src_idx (4V), slot_of (4TK) and counts (4E)
    ll_combine     : read the V slots (2VH), topk_idx, weights and slot_of
                     (16TK); write T rows (2TH)
    """
    return {
        "pack_fp8": 2 * T * H + N * H + 4 * N * (H // 128),
        "pack_fp8_ue8m0": 2 * T * H + N * H + N * (H // 128),
        "pack_fp8_tensor": 2 * T * H + N * H,
        "pack_fp8_prequant": T * H + 4 * T * (H // 128) + N * H + 4 * N * (H // 128),
        "combine": 2 * N * H + 2 * T * H + 4 * T * R + 12 * T * K,
        "cached_dispatch": 2 * T * H + 2 * N * H,
        "get_layout": 8 * T * K + T * R + 4 * (R + E),
        "ll_dispatch": 2 * T * H + 8 * T * K + 2 * V * H + 4 * V + 4 * T * K + 4 * E,
        "ll_combine": 2 * V * H + 16 * T * K + 2 * T * H,
    }[kind]


def _median_time(fn, budget_s, max_reps=5):
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start >= budget_s or len(times) >= max_reps:
            return statistics.median(times), len(times)


def measure_rows(steps, warmup, cpu_budget_s, flush, log_fn):
    """Every further step of the path on its own workload: the FP8 pack, the
    cached (handle-reuse) dispatch, the standalone layout and the low-latency
    pair.  Each is launched back to back over rotating buffer sets between two
    HIP events, like the step above; the CPU oracle is timed on a bounded
    sample of the same workload."""
    import numpy as np
    import torch

    from combine_get_dispatch_layout_amd import Buffer
    from combine_get_dispatch_layout_amd import _capi as C
    from combine_get_dispatch_layout_amd import workloads as wl

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    ex = C.make_exec(stream.cuda_stream, None, None, C.MOEDX_ASYNC)
    exr = ctypes.byref(ex)
    NSETS = 3
    o = None
    if cpu_budget_s > 0:
        import oracle as om
        o = om.Oracle()

    def record():
        ev = ctypes.c_void_p()
        C.check(C.moedx_event_record(ctypes.byref(ev), stream.cuda_stream))
        return ev.value

    def rot_ms(fns, n):
        flush()
        a = record()
        for i in range(n):
            fns[i % len(fns)]()
        b = record()
        torch.cuda.synchronize()
        ms = ctypes.c_float()
        C.check(C.moedx_event_elapsed_ms(a, b, ctypes.byref(ms)))
        C.moedx_event_destroy(a)
        C.moedx_event_destroy(b)
        return ms.value / n

    def timed(fns):
        # Warm-up: at least `warmup` launches and ROW_SETTLE_S of back-to-back
        # work, so that each row is timed after the clocks have settled from the
        # host-only work (oracle timing, input set-up) before it.
        t0 = time.perf_counter()
        n = 0
        while n < max(warmup, 1) or time.perf_counter() - t0 < ROW_SETTLE_S:
            rot_ms(fns, max(warmup, 1))
            n += max(warmup, 1)
        return rot_ms(fns, steps)

    # The exec the single-kernel row closures launch with: exr, or one whose
    # events are stamped at the kernel's own start and end.
    cur = [exr]

    def per_launch(fns):
        def launch(i, e):
            cur[0] = e
            fns[i % len(fns)]()
        try:
            return kernel_us_distribution(C, stream, launch, steps, flush)
        finally:
            cur[0] = exr

    def u16(t):
        return t.view(torch.int16).numpy().view(np.uint16)

    def entry(w, kind, ms, nbytes, extra, cpu=None):
        gbs = nbytes / (ms * 1e-3) / 1e9
        r = {"workload": w.name, "us": round(ms * 1e3, 2), "bytes": int(nbytes),
             "GBps": round(gbs, 1), "roofline_frac": round(gbs / HBM_PEAK_GBS, 4),
             "traffic": measured_traffic(kind),
             "tokens_per_s": round(w.tokens / (ms * 1e-3), 1)}
        r.update(extra)
        if cpu is not None:
            r["cpu_oracle"] = cpu
        return r

    def cpu_entry(nbytes, secs, reps, sample):
        return {"GBps": round(nbytes / secs / 1e9, 4), "cores": 1, "sample": sample,
                "reps": reps}

    def handle_rows(buf, h, ws):
        C.check(C.moedx_handle_finish(buf.ctx, h, exr))  # capacity mode: N comes with the prefixes
        dev_n = ctypes.c_void_p()
        shape = (ctypes.c_int64 * 2)()
        C.check(C.moedx_handle_tensor(h, C.MOEDX_T_NUM_RECV, ctypes.byref(dev_n), shape))
        off = dev_n.value - ws.data_ptr()
        return int(ws[off:off + 4].view(torch.int32).item())

    def normal_sets(w, fp8, seeds):
        T, H, K, E, R, Ch = w.tokens, w.hidden, w.topk, w.experts, w.ranks, w.channels
        inp = wl.make_inputs(w)
        buf = Buffer(E, R, num_channels=Ch, max_tokens=T)
        cap = T * min(K, R)
        nb = ctypes.c_size_t()
        C.check(C.moedx_handle_workspace_bytes(buf.ctx, T, K, cap, ctypes.byref(nb)))
        idx = inp.topk_idx.to(dev)
        sets = []
        for s in seeds:
            x = (inp.x if s is None else wl.fresh_x(w, s)).to(dev)
            ws = torch.empty(nb.value, dtype=torch.uint8, device=dev)
            h = ctypes.c_void_p()
            C.check(C.moedx_dispatch_prepare(buf.ctx, P(idx), T, K, None, None, None, P(ws), nb.value, cap,
                                             ctypes.byref(h), exr))
            if fp8:
                recv = torch.empty(cap, H, dtype=torch.uint8, device=dev)
                scales = torch.empty(cap, H // 128, dtype=torch.float32, device=dev)
            else:
                recv = torch.empty(cap, H, dtype=torch.bfloat16, device=dev)
                scales = None
            sets.append({"x": x, "ws": ws, "h": h, "recv": recv, "scales": scales})
        torch.cuda.synchronize()
        N = handle_rows(buf, sets[0]["h"], sets[0]["ws"])
        return inp, buf, idx, sets, N

    rows = {}

    # -- FP8 pack (per-1x128 E4M3) on the skewed 8192-token workload --------------
    w = wl.FP8_SKEWED
    log_fn(f"[bench] row pack_fp8: {w.name}")
    T, H, K, E = w.tokens, w.hidden, w.topk, w.experts
    inp, buf, idx, sets, N = normal_sets(w, True, [None] * input_copies(2 * T * H))

    def fp8_pack(s):
        return lambda: C.check(C.moedx_dispatch(
            buf.ctx, s["h"], P(s["x"]), T, H, C.MOEDX_QUANT_FP8_E4M3_1X128, None, None,
            P(s["recv"]), P(s["scales"]), None, None, cur[0]))

    fns = [fp8_pack(s) for s in sets]
    ms = timed(fns)
    dist = per_launch(fns)
    nbytes = row_bytes("pack_fp8", T, H, K, E, N=N)
    cpu = None
    if o is not None:
        ts = 512
        si = wl.make_inputs(w, tokens=ts)
        lay = o.layout(si.topk_idx.numpy(), E, w.ranks)
        pre = o.prefix(lay.is_token_in_rank, w.channels)
        xs = u16(si.x)
        secs, reps = _median_time(lambda: o.pack_fp8(xs, pre), cpu_budget_s / 4)
        cpu = cpu_entry(row_bytes("pack_fp8", ts, H, K, E, N=pre.num_recv), secs, reps,
                        f"oracle pack_fp8 on {ts} tokens of the same workload")
    rows["pack_fp8"] = entry(w, "pack_fp8", ms, nbytes, {"recv_rows": N, "dtype": "bf16->e4m3",
                                                          "per_launch_us": dist}, cpu)

    # the other scale modes and the pre-quantised pass-through, same workload
    def fp8_opt(s, opts, x_ptr, scales_ptr):
        return lambda: C.check(C.moedx_dispatch_fp8(buf.ctx, s["h"], x_ptr, T, H, ctypes.byref(opts),
                                                    P(s["recv"]), scales_ptr, cur[0]))

    ue8m0 = C.moedx_fp8(C.MOEDX_FP8_SCALE_UE8M0, 0, 0.0, None)
    tensor = C.moedx_fp8(C.MOEDX_FP8_SCALE_TENSOR, 0, 0.0123, None)
    u8 = [torch.empty(T * min(K, w.ranks), H // 128, dtype=torch.uint8, device=dev) for _ in sets]
    # pre-quantised input: the codes and scales of the first receive rows, in
    # enough copies to be read from HBM
    q0 = (sets[0]["recv"][:T], sets[0]["scales"][:T])
    pq = [(q0[0].clone(), q0[1].clone()) for _ in range(input_copies(T * H + 4 * T * (H // 128)))]
    pre_opts = [C.moedx_fp8(C.MOEDX_FP8_SCALE_AMAX, 1, 0.0, ctypes.c_void_p(q[1].data_ptr()))
                for q in pq]
    pq_sets = [sets[i % len(sets)] for i in range(len(pq))]
    variants = (
        ("pack_fp8_ue8m0", [fp8_opt(s, ue8m0, P(s["x"]), P(u)) for s, u in zip(sets, u8)],
         o.FP8_UE8M0 if o else None),
        ("pack_fp8_tensor", [fp8_opt(s, tensor, P(s["x"]), None) for s in sets],
         o.FP8_TENSOR if o else None),
        ("pack_fp8_prequant", [fp8_opt(s, op, P(q[0]), P(s["scales"]))
                               for s, q, op in zip(pq_sets, pq, pre_opts)], None),
    )
    for name, fns, omode in variants:
        log_fn(f"[bench] row {name}: {w.name}")
        ms = timed(fns)
        dist = per_launch(fns)
        cpu = None
        if o is not None:
            ts = 512
            si = wl.make_inputs(w, tokens=ts)
            lay = o.layout(si.topk_idx.numpy(), E, w.ranks)
            pre = o.prefix(lay.is_token_in_rank, w.channels)
            if omode is None:
                codes8 = np.zeros((ts, H), np.uint8)
                sc = np.zeros((ts, H // 128), np.float32)

                def run():
                    o.pack_rows_bytes(codes8, pre)
                    o.pack_rows_bytes(sc, pre)
            else:
                xs = u16(si.x)

                def run(xs=xs, omode=omode):
                    o.pack_fp8_mode(xs, pre, omode, 0.0123)
            secs, reps = _median_time(run, cpu_budget_s / 8)
            cpu = cpu_entry(row_bytes(name, ts, H, K, E, N=pre.num_recv), secs, reps,
                            f"oracle on {ts} tokens of the same workload")
        rows[name] = entry(w, name, ms, row_bytes(name, T, H, K, E, N=N),
                           {"recv_rows": N, "per_launch_us": dist}, cpu)
    # combine of bf16 expert outputs for the skewed routing (the dequantised rows
    # in a real layer; the values do not change the work)
    log_fn(f"[bench] row combine_fp8_skewed: {w.name}")
    gw4 = inp.topk_weights.to(dev)
    cap4 = T * min(K, w.ranks)
    for s in sets:
        s["y"] = torch.empty(cap4, H, dtype=torch.bfloat16, device=dev)
        s["out"] = torch.empty(T, H, dtype=torch.bfloat16, device=dev)

    def comb4(s):
        return lambda: C.check(C.moedx_combine(buf.ctx, s["h"], P(s["y"]), H, P(gw4), None,
                                               P(s["out"]), None, cur[0]))

    fns = [comb4(s) for s in sets]
    ms = timed(fns)
    rows["combine_fp8_skewed"] = entry(w, "combine_fp8_skewed", ms,
                                       row_bytes("combine", T, H, K, E, N=N, R=w.ranks),
                                       {"recv_rows": N, "dtype": "bf16",
                                        "per_launch_us": per_launch(fns)})

    # -- the first FP8 dispatch on a fresh handle (layout with every prefix at
    # prepare, then the FP8 pack, which also writes send_head / recv_src_idx),
    # and get_dispatch_layout alone, on the same workload
    log_fn(f"[bench] rows first_dispatch_fp8 / get_layout_fp8_skewed: {w.name}")
    R4 = w.ranks
    nb4 = ctypes.c_size_t()
    C.check(C.moedx_handle_workspace_bytes(buf.ctx, T, K, cap4, ctypes.byref(nb4)))
    for s in sets:
        s["ws_first"] = torch.empty(nb4.value, dtype=torch.uint8, device=dev)

    def first_fp8(s):
        def f():
            h = ctypes.c_void_p()
            C.check(C.moedx_dispatch_prepare(buf.ctx, P(idx), T, K, None, None, None,
                                             P(s["ws_first"]), nb4.value, cap4, ctypes.byref(h),
                                             exr))
            C.check(C.moedx_dispatch(buf.ctx, h, P(s["x"]), T, H, C.MOEDX_QUANT_FP8_E4M3_1X128,
                                     None, None, P(s["recv"]), P(s["scales"]), None, None, exr))
            C.moedx_handle_destroy(h)
        return f

    ms_f8 = timed([first_fp8(s) for s in sets])
    lay4 = 8 * T * K + T * R4 + 4 * (2 * R4 + E + 2 * R4 * w.channels)
    rows["first_dispatch_fp8"] = entry(
        w, "first_dispatch_fp8", ms_f8, lay4 + row_bytes("pack_fp8", T, H, K, E, N=N) + 4 * T * R4 + 4 * N,
        {"recv_rows": N, "dtype": "bf16->e4m3",
         "note": "prepare (the layout with every prefix: 128 groups of 64 tokens) + the FP8 pack "
                 "with the handle's send_head / recv_src_idx, on a fresh capacity-mode handle"})
    for s in sets:
        s["ntr"] = torch.empty(R4, dtype=torch.int32, device=dev)
        s["nte"] = torch.empty(E, dtype=torch.int32, device=dev)
        s["itr"] = torch.empty(T, R4, dtype=torch.uint8, device=dev)

    def get_layout4(s):
        return lambda: C.check(C.moedx_get_dispatch_layout(
            buf.ctx, P(idx), T, K, P(s["ntr"]), P(s["nte"]), P(s["itr"]), cur[0]))

    fns = [get_layout4(s) for s in sets]
    ms = timed(fns)
    rows["get_layout_fp8_skewed"] = entry(
        w, "get_layout_fp8_skewed", ms, row_bytes("get_layout", T, H, K, E, R=R4),
        {"bound_note": "latency (under 1 MB)", "per_launch_us": per_launch(fns)})
    for s in sets:
        C.moedx_handle_destroy(s["h"])
    del sets, buf, u8, pq

    # -- cached dispatch (handle reuse) on the 16384-token workload --------------
    w = wl.HANDLE_REUSE
    log_fn(f"[bench] row cached_dispatch: {w.name}")
    T, H, K, E = w.tokens, w.hidden, w.topk, w.experts
    inp, buf, idx, sets, N = normal_sets(w, False, list(w.reuse_seeds[:input_copies(2 * T * H)]))

    def cached(s):
        return lambda: C.check(C.moedx_dispatch(
            buf.ctx, s["h"], P(s["x"]), T, H, C.MOEDX_QUANT_NONE, None, None,
            P(s["recv"]), None, None, None, cur[0]))

    for s in sets:  # the first dispatch on each handle writes its rows
        cached(s)()
    fns = [cached(s) for s in sets]
    ms = timed(fns)
    dist = per_launch(fns)
    nbytes = row_bytes("cached_dispatch", T, H, K, E, N=N)
    cpu = None
    if o is not None:
        ts = 2048
        si = wl.make_inputs(w, tokens=ts)
        lay = o.layout(si.topk_idx.numpy(), E, w.ranks)
        pre = o.prefix(lay.is_token_in_rank, w.channels)
        xs, ids = u16(si.x), si.topk_idx.numpy()
        secs, reps = _median_time(lambda: o.pack_bf16(xs, ids, None, E, pre, with_topk=False),
                                     cpu_budget_s / 4)
        cpu = cpu_entry(row_bytes("cached_dispatch", ts, H, K, E, N=pre.num_recv), secs, reps,
                        f"oracle pack_bf16 on {ts} tokens of the same workload")
    rows["cached_dispatch"] = entry(w, "cached_dispatch", ms, nbytes,
                                    {"recv_rows": N, "dtype": "bf16", "per_launch_us": dist}, cpu)

    # -- the reuse repetition: cached pack, then the gate-weighted combine
    log_fn(f"[bench] rows combine_reuse / reuse_rep: {w.name}")
    gw5 = inp.topk_weights.to(dev)
    for s in sets:
        s["out"] = torch.empty(T, H, dtype=torch.bfloat16, device=dev)

    def comb5(s):
        return lambda: C.check(C.moedx_combine(buf.ctx, s["h"], P(s["recv"]), H, P(gw5), None,
                                               P(s["out"]), None, cur[0]))

    def rep5(s):
        p_, c_ = cached(s), comb5(s)
        return lambda: (p_(), c_())

    fns = [comb5(s) for s in sets]
    ms_c = timed(fns)
    b_c = row_bytes("combine", T, H, K, E, N=N, R=w.ranks)
    rows["combine_reuse"] = entry(w, "combine_reuse", ms_c, b_c,
                                  {"recv_rows": N, "dtype": "bf16", "per_launch_us": per_launch(fns)})
    ms_r = timed([rep5(s) for s in sets])
    rows["reuse_rep"] = entry(w, "reuse_rep", ms_r, nbytes + b_c,
                              {"recv_rows": N, "note": "cached dispatch + weighted combine, "
                                                      "back to back (one repetition)"})

    # -- what handle reuse saves: a first dispatch in exact mode on the same
    # workload = layout + scan, the host wait for N and the per-expert counts,
    # then the pack (rows, recv_topk_*, handle rows); a fresh handle each time
    log_fn(f"[bench] row first_dispatch_exact: {w.name}")
    nb_exact = ctypes.c_size_t()
    C.check(C.moedx_handle_workspace_bytes(buf.ctx, T, K, 0, ctypes.byref(nb_exact)))
    gw = inp.topk_weights.to(dev)
    blocking = C.make_exec(stream.cuda_stream, None, None, 0)
    for s in sets:
        s["ws_exact"] = torch.empty(nb_exact.value, dtype=torch.uint8, device=dev)
        s["rti"] = torch.empty(T * min(K, w.ranks), K, dtype=torch.int64, device=dev)
        s["rtw"] = torch.empty(T * min(K, w.ranks), K, dtype=torch.float32, device=dev)

    def first_exact(s):
        def f():
            h = ctypes.c_void_p()
            C.check(C.moedx_dispatch_prepare(buf.ctx, P(idx), T, K, None, None, None, P(s["ws_exact"]),
                                             nb_exact.value, 0, ctypes.byref(h),
                                             ctypes.byref(blocking)))
            C.check(C.moedx_dispatch(buf.ctx, h, P(s["x"]), T, H, C.MOEDX_QUANT_NONE, P(idx),
                                     P(gw), P(s["recv"]), None, P(s["rti"]), P(s["rtw"]), exr))
            C.moedx_handle_destroy(h)  # the host record only; the workspace stays alive
        return f

    ms_first = timed([first_exact(s) for s in sets])
    rows["first_dispatch_exact"] = entry(
        w, "first_dispatch_exact", ms_first,
        2 * T * H + 2 * N * H + 12 * T * K + 12 * N * K + 4 * T * w.ranks + 4 * N,
        {"recv_rows": N, "note": "layout + host wait for N + pack; cached_dispatch above "
                                 "is what handle reuse leaves"})
    for s in sets:
        C.moedx_handle_destroy(s["h"])
    del sets, buf

    # -- standalone get_dispatch_layout on the prefill workload -------------------
    w = wl.PREFILL
    log_fn(f"[bench] row get_layout: {w.name}")
    inp = wl.make_inputs(w)
    T, H, K, E, R = w.tokens, w.hidden, w.topk, w.experts, w.ranks
    buf = Buffer(E, R, num_channels=w.channels, max_tokens=T)
    lsets = []
    for _ in range(NSETS):
        lsets.append({"idx": inp.topk_idx.to(dev),
                      "ntpr": torch.empty(R, dtype=torch.int32, device=dev),
                      "ntpe": torch.empty(E, dtype=torch.int32, device=dev),
                      "itir": torch.empty(T, R, dtype=torch.uint8, device=dev)})

    def get_layout(s):
        return lambda: C.check(C.moedx_get_dispatch_layout(
            buf.ctx, P(s["idx"]), T, K, P(s["ntpr"]), P(s["ntpe"]), P(s["itir"]), cur[0]))

    fns = [get_layout(s) for s in lsets]
    ms = timed(fns)
    dist = per_launch(fns)
    cpu = None
    if o is not None:
        ids = inp.topk_idx.numpy()
        secs, reps = _median_time(lambda: o.layout(ids, E, R), cpu_budget_s / 8, max_reps=20)
        cpu = cpu_entry(row_bytes("get_layout", T, H, K, E, R=R), secs, reps,
                        f"oracle layout on the full {T}-token workload")
    rows["get_layout"] = entry(w, "get_layout", ms, row_bytes("get_layout", T, H, K, E, R=R),
                               {"bound_note": "latency (under 0.3 MB)", "per_launch_us": dist}, cpu)
    del lsets, buf

    # -- the first FP8 dispatch on the prefill routing (a fresh capacity-mode
    # handle each time: the layout's partials, then the FP8 pack that also
    # finishes the handle)
    log_fn(f"[bench] row first_dispatch_fp8_prefill: {w.name}")
    inp, buf, idx, sets, N = normal_sets(w, True, [None] * input_copies(2 * T * H))
    capp = T * min(K, R)
    nbp = ctypes.c_size_t()
    C.check(C.moedx_handle_workspace_bytes(buf.ctx, T, K, capp, ctypes.byref(nbp)))
    for s in sets:
        s["ws_first"] = torch.empty(nbp.value, dtype=torch.uint8, device=dev)

    def first_fp8_prefill(s):
        def f():
            h = ctypes.c_void_p()
            C.check(C.moedx_dispatch_prepare(buf.ctx, P(idx), T, K, None, None, None,
                                             P(s["ws_first"]), nbp.value, capp, ctypes.byref(h),
                                             exr))
            C.check(C.moedx_dispatch(buf.ctx, h, P(s["x"]), T, H, C.MOEDX_QUANT_FP8_E4M3_1X128,
                                     None, None, P(s["recv"]), P(s["scales"]), None, None, exr))
            C.moedx_handle_destroy(h)
        return f

    ms = timed([first_fp8_prefill(s) for s in sets])
    layp = 8 * T * K + T * R + 4 * (2 * R + E + 2 * R * w.channels)
    rows["first_dispatch_fp8_prefill"] = entry(
        w, "first_dispatch_fp8_prefill", ms,
        layp + row_bytes("pack_fp8", T, H, K, E, N=N) + 4 * T * R + 4 * N,
        {"recv_rows": N, "dtype": "bf16->e4m3",
         "note": "prepare (the layout's partials) + the FP8 pack that also finishes the handle "
                 "(prefixes, send_head, recv_src_idx) in the same launch, on a fresh "
                 "capacity-mode handle"})
    for s in sets:
        C.moedx_handle_destroy(s["h"])
    del sets, buf

    # -- the whole step on the tiny workload (launch-bound; its 0.4 MB stay in
    # the caches whatever the rotation)
    w = wl.TINY
    log_fn(f"[bench] row tiny_step: {w.name}")
    inp = wl.make_inputs(w)
    T, H, K, E, R, Ch = w.tokens, w.hidden, w.topk, w.experts, w.ranks, w.channels
    buf = Buffer(E, R, num_channels=Ch, max_tokens=T)
    cap1 = T * min(K, R)
    nb1 = ctypes.c_size_t()
    C.check(C.moedx_handle_workspace_bytes(buf.ctx, T, K, cap1, ctypes.byref(nb1)))
    idx1, gw1 = inp.topk_idx.to(dev), inp.topk_weights.to(dev)
    tsets = [{"x": inp.x.to(dev), "ws": torch.empty(nb1.value, dtype=torch.uint8, device=dev),
              "recv": torch.empty(cap1, H, dtype=torch.bfloat16, device=dev),
              "rti": torch.empty(cap1, K, dtype=torch.int64, device=dev),
              "rtw": torch.empty(cap1, K, dtype=torch.float32, device=dev),
              "out": torch.empty(T, H, dtype=torch.bfloat16, device=dev)} for _ in range(NSETS)]

    def tiny_step(s):
        def f():
            h = ctypes.c_void_p()
            C.check(C.moedx_dispatch_prepare(buf.ctx, P(idx1), T, K, None, None, None, P(s["ws"]),
                                             nb1.value, cap1, ctypes.byref(h), exr))
            C.check(C.moedx_dispatch(buf.ctx, h, P(s["x"]), T, H, C.MOEDX_QUANT_NONE, P(idx1),
                                     P(gw1), P(s["recv"]), None, P(s["rti"]), P(s["rtw"]), exr))
            C.check(C.moedx_combine(buf.ctx, h, P(s["recv"]), H, P(gw1), None, P(s["out"]), None,
                                    exr))
            C.moedx_handle_destroy(h)
        return f

    ms = timed([tiny_step(s) for s in tsets])
    ref_n = secs = reps = None
    if o is not None:
        xs1 = u16(inp.x)
        ids1, gws1 = inp.topk_idx.numpy(), inp.topk_weights.numpy()
        secs, reps = _median_time(lambda: oracle_step(o, xs1, ids1, gws1, E, R, Ch), cpu_budget_s / 16,
                                  max_reps=20)
        ref_n = oracle_step(o, xs1, ids1, gws1, E, R, Ch)[0]
    h0 = ctypes.c_void_p()
    C.check(C.moedx_dispatch_prepare(buf.ctx, P(idx1), T, K, None, None, None, P(tsets[0]["ws"]),
                                     nb1.value, cap1, ctypes.byref(h0), exr))
    N1 = handle_rows(buf, h0, tsets[0]["ws"])
    C.moedx_handle_destroy(h0)
    assert ref_n is None or ref_n == N1
    b1 = sum(algorithmic_bytes(T, H, K, E, R, Ch, N1).values())
    rows["tiny_step"] = entry(
        w, "tiny_step", ms, b1,
        {"recv_rows": N1, "dtype": "bf16",
         "note": "layout partials + first pack (finishing the handle) + gate-weighted combine, "
                 "capacity mode; launch-bound, inputs cache-resident"},
        cpu_entry(b1, secs, reps, f"oracle step on the full {T}-token workload") if o else None)
    del tsets, buf

    # -- low-latency dispatch and combine on the 128-token decode workload -------
    w = wl.LL_DECODE
    log_fn(f"[bench] rows ll_dispatch / ll_combine: {w.name}")
    inp = wl.make_inputs(w)
    T, H, K, E, cap = w.tokens, w.hidden, w.topk, w.experts, w.ll_capacity
    buf = Buffer(E, w.ranks, num_channels=1, max_tokens=T)
    nb = ctypes.c_size_t()
    C.check(C.moedx_ll_workspace_bytes(buf.ctx, T, K, cap, ctypes.byref(nb)))
    ids = inp.topk_idx.to(dev)
    wts = inp.topk_weights.to(dev)
    llsets = []
    for _ in range(NSETS):
        llsets.append({"x": inp.x.to(dev), "ws": torch.empty(nb.value, dtype=torch.uint8, device=dev),
                       "recv": torch.empty(E, cap, H, dtype=torch.bfloat16, device=dev),
                       "cnt": torch.empty(E, dtype=torch.int32, device=dev),
                       "out": torch.empty(T, H, dtype=torch.bfloat16, device=dev), "h": None})

    def ll_dispatch(s):
        def f():
            h = ctypes.c_void_p()
            C.check(C.moedx_ll_dispatch(buf.ctx, P(s["x"]), P(ids), T, K, H, cap, P(s["recv"]),
                                        P(s["cnt"]), P(s["ws"]), nb.value, ctypes.byref(h), cur[0]))
            if s["h"] is not None:
                C.moedx_handle_destroy(s["h"])
            s["h"] = h
        return f

    def ll_combine(s):
        return lambda: C.check(C.moedx_ll_combine(buf.ctx, P(s["recv"]), P(ids), P(wts), s["h"], H,
                                                  P(s["out"]), cur[0]))

    fns_d, fns_c = [ll_dispatch(s) for s in llsets], [ll_combine(s) for s in llsets]
    ms_d = timed(fns_d)
    dist_d = per_launch(fns_d)
    ms_c = timed(fns_c)
    dist_c = per_launch(fns_c)
    V = int((inp.topk_idx >= 0).sum())
    cpu_d = cpu_c = None
    if o is not None:
        xs, idn, wn = u16(inp.x), inp.topk_idx.numpy(), inp.topk_weights.numpy()
        res = {}

        def run_d():
            res["d"] = o.ll_dispatch(xs, idn, E, cap)

        secs, reps = _median_time(run_d, cpu_budget_s / 8)
        cpu_d = cpu_entry(row_bytes("ll_dispatch", T, H, K, E, V=V), secs, reps,
                          f"oracle ll_dispatch on the full {T}-token workload")
        recv_o, _, _, slot_o = res["d"]
        secs, reps = _median_time(lambda: o.ll_combine(recv_o, idn, wn, slot_o), cpu_budget_s / 8)
        cpu_c = cpu_entry(row_bytes("ll_combine", T, H, K, E, V=V), secs, reps,
                          f"oracle ll_combine on the full {T}-token workload")
    note = {"bound_note": "latency: a few MB per launch", "slots_filled": V,
            "cache_note": f"inputs ({inp.x.numel() * 2 / 1e6:.1f} MB of x, the handle) rotate over "
                          f"{NSETS} sets: they stay in the Infinity Cache, as a decode step's "
                          "activations would"}
    rows["ll_dispatch"] = entry(w, "ll_dispatch", ms_d, row_bytes("ll_dispatch", T, H, K, E, V=V),
                                dict(note, per_launch_us=dist_d), cpu_d)
    rows["ll_combine"] = entry(w, "ll_combine", ms_c, row_bytes("ll_combine", T, H, K, E, V=V),
                               dict(note, per_launch_us=dist_c), cpu_c)
    # the launch floor: the same call with no token launches one workgroup that
    # only writes the E counts (zeros), timed the way every row above is
    def ll_empty(s):
        def f():
            h = ctypes.c_void_p()
            C.check(C.moedx_ll_dispatch(buf.ctx, None, None, 0, K, H, cap, None, P(s["cnt"]),
                                        P(s["ws"]), nb.value, ctypes.byref(h), cur[0]))
            C.moedx_handle_destroy(h)
        return f

    fns = [ll_empty(s) for s in llsets]
    rows["launch_floor"] = {
        "us": round(timed(fns) * 1e3, 2), "per_launch_us": per_launch(fns),
        "note": "a one-workgroup kernel that writes 1 KB (the low-latency dispatch of an empty "
                "batch), timed as the rows above: what any launch costs on this path"}
    for s in llsets:
        if s["h"] is not None:
            C.moedx_handle_destroy(s["h"])
    del llsets, buf
    torch.cuda.synchronize()

    # Two workloads' whole timed regions, as the sums of rows above (each part
    # timed on its own rotation, as the headline step's dispatch and combine
    # are): the skewed FP8 workload's step (layout + scan + FP8 pack on a fresh
    # handle, then the bf16 combine) and the reuse workload's first call
    # (exact-mode first dispatch, then the combine), beside reuse_rep.
    def composite(name, parts, note):
        if not all(p in rows for p in parts):
            return
        us = sum(rows[p]["us"] for p in parts)
        nbytes = sum(rows[p]["bytes"] for p in parts)
        gbs = nbytes / (us * 1e-6) / 1e9
        rows[name] = {"workload": rows[parts[0]]["workload"], "us": round(us, 2),
                      "bytes": int(nbytes), "GBps": round(gbs, 1),
                      "roofline_frac": round(gbs / HBM_PEAK_GBS, 4), "parts": list(parts),
                      "note": note}

    composite("step_fp8_skewed", ("first_dispatch_fp8", "combine_fp8_skewed"),
              "sum of the two rows: the FP8 workload's timed region (first FP8 dispatch, then "
              "the bf16 combine of rows shaped like the receive buffer)")
    composite("first_call_reuse", ("first_dispatch_exact", "combine_reuse"),
              "sum of the two rows: the reuse workload's first call (exact mode: layout, host "
              "wait, pack; then the combine); reuse_rep is one repetition after it")
    return rows


def batch_sweep(token_counts, steps, log_fn):
    """The step (dispatch = layout + first pack on a fresh handle, then the
    combine; capacity mode) of the prefill workload's routing and hidden size at
    other batch sizes, every input read from HBM; one JSON line per batch size
    (the layout alone is timed beside it)."""
    import torch

    from combine_get_dispatch_layout_amd import Buffer
    from combine_get_dispatch_layout_amd import _capi as C
    from combine_get_dispatch_layout_amd import workloads as wl

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    ex = C.make_exec(stream.cuda_stream, None, None, C.MOEDX_ASYNC)
    exr = ctypes.byref(ex)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    sink = torch.empty((), dtype=torch.float32, device=dev)
    w = wl.PREFILL
    H, K, E, R, Ch = w.hidden, w.topk, w.experts, w.ranks, w.channels
    for T in token_counts:
        log_fn(f"[bench] batch sweep: {T} tokens")
        inp = wl.make_inputs(w, tokens=T)
        buf = Buffer(E, R, num_channels=Ch, max_tokens=T)
        cap = T * min(K, R)
        nb = ctypes.c_size_t()
        C.check(C.moedx_handle_workspace_bytes(buf.ctx, T, K, cap, ctypes.byref(nb)))
        nsets = input_copies(2 * T * H)
        idx, gw = inp.topk_idx.to(dev), inp.topk_weights.to(dev)
        sets = []
        for _ in range(nsets):
            s = {"x": inp.x.to(dev), "ws": torch.empty(nb.value, dtype=torch.uint8, device=dev),
                 "recv": torch.empty(cap, H, dtype=torch.bfloat16, device=dev),
                 "rti": torch.empty(cap, K, dtype=torch.int64, device=dev),
                 "rtw": torch.empty(cap, K, dtype=torch.float32, device=dev),
                 "out": torch.empty(T, H, dtype=torch.bfloat16, device=dev)}
            h = ctypes.c_void_p()
            C.check(C.moedx_dispatch_prepare(buf.ctx, P(idx), T, K, None, None, None, P(s["ws"]), nb.value, cap,
                                             ctypes.byref(h), exr))
            s["h"] = h
            sets.append(s)

        def first_pack(h, s):
            C.check(C.moedx_dispatch(buf.ctx, h, P(s["x"]), T, H, C.MOEDX_QUANT_NONE,
                                     P(idx), P(gw), P(s["recv"]), None, P(s["rti"]),
                                     P(s["rtw"]), exr))

        def op(name, i):
            s = sets[i % nsets]
            if name in ("layout", "dispatch"):
                h = ctypes.c_void_p()
                C.check(C.moedx_dispatch_prepare(buf.ctx, P(idx), T, K, None, None, None, P(s["ws"]), nb.value, cap,
                                                 ctypes.byref(h), exr))
                if name == "dispatch":
                    first_pack(h, s)
                C.moedx_handle_destroy(h)
            else:
                C.check(C.moedx_combine(buf.ctx, s["h"], P(s["recv"]), H, P(gw), None,
                                        P(s["out"]), None, exr))

        for i in range(nsets):
            first_pack(sets[i]["h"], sets[i])
        torch.cuda.synchronize()
        dev_n = ctypes.c_void_p()
        shape = (ctypes.c_int64 * 2)()
        C.check(C.moedx_handle_tensor(sets[0]["h"], C.MOEDX_T_NUM_RECV, ctypes.byref(dev_n), shape))
        off = dev_n.value - sets[0]["ws"].data_ptr()
        N = int(sets[0]["ws"][off:off + 4].view(torch.int32).item())
        us = {}
        for name in ("dispatch", "combine", "layout"):
            for _ in range(2):  # the first pass warms up
                torch.sum(flush_buf, dim=(0,), out=sink)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for i in range(steps):
                    op(name, i)
                b.record(stream)
                torch.cuda.synchronize()
                us[name] = round(a.elapsed_time(b) * 1e3 / steps, 2)
        byts = algorithmic_bytes(T, H, K, E, R, Ch, N)
        step_us = us["dispatch"] + us["combine"]
        gbs = sum(byts.values()) / (step_us * 1e-6) / 1e9
        dispatch_bytes = byts["layout"] + byts["pack"]
        print(json.dumps({"tokens": T, "hidden": H, "recv_rows": N, "buffer_sets": nsets,
                          "kernels_us": us, "step_us": round(step_us, 2), "GBps": round(gbs, 1),
                          "roofline_frac": round(gbs / HBM_PEAK_GBS, 4),
                          "dispatch_frac": round(dispatch_bytes / (us["dispatch"] * 1e-6) / 1e9
                                                 / HBM_PEAK_GBS, 4),
                          "combine_frac": round(byts["combine"] / (us["combine"] * 1e-6) / 1e9
                                                / HBM_PEAK_GBS, 4)}), flush=True)
        for s in sets:
            C.moedx_handle_destroy(s["h"])
        del sets, buf
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget-s", type=float, default=10.0,
                    help="seconds of CPU time for the oracle baseline (0 skips it)")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the further steps (FP8 pack, cached dispatch, standalone "
                         "layout, low-latency pair) on their own workloads")
    ap.add_argument("--batch-sweep", type=str, default=None, metavar="T1,T2,...",
                    help="instead of the step line, one line per batch size: the same step "
                         "with the prefill routing and hidden size at these token counts")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the exchange (logical ranks are buckets "
              "in one HBM); runs on more than one GPU are not part of this build.",
              file=sys.stderr)
        sys.exit(2)
    if args.batch_sweep:
        batch_sweep([int(v) for v in args.batch_sweep.split(",")], args.steps, log)
        return

    import torch

    from combine_get_dispatch_layout_amd import Buffer
    from combine_get_dispatch_layout_amd import _capi as C
    from combine_get_dispatch_layout_amd import workloads as wl

    w = wl.PREFILL
    T, H, K, E, R, Ch = w.tokens, w.hidden, w.topk, w.experts, w.ranks, w.channels
    log(f"[bench] generating {w.name}")
    inp = wl.make_inputs(w)
    inputs_sha256 = input_digests(inp)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cap = T * min(K, R)
    buf = Buffer(E, R, num_channels=Ch, max_tokens=T)
    ctx = buf.ctx
    nbytes = ctypes.c_size_t()
    C.check(C.moedx_handle_workspace_bytes(ctx, T, K, cap, ctypes.byref(nbytes)))
    # NSETS independent buffer sets, used in rotation so that no launch reads
    # data a recent launch touched: the 256 MB Infinity Cache holds a good part
    # of a freshly written receive buffer, and up to four 58.7 MB copies of x.
    NSETS = input_copies(2 * T * H)
    idx = inp.topk_idx.to(dev)
    gw = inp.topk_weights.to(dev)
    sets = []
    for _ in range(NSETS):
        sets.append({
            "x": inp.x.to(dev),
            "ws": torch.empty(nbytes.value, dtype=torch.uint8, device=dev),
            "recv": torch.empty(cap, H, dtype=torch.bfloat16, device=dev),
            "rti": torch.empty(cap, K, dtype=torch.int64, device=dev),
            "rtw": torch.empty(cap, K, dtype=torch.float32, device=dev),
            "out": torch.empty(T, H, dtype=torch.bfloat16, device=dev),
        })
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    sink = torch.empty((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    p_idx, p_gw = P(idx), P(gw)
    ex = C.make_exec(stream.cuda_stream, None, None, C.MOEDX_ASYNC)
    exr = ctypes.byref(ex)

    def flush():
        torch.sum(flush_buf, dim=(0,), out=sink)

    def prepare(s_, e=exr):
        h = ctypes.c_void_p()
        C.check(C.moedx_dispatch_prepare(ctx, p_idx, T, K, None, None, None, P(s_["ws"]), nbytes.value, cap,
                                         ctypes.byref(h), e))
        return h

    def pack(h, s_, e=exr):
        C.check(C.moedx_dispatch(ctx, h, P(s_["x"]), T, H, C.MOEDX_QUANT_NONE, p_idx, p_gw,
                                 P(s_["recv"]), None, P(s_["rti"]), P(s_["rtw"]), e))

    def combine(h, s_, e=exr):
        C.check(C.moedx_combine(ctx, h, P(s_["recv"]), H, p_gw, None, P(s_["out"]), None, e))

    def record():
        ev = ctypes.c_void_p()
        C.check(C.moedx_event_record(ctypes.byref(ev), stream.cuda_stream))
        return ev.value

    def elapsed_ms(a, b):
        ms = ctypes.c_float()
        C.check(C.moedx_event_elapsed_ms(a, b, ctypes.byref(ms)))
        C.moedx_event_destroy(a)
        C.moedx_event_destroy(b)
        return ms.value

    # The normal-kernel example's call order: get_dispatch_layout into its own
    # outputs, then the first dispatch given them (a scan of the handle from
    # is_token_in_rank and the expert totals, then the first pack).
    lay_out = [{"ntr": torch.empty(R, dtype=torch.int32, device=dev),
                "nte": torch.empty(E, dtype=torch.int32, device=dev),
                "itr": torch.empty(T, R, dtype=torch.uint8, device=dev)} for _ in range(NSETS)]

    def layout_call(lo, e=exr):
        C.check(C.moedx_get_dispatch_layout(ctx, p_idx, T, K, P(lo["ntr"]), P(lo["nte"]),
                                            P(lo["itr"]), e))

    def prepare_from(s_, lo, e=exr):
        h = ctypes.c_void_p()
        C.check(C.moedx_dispatch_prepare(ctx, p_idx, T, K, P(lo["ntr"]), P(lo["itr"]),
                                         P(lo["nte"]), P(s_["ws"]), nbytes.value, cap,
                                         ctypes.byref(h), e))
        return h

    def layout_then_dispatch(j):
        layout_call(lay_out[j])
        h = prepare_from(sets[j], lay_out[j])
        pack(h, sets[j])
        C.moedx_handle_destroy(h)

    # Each set's handle, finished by its first pack; the combine runs on these.
    handles = [prepare(s_) for s_ in sets]
    for h, s_ in zip(handles, sets):
        pack(h, s_)

    def dispatch(s_, e=exr, e_pack=None):
        """The step's dispatch on a fresh handle: the layout's partials, then the
        first pack, which also finishes the handle's prefixes."""
        h = prepare(s_, e)
        pack(h, s_, e_pack if e_pack is not None else e)
        C.moedx_handle_destroy(h)

    def op_avg_ms(op, n):
        """Average duration of n back-to-back runs of one op over rotating sets."""
        flush()
        a = record()
        for i in range(n):
            j = i % NSETS
            if op == "layout":
                C.moedx_handle_destroy(prepare(sets[j]))
            elif op == "dispatch":
                dispatch(sets[j])
            elif op == "layout_then_dispatch":
                layout_then_dispatch(j)
            else:
                combine(handles[j], sets[j])
        b = record()
        torch.cuda.synchronize()
        return elapsed_ms(a, b) / n

    def op_kernel_us(op, n):
        """Kernel durations of one kernel per run over n back-to-back runs on
        rotating sets: p10 / median / p90 / mean ("pack": the first pack of each
        dispatch, its layout launch unstamped before it)."""
        def launch(i, e):
            j = i % NSETS
            if op == "layout":
                C.moedx_handle_destroy(prepare(sets[j], e))
            elif op == "pack":
                dispatch(sets[j], exr, e)
            else:
                combine(handles[j], sets[j], e)
        return kernel_us_distribution(C, stream, launch, n, flush)

    def pipelined_ms(n):
        """n whole steps back to back (layout, first pack, combine each), rotating sets."""
        flush()
        a = record()
        for i in range(n):
            s_ = sets[i % NSETS]
            h = prepare(s_)
            pack(h, s_)
            combine(h, s_)
            C.moedx_handle_destroy(h)
        b = record()
        torch.cuda.synchronize()
        return elapsed_ms(a, b) / n

    log(f"[bench] warmup {args.warmup}")
    for op in ("layout", "dispatch", "combine", "layout_then_dispatch"):
        op_avg_ms(op, max(args.warmup, 1))
    pipelined_ms(max(args.warmup, 1))
    torch.cuda.synchronize()
    h = handles[0]
    dev_n = ctypes.c_void_p()
    shape = (ctypes.c_int64 * 2)()
    C.check(C.moedx_handle_tensor(h, C.MOEDX_T_NUM_RECV, ctypes.byref(dev_n), shape))
    off = dev_n.value - sets[0]["ws"].data_ptr()
    N = int(sets[0]["ws"][off:off + 4].view(torch.int32).item())
    bytes_ = algorithmic_bytes(T, H, K, E, R, Ch, N)
    step_bytes = sum(bytes_.values())
    log(f"[bench] N={N} receive rows; {step_bytes / 1e6:.1f} MB per step")

    log(f"[bench] timing: {args.steps} launches per op (HBM-cold rotation), {args.steps} pipelined steps")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_disp = op_avg_ms("dispatch", args.steps)
    t_comb = op_avg_ms("combine", args.steps)
    t_lay = op_avg_ms("layout", args.steps)
    ms_pipe = pipelined_ms(args.steps)
    wall = time.perf_counter() - wall0
    dist = {op: op_kernel_us(op, args.steps) for op in ("layout", "pack", "combine")}
    t_pack = dist["pack"]["mean"] * 1e-3  # ms: the first pack alone, kernel-stamped
    log("[bench] the pages' call order: get_dispatch_layout, dispatch given its outputs, combine")
    st0 = buf.stats()
    t_ltd = op_avg_ms("layout_then_dispatch", args.steps)
    st1 = buf.stats()
    ltd_launches = {k: round((st1[k] - st0[k]) / args.steps, 3)
                    for k in ("layout_launches", "scan_launches", "pack_launches")}

    # Exact mode through the API on the host clock: the host waits for N after
    # the layout (no capacity bound), then the pack and the combine run.
    nb_exact = ctypes.c_size_t()
    C.check(C.moedx_handle_workspace_bytes(ctx, T, K, 0, ctypes.byref(nb_exact)))
    ws_exact = torch.empty(nb_exact.value, dtype=torch.uint8, device=dev)
    blocking = C.make_exec(stream.cuda_stream, None, None, 0)

    def exact_step(s_):
        h_ = ctypes.c_void_p()
        C.check(C.moedx_dispatch_prepare(ctx, p_idx, T, K, None, None, None, P(ws_exact), nb_exact.value, 0,
                                         ctypes.byref(h_), ctypes.byref(blocking)))
        pack(h_, s_)
        combine(h_, s_, ctypes.byref(blocking))
        C.moedx_handle_destroy(h_)

    wall_exact = []
    for i in range(max(args.warmup, 1) + args.steps):
        t0 = time.perf_counter()
        exact_step(sets[i % NSETS])
        if i >= max(args.warmup, 1):
            wall_exact.append((time.perf_counter() - t0) * 1e6)
    wall_exact.sort()
    ms = t_disp + t_comb
    gbs = step_bytes / (ms * 1e-3) / 1e9
    for h in handles:
        C.moedx_handle_destroy(h)

    log("[bench] plain device read, write and copy of one receive buffer's size (context: "
        "practical ceilings)")
    ceil = hbm_ceilings(2 * N * H, max(args.steps, 10), flush)
    copy_gbs = ceil["copy_GBps"]

    t_comb_k = dist["combine"]["mean"] * 1e-3
    kern = {"pack": (t_pack, bytes_["pack"]), "combine": (t_comb_k, bytes_["combine"])}
    dom = max(kern, key=lambda k: kern[k][0])
    dom_ms, dom_bytes = kern[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = measured_traffic(dom)

    cpu = None
    if args.cpu_budget_s > 0:
        threads = cpu_threads()
        log(f"[bench] CPU oracle baseline on {threads} threads and on 1 "
            f"(~{args.cpu_budget_s:.0f} s)")
        t_all, reps_all, n_all = cpu_baseline(inp, w, args.cpu_budget_s / 3, threads)
        t_one, reps_one, n_one = cpu_baseline(inp, w, 2 * args.cpu_budget_s / 3, 1)
        assert n_all == N and n_one == N
        cpu = {"value": round(step_bytes / t_all / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle", "tokens_per_s": round(T / t_all, 1), "cpu_model": cpu_model(),
               "affinity_cpus": len(os.sched_getaffinity(0)),
               "sample": f"median of {reps_all} full {T}x{H} steps (layout+prefix+pack+weighted "
                         f"combine) of the C oracle, its per-token parts over {threads} token "
                         f"ranges on {threads} threads (the prefix scan on one)",
               "single_thread": {"value": round(step_bytes / t_one / 1e9, 4), "unit": "GB/s",
                                 "cores": 1, "tokens_per_s": round(T / t_one, 1),
                                 "sample": f"median of {reps_one} full steps, one thread"}}

    rows = None
    if not args.no_rows:
        rows = measure_rows(args.steps, args.warmup, args.cpu_budget_s, flush, log)

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
        "inputs_sha256": inputs_sha256,
        "config": {"workload": w.name, "tokens": T, "hidden": H, "experts": E, "topk": K,
                   "ranks": R, "channels": Ch, "routing": w.routing, "recv_rows": N,
                   "mode": "capacity (no host sync)",
                   "timing": "dispatch (layout partials + first pack on a fresh handle) plus "
                             "combine, each the mean over back-to-back runs rotating over "
                             f"{NSETS} buffer sets, so that every input is read from HBM (not "
                             "the Infinity Cache); HIP events"},
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "step_roofline_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "ops_us": {"dispatch": round(t_disp * 1e3, 2), "combine": round(t_comb * 1e3, 2),
                   "layout_alone": round(t_lay * 1e3, 2)},
        "kernels_us": {"layout": dist["layout"]["mean"], "pack": dist["pack"]["mean"],
                       "combine": dist["combine"]["mean"]},
        "kernels_us_per_launch": dist,
        "kernel_GBps": {"pack": round(bytes_["pack"] / (t_pack * 1e-3) / 1e9, 1),
                        "combine": round(bytes_["combine"] / (t_comb_k * 1e-3) / 1e9, 1)},
        "layout_then_dispatch": {
            "dispatch_us": round(t_ltd * 1e3, 2), "combine_us": round(t_comb * 1e3, 2),
            "step_us": round((t_ltd + t_comb) * 1e3, 2),
            "GBps": round(step_bytes / ((t_ltd + t_comb) * 1e-3) / 1e9, 1),
            "roofline_frac": round(step_bytes / ((t_ltd + t_comb) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tokens_per_s": round(T / ((t_ltd + t_comb) * 1e-3), 1),
            "launches_per_dispatch": ltd_launches,
            "note": "the normal-kernel example's order: get_dispatch_layout, then the first "
                    "dispatch given num_tokens_per_rank / is_token_in_rank / "
                    "num_tokens_per_expert (its handle borrows the partials the layout left "
                    "in the ctx: no second layout and no scan, the first pack finishes the "
                    "handle), then the same combine; same buffer rotation and byte count as "
                    "the step"},
        "pipelined_ms_per_step": round(ms_pipe, 5),
        "exact_mode_api_wall_us": {
            "median": round(statistics.median(wall_exact), 1),
            "p10": round(wall_exact[int(0.1 * (len(wall_exact) - 1))], 1),
            "p90": round(wall_exact[int(round(0.9 * (len(wall_exact) - 1)))], 1),
            "note": "host clock; layout, host wait for N and the per-expert counts, pack, "
                    "combine, host wait"},
        "pipelined_GBps_cache_assisted": round(step_bytes / (ms_pipe * 1e-3) / 1e9, 1),
        "copy_ceiling_GBps": round(copy_gbs, 1),
        "hbm_ceilings": ceil,
        "algorithmic_bytes": bytes_,
        "wall_s_timed": round(wall, 4),
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
