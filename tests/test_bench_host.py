"""Host-side pieces of bench.py that need no GPU: the one-GPU guard, the input
rotation that keeps every timed launch reading from HBM, and the traffic
figures that are reported only for the kernel source they were measured on."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_rotation_reads_at_least_twice_the_infinity_cache_between_reuses():
    for nbytes in (1 << 20, 58_720_256, 117_440_512, 233_000_000, 1 << 30):
        n = bench.input_copies(nbytes)
        assert n >= 3
        # between two reads of one copy, the other n - 1 copies are read
        assert (n - 1) * nbytes >= 2 * bench.INFINITY_CACHE_BYTES


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    summary = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))
    for op, rec in summary["ops"].items():
        assert rec["traffic_bytes_per_launch"] > 0
        # the figure while the source matches the one profiled, nothing after a change
        same = rec["source_sha256_16"] == bench.source_digest(rec["source"])
        assert bench.measured_traffic(op) == (rec["traffic_bytes_per_launch"] if same else None)
    # a different source (here: another kernel file) gives no figure
    monkeypatch.setitem(bench.TRAFFIC_SOURCES, "pack", "combine.hip")
    assert bench.measured_traffic("pack") is None
    assert bench.measured_traffic("no_such_op") is None


def test_all_cores_oracle_leg_equals_the_single_thread_step():
    """The CPU baseline's all-cores leg only splits the oracle's calls over
    token ranges: its receive rows and combined rows equal the one-thread
    oracle's."""
    import concurrent.futures as cf

    import numpy as np
    import torch

    import oracle as om
    from combine_get_dispatch_layout_amd import workloads as wl

    w = wl.PREFILL
    inp = wl.make_inputs(w, tokens=301)
    o = om.Oracle()
    x = inp.x.view(torch.int16).numpy().view(np.uint16)[:, :256].copy()
    idx, gw = inp.topk_idx.numpy(), inp.topk_weights.numpy()
    n1, rx1, out1 = bench.oracle_step(o, x, idx, gw, w.experts, w.ranks, w.channels)
    with cf.ThreadPoolExecutor(max_workers=4) as pool:
        n4, rx4, out4 = bench.oracle_step(o, x, idx, gw, w.experts, w.ranks, w.channels, 7, pool)
    assert n1 == n4
    assert np.array_equal(rx1, rx4)
    assert np.array_equal(out1, out4)
    assert bench.cpu_threads() >= 1


def test_headline_input_digests_are_stable():
    """The bench line records a digest of each generated input of the prefill
    workload; the seeded generator gives the same bytes on every run."""
    from combine_get_dispatch_layout_amd import workloads as wl
    d = bench.input_digests(wl.make_inputs(wl.PREFILL))
    assert d == {"x": "dc0bef52dad6fc0f", "topk_idx": "97eb46dbb565f6c3",
                 "topk_weights": "ee85ac06ed5a21f0"}
