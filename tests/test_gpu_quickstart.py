"""The README's Python quick start, run as written, with its results checked:
layout counts against their definitions, receive rows against the gather they
must equal, the gate-weighted combine of the identity expert against x
(bitwise: the gates of a token sum to one within a few fp32 ulps, far inside
half a bf16 ulp), the cached dispatch likewise, and sampled FP8 rows against
the oracle."""

import os
import re

import numpy as np
import pytest
import torch

from tests.gpu_common import device

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _snippet():
    text = open(os.path.join(ROOT, "README.md")).read()
    m = re.search(r"## Python quick start\s+```python\n(.*?)```", text, re.S)
    assert m, "README has no Python quick start block"
    return m.group(1)


def test_readme_quick_start(oracle):
    device()
    print("[quickstart] README snippet", flush=True)
    torch.manual_seed(0)
    ns = {}
    exec(compile(_snippet(), "README.md", "exec"), ns)
    torch.cuda.synchronize()
    T, E, K, R = ns["T"], ns["E"], ns["K"], ns["R"]
    x, idx = ns["x"], ns["topk_idx"]
    P = E // R
    # layout
    assert torch.equal(ns["nte"].long().cpu(), torch.bincount(idx.flatten().cpu(), minlength=E))
    in_rank = torch.zeros(T, R, dtype=torch.bool)
    in_rank[torch.arange(T).unsqueeze(1), (idx.cpu() // P)] = True
    assert torch.equal(ns["in_rank"].cpu(), in_rank)
    assert torch.equal(ns["ntr"].long().cpu(), in_rank.sum(0))
    # rows: bucket-major, ascending token inside a bucket
    src = in_rank.t().nonzero()[:, 1]
    h = ns["handle"].fields()
    assert torch.equal(h["recv_src_idx"].long().cpu(), src)
    recv = ns["recv_x"]
    assert recv.shape[0] == src.numel()
    assert torch.equal(recv.view(torch.int16).cpu(), x.view(torch.int16).cpu()[src])
    # gate-weighted combine of the identity expert gives x back
    assert torch.equal(ns["out"].view(torch.int16).cpu(), x.view(torch.int16).cpu())
    # the cached dispatch moved fresh rows through the same handle
    assert torch.equal(ns["recv2"].view(torch.int16).cpu(), ns["x2"].view(torch.int16).cpu()[src])
    # FP8: codes and scales of sampled rows against the oracle
    codes, scales = ns["codes"].cpu().numpy(), ns["scales"].cpu().numpy()
    xs = x.view(torch.int16).cpu().numpy().view(np.uint16)
    rows = np.random.default_rng(0).choice(src.numel(), size=16, replace=False)
    for row in rows:
        ref_codes, ref_scales = oracle.quant_row_fp8(xs[src[row]])
        np.testing.assert_array_equal(codes[row], ref_codes)
        np.testing.assert_array_equal(scales[row].view(np.uint32),
                                      np.asarray(ref_scales, np.float32).view(np.uint32))
