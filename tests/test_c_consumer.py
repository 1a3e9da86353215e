"""The C ABI from plain C: tests/c_consumer.c includes include/moedx.h and
links libmoedx.so with gcc (C11, warnings as errors), with no C++ and no
Python in the program.  On the CPU it checks the host-side validation; on the
GPU it runs one exact-mode step (layout, prepare from the layout's outputs,
first dispatch, gate-weighted combine) whose outputs are compared with the
oracle."""

import os
import struct
import subprocess

import numpy as np
import pytest
import torch

import oracle as om
from combine_get_dispatch_layout_amd import workloads as wl
from tests import device_check
from tests.helpers import bf16_bits


def _binary(tmp_path=None):
    if tmp_path is not None:  # a fresh build (CPU test: the compile itself is checked)
        return device_check.build_c_consumer(str(tmp_path / "c_consumer"))
    if not os.path.exists(device_check.C_BIN):
        device_check.build_c_consumer()
    return device_check.C_BIN


def test_header_is_plain_c_and_validation_runs_without_gpu(tmp_path):
    lib = os.path.join(os.path.dirname(device_check.HERE), "combine_get_dispatch_layout_amd",
                       "libmoedx.so")
    if not os.path.exists(lib):
        from combine_get_dispatch_layout_amd import build
        build.build()
    exe = _binary(tmp_path)
    env = dict(os.environ, LD_LIBRARY_PATH=os.path.dirname(lib) + ":" + os.environ.get(
        "LD_LIBRARY_PATH", ""))
    r = subprocess.run([exe, "validate"], capture_output=True, text=True, env=env, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "validate ok" in r.stdout


@pytest.mark.gpu
def test_c_program_step_matches_oracle(oracle, tmp_path):
    T, K, E, R, C, H = 700, 6, 64, 8, 5, 512
    rng = np.random.default_rng(77)
    idx = wl.random_routing(rng, T, E, K, p_empty=0.05)
    g = torch.Generator().manual_seed(77)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    w = torch.softmax(torch.randn(T, K, generator=g), -1).numpy().astype(np.float32)
    xb = bf16_bits(x)
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(struct.pack("<6i", T, K, E, R, C, H))
        f.write(idx.astype("<i8").tobytes())
        f.write(xb.astype("<u2").tobytes())
        f.write(w.astype("<f4").tobytes())
    print(f"[c] T={T} K={K} E={E} R={R} C={C} H={H}", flush=True)
    r = subprocess.run([_binary(), "run", str(inp), str(out)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    buf = open(out, "rb").read()
    off = 0

    def take(dtype, n):
        nonlocal off
        a = np.frombuffer(buf, dtype=dtype, count=n, offset=off)
        off += a.nbytes
        return a

    N = int(take("<i4", 1)[0])
    ntr, nte = take("<i4", R), take("<i4", E)
    itr = take("u1", T * R).reshape(T, R)
    recv = take("<u2", N * H).reshape(N, H)
    rti = take("<i8", N * K).reshape(N, K)
    rtw = take("<f4", N * K).reshape(N, K)
    comb = take("<u2", T * H).reshape(T, H)
    assert off == len(buf)
    ref = om.dispatch(oracle, xb, idx, w, E, R, C)
    assert N == ref.prefix.num_recv
    np.testing.assert_array_equal(ntr, ref.layout.num_tokens_per_rank)
    np.testing.assert_array_equal(nte, ref.layout.num_tokens_per_expert)
    np.testing.assert_array_equal(itr, ref.layout.is_token_in_rank)
    np.testing.assert_array_equal(recv, ref.recv_x)
    np.testing.assert_array_equal(rti, ref.recv_topk_idx)
    np.testing.assert_array_equal(rtw.view(np.uint32), ref.recv_topk_weights.view(np.uint32))
    want, _ = oracle.combine(ref.recv_x, idx, E, ref.prefix, gate_weights=w)
    from tests.gpu_common import assert_bf16_within_1ulp
    assert_bf16_within_1ulp("combine", comb, want)
