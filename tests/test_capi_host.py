"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call."""

import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "combine_get_dispatch_layout_amd", "libmoedx.so")


@pytest.fixture(scope="module")
def capi():
    if not os.path.exists(LIB):
        from combine_get_dispatch_layout_amd import build
        build.build()
    from combine_get_dispatch_layout_amd import _capi
    return _capi


def test_header_symbols_are_exported(capi):
    names = capi.header_symbols()
    assert len(names) >= 20
    raw = ctypes.CDLL(capi.LIB_PATH)
    missing = [n for n in names if not hasattr(raw, n)]
    assert not missing, missing
    # the binding declares exactly the header's functions
    assert sorted(capi.SIGNATURES) == names


def test_only_api_symbols_are_exported(capi):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", capi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert {n for n in exported if n.startswith("moedx_")} == set(capi.header_symbols())


@pytest.mark.parametrize("args,code", [
    ((0, 16, 3, 2, 128, 0), -1),      # E % R != 0
    ((0, 16, 0, 2, 128, 0), -1),      # R < 1
    ((0, 16, 65, 2, 128, 0), -1),     # R > 64
    ((0, 2048, 8, 2, 128, 0), -1),    # E > 1024
    ((0, 16, 4, 0, 128, 0), -1),      # C < 1
    ((0, 16, 4, 2, -1, 0), -1),       # max_tokens < 0
    ((0, 16, 4, 2, 128, 7), -1),      # unknown flags
    ((-1, 16, 4, 2, 128, 0), -1),     # device < 0
])
def test_create_validates_before_hip(capi, args, code):
    ctx = ctypes.c_void_p(123)
    rc = capi.moedx_create(ctypes.byref(ctx), *args)
    assert rc == code
    assert ctx.value is None
    assert capi.last_error()


def test_null_arguments_are_rejected(capi):
    assert capi.moedx_event_wait(None, None) == capi.MOEDX_EINVAL
    assert capi.moedx_event_synchronize(None) == capi.MOEDX_EINVAL
    assert capi.moedx_event_record(None, None) == capi.MOEDX_EINVAL
    assert capi.moedx_handle_num_recv(None, None) == capi.MOEDX_EINVAL
    assert capi.moedx_handle_tensor(None, 0, None, None) == capi.MOEDX_EINVAL
    assert capi.moedx_ctx_stats(None, None) == capi.MOEDX_EINVAL
    assert capi.moedx_dispatch_prepare(None, None, 0, 1, None, None, None, None, 0, 0, None, None) == capi.MOEDX_EINVAL
    assert capi.moedx_combine(None, None, None, 8, None, None, None, None, None) == capi.MOEDX_EINVAL
    assert capi.moedx_handle_finish(None, None, None) == capi.MOEDX_EINVAL
    assert capi.moedx_dispatch_fp8(None, None, None, 0, 128, None, None, None, None) == capi.MOEDX_EINVAL
    assert capi.moedx_ll_dispatch_recv(None, None, None, None, 8, None, None) == capi.MOEDX_EINVAL
    assert capi.moedx_ll_combine(None, None, None, None, None, 8, None, None) == capi.MOEDX_EINVAL
    assert capi.moedx_destroy(None) == capi.MOEDX_OK
    assert capi.moedx_handle_destroy(None) == capi.MOEDX_OK
    assert capi.moedx_event_destroy(None) == capi.MOEDX_OK


def test_releases_wait_for_the_end_of_a_capture():
    """Finalizer releases queue while a stream capture runs and happen at the
    next release or call outside a capture, most recent first."""
    from combine_get_dispatch_layout_amd import buffer as bm

    done = []
    assert not bm._deferred
    bm._release(done.append, 1, _capturing=lambda: True)
    bm._release(done.append, 2, _capturing=lambda: True)
    assert done == [] and len(bm._deferred) == 2
    bm._flush_deferred(_capturing=lambda: True)  # still capturing: nothing happens
    assert done == []
    bm._release(done.append, 3, _capturing=lambda: False,
                _flush=lambda: bm._flush_deferred(_capturing=lambda: False))
    assert done == [3, 2, 1] and not bm._deferred


def test_ctx_set_stream_rejects_null(capi):
    assert capi.moedx_ctx_set_stream(None, ctypes.c_void_p(256)) == capi.MOEDX_EINVAL


def test_static_layout_validates_before_hip(capi):
    """The allocation-free layout rejects bad shapes before any HIP call (dummy
    non-null pointers are never touched)."""
    p = ctypes.c_void_p(256)
    assert capi.moedx_get_dispatch_layout_static(p, 10, 2, 16, 3, p, p, p, None) == capi.MOEDX_EINVAL
    assert capi.moedx_get_dispatch_layout_static(p, 10, 0, 16, 4, p, p, p, None) == capi.MOEDX_EINVAL
    assert capi.moedx_get_dispatch_layout_static(p, 10, 2, 16, 65, p, p, p, None) == capi.MOEDX_EINVAL
    assert capi.moedx_get_dispatch_layout_static(p, -1, 2, 16, 4, p, p, p, None) == capi.MOEDX_EINVAL
    assert capi.moedx_get_dispatch_layout_static(None, 10, 2, 16, 4, p, p, p, None) == capi.MOEDX_EINVAL
    assert capi.moedx_get_dispatch_layout_static(p, (1 << 24) + 1, 8, 1024, 64, p, p, p, None) \
        == capi.MOEDX_EINVAL
    assert capi.moedx_get_dispatch_layout_static(p, 10, 2, 2048, 64, p, p, p, None) == capi.MOEDX_EINVAL
