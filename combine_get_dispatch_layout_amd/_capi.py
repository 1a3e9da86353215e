"""ctypes binding of libmoedx.so: the C entry points under their own names.

Argument marshalling only; every step of the path runs in the library's HIP
kernels.  Loading fails loudly when the library has not been built; there is
no fallback.
"""

from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoedx.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "moedx.h")

# status codes
MOEDX_OK = 0
MOEDX_EINVAL = -1
MOEDX_ENOMEM = -2
MOEDX_EHIP = -3
MOEDX_ECAPACITY = -4
MOEDX_ESTATE = -5

MOEDX_ON_CTX_STREAM = 1
MOEDX_ASYNC = 2

MOEDX_QUANT_NONE = 0
MOEDX_QUANT_FP8_E4M3_1X128 = 1

MOEDX_FP8_SCALE_AMAX = 0
MOEDX_FP8_SCALE_POW2 = 1
MOEDX_FP8_SCALE_UE8M0 = 2
MOEDX_FP8_SCALE_TENSOR = 3

# handle tensors
MOEDX_T_RANK_PREFIX_MATRIX = 0
MOEDX_T_CHANNEL_PREFIX_MATRIX = 1
MOEDX_T_RECV_CHANNEL_PREFIX_MATRIX = 2
MOEDX_T_RECV_SRC_IDX = 3
MOEDX_T_IS_TOKEN_IN_RANK = 4
MOEDX_T_SEND_HEAD = 5
MOEDX_T_NUM_TOKENS_PER_RANK = 6
MOEDX_T_NUM_TOKENS_PER_EXPERT = 7
MOEDX_T_NUM_RECV = 8
MOEDX_T_LL_SRC_IDX = 9
MOEDX_T_LL_SLOT_OF = 10


class moedx_exec(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("prev", ctypes.c_void_p),
                ("done", ctypes.c_void_p), ("flags", ctypes.c_uint32),
                ("kernel_start", ctypes.c_void_p), ("kernel_stop", ctypes.c_void_p)]


class moedx_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "layout_launches", "pack_launches", "pack_fp8_launches",
        "combine_launches", "ll_dispatch_launches", "ll_combine_launches", "host_syncs",
        "scan_launches")]


class moedx_fp8(ctypes.Structure):
    _fields_ = [("scale_mode", ctypes.c_int), ("prequantized", ctypes.c_int),
                ("tensor_scale", ctypes.c_float), ("x_scales", ctypes.c_void_p)]


class MoedxError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"moedx error {code}: {msg}")
        self.code = code


_P = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_EX = ctypes.POINTER(moedx_exec)

SIGNATURES = {
    "moedx_last_error": (ctypes.c_char_p, []),
    "moedx_create": (_I, [_PP, _I, _I, _I, _I, _I, ctypes.c_uint32]),
    "moedx_destroy": (_I, [_P]),
    "moedx_ctx_stats": (_I, [_P, ctypes.POINTER(moedx_stats)]),
    "moedx_ctx_stream": (_I, [_P, _PP]),
    "moedx_ctx_set_stream": (_I, [_P, _P]),
    "moedx_event_record": (_I, [_PP, _P]),
    "moedx_event_create": (_I, [_PP]),
    "moedx_event_wait": (_I, [_P, _P]),
    "moedx_event_synchronize": (_I, [_P]),
    "moedx_event_elapsed_ms": (_I, [_P, _P, ctypes.POINTER(ctypes.c_float)]),
    "moedx_event_destroy": (_I, [_P]),
    "moedx_get_dispatch_layout": (_I, [_P, _P, _I, _I, _P, _P, _P, _EX]),
    "moedx_get_dispatch_layout_static": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P]),
    "moedx_handle_workspace_bytes": (_I, [_P, _I, _I, _I64, ctypes.POINTER(_SZ)]),
    "moedx_dispatch_prepare": (_I, [_P, _P, _I, _I, _P, _P, _P, _P, _SZ, _I64, _PP, _EX]),
    "moedx_handle_num_recv": (_I, [_P, ctypes.POINTER(_I64)]),
    "moedx_handle_recv_tokens_per_expert": (_I, [_P, _P]),
    "moedx_handle_tensor": (_I, [_P, _I, _PP, ctypes.POINTER(_I64)]),
    "moedx_handle_finish": (_I, [_P, _P, _EX]),
    "moedx_handle_destroy": (_I, [_P]),
    "moedx_dispatch": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _EX]),
    "moedx_dispatch_fp8": (_I, [_P, _P, _P, _I, _I, ctypes.POINTER(moedx_fp8), _P, _P, _EX]),
    "moedx_combine": (_I, [_P, _P, _P, _I, _P, _P, _P, _P, _EX]),
    "moedx_ll_workspace_bytes": (_I, [_P, _I, _I, _I, ctypes.POINTER(_SZ)]),
    "moedx_ll_dispatch": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _SZ, _PP, _EX]),
    "moedx_ll_dispatch_recv": (_I, [_P, _P, _P, _P, _I, _P, _EX]),
    "moedx_ll_combine": (_I, [_P, _P, _P, _P, _P, _I, _P, _EX]),
}


def header_symbols(path: str = HEADER) -> list:
    """Names of the functions include/moedx.h declares."""
    text = open(path).read()
    return sorted(set(re.findall(r"MOEDX_API\s+[\w\s\*]*?\b(moedx_\w+)\s*\(", text)))


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m combine_get_dispatch_layout_amd.build` "
            "(the MoE dispatch path has no fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = load()


def last_error() -> str:
    return lib.moedx_last_error().decode(errors="replace")


def check(rc: int) -> None:
    if rc != MOEDX_OK:
        raise MoedxError(rc, last_error())


def make_exec(stream: int = 0, prev=None, done=None, flags: int = 0, kernel_start=None,
              kernel_stop=None) -> moedx_exec:
    """prev / kernel_start / kernel_stop: event pointers (int) or None; done: a
    ctypes.c_void_p to receive the completion event, or None."""
    return moedx_exec(ctypes.c_void_p(stream or None), ctypes.c_void_p(prev or None),
                      ctypes.cast(ctypes.byref(done), ctypes.c_void_p) if done is not None else None,
                      flags, ctypes.c_void_p(kernel_start or None),
                      ctypes.c_void_p(kernel_stop or None))


# The entry points under their C names.
globals().update({name: getattr(lib, name) for name in SIGNATURES})
