"""CPU oracle for the MoE dispatch layout / pack / combine path.

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The product path (the
HIP library and its Python binding) never imports this package.

The arithmetic lives in ``oracle.c`` (plain scalar C, gcc ``-O2
-ffp-contract=off``); this module only marshals numpy arrays to it.  It shares
no code with the HIP library.

Arrays: bf16 data travels as ``np.uint16`` bit patterns, FP8 codes as
``np.uint8``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(src: str = _SRC, out: str = _LIB, extra: Optional[list] = None) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    cmd = ["gcc", *CFLAGS, *(extra or []), src, "-o", out + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(out + ".tmp", out)
    return out


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    sig = {
        "oracle_bf16_round": (ctypes.c_uint16, [ctypes.c_float]),
        "oracle_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "oracle_e4m3_encode": (ctypes.c_uint8, [ctypes.c_float]),
        "oracle_e4m3_decode": (ctypes.c_float, [ctypes.c_uint8]),
        "oracle_bf16_round_array": (None, [_P, _I64, _P]),
        "oracle_e4m3_encode_array": (None, [_P, _I64, _P]),
        "oracle_layout": (_I32, [_P, _I64, _I32, _I32, _I32, _P, _P, _P]),
        "oracle_prefix": (None, [_P, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P]),
        "oracle_pack_bf16": (None, [_P, _I64, _I64, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P]),
        "oracle_quant_row_fp8": (None, [_P, _I64, _P, _P]),
        "oracle_pack_fp8": (None, [_P, _I64, _I64, _I32, _P, _P, _P, _P]),
        "oracle_pow2_scale": (ctypes.c_float, [ctypes.c_float]),
        "oracle_quant_row_fp8_mode": (None, [_P, _I64, _I32, ctypes.c_float, _P, _P, _P]),
        "oracle_pack_fp8_mode": (None, [_P, _I64, _I64, _I32, _P, _P, _I32, ctypes.c_float, _P, _P,
                                        _P]),
        "oracle_pack_rows_bytes": (None, [_P, _I64, _I64, _I32, _P, _P, _P]),
        "oracle_combine": (None, [_P, _I64, _I64, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P]),
        "oracle_ll_dispatch": (_I32, [_P, _I64, _I64, _P, _I32, _I32, _I64, _P, _P, _P, _P]),
        "oracle_ll_combine": (None, [_P, _I64, _I64, _P, _P, _I64, _I32, _P, _P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib_cache: dict = {}


def load(path: str = _LIB) -> ctypes.CDLL:
    """Load (building first if absent) an oracle library."""
    if path not in _lib_cache:
        if not os.path.exists(path):
            build(out=path)
        _lib_cache[path] = _declare(ctypes.CDLL(path))
    return _lib_cache[path]


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


@dataclass
class Layout:
    num_tokens_per_rank: np.ndarray    # [R] int32
    num_tokens_per_expert: np.ndarray  # [E] int32
    is_token_in_rank: np.ndarray       # [T, R] uint8 (0/1)


@dataclass
class Prefix:
    rank_prefix_matrix: np.ndarray          # [R] int32, inclusive
    channel_prefix_matrix: np.ndarray       # [R, C] int32, inclusive
    recv_channel_prefix_matrix: np.ndarray  # [R, C] int32, exclusive
    send_head: np.ndarray                   # [T, R] int32, -1 where absent
    recv_src_idx: np.ndarray                # [N] int32
    num_recv: int                           # N


class Oracle:
    """Thin numpy front end over one compiled oracle library."""

    def __init__(self, path: str = _LIB):
        self.lib = load(path)

    # -- codecs ---------------------------------------------------------
    def bf16_round(self, f32: np.ndarray) -> np.ndarray:
        a = _c(f32, np.float32).reshape(-1)
        out = np.empty(a.shape, np.uint16)
        self.lib.oracle_bf16_round_array(_ptr(a), a.size, _ptr(out))
        return out.reshape(np.shape(f32))

    def e4m3_encode(self, f32: np.ndarray) -> np.ndarray:
        a = _c(f32, np.float32).reshape(-1)
        out = np.empty(a.shape, np.uint8)
        self.lib.oracle_e4m3_encode_array(_ptr(a), a.size, _ptr(out))
        return out.reshape(np.shape(f32))

    def e4m3_decode(self, codes: np.ndarray) -> np.ndarray:
        c = np.asarray(codes, dtype=np.uint8).reshape(-1)
        f = self.lib.oracle_e4m3_decode
        return np.array([f(int(v)) for v in c], dtype=np.float32).reshape(np.shape(codes))

    # -- layout and handle ----------------------------------------------
    def layout(self, topk_idx: np.ndarray, num_experts: int, num_ranks: int,
               out_itr: Optional[np.ndarray] = None) -> Layout:
        """out_itr: a C-contiguous uint8 [T, R] array (a row range of a larger
        one, say) that receives is_token_in_rank."""
        idx = _c(topk_idx, np.int64)
        T, K = idx.shape
        ntr = np.empty(num_ranks, np.int32)
        nte = np.empty(num_experts, np.int32)
        itr = np.empty((T, num_ranks), np.uint8) if out_itr is None else out_itr
        assert itr.shape == (T, num_ranks) and itr.dtype == np.uint8 and itr.flags["C_CONTIGUOUS"]
        rc = self.lib.oracle_layout(_ptr(idx), T, K, num_experts, num_ranks,
                                    _ptr(ntr), _ptr(nte), _ptr(itr))
        if rc != 0:
            raise ValueError("topk_idx holds an id outside {-1} u [0,E) or a repeated expert")
        return Layout(ntr, nte, itr)

    def prefix(self, is_token_in_rank: np.ndarray, num_channels: int) -> Prefix:
        itr = _c(is_token_in_rank, np.uint8)
        T, R = itr.shape
        C = num_channels
        rpm = np.empty(R, np.int32)
        cpm = np.empty((R, C), np.int32)
        rcpm = np.empty((R, C), np.int32)
        sh = np.empty((T, R), np.int32)
        src = np.empty(max(int(itr.sum()), 1), np.int32)
        n = ctypes.c_int64(0)
        self.lib.oracle_prefix(_ptr(itr), T, R, C, _ptr(rpm), _ptr(cpm), _ptr(rcpm), _ptr(sh),
                               _ptr(src), ctypes.byref(n))
        return Prefix(rpm, cpm, rcpm, sh, src[: n.value].copy(), int(n.value))

    # -- pack -------------------------------------------------------------
    def pack_bf16(self, x_u16: np.ndarray, topk_idx, topk_weights, num_experts: int,
                  pre: Prefix, with_topk: bool = True, out: Optional[tuple] = None):
        """out: preallocated (recv_x [N, H], recv_topk_idx [N, K] or None,
        recv_topk_weights [N, K] or None), written in place (a token range of
        x with the same rows of pre.send_head writes that range's rows)."""
        x = _c(x_u16, np.uint16)
        T, H = x.shape
        idx = _c(topk_idx, np.int64)
        K = idx.shape[1]
        R = pre.send_head.shape[1]
        assert pre.send_head.shape[0] == T
        N = pre.num_recv
        if out is not None:
            recv_x, rti, rtw = out
            assert recv_x.shape == (N, H) and recv_x.dtype == np.uint16
        else:
            recv_x = np.zeros((N, H), np.uint16)
            rti = np.empty((N, K), np.int64) if with_topk else None
            rtw = np.empty((N, K), np.float32) if (with_topk and topk_weights is not None) else None
        w = _c(topk_weights, np.float32) if topk_weights is not None else None
        self.lib.oracle_pack_bf16(_ptr(x), T, H, _ptr(idx), _ptr(w), K, num_experts, R,
                                  _ptr(pre.send_head), _ptr(pre.rank_prefix_matrix),
                                  _ptr(recv_x), _ptr(rti), _ptr(rtw))
        return recv_x, rti, rtw

    def quant_row_fp8(self, xrow_u16: np.ndarray):
        x = _c(xrow_u16, np.uint16).reshape(-1)
        H = x.size
        codes = np.empty(H, np.uint8)
        scales = np.empty(max(H // 128, 1), np.float32)
        self.lib.oracle_quant_row_fp8(_ptr(x), H, _ptr(codes), _ptr(scales))
        return codes, scales[: H // 128]

    def pack_fp8(self, x_u16: np.ndarray, pre: Prefix):
        x = _c(x_u16, np.uint16)
        T, H = x.shape
        R = pre.send_head.shape[1]
        N = pre.num_recv
        codes = np.zeros((N, H), np.uint8)
        scales = np.zeros((N, H // 128), np.float32)
        self.lib.oracle_pack_fp8(_ptr(x), T, H, R, _ptr(pre.send_head),
                                 _ptr(pre.rank_prefix_matrix), _ptr(codes), _ptr(scales))
        return codes, scales

    # FP8 scale modes (oracle_quant_row_fp8_mode): per-group amax / 448, the
    # power-of-two scale, the same as UE8M0 exponent bytes, one tensor scale.
    FP8_AMAX, FP8_POW2, FP8_UE8M0, FP8_TENSOR = 0, 1, 2, 3

    def pow2_scale(self, ap: float) -> float:
        return float(self.lib.oracle_pow2_scale(ap))

    def quant_row_fp8_mode(self, xrow_u16: np.ndarray, mode: int, tensor_scale: float = 0.0):
        """(codes [H] u8, scales [H/128]: fp32, u8 (UE8M0) or None (tensor))."""
        x = _c(xrow_u16, np.uint16).reshape(-1)
        H = x.size
        G = H // 128
        codes = np.empty(H, np.uint8)
        sf = np.zeros(max(G, 1), np.float32)
        su = np.zeros(max(G, 1), np.uint8)
        self.lib.oracle_quant_row_fp8_mode(_ptr(x), H, mode, tensor_scale, _ptr(codes), _ptr(sf),
                                           _ptr(su))
        scales = {self.FP8_UE8M0: su[:G], self.FP8_TENSOR: None}.get(mode, sf[:G])
        return codes, scales

    def pack_fp8_mode(self, x_u16: np.ndarray, pre: Prefix, mode: int, tensor_scale: float = 0.0):
        x = _c(x_u16, np.uint16)
        T, H = x.shape
        G = H // 128
        R = pre.send_head.shape[1]
        N = pre.num_recv
        codes = np.zeros((N, H), np.uint8)
        sf = np.zeros((N, G), np.float32) if mode in (self.FP8_AMAX, self.FP8_POW2) else None
        su = np.zeros((N, G), np.uint8) if mode == self.FP8_UE8M0 else None
        self.lib.oracle_pack_fp8_mode(_ptr(x), T, H, R, _ptr(pre.send_head),
                                      _ptr(pre.rank_prefix_matrix), mode, tensor_scale,
                                      _ptr(codes), _ptr(sf), _ptr(su))
        return codes, (su if mode == self.FP8_UE8M0 else sf)

    def pack_rows_bytes(self, src: np.ndarray, pre: Prefix) -> np.ndarray:
        """Receive rows of a [T, W] byte array (pre-quantised codes or scales)."""
        a = np.ascontiguousarray(src).view(np.uint8)
        T = a.shape[0]
        a = a.reshape(T, -1)
        W = a.shape[1]
        R = pre.send_head.shape[1]
        out = np.zeros((pre.num_recv, W), np.uint8)
        self.lib.oracle_pack_rows_bytes(_ptr(a), T, W, R, _ptr(pre.send_head),
                                        _ptr(pre.rank_prefix_matrix), _ptr(out))
        return out

    # -- combine ------------------------------------------------------------
    def combine(self, y_u16: np.ndarray, topk_idx, num_experts: int, pre: Prefix,
                gate_weights=None, recv_topk_weights=None, out: Optional[np.ndarray] = None):
        """out: a preallocated C-contiguous uint16 [T, H] array (a token range of
        a larger one, with the same rows of topk_idx, pre.send_head and
        gate_weights) that receives the combined rows."""
        y = _c(y_u16, np.uint16)
        H = y.shape[1]
        idx = _c(topk_idx, np.int64)
        T, K = idx.shape
        R = pre.send_head.shape[1]
        assert pre.send_head.shape[0] == T
        gw = _c(gate_weights, np.float32) if gate_weights is not None else None
        rtw = _c(recv_topk_weights, np.float32) if recv_topk_weights is not None else None
        if out is None:
            out = np.empty((T, H), np.uint16)
        assert out.shape == (T, H) and out.dtype == np.uint16 and out.flags["C_CONTIGUOUS"]
        cw = np.empty((T, K), np.float32) if rtw is not None else None
        self.lib.oracle_combine(_ptr(y), T, H, _ptr(idx), K, num_experts, R,
                                _ptr(pre.send_head), _ptr(pre.rank_prefix_matrix),
                                _ptr(gw), _ptr(rtw), _ptr(out), _ptr(cw))
        return out, cw

    # -- low-latency layout -------------------------------------------------
    def ll_dispatch(self, x_u16: Optional[np.ndarray], topk_idx, num_experts: int, cap: int,
                    hidden: Optional[int] = None):
        idx = _c(topk_idx, np.int64)
        T, K = idx.shape
        x = _c(x_u16, np.uint16) if x_u16 is not None else None
        H = x.shape[1] if x is not None else (hidden or 0)
        recv_x = np.zeros((num_experts, cap, H), np.uint16) if x is not None else None
        cnt = np.empty(num_experts, np.int32)
        src = np.empty((num_experts, cap), np.int32)
        slot = np.empty((T, K), np.int32)
        rc = self.lib.oracle_ll_dispatch(_ptr(x), T, H, _ptr(idx), K, num_experts, cap,
                                         _ptr(recv_x), _ptr(cnt), _ptr(src), _ptr(slot))
        if rc != 0:
            raise ValueError("an expert receives more tokens than the slot capacity")
        return recv_x, cnt, src, slot

    def ll_combine(self, y_u16: np.ndarray, topk_idx, topk_weights, slot_of):
        y = _c(y_u16, np.uint16)
        E, cap, H = y.shape
        idx = _c(topk_idx, np.int64)
        T, K = idx.shape
        w = _c(topk_weights, np.float32)
        so = _c(slot_of, np.int32)
        out = np.empty((T, H), np.uint16)
        self.lib.oracle_ll_combine(_ptr(y), cap, H, _ptr(idx), _ptr(w), T, K, _ptr(so), _ptr(out))
        return out


@dataclass
class Dispatch:
    layout: Layout
    prefix: Prefix
    recv_x: np.ndarray
    recv_topk_idx: Optional[np.ndarray]
    recv_topk_weights: Optional[np.ndarray]


def dispatch(o: Oracle, x_u16, topk_idx, topk_weights, num_experts, num_ranks, num_channels,
             with_rows: bool = True) -> Dispatch:
    """Layout, handle and bf16 pack, in the order a first dispatch runs them."""
    lay = o.layout(topk_idx, num_experts, num_ranks)
    pre = o.prefix(lay.is_token_in_rank, num_channels)
    if with_rows:
        rx, rti, rtw = o.pack_bf16(x_u16, topk_idx, topk_weights, num_experts, pre)
    else:
        rx = rti = rtw = None
    return Dispatch(lay, pre, rx, rti, rtw)
