"""Python front end with the call shapes of the pages, over libmoedx.so.

``Buffer`` mirrors the normal and low-latency usage examples of the
EnflameTechnology/DeepEP README (get_dispatch_layout, dispatch, combine,
low_latency_dispatch, low_latency_combine, capture); ``EventOverlap`` mirrors
the event wrapper of "How DeepEP Achieves Communication-Computation
Overlapping with EventOverlap" (current_stream_wait and the context manager).
PyTorch only provides device memory and the current stream; every step runs in
the library's HIP kernels.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _capi as C


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    p = t.data_ptr()
    if p == 0 and t.numel() == 0:  # an empty view still names its allocation
        p = t.untyped_storage().data_ptr()
    return ctypes.c_void_p(p or None)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


# Releases that must wait until no stream capture is running.  Destroying a
# context synchronises its stream and frees device and pinned memory, and an
# event destroy is not a capturable call either; any of them during a capture
# invalidates the graph being recorded.  A finalizer can run at any point (the
# garbage collector may collect an old Buffer in the middle of someone else's
# capture), so while the current stream is capturing the release is queued and
# done by the next call that runs outside a capture.
_deferred: list = []


def _capturing() -> bool:
    try:
        return torch.cuda.is_available() and torch.cuda.is_current_stream_capturing()
    except Exception:  # interpreter shutdown: torch may already be gone
        return False


def _flush_deferred(_deferred=_deferred, _capturing=_capturing) -> None:
    while _deferred and not _capturing():
        fn, ptr = _deferred.pop()
        fn(ptr)


# Finalizers reach these through default arguments and class attributes: at
# interpreter exit the module's globals may already be gone.
def _release(fn, ptr, _deferred=_deferred, _capturing=_capturing,
             _flush=_flush_deferred) -> None:
    if _capturing():
        _deferred.append((fn, ptr))
        return
    fn(ptr)
    _flush()


class EventOverlap:
    """Owns one library event.  ``event is None`` means "already complete"
    (what a call with async_finish=False hands back, for tuple arity)."""

    def __init__(self, event: Optional[int] = None):
        self.event = event

    def current_stream_wait(self) -> None:
        if self.event is not None:
            C.check(C.moedx_event_wait(self.event, _stream()))

    def synchronize(self) -> None:
        if self.event is not None:
            C.check(C.moedx_event_synchronize(self.event))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.current_stream_wait()

    # Held by the class: at interpreter exit module globals may already be gone.
    _destroy = staticmethod(C.moedx_event_destroy)
    _release = staticmethod(_release)

    def __del__(self):
        if getattr(self, "event", None) is not None:
            self._release(self._destroy, self.event)
            self.event = None


_MATRICES = {C.MOEDX_T_CHANNEL_PREFIX_MATRIX, C.MOEDX_T_RECV_CHANNEL_PREFIX_MATRIX,
             C.MOEDX_T_IS_TOKEN_IN_RANK, C.MOEDX_T_SEND_HEAD, C.MOEDX_T_LL_SRC_IDX,
             C.MOEDX_T_LL_SLOT_OF}


class Handle:
    """A prepared layout: the library handle plus the device workspace that
    holds its arrays (kept alive as long as the handle)."""

    def __init__(self, ptr: int, workspace: torch.Tensor, T: int, K: int, low_latency: bool,
                 capacity: int = 0, buffer: "Optional[Buffer]" = None):
        self.ptr = ptr
        self.workspace = workspace
        self.T, self.K = T, K
        self.low_latency = low_latency
        self.capacity = capacity
        self.buffer = buffer  # the Buffer whose ctx prepared it (normal handles)

    def finish(self) -> None:
        """Write a capacity-mode handle's prefixes, totals and N on the current
        stream now rather than on its first dispatch or combine (nothing runs
        when they are already written)."""
        if self.low_latency or self.buffer is None:
            return
        ex = C.make_exec(_stream(), None, None, C.MOEDX_ASYNC)
        C.check(C.moedx_handle_finish(self.buffer.ctx, self.ptr, ctypes.byref(ex)))

    def tensor(self, which: int, dtype: torch.dtype) -> torch.Tensor:
        """View of one handle array (MOEDX_T_*) inside the workspace."""
        dev = ctypes.c_void_p()
        shape = (ctypes.c_int64 * 2)()
        C.check(C.moedx_handle_tensor(self.ptr, which, ctypes.byref(dev), shape))
        n0, n1 = int(shape[0]), int(shape[1])
        off = (dev.value or 0) - self.workspace.data_ptr()
        nbytes = n0 * n1 * torch.empty((), dtype=dtype).element_size()
        assert 0 <= off and off + nbytes <= self.workspace.numel()
        v = self.workspace[off: off + nbytes].view(dtype)
        return v.view(n0, n1) if which in _MATRICES else v

    @property
    def num_recv(self) -> int:
        n = ctypes.c_int64()
        C.check(C.moedx_handle_num_recv(self.ptr, ctypes.byref(n)))
        return int(n.value)

    def recv_tokens_per_expert(self, num_experts: int) -> list:
        a = (ctypes.c_int32 * num_experts)()
        C.check(C.moedx_handle_recv_tokens_per_expert(self.ptr, a))
        return list(a)

    # handle fields named on the handle-reuse page
    def fields(self) -> dict:
        self.finish()
        if self.low_latency:
            return {"src_idx": self.tensor(C.MOEDX_T_LL_SRC_IDX, torch.int32),
                    "slot_of": self.tensor(C.MOEDX_T_LL_SLOT_OF, torch.int32)}
        return {
            "rank_prefix_matrix": self.tensor(C.MOEDX_T_RANK_PREFIX_MATRIX, torch.int32),
            "channel_prefix_matrix": self.tensor(C.MOEDX_T_CHANNEL_PREFIX_MATRIX, torch.int32),
            "recv_channel_prefix_matrix": self.tensor(C.MOEDX_T_RECV_CHANNEL_PREFIX_MATRIX, torch.int32),
            "recv_src_idx": self.tensor(C.MOEDX_T_RECV_SRC_IDX, torch.int32),
            "is_token_in_rank": self.tensor(C.MOEDX_T_IS_TOKEN_IN_RANK, torch.uint8),
            "send_head": self.tensor(C.MOEDX_T_SEND_HEAD, torch.int32),
            "num_tokens_per_rank": self.tensor(C.MOEDX_T_NUM_TOKENS_PER_RANK, torch.int32),
            "num_tokens_per_expert": self.tensor(C.MOEDX_T_NUM_TOKENS_PER_EXPERT, torch.int32),
            "num_recv": self.tensor(C.MOEDX_T_NUM_RECV, torch.int32),
        }

    _destroy = staticmethod(C.moedx_handle_destroy)

    def __del__(self):
        if getattr(self, "ptr", None):
            self._destroy(self.ptr)
            self.ptr = None


class Buffer:
    """One GPU's share of the expert-parallel exchange: ``num_ranks`` logical
    ranks are buckets of ``num_experts / num_ranks`` experts in this GPU's HBM."""

    def __init__(self, num_experts: int, num_ranks: int, num_channels: int = 24,
                 max_tokens: int = 16384, device: Optional[int] = None):
        self.device = torch.cuda.current_device() if device is None else device
        self.num_experts, self.num_ranks, self.num_channels = num_experts, num_ranks, num_channels
        self.max_tokens = max_tokens
        _flush_deferred()
        ctx = ctypes.c_void_p()
        C.check(C.moedx_create(ctypes.byref(ctx), self.device, num_experts, num_ranks,
                               num_channels, max_tokens, 0))
        self.ctx = ctx.value
        # The comm stream (allocate_on_comm_stream) is one of PyTorch's own
        # pool streams, which live as long as the process: tensors an op used
        # there record it (_keep), and the caching allocator records an event
        # on it when such a tensor is freed, possibly after this Buffer is gone.
        self._ctx_stream = torch.cuda.Stream(device=self.device)
        C.check(C.moedx_ctx_set_stream(self.ctx, self._ctx_stream.cuda_stream))

    _destroy = staticmethod(C.moedx_destroy)
    _release = staticmethod(_release)

    def __del__(self):
        if getattr(self, "ctx", None):
            self._release(self._destroy, self.ctx)
            self.ctx = None

    # -- plumbing ---------------------------------------------------------------
    def ctx_stream(self) -> "torch.cuda.Stream":
        """The ctx's own stream (where allocate_on_comm_stream runs an op)."""
        return self._ctx_stream

    def _keep(self, on_ctx_stream: bool, *tensors) -> None:
        """An op on the ctx stream uses memory that PyTorch's caching allocator
        handed out on the caller's stream: record the ctx stream on every such
        tensor, so that no block is given to a new allocation before the ctx
        stream's work on it has finished (even when the tensor is a temporary
        dropped as the call returns)."""
        if not on_ctx_stream:
            return
        s = self.ctx_stream()
        for t in tensors:
            if isinstance(t, torch.Tensor) and t.is_cuda and t.numel() > 0:
                t.record_stream(s)

    def _exec(self, previous_event, async_finish, allocate_on_comm_stream, no_sync=False):
        if _deferred:
            _flush_deferred()
        done = ctypes.c_void_p() if async_finish else None
        flags = (C.MOEDX_ON_CTX_STREAM if allocate_on_comm_stream else 0) | (
            C.MOEDX_ASYNC if no_sync else 0)
        prev = previous_event.event if previous_event is not None else None
        return C.make_exec(_stream(), prev, done, flags), done

    @staticmethod
    def _event(done) -> EventOverlap:
        return EventOverlap(done.value if done is not None else None)

    def stats(self) -> dict:
        s = C.moedx_stats()
        C.check(C.moedx_ctx_stats(self.ctx, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in C.moedx_stats._fields_}

    @staticmethod
    def capture() -> EventOverlap:
        ev = ctypes.c_void_p()
        C.check(C.moedx_event_record(ctypes.byref(ev), _stream()))
        return EventOverlap(ev.value)

    # -- layout -----------------------------------------------------------------
    def get_dispatch_layout(self, topk_idx: torch.Tensor, num_experts: int,
                            previous_event: Optional[EventOverlap] = None,
                            async_finish: bool = False, allocate_on_comm_stream: bool = False,
                            no_sync: bool = False):
        """Returns (num_tokens_per_rank, None, num_tokens_per_expert,
        is_token_in_rank, event); the None stands for the per-RDMA-rank counts,
        which do not exist on one GPU.  ``no_sync`` returns without blocking
        (stream order only), as under graph capture."""
        assert num_experts == self.num_experts
        topk_idx = topk_idx.contiguous()
        T, K = topk_idx.shape
        dev = topk_idx.device
        ntr = torch.empty(self.num_ranks, dtype=torch.int32, device=dev)
        nte = torch.empty(num_experts, dtype=torch.int32, device=dev)
        itr = torch.empty(T, self.num_ranks, dtype=torch.bool, device=dev)
        ex, done = self._exec(previous_event, async_finish, allocate_on_comm_stream, no_sync)
        C.check(C.moedx_get_dispatch_layout(self.ctx, _ptr(topk_idx), T, K, _ptr(ntr), _ptr(nte),
                                            _ptr(itr), ctypes.byref(ex)))
        self._keep(allocate_on_comm_stream, topk_idx, ntr, nte, itr)
        return ntr, None, nte, itr, self._event(done)

    # -- normal dispatch / combine --------------------------------------------------
    def prepare(self, topk_idx: torch.Tensor, num_worst_tokens: int = 0,
                previous_event=None, async_finish=False, allocate_on_comm_stream=False,
                no_sync=False, num_tokens_per_rank=None, is_token_in_rank=None,
                num_tokens_per_expert=None):
        """Layout + scan into a new handle (exact mode, or capacity mode with
        ``num_worst_tokens`` receive rows; a capacity-mode handle's prefixes,
        totals and N are written by its first dispatch or combine).  Given
        get_dispatch_layout's ``is_token_in_rank`` and ``num_tokens_per_expert``
        (and optionally ``num_tokens_per_rank``), no layout runs: the handle is
        scanned from them."""
        topk_idx = topk_idx.contiguous()
        T, K = topk_idx.shape
        from_layout = is_token_in_rank is not None or num_tokens_per_expert is not None
        if from_layout:
            assert is_token_in_rank is not None and num_tokens_per_expert is not None, \
                "is_token_in_rank and num_tokens_per_expert go together"
            assert tuple(is_token_in_rank.shape) == (T, self.num_ranks)
            assert is_token_in_rank.dtype in (torch.bool, torch.uint8)
            assert tuple(num_tokens_per_expert.shape) == (self.num_experts,)
            assert num_tokens_per_expert.dtype == torch.int32
            is_token_in_rank = is_token_in_rank.contiguous()
            num_tokens_per_expert = num_tokens_per_expert.contiguous()
            if num_tokens_per_rank is not None:
                assert tuple(num_tokens_per_rank.shape) == (self.num_ranks,)
                num_tokens_per_rank = num_tokens_per_rank.contiguous()
        else:
            num_tokens_per_rank = None
        nbytes = ctypes.c_size_t()
        C.check(C.moedx_handle_workspace_bytes(self.ctx, T, K, num_worst_tokens, ctypes.byref(nbytes)))
        ws = torch.empty(nbytes.value, dtype=torch.uint8, device=topk_idx.device)
        h = ctypes.c_void_p()
        ex, done = self._exec(previous_event, async_finish, allocate_on_comm_stream, no_sync)
        C.check(C.moedx_dispatch_prepare(self.ctx, _ptr(topk_idx), T, K, _ptr(num_tokens_per_rank),
                                         _ptr(is_token_in_rank), _ptr(num_tokens_per_expert),
                                         _ptr(ws), nbytes.value, num_worst_tokens,
                                         ctypes.byref(h), ctypes.byref(ex)))
        self._keep(allocate_on_comm_stream, topk_idx, ws, is_token_in_rank, num_tokens_per_expert)
        return Handle(h.value, ws, T, K, False, num_worst_tokens, self), self._event(done)

    def dispatch(self, x, handle: Optional[Handle] = None, num_tokens_per_rank=None,
                 num_tokens_per_rdma_rank=None, is_token_in_rank=None, num_tokens_per_expert=None,
                 topk_idx: Optional[torch.Tensor] = None, topk_weights: Optional[torch.Tensor] = None,
                 previous_event: Optional[EventOverlap] = None, async_finish: bool = False,
                 allocate_on_comm_stream: bool = False, num_worst_tokens: int = 0,
                 fp8: bool = False, round_scale: bool = False, use_ue8m0: bool = False,
                 fp8_quant_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                 out_scales: Optional[torch.Tensor] = None, no_sync: bool = False):
        """Returns (recv_x, recv_topk_idx, recv_topk_weights,
        num_recv_tokens_per_expert_list, handle, event); recv_x is
        (codes, scales) for FP8 (scales None with a per-tensor scale).  ``x``
        may be a pre-quantised (codes uint8 [T, H], scales) pair, dispatched
        unchanged.  FP8 scales: per 1x128 block amax / 448 by default;
        ``round_scale`` rounds them up to powers of two; ``use_ue8m0`` stores
        them as UE8M0 exponent bytes (and implies ``round_scale``);
        ``fp8_quant_scale`` is one scale for the whole tensor (exclusive with
        ``use_ue8m0``).  With ``handle`` (cached dispatch) topk_idx and
        topk_weights must be None and only recv_x is produced.  On a first
        dispatch, get_dispatch_layout's outputs (``is_token_in_rank`` and
        ``num_tokens_per_expert``, with ``num_tokens_per_rank`` if at hand) are
        reused: the handle is scanned from them and no layout runs again."""
        prequant = isinstance(x, tuple)
        x_scales = None
        if prequant:
            x, x_scales = x
            x_scales = x_scales.contiguous() if x_scales is not None else None
            fp8 = True
        assert not (use_ue8m0 and fp8_quant_scale is not None), \
            "fp8_quant_scale and use_ue8m0 are exclusive"
        fp8 = fp8 or round_scale or use_ue8m0 or fp8_quant_scale is not None
        x = x.contiguous()
        T, H = x.shape
        first = handle is None
        if first:
            assert topk_idx is not None, "a first dispatch needs topk_idx"
            reuse = is_token_in_rank is not None and num_tokens_per_expert is not None
            handle, _ = self.prepare(
                topk_idx, num_worst_tokens, previous_event, False, allocate_on_comm_stream,
                no_sync=True, num_tokens_per_rank=num_tokens_per_rank if reuse else None,
                is_token_in_rank=is_token_in_rank if reuse else None,
                num_tokens_per_expert=num_tokens_per_expert if reuse else None)
            previous_event = None
        else:
            assert topk_idx is None and topk_weights is None, \
                "a cached dispatch takes no topk_idx / topk_weights"
        rows = handle.capacity if handle.capacity > 0 else handle.num_recv
        K = handle.K
        dev = x.device
        # At least one row is allocated so that an empty receive side still
        # passes a valid device pointer; the returned views have `rows` rows.
        alloc = max(rows, 1)
        mode = (C.MOEDX_FP8_SCALE_TENSOR if fp8_quant_scale is not None else
                C.MOEDX_FP8_SCALE_UE8M0 if use_ue8m0 else
                C.MOEDX_FP8_SCALE_POW2 if round_scale else C.MOEDX_FP8_SCALE_AMAX)
        if fp8:
            recv_x = out if out is not None else torch.empty(alloc, H, dtype=torch.uint8, device=dev)
            sdt = torch.uint8 if mode == C.MOEDX_FP8_SCALE_UE8M0 else torch.float32
            recv_s = None if mode == C.MOEDX_FP8_SCALE_TENSOR else (
                out_scales if out_scales is not None else
                torch.empty(alloc, H // 128, dtype=sdt, device=dev))
        else:
            recv_x = out if out is not None else torch.empty(alloc, H, dtype=torch.bfloat16, device=dev)
            recv_s = None
        rti = rtw = None
        if first and not fp8:
            rti = torch.empty(alloc, K, dtype=torch.int64, device=dev)
            if topk_weights is not None:
                rtw = torch.empty(alloc, K, dtype=torch.float32, device=dev)
        ex, done = self._exec(previous_event, async_finish, allocate_on_comm_stream, no_sync)
        if fp8 and (mode != C.MOEDX_FP8_SCALE_AMAX or prequant):
            opts = C.moedx_fp8(mode, int(prequant),
                               float(fp8_quant_scale) if fp8_quant_scale is not None else 0.0,
                               _ptr(x_scales))
            C.check(C.moedx_dispatch_fp8(self.ctx, handle.ptr, _ptr(x), T, H, ctypes.byref(opts),
                                         _ptr(recv_x), _ptr(recv_s), ctypes.byref(ex)))
        else:
            tw = topk_weights.contiguous() if topk_weights is not None else None
            ti = topk_idx.contiguous() if (first and not fp8) else None
            C.check(C.moedx_dispatch(self.ctx, handle.ptr, _ptr(x), T, H,
                                     C.MOEDX_QUANT_FP8_E4M3_1X128 if fp8 else C.MOEDX_QUANT_NONE,
                                     _ptr(ti), _ptr(tw if (first and not fp8) else None),
                                     _ptr(recv_x), _ptr(recv_s), _ptr(rti), _ptr(rtw),
                                     ctypes.byref(ex)))
            self._keep(allocate_on_comm_stream, ti, tw)
        self._keep(allocate_on_comm_stream, x, x_scales, recv_x, recv_s, rti, rtw, topk_idx,
                   topk_weights if first else None)
        per_expert = handle.recv_tokens_per_expert(self.num_experts) if (
            first and handle.capacity == 0) else None
        if out is None:
            recv_x = recv_x[:rows]
        if recv_s is not None and out_scales is None:
            recv_s = recv_s[:rows]
        rti = rti[:rows] if rti is not None else None
        rtw = rtw[:rows] if rtw is not None else None
        rx = (recv_x, recv_s) if fp8 else recv_x
        return rx, rti, rtw, per_expert, handle, self._event(done)

    def combine(self, x: torch.Tensor, handle: Handle, topk_weights: Optional[torch.Tensor] = None,
                gate_weights: Optional[torch.Tensor] = None,
                previous_event: Optional[EventOverlap] = None, async_finish: bool = False,
                allocate_on_comm_stream: bool = False, out: Optional[torch.Tensor] = None,
                no_sync: bool = False):
        """Returns (combined_x, combined_topk_weights, event).  ``topk_weights``
        is the per-row weight payload ([rows, K]) reduced like the rows;
        ``gate_weights`` ([T, K]) scales each bucket's row by its summed gate
        weight."""
        x = x.contiguous()
        H = x.shape[1]
        T, K = handle.T, handle.K
        combined = out if out is not None else torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
        cw = torch.empty(T, K, dtype=torch.float32, device=x.device) if topk_weights is not None else None
        ex, done = self._exec(previous_event, async_finish, allocate_on_comm_stream, no_sync)
        gw = gate_weights.contiguous() if gate_weights is not None else None
        tw = topk_weights.contiguous() if topk_weights is not None else None
        C.check(C.moedx_combine(self.ctx, handle.ptr, _ptr(x), H, _ptr(gw), _ptr(tw),
                                _ptr(combined), _ptr(cw), ctypes.byref(ex)))
        self._keep(allocate_on_comm_stream, x, gw, tw, combined, cw)
        return combined, cw, self._event(done)

    # -- low-latency ------------------------------------------------------------
    def low_latency_dispatch(self, x: torch.Tensor, topk_idx: torch.Tensor,
                             num_max_dispatch_tokens_per_rank: int, num_experts: int,
                             previous_event=None, async_finish: bool = False,
                             return_recv_hook: bool = False, no_sync: bool = False):
        """Returns (recv_x [E, cap, H], recv_count [E] int32, handle, event, hook).
        With return_recv_hook the call fills counts and the handle only, and
        the rows arrive when hook() runs (a second kernel launch on the
        current stream); otherwise hook is None."""
        assert num_experts == self.num_experts
        x = x.contiguous()
        topk_idx = topk_idx.contiguous()
        T, H = x.shape
        K = topk_idx.shape[1]
        cap = num_max_dispatch_tokens_per_rank
        dev = x.device
        nbytes = ctypes.c_size_t()
        C.check(C.moedx_ll_workspace_bytes(self.ctx, T, K, cap, ctypes.byref(nbytes)))
        ws = torch.empty(nbytes.value, dtype=torch.uint8, device=dev)
        recv_x = torch.empty(num_experts, cap, H, dtype=torch.bfloat16, device=dev)
        cnt = torch.empty(num_experts, dtype=torch.int32, device=dev)
        h = ctypes.c_void_p()
        ex, done = self._exec(previous_event, async_finish, False, no_sync)
        C.check(C.moedx_ll_dispatch(self.ctx, _ptr(x), _ptr(topk_idx), T, K, H, cap,
                                    None if return_recv_hook else _ptr(recv_x), _ptr(cnt),
                                    _ptr(ws), nbytes.value, ctypes.byref(h), ctypes.byref(ex)))
        handle = Handle(h.value, ws, T, K, True)
        hook = None
        if return_recv_hook:
            def hook():
                rex = C.make_exec(_stream(), None, None, C.MOEDX_ASYNC)
                C.check(C.moedx_ll_dispatch_recv(self.ctx, handle.ptr, _ptr(x), _ptr(topk_idx), H,
                                                 _ptr(recv_x), ctypes.byref(rex)))
        return recv_x, cnt, handle, self._event(done), hook

    def low_latency_combine(self, x: torch.Tensor, topk_idx: torch.Tensor,
                            topk_weights: torch.Tensor, handle: Handle, previous_event=None,
                            async_finish: bool = False, return_recv_hook: bool = False,
                            out: Optional[torch.Tensor] = None, no_sync: bool = False):
        """Returns (combined [T, H] bf16, event, hook).  With return_recv_hook
        the reduction runs when hook() is called (on the current stream) and
        event is None; otherwise hook is None."""
        x = x.contiguous()
        H = x.shape[-1]
        T = handle.T
        combined = out if out is not None else torch.empty(T, H, dtype=torch.bfloat16, device=x.device)
        ti, tw = topk_idx.contiguous(), topk_weights.contiguous()

        def run(ex):
            C.check(C.moedx_ll_combine(self.ctx, _ptr(x), _ptr(ti), _ptr(tw), handle.ptr, H,
                                       _ptr(combined), ctypes.byref(ex)))

        if return_recv_hook:
            prev = previous_event.event if previous_event is not None else None

            def hook():
                run(C.make_exec(_stream(), prev, None, C.MOEDX_ASYNC))
            return combined, EventOverlap(None), hook
        ex, done = self._exec(previous_event, async_finish, False, no_sync)
        run(ex)
        return combined, self._event(done), None
