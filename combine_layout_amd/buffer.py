"""Python binding of the C ABI: the afdEP-comm ``Buffer`` calls on one GPU.

Argument marshalling only: every step of the round runs in the HIP library.
torch provides device memory (workspace, arenas, outputs) and the stream.

Method names and keywords follow the afdEP-comm API contract page
("Roles and tensors"); because one Buffer plays every role on one GPU, each
role call takes the source index s or the partition index f first.
"""
from __future__ import annotations

import ctypes
from typing import List, NamedTuple, Optional

import torch

from . import _native as nat

topk_idx_dtype = torch.int32


class Received(NamedTuple):
    rows: torch.Tensor              # [receive_rows, H] bf16 or float8_e4m3fn, expert-major
    scales: Optional[torch.Tensor]  # [receive_rows, H/128] float32 (FP8 only)
    weights: torch.Tensor           # [receive_rows] float32
    ends: torch.Tensor              # [E/F] int32, device prefix sums of the local experts
    receipt: nat.Receipt
    receive_rows: int
    host_counts: Optional[List[int]]


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class _DeviceBytes:
    """A device byte range the library owns (the static scratch array), seen
    by torch through the CUDA array interface."""

    def __init__(self, ptr: int, nbytes: int):
        self.__cuda_array_interface__ = {"shape": (nbytes,), "typestr": "|u1", "data": (ptr, False),
                                         "strides": None, "version": 3}


class Buffer:
    """One context over caller-owned (torch) device memory.

    num_sources N, num_partitions F, num_experts E, topk K, hidden H,
    expert_alignment alpha, capacity (largest bucket), dtype "bf16" | "fp8",
    combine "once" | "per_stage" | "per_stage_fp8" (how the combine rounds;
    the per-stage modes need two or more partitions).
    Receive arenas are sized for ``arena_bucket`` (default: capacity).
    dispatch "auto" | "split" | "one_launch" (afd_dispatch_mode).
    static_workspace=True makes the context with afd_create_static: no
    workspace is allocated, the library's static scratch array on the device
    serves (one such Buffer per device at a time)."""

    def __init__(self, num_sources, num_partitions, num_experts, topk, hidden, expert_alignment=1,
                 capacity=2048, dtype="bf16", device=None, arena_bucket=None, combine="once",
                 static_workspace=False, dispatch="auto"):
        self.lib = nat.load()
        self.device = torch.device(device if device is not None else "cuda", torch.cuda.current_device()) \
            if device is None or isinstance(device, str) and device == "cuda" else torch.device(device)
        self.fp8 = dtype == "fp8"
        if combine not in nat.COMBINE_MODES:
            raise ValueError(f"combine must be one of {sorted(nat.COMBINE_MODES)}")
        self.combine = combine
        if dispatch not in nat.DISPATCH_MODES:
            raise ValueError(f"dispatch must be one of {sorted(nat.DISPATCH_MODES)}")
        self.cfg = nat.Config(num_sources, num_partitions, num_experts, topk, hidden, expert_alignment, capacity,
                              nat.AFD_FP8_E4M3 if self.fp8 else nat.AFD_BF16, nat.COMBINE_MODES[combine],
                              nat.DISPATCH_MODES[dispatch])
        self.N, self.F, self.E, self.K, self.H = num_sources, num_partitions, num_experts, topk, hidden
        self.E_loc = num_experts // num_partitions
        self.alpha, self.capacity = expert_alignment, capacity
        ws = ctypes.c_size_t(0)
        rb = ctypes.c_int64(0)
        bucket = arena_bucket if arena_bucket is not None else capacity
        nat.check(self.lib.afd_query(ctypes.byref(self.cfg), bucket, ctypes.byref(ws), ctypes.byref(rb)), "afd_query")
        self.static_workspace = static_workspace
        self.workspace = None if static_workspace else torch.empty(ws.value, dtype=torch.uint8, device=self.device)
        self.rows_cap = rb.value
        self.arenas = []
        for _ in range(num_partitions):
            rows = torch.empty((self.rows_cap, hidden), dtype=torch.uint8 if self.fp8 else torch.bfloat16,
                               device=self.device)
            scales = torch.empty((self.rows_cap, hidden // 128), dtype=torch.float32, device=self.device) \
                if self.fp8 else None
            roww = torch.empty(self.rows_cap, dtype=torch.float32, device=self.device)
            self.arenas.append((rows, scales, roww))
        ctx = ctypes.c_void_p(0)
        if static_workspace:
            with torch.cuda.device(self.device):
                nat.check(self.lib.afd_create_static(ctypes.byref(self.cfg), ctypes.byref(ctx)), "afd_create_static")
        else:
            nat.check(self.lib.afd_create(ctypes.byref(self.cfg), _ptr(self.workspace), ws.value,
                                          ctypes.byref(ctx)), "afd_create")
        self.ctx = ctx
        self._bind()
        self._round_refs = {}
        self._out = [None] * num_sources
        self._T = [0] * num_sources

    def _bind(self):
        for f, (rows, scales, roww) in enumerate(self.arenas):
            nat.check(self.lib.afd_bind_partition(self.ctx, f, _ptr(rows), _ptr(scales), _ptr(roww),
                                                  self.rows_cap), "afd_bind_partition")

    def bind_arenas(self, bucket):
        """Allocate and bind receive arenas sized for `bucket` tokens per
        source.  Allowed between rounds, or after a worker_receive refused
        the round for a smaller arena (then receive again)."""
        rb = self.rows_bound(bucket)
        arenas = []
        for _ in range(self.F):
            rows = torch.empty((rb, self.H), dtype=torch.uint8 if self.fp8 else torch.bfloat16, device=self.device)
            scales = torch.empty((rb, self.H // 128), dtype=torch.float32, device=self.device) if self.fp8 else None
            arenas.append((rows, scales, torch.empty(rb, dtype=torch.float32, device=self.device)))
        old = self.arenas, self.rows_cap
        self.arenas, self.rows_cap = arenas, rb
        try:
            self._bind()
        except nat.AfdError:
            self.arenas, self.rows_cap = old
            self._bind()
            raise

    # -- helpers -------------------------------------------------------------
    def _ws_view(self, ptr: int, nbytes: int) -> torch.Tensor:
        if self.workspace is None:
            return torch.as_tensor(_DeviceBytes(ptr, nbytes), device=self.device)
        off = ptr - self.workspace.data_ptr()
        assert 0 <= off and off + nbytes <= self.workspace.numel()
        return self.workspace[off:off + nbytes]

    def rows_bound(self, bucket: int) -> int:
        rb = ctypes.c_int64(0)
        nat.check(self.lib.afd_query(ctypes.byref(self.cfg), bucket, None, ctypes.byref(rb)), "afd_query")
        return rb.value

    # -- the four role calls ---------------------------------------------------
    def source_dispatch(self, s, x, ids, weights, x_scale=None, *, bucket, read_host_counts=False, out=None,
                        cached=False):
        """cached=True reuses the receive layout of the last round (the
        ElasticBuffer page's cached dispatch): ids are not read (pass None),
        T must match that round's, and read_host_counts is not available."""
        if cached:
            T = int(weights.shape[0]) if weights is not None else 0
        else:
            T = int(ids.shape[0]) if ids is not None else 0
        if T > 0:
            if self.fp8:
                if x.element_size() != 1:
                    raise TypeError("FP8 dispatch takes float8_e4m3fn (or uint8) activations")
            elif x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
                raise TypeError("BF16 dispatch takes bfloat16 activations")
            if not cached and ids.dtype != topk_idx_dtype:
                raise TypeError("ids must be buffer.topk_idx_dtype (int32)")
            if weights.dtype != torch.float32:
                raise TypeError("weights must be float32")
            if tuple(x.shape) != (T, self.H) or tuple(weights.shape) != (T, self.K) or \
                    (not cached and tuple(ids.shape) != (T, self.K)):
                raise ValueError("x must be [T, H]; ids and weights [T, K]")
            if not (x.is_contiguous() and weights.is_contiguous() and (cached or ids.is_contiguous())):
                raise ValueError("x, ids and weights must be contiguous")
        sst = ssg = 0
        if x_scale is not None:
            if x_scale.dtype != torch.float32 or tuple(x_scale.shape) != (T, self.H // 128):
                raise ValueError("x_scale must be float32 [T, H/128]")
            sst, ssg = x_scale.stride()
        if out is None and T > 0:
            out = torch.empty((T, self.H), dtype=torch.bfloat16, device=self.device)
        if cached:
            if read_host_counts:
                raise ValueError("a cached dispatch never reads host counts")
            st = self.lib.afd_source_dispatch_cached(self.ctx, s, T, _ptr(x if T else None),
                                                     _ptr(weights if T else None), _ptr(x_scale), sst, ssg,
                                                     _ptr(out), bucket, _stream(self.device))
        else:
            st = self.lib.afd_source_dispatch(self.ctx, s, T, _ptr(x if T else None), _ptr(ids if T else None),
                                              _ptr(weights if T else None), _ptr(x_scale), sst, ssg, _ptr(out),
                                              bucket, 1 if read_host_counts else 0, _stream(self.device))
        nat.check(st, "source_dispatch")
        self._round_refs[("src", s)] = (x, ids, weights, x_scale, out)
        self._out[s] = out
        self._T[s] = T

    def worker_receive(self, f, *, bucket, read_host_counts=False) -> Received:
        rec = nat.Receive()
        hc = (ctypes.c_int32 * self.E_loc)() if read_host_counts else None
        st = self.lib.afd_worker_receive(self.ctx, f, bucket, 1 if read_host_counts else 0,
                                         ctypes.cast(hc, ctypes.c_void_p) if hc is not None else None,
                                         ctypes.byref(rec), _stream(self.device))
        if st not in (nat.AFD_OK, nat.AFD_E_ROUTE):
            nat.check(st, "worker_receive")
        rows_t, scales_t, roww_t = self.arenas[f]
        assert rec.rows == rows_t.data_ptr() and rec.weights == roww_t.data_ptr()
        n = rec.receive_rows
        rows = rows_t[:n]
        if self.fp8:
            try:
                rows = rows.view(torch.float8_e4m3fn)
            except (RuntimeError, TypeError):
                pass
        ends = self._ws_view(rec.ends, 4 * self.E_loc).view(torch.int32)
        receipt = nat.Receipt(rec.receipt.round, rec.receipt.partition, 0)
        out = Received(rows, scales_t[:n] if scales_t is not None else None, roww_t[:n], ends, receipt, n,
                       list(hc) if hc is not None else None)
        if st == nat.AFD_E_ROUTE:
            raise nat.AfdError(st, "worker_receive: invalid routes (the round completed with them skipped)")
        return out

    def worker_reply(self, f, rows, receipt):
        if rows.dtype != torch.bfloat16 or not rows.is_contiguous() or rows.shape[-1] != self.H:
            raise ValueError("replies must be contiguous bfloat16 [receive_rows, H]")
        st = self.lib.afd_worker_reply(self.ctx, f, _ptr(rows), int(rows.shape[0]), ctypes.byref(receipt),
                                       _stream(self.device))
        nat.check(st, "worker_reply")
        self._round_refs[("reply", f)] = rows

    def source_collect(self, s, *, view=False) -> torch.Tensor:
        res = ctypes.c_void_p(0)
        stride = ctypes.c_int64(0)
        st = self.lib.afd_source_collect(self.ctx, s, 1 if view else 0, ctypes.byref(res), ctypes.byref(stride),
                                         _stream(self.device))
        nat.check(st, "source_collect")
        T = self._T[s]
        if T == 0:
            return torch.empty((0, self.H), dtype=torch.bfloat16, device=self.device)
        out = self._out[s]
        if out is not None and res.value == out.data_ptr():
            return out
        return self._ws_view(res.value, T * self.H * 2).view(torch.bfloat16).view(T, self.H)

    def partials(self, s, f) -> torch.Tensor:
        """Per-stage combine: source s's stage-one rows from partition f, a
        uint8 view [T, row_bytes] of the workspace (BF16 partials, or E4M3
        codes followed by the scale bytes).  Rows of tokens without a live
        choice in f are unspecified."""
        ptr = ctypes.c_void_p(0)
        rb = ctypes.c_int64(0)
        nat.check(self.lib.afd_get_partials(self.ctx, s, f, ctypes.byref(ptr), ctypes.byref(rb)), "get_partials")
        T = self._T[s]
        return self._ws_view(ptr.value, max(T, 1) * rb.value).view(-1, rb.value)[:T]

    def round_info(self) -> dict:
        """Which kernels the last enqueued round runs: dispatch path
        ("one_kernel", "tiled", "cached", "empty"), kernel counts, tokens and
        layout tiles."""
        ri = nat.RoundInfo()
        nat.check(self.lib.afd_get_round_info(self.ctx, ctypes.byref(ri)), "get_round_info")
        return {"round": ri.round, "dispatch_path": nat.DISPATCH_PATHS.get(ri.dispatch_path, ri.dispatch_path),
                "dispatch_kernels": ri.dispatch_kernels, "combine_kernels": ri.combine_kernels,
                "tokens": ri.tokens, "layout_tiles": ri.layout_tiles, "tile_tokens": ri.tile_tokens}

    # -- errors / teardown ---------------------------------------------------
    def get_error(self, clear=False, with_status=False):
        """The sticky first invalid route (code, s, t, k); with_status=True
        also returns the call's status (AFD_E_TIMEOUT when a one-launch
        dispatch gave up waiting)."""
        code, s, t, k = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        st = self.lib.afd_get_error(self.ctx, _stream(self.device), 1 if clear else 0, ctypes.byref(code),
                                    ctypes.byref(s), ctypes.byref(t), ctypes.byref(k))
        if st not in (nat.AFD_OK, nat.AFD_E_ROUTE, nat.AFD_E_TIMEOUT):
            nat.check(st, "get_error")
        err = (code.value, s.value, t.value, k.value)
        return (err, st) if with_status else err

    def set_dispatch_wait(self, polls):
        """Polls a one-launch dispatch's workgroups make before giving up
        (negative: give up at once)."""
        nat.check(self.lib.afd_set_dispatch_wait(self.ctx, int(polls)), "set_dispatch_wait")

    def close(self):
        if getattr(self, "ctx", None):
            self.lib.afd_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
