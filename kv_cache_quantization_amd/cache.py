"""Torch-facing wrapper of one KIVI cache (a layer's K/V for B x H streams).

PyTorch supplies the device buffer, the decode workspace, the output tensor
and the current HIP stream; all computation is in libkivi's kernels.
"""
from __future__ import annotations

import torch

from . import kivi as _k


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class KiviCache:
    """Packed KIVI cache bound to a torch-allocated device buffer."""

    def __init__(self, batch: int, n_kv_heads: int, n_q_heads: int, max_tokens: int,
                 bits: int = 2, group: int = 32, residual: int = 128, head_dim: int = 128,
                 kv_dtype: torch.dtype = torch.float16, device="cuda",
                 policy: int = _k.KIVI_FLUSH_WINDOW, key_outliers: int = 0):
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.kv_dtype = kv_dtype
        dt = _k.KIVI_F16 if kv_dtype == torch.float16 else _k.KIVI_F32
        if kv_dtype not in (torch.float16, torch.float32):
            raise TypeError("kv_dtype must be float16 or float32")
        self.cfg = _k.make_config(batch, n_kv_heads, n_q_heads, head_dim, bits, group,
                                  residual, max_tokens, dt, policy, key_outliers)
        nbytes = _k.kivi_cache_bytes(self.cfg)
        if nbytes == 0:
            raise _k.KiviError(_k.KIVI_ERR_INVALID_ARG, "kivi_cache_bytes")
        # 256-byte alignment: over-allocate and offset.
        self._raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        off = (-self._raw.data_ptr()) % 256
        self.buffer = self._raw[off:off + nbytes]
        self.handle = _k.kivi_cache_create(self.cfg, self.buffer.data_ptr(), nbytes)
        self._ws = None
        self._attn_ws = None

    def reset(self) -> None:
        """Forget every token: a fresh host handle over the same buffer."""
        _k.kivi_cache_destroy(self.handle)
        self.handle = None
        self.handle = _k.kivi_cache_create(self.cfg, self.buffer.data_ptr(), self.buffer.numel())

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            self.handle = None
            try:
                _k.kivi_cache_destroy(h)
            except (TypeError, AttributeError):
                # interpreter shutdown: the binding module is already torn
                # down, and the host handle goes with the process
                pass

    # -- shape helpers ------------------------------------------------------
    @property
    def streams(self) -> int:
        return self.cfg.batch * self.cfg.n_kv_heads

    def layout(self) -> _k.kivi_layout:
        return _k.kivi_get_layout(self.handle)

    def plan_append(self, n_new: int) -> _k.kivi_append_plan:
        return _k.kivi_plan_append(self.handle, n_new)

    def decode_plan(self):
        return _k.kivi_decode_plan(self.handle)

    # -- hot path -------------------------------------------------------------
    def append(self, k: torch.Tensor, v: torch.Tensor, defer_flush: bool = False) -> None:
        """Append [B, H, n_new, D] rows (contiguous, kv dtype, on the device).
        defer_flush: only copy into the ring (KIVI_DEFER_FLUSH); a later
        flush() or plain append quantizes the aged groups."""
        c = self.cfg
        shape = (c.batch, c.n_kv_heads, k.shape[2], c.head_dim)
        for t in (k, v):
            if tuple(t.shape) != shape or t.dtype != self.kv_dtype or not t.is_contiguous() \
                    or t.device != self.device:
                raise ValueError("append expects contiguous %s %s on %s" %
                                 (self.kv_dtype, shape, self.device))
        n_new = k.shape[2]
        _k.kivi_append(self.handle, k.data_ptr() if n_new else None,
                       v.data_ptr() if n_new else None, n_new,
                       _k.KIVI_DEFER_FLUSH if defer_flush else 0,
                       _stream_handle(self.device))

    def flush(self) -> None:
        _k.kivi_flush(self.handle, _stream_handle(self.device))

    def workspace(self) -> torch.Tensor:
        if self._ws is None:
            n = _k.kivi_decode_workspace_bytes(self.handle)
            self._ws = torch.empty(n, dtype=torch.uint8, device=self.device)
        return self._ws

    def decode(self, q: torch.Tensor, softmax_scale: float = 0.0,
               out: torch.Tensor | None = None) -> torch.Tensor:
        """softmax(scale q K^T) V over every cached token; q: [B, Hq, D]."""
        c = self.cfg
        if tuple(q.shape) != (c.batch, c.n_q_heads, c.head_dim) or not q.is_contiguous() \
                or q.dtype not in (torch.float16, torch.float32) or q.device != self.device:
            raise ValueError("decode expects contiguous fp16/fp32 q of shape %s" %
                             ((c.batch, c.n_q_heads, c.head_dim),))
        if out is None:
            out = torch.empty((c.batch, c.n_q_heads, c.head_dim), dtype=torch.float32,
                              device=self.device)
        ws = self.workspace()
        qd = _k.KIVI_F16 if q.dtype == torch.float16 else _k.KIVI_F32
        _k.kivi_decode_attn(self.handle, q.data_ptr(), qd, float(softmax_scale), out.data_ptr(),
                            ws.data_ptr(), ws.numel(), _stream_handle(self.device))
        return out

    def append_decode(self, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor,
                      softmax_scale: float = 0.0, out: torch.Tensor | None = None) -> torch.Tensor:
        """append(k, v) then decode(q) in one call (kivi_append_decode): when
        nothing ages out of the residual the new rows reach the ring through
        the decode launch itself."""
        c = self.cfg
        shape = (c.batch, c.n_kv_heads, k.shape[2], c.head_dim)
        for t in (k, v):
            if tuple(t.shape) != shape or t.dtype != self.kv_dtype or not t.is_contiguous() \
                    or t.device != self.device:
                raise ValueError("append_decode expects contiguous %s %s on %s" %
                                 (self.kv_dtype, shape, self.device))
        if tuple(q.shape) != (c.batch, c.n_q_heads, c.head_dim) or not q.is_contiguous() \
                or q.dtype not in (torch.float16, torch.float32) or q.device != self.device:
            raise ValueError("append_decode expects contiguous fp16/fp32 q of shape %s" %
                             ((c.batch, c.n_q_heads, c.head_dim),))
        if out is None:
            out = torch.empty((c.batch, c.n_q_heads, c.head_dim), dtype=torch.float32,
                              device=self.device)
        ws = self.workspace()
        n_new = k.shape[2]
        qd = _k.KIVI_F16 if q.dtype == torch.float16 else _k.KIVI_F32
        _k.kivi_append_decode(self.handle, k.data_ptr() if n_new else None,
                              v.data_ptr() if n_new else None, n_new, q.data_ptr(), qd,
                              float(softmax_scale), out.data_ptr(), ws.data_ptr(), ws.numel(),
                              _stream_handle(self.device))
        return out

    def attn(self, q: torch.Tensor, causal: bool = False, softmax_scale: float = 0.0,
             out: torch.Tensor | None = None) -> torch.Tensor:
        """T queries per head over every cached token; q: [B, Hq, T, D].
        causal: the queries are the last T cached tokens (query t sees tokens
        0 .. n - T + t)."""
        c = self.cfg
        if q.dim() != 4 or tuple(q.shape[:2]) != (c.batch, c.n_q_heads) or \
                q.shape[3] != c.head_dim or q.shape[2] < 1 or not q.is_contiguous() or \
                q.dtype not in (torch.float16, torch.float32) or q.device != self.device:
            raise ValueError("attn expects contiguous fp16/fp32 q of shape (%d, %d, T, %d)" %
                             (c.batch, c.n_q_heads, c.head_dim))
        T = q.shape[2]
        if out is None:
            out = torch.empty((c.batch, c.n_q_heads, T, c.head_dim), dtype=torch.float32,
                              device=self.device)
        n = _k.kivi_attn_workspace_bytes(self.handle, T)
        if n > 0 and (self._attn_ws is None or self._attn_ws.numel() < n):
            self._attn_ws = torch.empty(n, dtype=torch.uint8, device=self.device)
        ws = self._attn_ws if n > 0 else None
        qd = _k.KIVI_F16 if q.dtype == torch.float16 else _k.KIVI_F32
        _k.kivi_attn(self.handle, q.data_ptr(), qd, T, int(bool(causal)), float(softmax_scale),
                     out.data_ptr(), ws.data_ptr() if ws is not None else None,
                     ws.numel() if ws is not None else 0, _stream_handle(self.device))
        return out

    # -- raw views (tests read the packed cache through the layout) -----------
    def blocks_view(self) -> torch.Tensor:
        lo = self.layout()
        c = self.cfg
        nbytes = self.streams * lo.max_groups * lo.block_bytes
        return self.buffer[lo.blocks:lo.blocks + nbytes].view(
            self.streams, lo.max_groups, lo.block_bytes)

    def kside_view(self):
        """[streams, max_kside_units, 2, D] fp16 key units of the split layout
        (G > 32: K scale, K zero of each key group), or None at G = 32."""
        lo = self.layout()
        if lo.kside_unit_tokens == 0:
            return None
        D = self.cfg.head_dim
        nbytes = self.streams * lo.max_kside_units * 4 * D
        return self.buffer[lo.kside:lo.kside + nbytes].view(torch.float16).view(
            self.streams, lo.max_kside_units, 2, D)

    def outlier_records_view(self) -> torch.Tensor:
        """[streams, max_groups, 256] bytes of the outlier records (key_outliers > 0)."""
        lo = self.layout()
        nbytes = self.streams * lo.max_groups * 256
        return self.buffer[lo.outliers:lo.outliers + nbytes].view(self.streams, lo.max_groups, 256)

    def ring_views(self):
        lo = self.layout()
        c = self.cfg
        es = 2 if self.kv_dtype == torch.float16 else 4
        nbytes = self.streams * lo.ring_capacity * c.head_dim * es
        rk = self.buffer[lo.ring_k:lo.ring_k + nbytes].view(self.kv_dtype)
        rv = self.buffer[lo.ring_v:lo.ring_v + nbytes].view(self.kv_dtype)
        shape = (c.batch, c.n_kv_heads, lo.ring_capacity, c.head_dim)
        return rk.view(shape), rv.view(shape)
