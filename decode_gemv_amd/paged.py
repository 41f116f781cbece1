"""Thin torch-facing wrapper of the packkv paged-cache C ABI.

The records of every stream share one pool of fixed-size pages, found
through per-stream block tables, and each stream holds its own number of
tokens.  Encoding, appending, page allocation and release, and fused decode
attention all run in the HIP library on the current torch stream; this class
only allocates the caller-owned device arrays and marshals arguments.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch

from . import _lib
from .cache import D, _ptr, _stream


class PagedKVCache:
    """A paged packed K/V cache of ``n_streams`` streams of up to ``max_tokens``
    tokens each, over a pool of ``n_pages`` pages of ``page_bytes``."""

    def __init__(self, n_streams: int, max_tokens: int, n_pages: int, page_bytes: int = 65536,
                 bits: int = 4, block: int = 64, permute: int = 1, device: str = "cuda",
                 payload_order: int = 0):
        lib = _lib.load()
        self.cfg = _lib.Config(D, bits, block, 32, int(permute), int(payload_order))
        sz = _lib.PagedSizes()
        _lib.check(lib.packkv_paged_sizes(ctypes.byref(self.cfg), n_streams, max_tokens, n_pages, page_bytes,
                                          ctypes.byref(sz)), "packkv_paged_sizes")
        self.sizes = sz
        self.n_streams, self.max_tokens, self.bits, self.block = n_streams, max_tokens, bits, block
        self.n_pages, self.page_bytes = n_pages, page_bytes
        self.max_blocks = sz.max_blocks
        dev = torch.device(device)
        self.pool = torch.zeros(sz.pool_bytes, dtype=torch.uint8, device=dev)
        self.k_table = torch.zeros(n_streams * sz.max_blocks, dtype=torch.int64, device=dev)
        self.v_table = torch.zeros_like(self.k_table)
        self.lengths_dev = torch.zeros(n_streams, dtype=torch.int32, device=dev)
        self.alloc = torch.zeros(sz.alloc_bytes // 4, dtype=torch.int32, device=dev)
        self.perm = torch.full((sz.perm_bytes,), 0xFF, dtype=torch.uint8, device=dev)
        self.tail_k = torch.zeros(n_streams * block * D, dtype=torch.float16, device=dev)
        self.tail_v = torch.zeros_like(self.tail_k)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self._host_len = (ctypes.c_int32 * n_streams)()
        self._c = _lib.PagedT(self.cfg, n_streams, n_pages, max_tokens, page_bytes, _ptr(self.pool),
                              _ptr(self.k_table), _ptr(self.v_table), _ptr(self.lengths_dev), _ptr(self.alloc),
                              _ptr(self.perm), _ptr(self.tail_k), _ptr(self.tail_v), _ptr(self.status),
                              ctypes.addressof(self._host_len))
        self._aws: dict = {}
        _lib.check(lib.packkv_paged_init(ctypes.byref(self._c), _stream()), "packkv_paged_init")

    # ------------------------------------------------------------------ state
    @property
    def lengths(self) -> list:
        """Tokens held by each stream (the library's host copy)."""
        return list(self._host_len)

    def free_pages(self) -> int:
        """Pages on the free stack (reads the device; synchronises)."""
        return int(self.alloc[0].item())

    def tables(self):
        """Host copies of the K and V block tables as (start bytes, size) int64
        arrays [S][max_blocks]."""
        out = []
        for t in (self.k_table, self.v_table):
            a = t.view(self.n_streams, self.max_blocks).cpu().numpy().view(np.uint64)
            out.append(((a & 0xFFFFFFFF).astype(np.int64) * 16, (a >> 32).astype(np.int64)))
        return out

    def records(self, pool_host: Optional[np.ndarray] = None) -> list:
        """Per stream, the list of (K record bytes, V record bytes) of its
        blocks, read from a host copy of the pool through the block tables."""
        pool = self.pool.cpu().numpy() if pool_host is None else pool_host
        (ks, kz), (vs, vz) = self.tables()
        res = []
        for s, n in enumerate(self.lengths):
            nb = -(-n // self.block)
            res.append([(pool[ks[s, j]:ks[s, j] + kz[s, j]].tobytes(), pool[vs[s, j]:vs[s, j] + vz[s, j]].tobytes())
                        for j in range(nb)])
        return res

    def perm_table(self) -> torch.Tensor:
        return self.perm.view(self.n_streams, self.max_blocks, self.block)

    # ------------------------------------------------------------- encoding
    def prefill(self, stream0: int, k: torch.Tensor, v: torch.Tensor) -> None:
        """Prefill the empty streams stream0 .. stream0 + n - 1 with k, v fp16
        [n][T][D] (contiguous, on the device)."""
        self._check_kv(k, v)
        _lib.check(_lib.load().packkv_paged_prefill(ctypes.byref(self._c), stream0, k.shape[0], _ptr(k), _ptr(v),
                                                    k.shape[1], _stream()), "packkv_paged_prefill")

    def append(self, k: torch.Tensor, v: torch.Tensor) -> None:
        """One decode step: k, v fp16 [S][1][D], one token per stream."""
        self._check_kv(k, v)
        if k.shape[0] != self.n_streams or k.shape[1] != 1:
            raise ValueError("append takes one token per stream: [S][1][D]")
        _lib.check(_lib.load().packkv_paged_append(ctypes.byref(self._c), _ptr(k), _ptr(v), _stream()),
                   "packkv_paged_append")

    def release(self, s: int) -> None:
        """Stream s back to empty; its pages return to the pool."""
        _lib.check(_lib.load().packkv_paged_release(ctypes.byref(self._c), s, _stream()), "packkv_paged_release")

    @staticmethod
    def _check_kv(k, v):
        if k.dtype != torch.float16 or v.dtype != torch.float16 or not k.is_contiguous() or \
                not v.is_contiguous() or k.shape != v.shape or k.dim() != 3 or k.shape[2] != D or not k.is_cuda:
            raise ValueError("k and v must be contiguous fp16 CUDA tensors [n][T][D]")

    # ------------------------------------------------------------- decoding
    def attention_workspace(self, group: int) -> torch.Tensor:
        """Zero-filled workspace for `group` queries per stream (reused)."""
        need = int(_lib.load().packkv_paged_attention_workspace_bytes(ctypes.byref(self._c), group))
        ws = self._aws.get(group)
        if ws is None or ws.numel() < need:
            ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=self.pool.device)
            self._aws[group] = ws
        return ws

    def attention(self, q: torch.Tensor, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Fused decode attention, each stream over its own tokens; q fp16
        [S][G][D] -> out fp32 [S][G][D] (zero for an empty stream)."""
        S, G, d = q.shape
        if q.dtype != torch.float16 or S != self.n_streams or d != D or not q.is_contiguous():
            raise ValueError("q must be contiguous fp16 [S][G][D]")
        if out is None:
            out = torch.empty(S, G, D, dtype=torch.float32, device=q.device)
        if out.dtype != torch.float32 or tuple(out.shape) != (S, G, D) or not out.is_contiguous():
            raise ValueError("out must be contiguous fp32 [S][G][D]")
        ws = self.attention_workspace(G) if workspace is None else workspace
        sc = D ** -0.5 if scale is None else float(scale)
        _lib.check(_lib.load().packkv_paged_attention(ctypes.byref(self._c), _ptr(q), G, sc, _ptr(out), _ptr(ws),
                                                      ws.numel() * ws.element_size(), _stream()),
                   "packkv_paged_attention")
        return out

    def check(self) -> int:
        """Synchronise and return (and clear) the device error latch."""
        return int(_lib.load().packkv_paged_check(ctypes.byref(self._c), _stream()))
