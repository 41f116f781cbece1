"""Thin torch-facing wrapper of the packkv C ABI.

Only argument marshalling happens here: every step of the path (encode,
append, the two fused GEMVs, softmax, decompress) runs in the HIP library on
the current torch stream.  torch provides the device memory.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

# head_dim of the paged cache (the contiguous cache takes 64, 128 or 256)
D = 128


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


class PackedKVCache:
    """A packed K/V cache of ``n_streams`` streams (batch x KV heads).

    All arrays are caller-owned torch tensors on ``device``; sizes come from
    ``packkv_cache_sizes``.
    """

    def __init__(self, n_streams: int, max_tokens: int, bits: int = 4, block: int = 64,
                 permute: int = 1, device: str = "cuda", head_dim: int = 128, payload_order: int = 0):
        # permute: 0 identity, 1 greedy grouping, 2 sort key (True/False = 1/0);
        # payload_order: 0 by channel, 1 K rows by decreasing width (b <= 4)
        lib = _lib.load()
        self.head_dim = head_dim
        self.cfg = _lib.Config(head_dim, bits, block, 32, int(permute), int(payload_order))
        sz = _lib.Sizes()
        _lib.check(lib.packkv_cache_sizes(ctypes.byref(self.cfg), n_streams, max_tokens, ctypes.byref(sz)),
                   "packkv_cache_sizes")
        self.sizes = sz
        self.n_streams, self.max_tokens, self.bits, self.block = n_streams, max_tokens, bits, block
        self.max_blocks = sz.max_blocks
        dev = torch.device(device)
        self.k_arena = torch.zeros(sz.arena_bytes, dtype=torch.uint8, device=dev)
        self.v_arena = torch.zeros(sz.arena_bytes, dtype=torch.uint8, device=dev)
        self.k_off = torch.zeros(n_streams * (sz.max_blocks + 1), dtype=torch.int32, device=dev)
        self.v_off = torch.zeros_like(self.k_off)
        self.perm = torch.full((sz.perm_bytes,), 0xFF, dtype=torch.uint8, device=dev)
        self.tail_k = torch.zeros(n_streams * block * self.head_dim, dtype=torch.float16, device=dev)
        self.tail_v = torch.zeros_like(self.tail_k)
        self.status = torch.zeros(1, dtype=torch.int32, device=dev)
        self._c = _lib.CacheT(self.cfg, n_streams, max_tokens, 0, sz.arena_stride,
                              _ptr(self.k_arena), _ptr(self.v_arena), _ptr(self.k_off), _ptr(self.v_off),
                              _ptr(self.perm), _ptr(self.tail_k), _ptr(self.tail_v), _ptr(self.status))
        self._ws: dict = {}
        self._aws: dict = {}

    # ------------------------------------------------------------------ state
    @property
    def n_tokens(self) -> int:
        return int(self._c.n_tokens)

    @property
    def arena_stride(self) -> int:
        return int(self.sizes.arena_stride)

    def offsets(self, which: str) -> torch.Tensor:
        off = self.k_off if which == "K" else self.v_off
        return off.view(self.n_streams, self.max_blocks + 1)

    def perm_table(self) -> torch.Tensor:
        return self.perm.view(self.n_streams, self.max_blocks, self.block)

    def arena(self, which: str) -> torch.Tensor:
        a = self.k_arena if which == "K" else self.v_arena
        return a.view(self.n_streams, self.arena_stride)

    # ------------------------------------------------------------ checkpoint
    _STATE = ("k_arena", "v_arena", "k_off", "v_off", "perm", "tail_k", "tail_v")

    def state_dict(self) -> dict:
        """The cache's whole state as host tensors: both arenas, both offset
        tables, the permutation, the raw tail staging and the token count.
        Synchronises the current stream first."""
        torch.cuda.current_stream().synchronize()
        st = {name: getattr(self, name).cpu() for name in self._STATE}
        st["n_tokens"] = self.n_tokens
        st["config"] = (self.n_streams, self.max_tokens, self.bits, self.block, int(self.cfg.permute),
                        self.head_dim, int(self.cfg.payload_order))
        return st

    def load_state_dict(self, st: dict) -> None:
        """Restores a state taken by state_dict from a cache of the same
        configuration; appends then continue where that cache stopped."""
        mine = (self.n_streams, self.max_tokens, self.bits, self.block, int(self.cfg.permute), self.head_dim,
                int(self.cfg.payload_order))
        if tuple(st["config"]) != mine:
            raise ValueError(f"state of a cache configured {tuple(st['config'])}, this one is {mine}")
        for name in self._STATE:
            dst = getattr(self, name)
            src = st[name]
            if src.shape != dst.shape or src.dtype != dst.dtype:
                raise ValueError(f"{name}: shape or dtype differs")
            dst.copy_(src, non_blocking=False)
        self._c.n_tokens = int(st["n_tokens"])
        self.status.zero_()

    # ------------------------------------------------------------- encoding
    def compress(self, k: torch.Tensor, v: torch.Tensor) -> None:
        """Prefill: k, v fp16 [S][T][D] contiguous on the device."""
        self._check_kv(k, v)
        _lib.check(_lib.load().packkv_compress_block(ctypes.byref(self._c), _ptr(k), _ptr(v), k.shape[1],
                                                     _stream()), "packkv_compress_block")

    def append(self, k: torch.Tensor, v: torch.Tensor) -> None:
        """Decode: append k, v fp16 [S][n][D]."""
        self._check_kv(k, v)
        _lib.check(_lib.load().packkv_append_tokens(ctypes.byref(self._c), _ptr(k), _ptr(v), k.shape[1],
                                                    _stream()), "packkv_append_tokens")

    def _check_kv(self, k, v):
        if k.dtype != torch.float16 or v.dtype != torch.float16 or not k.is_contiguous() or \
                not v.is_contiguous() or k.shape != v.shape or k.dim() != 3 or \
                k.shape[0] != self.n_streams or k.shape[2] != self.head_dim or not k.is_cuda:
            raise ValueError("k and v must be contiguous fp16 CUDA tensors [S][T][D]")

    # ------------------------------------------------------------- decoding
    def qk(self, q: torch.Tensor, scores: Optional[torch.Tensor] = None) -> torch.Tensor:
        """scores[s][g][t] = q[s][g] . K_hat[s][t] (slot order); q fp16 [S][G][D]."""
        S, G, d = q.shape
        if q.dtype != torch.float16 or S != self.n_streams or d != self.head_dim or not q.is_contiguous():
            raise ValueError("q must be contiguous fp16 [S][G][D]")
        T = self.n_tokens
        if scores is None:
            scores = torch.empty(S, G, T, dtype=torch.float32, device=q.device)
        if scores.dtype != torch.float32 or scores.shape[:2] != (S, G) or scores.stride(2) != 1 \
                or scores.stride(1) != scores.shape[2] or scores.stride(0) != G * scores.shape[2]:
            raise ValueError("scores must be contiguous fp32 [S][G][ld]")
        _lib.check(_lib.load().packkv_qk_gemv(ctypes.byref(self._c), _ptr(q), G, _ptr(scores),
                                              scores.shape[2], _stream()), "packkv_qk_gemv")
        return scores

    def workspace(self, group: int) -> torch.Tensor:
        """The V GEMV workspace for `group` queries per stream, zero-filled when
        first made (its per-stream counters must start at zero; each call
        leaves them at zero), then reused."""
        need = int(_lib.load().packkv_pv_workspace_bytes(ctypes.byref(self._c), group))
        ws = self._ws.get(group)
        if ws is None or ws.numel() < need:
            ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=self.k_arena.device)
            self._ws[group] = ws
        return ws

    def pv(self, p: torch.Tensor, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        """out[s][g][c] = sum_t p[s][g][t] V_hat[s][t][c]; p fp32 [S][G][ld] in slot order."""
        S, G, ld = p.shape
        if p.dtype != torch.float32 or S != self.n_streams or not p.is_contiguous():
            raise ValueError("p must be contiguous fp32 [S][G][ld]")
        if out is None:
            out = torch.empty(S, G, self.head_dim, dtype=torch.float32, device=p.device)
        ws = self.workspace(G) if workspace is None else workspace
        _lib.check(_lib.load().packkv_pv_gemv(ctypes.byref(self._c), _ptr(p), ld, G, _ptr(out), _ptr(ws),
                                              ws.numel() * ws.element_size(), _stream()),
                   "packkv_pv_gemv")
        return out

    def attention_workspace(self, group: int) -> torch.Tensor:
        """The fused-attention workspace for `group` queries per stream,
        zero-filled when first made, then reused."""
        need = int(_lib.load().packkv_attention_workspace_bytes(ctypes.byref(self._c), group))
        ws = self._aws.get(group)
        if ws is None or ws.numel() < need:
            ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=self.k_arena.device)
            self._aws[group] = ws
        return ws

    def attention(self, q: torch.Tensor, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        """out[s][g] = softmax(scale * q[s][g] . K_hat[s]^T) V_hat[s] in one launch;
        q fp16 [S][G][D], scale defaults to 1/sqrt(D)."""
        S, G, d = q.shape
        if q.dtype != torch.float16 or S != self.n_streams or d != self.head_dim or not q.is_contiguous():
            raise ValueError("q must be contiguous fp16 [S][G][D]")
        if out is None:
            out = torch.empty(S, G, self.head_dim, dtype=torch.float32, device=q.device)
        if out.dtype != torch.float32 or tuple(out.shape) != (S, G, self.head_dim) or not out.is_contiguous():
            raise ValueError("out must be contiguous fp32 [S][G][D]")
        ws = self.attention_workspace(G) if workspace is None else workspace
        sc = self.head_dim ** -0.5 if scale is None else float(scale)
        _lib.check(_lib.load().packkv_attention_decode(ctypes.byref(self._c), _ptr(q), G, sc, _ptr(out), _ptr(ws),
                                                       ws.numel() * ws.element_size(), _stream()),
                   "packkv_attention_decode")
        return out

    def attention_noalloc(self, q: torch.Tensor, out: torch.Tensor, scale: Optional[float] = None) -> torch.Tensor:
        """attention() through packkv_attention_decode_noalloc: no workspace,
        the library's own per-GPU scratch array instead (the caller passes
        out, fp32 [S][G][D]); bit-identical results."""
        S, G, d = q.shape
        if q.dtype != torch.float16 or S != self.n_streams or d != self.head_dim or not q.is_contiguous():
            raise ValueError("q must be contiguous fp16 [S][G][D]")
        if out.dtype != torch.float32 or tuple(out.shape) != (S, G, self.head_dim) or not out.is_contiguous():
            raise ValueError("out must be contiguous fp32 [S][G][D]")
        sc = self.head_dim ** -0.5 if scale is None else float(scale)
        _lib.check(_lib.load().packkv_attention_decode_noalloc(ctypes.byref(self._c), _ptr(q), G, sc, _ptr(out),
                                                               _stream()), "packkv_attention_decode_noalloc")
        return out

    def decompress(self, which: str, mode: int) -> torch.Tensor:
        """mode 0: uint8 q [S][T][D] slot order; mode 1: fp32 x_hat [S][T][D] token order."""
        T = self.n_tokens
        dt = torch.uint8 if mode == 0 else torch.float32
        out = torch.zeros(self.n_streams, T, self.head_dim, dtype=dt, device=self.k_arena.device)
        _lib.check(_lib.load().packkv_decompress(ctypes.byref(self._c), 0 if which == "K" else 1, mode,
                                                 _ptr(out), _stream()), "packkv_decompress")
        return out

    def check(self) -> int:
        """Synchronise and return (and clear) the device error latch."""
        return int(_lib.load().packkv_check(ctypes.byref(self._c), _stream()))

    def stats(self) -> dict:
        out = torch.zeros(32, dtype=torch.int64, device=self.k_arena.device)
        _lib.check(_lib.load().packkv_stats(ctypes.byref(self._c), _ptr(out), _stream()), "packkv_stats")
        o = out.cpu().tolist()
        # widths 0..4 then 5..8 (the latter only at b > 4)
        nw = self.bits + 1
        return {"k_width_hist": (o[0:5] + o[16:20])[:max(5, nw)], "v_width_hist": (o[5:10] + o[20:24])[:max(5, nw)],
                "k_bytes": o[10], "v_bytes": o[11], "k_words": o[12], "v_words": o[13], "k_runs": o[14],
                "v_runs": o[15]}


def stream_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """The streaming-read ceiling probe: read a 16-byte-aligned device buffer
    once; sink (int32 [4096], on the device) receives the XOR of each
    workgroup's words, so folding a zero-filled sink gives the buffer's XOR."""
    if sink.dtype != torch.int32 or sink.numel() < 4096 or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous int32 tensor of at least 4096 words")
    nbytes = buf.numel() * buf.element_size()
    _lib.check(_lib.load().packkv_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream()), "packkv_stream_read")


def attention_multi_workspace(caches, group: int) -> torch.Tensor:
    """A zero-filled workspace for attention_multi over `caches` (reusable)."""
    need = int(_lib.load().packkv_attention_multi_workspace_bytes(ctypes.byref(caches[0]._c), group, len(caches)))
    return torch.zeros(max(need, 16), dtype=torch.uint8, device=caches[0].k_arena.device)


def attention_multi(caches, q: torch.Tensor, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """PackedKVCache.attention for several caches of one shape (e.g. a
    model's layers) in one launch: q fp16 [L][S][G][D] -> out fp32 [L][S][G][D]."""
    L, S, G, d = q.shape
    if L != len(caches) or L < 1:
        raise ValueError("q must have one [S][G][D] slice per cache")
    D = caches[0].head_dim
    if q.dtype != torch.float16 or d != D or not q.is_contiguous():
        raise ValueError("q must be contiguous fp16 [L][S][G][D]")
    if out is None:
        out = torch.empty(L, S, G, D, dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (L, S, G, D) or not out.is_contiguous():
        raise ValueError("out must be contiguous fp32 [L][S][G][D]")
    ws = attention_multi_workspace(caches, G) if workspace is None else workspace
    sc = D ** -0.5 if scale is None else float(scale)
    arr = (ctypes.POINTER(_lib.CacheT) * L)(*[ctypes.pointer(c._c) for c in caches])
    _lib.check(_lib.load().packkv_attention_decode_multi(arr, L, _ptr(q), G, sc, _ptr(out), _ptr(ws),
                                                         ws.numel() * ws.element_size(), _stream()),
               "packkv_attention_decode_multi")
    return out


def softmax_rows(scores: torch.Tensor, T: int, scale: float, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """p = softmax(scores * scale) over the first T entries of each row ([..., ld] fp32)."""
    if scores.dtype != torch.float32 or not scores.is_contiguous():
        raise ValueError("scores must be contiguous fp32")
    ld = scores.shape[-1]
    rows = scores.numel() // ld
    if out is None:
        out = torch.empty_like(scores)
    _lib.check(_lib.load().packkv_softmax_rows(_ptr(scores), _ptr(out), rows, T, ld, scale, _stream()),
               "packkv_softmax_rows")
    return out
