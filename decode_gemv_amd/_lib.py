"""ctypes view of the packkv C ABI (include/packkv.h).

Loading the shared library does not touch the GPU.  If the library has not
been built, importing fails loudly: there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpackkv.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "packkv.h")

OK, EINVAL, EUNSUPPORTED, ECAPACITY, ECORRUPT, EHIP, ESTATE = range(7)

c_int32, c_int64, c_uint64, c_void_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p


class Config(ctypes.Structure):
    _fields_ = [("head_dim", c_int32), ("bits", c_int32), ("block_tokens", c_int32),
                ("run_tokens", c_int32), ("permute", c_int32), ("payload_order", c_int32)]


class CacheT(ctypes.Structure):
    _fields_ = [("cfg", Config), ("n_streams", c_int32), ("max_tokens", c_int64),
                ("n_tokens", c_int64), ("arena_stride", c_uint64),
                ("k_arena", c_void_p), ("v_arena", c_void_p),
                ("k_off", c_void_p), ("v_off", c_void_p), ("perm", c_void_p),
                ("tail_k", c_void_p), ("tail_v", c_void_p), ("status", c_void_p)]


class Sizes(ctypes.Structure):
    _fields_ = [("arena_stride", c_uint64), ("arena_bytes", c_uint64), ("off_bytes", c_uint64),
                ("perm_bytes", c_uint64), ("tail_bytes", c_uint64), ("max_blocks", c_int64)]


class PagedT(ctypes.Structure):
    _fields_ = [("cfg", Config), ("n_streams", c_int32), ("n_pages", c_int32), ("max_tokens", c_int64),
                ("page_bytes", c_uint64), ("pool", c_void_p), ("k_table", c_void_p), ("v_table", c_void_p),
                ("lengths", c_void_p), ("alloc", c_void_p), ("perm", c_void_p), ("tail_k", c_void_p),
                ("tail_v", c_void_p), ("status", c_void_p), ("host_lengths", c_void_p)]


class PagedSizes(ctypes.Structure):
    _fields_ = [("pool_bytes", c_uint64), ("table_bytes", c_uint64), ("alloc_bytes", c_uint64),
                ("lengths_bytes", c_uint64), ("perm_bytes", c_uint64), ("tail_bytes", c_uint64),
                ("slot_bytes", c_uint64), ("min_page_bytes", c_uint64), ("max_blocks", c_int64)]


class PackKVError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"{what}: packkv status {code} ({status_str(code)})")


_SIGS = {
    "packkv_cache_sizes": (c_int32, [ctypes.POINTER(Config), c_int32, c_int64, ctypes.POINTER(Sizes)]),
    "packkv_arena_stride_bytes": (c_uint64, [ctypes.POINTER(Config), c_int64]),
    "packkv_pv_workspace_bytes": (c_uint64, [ctypes.POINTER(CacheT), c_int32]),
    "packkv_attention_workspace_bytes": (c_uint64, [ctypes.POINTER(CacheT), c_int32]),
    "packkv_attention_decode": (c_int32, [ctypes.POINTER(CacheT), c_void_p, c_int32, ctypes.c_float, c_void_p,
                                          c_void_p, c_uint64, c_void_p]),
    "packkv_attention_decode_multi": (c_int32, [ctypes.POINTER(ctypes.POINTER(CacheT)), c_int32, c_void_p,
                                                c_int32, ctypes.c_float, c_void_p, c_void_p, c_uint64,
                                                c_void_p]),
    "packkv_attention_multi_workspace_bytes": (c_uint64, [ctypes.POINTER(CacheT), c_int32, c_int32]),
    "packkv_attention_decode_noalloc": (c_int32, [ctypes.POINTER(CacheT), c_void_p, c_int32, ctypes.c_float,
                                                  c_void_p, c_void_p]),
    "packkv_compress_block": (c_int32, [ctypes.POINTER(CacheT), c_void_p, c_void_p, c_int64, c_void_p]),
    "packkv_append_tokens": (c_int32, [ctypes.POINTER(CacheT), c_void_p, c_void_p, c_int32, c_void_p]),
    "packkv_qk_gemv": (c_int32, [ctypes.POINTER(CacheT), c_void_p, c_int32, c_void_p, c_int64, c_void_p]),
    "packkv_pv_gemv": (c_int32, [ctypes.POINTER(CacheT), c_void_p, c_int64, c_int32, c_void_p,
                                 c_void_p, c_uint64, c_void_p]),
    "packkv_decompress": (c_int32, [ctypes.POINTER(CacheT), c_int32, c_int32, c_void_p, c_void_p]),
    "packkv_softmax_rows": (c_int32, [c_void_p, c_void_p, c_int32, c_int64, c_int64, ctypes.c_float,
                                      c_void_p]),
    "packkv_check": (c_int32, [ctypes.POINTER(CacheT), c_void_p]),
    "packkv_stream_read": (c_int32, [c_void_p, c_uint64, c_void_p, c_void_p]),
    "packkv_stats": (c_int32, [ctypes.POINTER(CacheT), c_void_p, c_void_p]),
    "packkv_status_str": (ctypes.c_char_p, [c_int32]),
    "packkv_paged_sizes": (c_int32, [ctypes.POINTER(Config), c_int32, c_int64, c_int32, c_uint64,
                                     ctypes.POINTER(PagedSizes)]),
    "packkv_paged_init": (c_int32, [ctypes.POINTER(PagedT), c_void_p]),
    "packkv_paged_prefill": (c_int32, [ctypes.POINTER(PagedT), c_int32, c_int32, c_void_p, c_void_p, c_int64,
                                       c_void_p]),
    "packkv_paged_append": (c_int32, [ctypes.POINTER(PagedT), c_void_p, c_void_p, c_void_p]),
    "packkv_paged_release": (c_int32, [ctypes.POINTER(PagedT), c_int32, c_void_p]),
    "packkv_paged_attention_workspace_bytes": (c_uint64, [ctypes.POINTER(PagedT), c_int32]),
    "packkv_paged_attention": (c_int32, [ctypes.POINTER(PagedT), c_void_p, c_int32, ctypes.c_float, c_void_p,
                                         c_void_p, c_uint64, c_void_p]),
    "packkv_paged_check": (c_int32, [ctypes.POINTER(PagedT), c_void_p]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree libpackkv.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m decode_gemv_amd.build` "
                              "(the HIP library is required; there is no fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def header_functions() -> list:
    """Names of the functions include/packkv.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(packkv_\w+)\s*\(", text)))


def status_str(code: int) -> str:
    try:
        return load().packkv_status_str(code).decode()
    except Exception:  # pragma: no cover - only used for messages
        return "?"


def check(code: int, what: str) -> None:
    if code != OK:
        raise PackKVError(code, what)
