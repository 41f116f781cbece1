"""decode_gemv_amd - PackKV's compressed KV cache and fused decompress-GEMVs on MI355X.

The hot path lives in the HIP library ``libpackkv.so`` (C ABI in
``include/packkv.h``); this package only marshals torch tensors into it.
"""

from ._lib import PackKVError, load as load_library  # noqa: F401
from .cache import PackedKVCache, attention_multi, attention_multi_workspace, softmax_rows, stream_read  # noqa: F401,E501
from .paged import PagedKVCache  # noqa: F401

__all__ = ["PackedKVCache", "PagedKVCache", "attention_multi", "attention_multi_workspace", "softmax_rows",
           "stream_read", "PackKVError", "load_library"]
