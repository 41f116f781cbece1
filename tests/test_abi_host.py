"""The C-ABI library loads, exports every declared symbol, and validates on the host.

No test here launches a kernel: every call below fails (or succeeds) in host
code before the library touches the GPU.
"""

import ctypes
import os

import pytest

from decode_gemv_amd import _lib


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return _lib.load()


def test_every_header_function_is_exported(lib):
    names = _lib.header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/packkv.h but not exported"
    assert set(names) == set(_lib._SIGS), "binding signatures and header disagree"


def cfg(bits=4, block=64, D=128, R=32, permute=1):
    return _lib.Config(D, bits, block, R, permute)


@pytest.mark.parametrize("bad,code", [
    (dict(D=64), _lib.EUNSUPPORTED), (dict(bits=5), _lib.EUNSUPPORTED), (dict(bits=1), _lib.EUNSUPPORTED),
    (dict(block=32), _lib.EUNSUPPORTED), (dict(R=16), _lib.EUNSUPPORTED), (dict(permute=3), _lib.EINVAL),
])
def test_unsupported_configs_are_rejected(lib, bad, code):
    s = _lib.Sizes()
    assert lib.packkv_cache_sizes(ctypes.byref(cfg(**bad)), 4, 1000, ctypes.byref(s)) == code
    assert lib.packkv_arena_stride_bytes(ctypes.byref(cfg(**bad)), 1000) == 0


@pytest.mark.parametrize("bits,block", [(2, 64), (3, 64), (4, 64), (4, 128), (3, 128)])
def test_sizes_follow_the_worst_case_record(lib, bits, block):
    s = _lib.Sizes()
    assert lib.packkv_cache_sizes(ctypes.byref(cfg(bits, block)), 3, 1000, ctypes.byref(s)) == 0
    nb = -(-1000 // block)
    nr = block // 32
    krec = -(-(512 + nr * 128) // 16) * 16 + 4 * nr * 128 * bits
    vrec = -(-(4 * block + nr * 128) // 16) * 16 + 4 * nr * 128 * bits
    assert s.max_blocks == nb
    assert s.arena_stride % 256 == 0 and s.arena_stride >= nb * max(krec, vrec) + 64
    assert s.arena_bytes == 3 * s.arena_stride
    assert s.off_bytes == 3 * (nb + 1) * 4 and s.perm_bytes == 3 * nb * block
    assert s.tail_bytes == 3 * block * 128 * 2
    assert lib.packkv_arena_stride_bytes(ctypes.byref(cfg(bits, block)), 1000) == s.arena_stride


def test_invalid_arguments_fail_before_any_launch(lib):
    c = _lib.CacheT(cfg(), 2, 100, 0, 0, None, None, None, None, None, None, None, None)
    assert lib.packkv_compress_block(ctypes.byref(c), None, None, 10, None) == _lib.EINVAL
    assert lib.packkv_qk_gemv(ctypes.byref(c), None, 1, None, 10, None) == _lib.EINVAL
    assert lib.packkv_pv_workspace_bytes(ctypes.byref(c), 1) == 0
    assert lib.packkv_softmax_rows(None, None, 1, 10, 10, 1.0, None) == _lib.EINVAL
    # a cache whose pointers are set but whose stride is too small
    fake = 4096
    c2 = _lib.CacheT(cfg(), 2, 100, 0, 256, fake, fake, fake, fake, fake, fake, fake, fake)
    assert lib.packkv_compress_block(ctypes.byref(c2), fake, fake, 10, None) == _lib.EINVAL
    s = _lib.Sizes()
    lib.packkv_cache_sizes(ctypes.byref(cfg()), 2, 100, ctypes.byref(s))
    c3 = _lib.CacheT(cfg(), 2, 100, 0, s.arena_stride, fake, fake, fake, fake, fake, fake, fake, fake)
    assert lib.packkv_compress_block(ctypes.byref(c3), fake, fake, 101, None) == _lib.ECAPACITY
    assert lib.packkv_compress_block(ctypes.byref(c3), fake, fake, 0, None) == _lib.EINVAL
    assert lib.packkv_qk_gemv(ctypes.byref(c3), fake, 1, fake, 10, None) == _lib.ESTATE
    c3.n_tokens = 50
    assert lib.packkv_compress_block(ctypes.byref(c3), fake, fake, 10, None) == _lib.ESTATE
    assert lib.packkv_qk_gemv(ctypes.byref(c3), fake, 0, fake, 50, None) == _lib.EINVAL
    assert lib.packkv_qk_gemv(ctypes.byref(c3), fake, 1, fake, 49, None) == _lib.EINVAL
    assert lib.packkv_append_tokens(ctypes.byref(c3), fake, fake, 51, None) == _lib.ECAPACITY
    assert lib.packkv_decompress(ctypes.byref(c3), 2, 0, fake, None) == _lib.EINVAL
    assert lib.packkv_pv_gemv(ctypes.byref(c3), fake, 50, 1, fake, fake, 0, None) == _lib.EINVAL
    need = lib.packkv_attention_workspace_bytes(ctypes.byref(c3), 1)
    assert need > 0
    assert lib.packkv_attention_decode(ctypes.byref(c3), None, 1, 0.1, fake, fake, need, None) == _lib.EINVAL
    assert lib.packkv_attention_decode(ctypes.byref(c3), fake, 0, 0.1, fake, fake, need, None) == _lib.EINVAL
    assert lib.packkv_attention_decode(ctypes.byref(c3), fake, 1, 0.0, fake, fake, need, None) == _lib.EINVAL
    assert lib.packkv_attention_decode(ctypes.byref(c3), fake, 1, float("nan"), fake, fake, need, None) == _lib.EINVAL
    assert lib.packkv_attention_decode(ctypes.byref(c3), fake, 1, 0.1, fake, fake, need - 1, None) == _lib.EINVAL
    c3.n_tokens = 0
    assert lib.packkv_attention_decode(ctypes.byref(c3), fake, 1, 0.1, fake, fake, need, None) == _lib.ESTATE


def test_multi_cache_attention_checks_before_any_launch(lib):
    fake = 4096
    s = _lib.Sizes()
    lib.packkv_cache_sizes(ctypes.byref(cfg()), 2, 100, ctypes.byref(s))
    mk = lambda n_tokens=50, S=2, max_tokens=100: _lib.CacheT(cfg(), S, max_tokens, n_tokens, s.arena_stride,
                                                               fake, fake, fake, fake, fake, fake, fake, fake)
    a, b = mk(), mk()
    one = lib.packkv_attention_workspace_bytes(ctypes.byref(a), 1)
    assert lib.packkv_attention_multi_workspace_bytes(ctypes.byref(a), 1, 3) == 3 * one
    assert lib.packkv_attention_multi_workspace_bytes(ctypes.byref(a), 1, 0) == 0
    P = ctypes.POINTER(_lib.CacheT)
    arr = lambda *cs: (P * len(cs))(*[ctypes.pointer(c) for c in cs])
    ok2 = arr(a, b)
    assert lib.packkv_attention_decode_multi(None, 2, fake, 1, 0.1, fake, fake, 2 * one, None) == _lib.EINVAL
    assert lib.packkv_attention_decode_multi(ok2, 0, fake, 1, 0.1, fake, fake, 2 * one, None) == _lib.EINVAL
    assert lib.packkv_attention_decode_multi(ok2, 2, fake, 1, 0.1, fake, fake, 2 * one - 1, None) == _lib.EINVAL
    assert lib.packkv_attention_decode_multi(ok2, 2, None, 1, 0.1, fake, fake, 2 * one, None) == _lib.EINVAL
    # caches that differ in length, stream count or capacity
    for other in (mk(n_tokens=49), mk(S=3), mk(max_tokens=99)):
        assert lib.packkv_attention_decode_multi(arr(a, other), 2, fake, 1, 0.1, fake, fake, 4 * one,
                                                 None) == _lib.EINVAL
    empty = arr(mk(n_tokens=0), mk(n_tokens=0))
    assert lib.packkv_attention_decode_multi(empty, 2, fake, 1, 0.1, fake, fake, 2 * one, None) == _lib.ESTATE


def test_status_strings(lib):
    for code in range(7):
        assert lib.packkv_status_str(code)
    assert lib.packkv_status_str(99) == b"unknown status"
