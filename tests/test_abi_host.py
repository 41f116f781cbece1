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


def cfg(bits=4, block=64, D=128, R=32, permute=1, order=0):
    return _lib.Config(D, bits, block, R, permute, order)


@pytest.mark.parametrize("bad,code", [
    (dict(D=96), _lib.EUNSUPPORTED), (dict(D=512), _lib.EUNSUPPORTED), (dict(bits=9), _lib.EUNSUPPORTED),
    (dict(bits=1), _lib.EUNSUPPORTED),
    (dict(block=32), _lib.EUNSUPPORTED), (dict(R=16), _lib.EUNSUPPORTED), (dict(permute=3), _lib.EINVAL),
    (dict(order=2), _lib.EINVAL), (dict(order=-1), _lib.EINVAL), (dict(bits=5, order=1), _lib.EUNSUPPORTED),
    (dict(bits=8, order=1), _lib.EUNSUPPORTED),
])
def test_unsupported_configs_are_rejected(lib, bad, code):
    s = _lib.Sizes()
    assert lib.packkv_cache_sizes(ctypes.byref(cfg(**bad)), 4, 1000, ctypes.byref(s)) == code
    assert lib.packkv_arena_stride_bytes(ctypes.byref(cfg(**bad)), 1000) == 0


@pytest.mark.parametrize("bits,block", [(2, 64), (3, 64), (4, 64), (4, 128), (3, 128), (5, 64), (8, 128)])
def test_sizes_follow_the_worst_case_record(lib, bits, block):
    s = _lib.Sizes()
    assert lib.packkv_cache_sizes(ctypes.byref(cfg(bits, block)), 3, 1000, ctypes.byref(s)) == 0
    nb = -(-1000 // block)
    nr = block // 32
    hb = 1 if bits <= 4 else 2                    # header entry bytes
    krec = -(-(512 + hb * nr * 128) // 16) * 16 + 4 * nr * 128 * bits
    vrec = -(-(4 * block + hb * nr * 128) // 16) * 16 + 4 * nr * 128 * bits
    assert s.max_blocks == nb
    assert s.arena_stride % 256 == 0 and s.arena_stride >= nb * max(krec, vrec) + 64
    assert s.arena_bytes == 3 * s.arena_stride
    assert s.off_bytes == 3 * (nb + 1) * 4 and s.perm_bytes == 3 * nb * block
    assert s.tail_bytes == 3 * block * 128 * 2
    assert lib.packkv_arena_stride_bytes(ctypes.byref(cfg(bits, block)), 1000) == s.arena_stride


@pytest.mark.parametrize("D,bits,block", [(64, 4, 64), (64, 8, 128), (256, 2, 64), (256, 8, 128)])
def test_sizes_follow_the_head_dim(lib, D, bits, block):
    """Records scale with head_dim: K params 4D, V params 4B, one header entry
    per (run, channel), b words per (run, channel) at full width."""
    s = _lib.Sizes()
    assert lib.packkv_cache_sizes(ctypes.byref(cfg(bits, block, D=D)), 2, 1000, ctypes.byref(s)) == 0
    nb, nr, hb = -(-1000 // block), block // 32, 1 if bits <= 4 else 2
    krec = -(-(4 * D + hb * nr * D) // 16) * 16 + 4 * nr * D * bits
    vrec = -(-(4 * block + hb * nr * D) // 16) * 16 + 4 * nr * D * bits
    assert s.arena_stride >= nb * max(krec, vrec) + 64 and s.arena_stride % 256 == 0
    assert s.tail_bytes == 2 * block * D * 2


def test_paged_cache_takes_head_dim_128_only(lib):
    s = _lib.PagedSizes()
    for D in (64, 256):
        c = cfg(4, 64, D=D)
        assert lib.packkv_paged_sizes(ctypes.byref(c), 2, 1000, 16, 65536, ctypes.byref(s)) == _lib.EUNSUPPORTED
    assert lib.packkv_paged_sizes(ctypes.byref(cfg(4, 64)), 2, 1000, 16, 65536, ctypes.byref(s)) == 0


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
    # the encoder reads appended tokens with 16-byte loads: misaligned input
    # is refused before any launch
    assert lib.packkv_append_tokens(ctypes.byref(c3), fake + 2, fake, 1, None) == _lib.EINVAL
    assert lib.packkv_append_tokens(ctypes.byref(c3), fake, fake + 8, 1, None) == _lib.EINVAL
    assert lib.packkv_compress_block(ctypes.byref(c3), fake + 4, fake, 10, None) == _lib.EINVAL
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


def paged_cfg(lib, S=3, max_tokens=1000, n_pages=8, page=None, bits=4, block=64):
    s = _lib.PagedSizes()
    c = cfg(bits, block)
    assert lib.packkv_paged_sizes(ctypes.byref(c), S, max_tokens, n_pages, 1 << 20, ctypes.byref(s)) == 0
    page = page or s.min_page_bytes
    fake = 4096
    host = (ctypes.c_int32 * S)()
    p = _lib.PagedT(c, S, n_pages, max_tokens, page, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                    ctypes.addressof(host))
    return p, host, s


@pytest.mark.parametrize("bits,block", [(2, 64), (4, 64), (3, 128), (4, 128)])
def test_paged_sizes(lib, bits, block):
    s = _lib.PagedSizes()
    c = cfg(bits, block)
    assert lib.packkv_paged_sizes(ctypes.byref(c), 3, 1000, 10, 1 << 16, ctypes.byref(s)) == 0
    nr = block // 32
    krec = -(-(512 + nr * 128) // 16) * 16 + 4 * nr * 128 * bits
    vrec = -(-(4 * block + nr * 128) // 16) * 16 + 4 * nr * 128 * bits
    assert s.slot_bytes == max(krec, vrec)
    assert s.min_page_bytes % 256 == 0 and s.slot_bytes <= s.min_page_bytes < s.slot_bytes + 256
    assert s.pool_bytes == 10 * (1 << 16) + 3 * 2 * s.slot_bytes + 256
    mb = -(-1000 // block)
    assert s.max_blocks == mb and s.table_bytes == 3 * mb * 8
    assert s.alloc_bytes == (2 + 4 * 3 + 10) * 4 and s.lengths_bytes == 12
    assert s.perm_bytes == 3 * mb * block and s.tail_bytes == 3 * block * 128 * 2
    bad = lambda **kw: lib.packkv_paged_sizes(ctypes.byref(c), kw.get("S", 3), 1000, kw.get("n", 10),
                                              kw.get("page", 1 << 16), ctypes.byref(s))
    assert bad(page=s.min_page_bytes + 128) == _lib.EINVAL          # not a multiple of 256
    assert bad(page=s.min_page_bytes - 256) == _lib.EINVAL          # below one record
    assert bad(n=0) == _lib.EINVAL
    assert bad(n=(1 << 36) // (1 << 16)) == _lib.EINVAL            # pool past 2^32 16-byte units
    assert bad(S=0) == _lib.EINVAL


def test_paged_calls_check_before_any_launch(lib):
    p, host, s = paged_cfg(lib)
    fake = 4096
    P = ctypes.byref(p)
    need = lib.packkv_paged_attention_workspace_bytes(P, 1)
    assert need > 0
    # every stream empty: nothing to attend to
    assert lib.packkv_paged_attention(P, fake, 1, 0.1, fake, fake, need, None) == _lib.ESTATE
    host[1] = 10
    assert lib.packkv_paged_attention(P, fake, 1, 0.1, fake, fake, need - 1, None) == _lib.EINVAL
    assert lib.packkv_paged_attention(P, None, 1, 0.1, fake, fake, need, None) == _lib.EINVAL
    assert lib.packkv_paged_attention(P, fake, 0, 0.1, fake, fake, need, None) == _lib.EINVAL
    assert lib.packkv_paged_attention(P, fake, 1, float("inf"), fake, fake, need, None) == _lib.EINVAL
    # prefill: a stream that holds tokens, a range past S, too many tokens, misalignment
    assert lib.packkv_paged_prefill(P, 1, 1, fake, fake, 10, None) == _lib.ESTATE
    assert lib.packkv_paged_prefill(P, 0, 2, fake, fake, 10, None) == _lib.ESTATE
    assert lib.packkv_paged_prefill(P, 2, 2, fake, fake, 10, None) == _lib.EINVAL
    assert lib.packkv_paged_prefill(P, 0, 1, fake, fake, 1001, None) == _lib.ECAPACITY
    assert lib.packkv_paged_prefill(P, 0, 1, fake + 2, fake, 10, None) == _lib.EINVAL
    assert lib.packkv_paged_prefill(P, 0, 1, fake, fake, 0, None) == _lib.EINVAL
    # append: one full stream stops the step
    host[2] = 1000
    assert lib.packkv_paged_append(P, fake, fake, None) == _lib.ECAPACITY
    assert lib.packkv_paged_append(P, None, fake, None) == _lib.EINVAL
    assert list(host) == [0, 10, 1000]                             # nothing changed
    assert lib.packkv_paged_release(P, 3, None) == _lib.EINVAL
    assert lib.packkv_paged_release(P, -1, None) == _lib.EINVAL
    # a page below one record, or a missing array
    p.page_bytes = s.min_page_bytes - 256
    assert lib.packkv_paged_release(P, 0, None) == _lib.EINVAL
    p.page_bytes = s.min_page_bytes
    p.host_lengths = None
    assert lib.packkv_paged_release(P, 0, None) == _lib.EINVAL


def test_stream_read_checks_its_arguments(lib):
    fake = 4096
    assert lib.packkv_stream_read(None, 64, fake, None) == _lib.EINVAL
    assert lib.packkv_stream_read(fake, 64, None, None) == _lib.EINVAL
    assert lib.packkv_stream_read(fake + 8, 64, fake, None) == _lib.EINVAL     # not 16-byte aligned
    assert lib.packkv_stream_read(fake, 60, fake, None) == _lib.EINVAL         # not a multiple of 16
    assert lib.packkv_stream_read(fake, 0, fake, None) == _lib.EINVAL


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_width_sorted_payload_keeps_the_sizes(lib, bits):
    """Payload order 1 is accepted up to 4 bits and sizes nothing differently."""
    a, b = _lib.Sizes(), _lib.Sizes()
    assert lib.packkv_cache_sizes(ctypes.byref(cfg(bits)), 3, 1000, ctypes.byref(a)) == 0
    assert lib.packkv_cache_sizes(ctypes.byref(cfg(bits, order=1)), 3, 1000, ctypes.byref(b)) == 0
    assert bytes(a) == bytes(b)
