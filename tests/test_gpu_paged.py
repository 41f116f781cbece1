"""GPU parity of the paged cache: records reached through the block tables
are byte-identical to the oracle's records of each stream's tokens, the
allocator's placement is valid, and fused attention over ragged streams
matches the oracle (rel-L2 <= 1e-4) and, at equal lengths, the contiguous
cache bit for bit.
"""

import numpy as np
import pytest

from gpu_common import say, make_kv, oracle_streams, rel_l2, worst_row_rel, check_placement
from oracle import stream as ostream, attention

pytestmark = pytest.mark.gpu
TOL = 1e-4

CASES = [
    # id, bits, block, permute, law, page records (pages hold about this many records)
    ("b4B64-gauss", 4, 64, 1, "gauss", 2),
    ("b3B128-struct", 3, 128, 1, "struct", 3),
    ("b2B64-mixed-sortkey", 2, 64, 2, "mixed", 5),
    ("b4B64-identity", 4, 64, 0, "struct", 1),
    ("b8B64-gauss", 8, 64, 1, "gauss", 2),
    ("b6B128-struct", 6, 128, 2, "struct", 3),
    # width-sorted K payload (payload order 1)
    ("b3B128-struct-wsorted", 3, 128, 1, "struct", 3, 1),
    ("b4B64-mixed-wsorted", 4, 64, 2, "mixed", 2, 1),
]


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch, torch.device("cuda:0")


def paged(torch, dev, S, max_tokens, n_pages, page_records, bits, block, permute, payload_order=0):
    from decode_gemv_amd import PagedKVCache
    from decode_gemv_amd import _lib
    import ctypes
    sz = _lib.PagedSizes()
    cfg = _lib.Config(128, bits, block, 32, permute, payload_order)
    assert _lib.load().packkv_paged_sizes(ctypes.byref(cfg), S, max_tokens, 1, 1 << 20, ctypes.byref(sz)) == 0
    page = -(-page_records * sz.slot_bytes // 256) * 256
    return PagedKVCache(S, max_tokens, n_pages, page_bytes=page, bits=bits, block=block, permute=permute,
                        device=str(dev), payload_order=payload_order)


def check_records(c, refs, lengths):
    recs = c.records()
    perm = c.perm_table().cpu().numpy()
    B = c.block
    for s, (ref, n) in enumerate(zip(refs, lengths)):
        assert c.lengths[s] == n
        if n == 0:
            assert recs[s] == []
            continue
        ko, vo = ref.offsets("K"), ref.offsets("V")
        ka, va = ref.arena("K"), ref.arena("V")
        assert len(recs[s]) == len(ko) - 1
        for j, (kr, vr) in enumerate(recs[s]):
            assert kr == ka[ko[j]:ko[j + 1]], f"K record differs, stream {s}, block {j}"
            assert vr == va[vo[j]:vo[j + 1]], f"V record differs, stream {s}, block {j}"
        nb = len(ko) - 1
        assert np.array_equal(perm[s, :nb], ref.perm_table()), f"perm differs, stream {s}"
        nt = n % B
        tk = c.tail_k.view(c.n_streams, B, 128)[s, :nt].cpu().numpy()
        tv = c.tail_v.view(c.n_streams, B, 128)[s, :nt].cpu().numpy()
        assert np.array_equal(tk.view(np.uint16), ref.tail_k.view(np.uint16))
        assert np.array_equal(tv.view(np.uint16), ref.tail_v.view(np.uint16))


def check_attention(torch, dev, c, refs, lengths, G, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((c.n_streams, G, 128)).astype(np.float16)
    got = c.attention(torch.from_numpy(q).to(dev)).cpu().numpy()
    assert c.check() == 0
    for s, (ref, n) in enumerate(zip(refs, lengths)):
        if n == 0:
            assert not got[s].any(), "an empty stream's output is zero"
            continue
        kh, vh, _, _ = ostream.decode_stream(ref)
        want = attention.pv(attention.softmax(attention.qk(q[s], kh), 128), vh)
        assert rel_l2(got[s], want) <= TOL and worst_row_rel(got[s], want) <= TOL, \
            (s, rel_l2(got[s], want), worst_row_rel(got[s], want))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ragged_prefill_and_appends_match_oracle(torch_dev, case):
    """Streams prefilled to different lengths (one left empty), then decode
    steps on every stream: records, permutation, tail staging and attention
    equal the oracle's for each stream's tokens at every checkpoint."""
    torch, dev = torch_dev
    cid, bits, block, permute, law, page_records = case[:6]
    order = case[6] if len(case) > 6 else 0
    B = block
    start = [0, 1, B, B + 86, 5 * B + 13]
    steps = 70
    S = len(start)
    total = max(start) + steps
    K, V = make_kv(law, S, total, block, seed=3)
    c = paged(torch, dev, S, total + 4, 64, page_records, bits, block, permute, order)
    for s, n in enumerate(start):
        if n:
            say("paged prefill", cid, s, n)
            c.prefill(s, torch.from_numpy(K[s:s + 1, :n].copy()).to(dev),
                      torch.from_numpy(V[s:s + 1, :n].copy()).to(dev))
    assert c.check() == 0
    lengths = list(start)

    def refs_now():
        return [oracle_streams(K[s:s + 1, :n], V[s:s + 1, :n], bits, block, permute, order)[0] if n else None
                for s, n in enumerate(lengths)]

    refs = refs_now()
    check_records(c, refs, lengths)
    check_placement(c)
    check_attention(torch, dev, c, refs, lengths, 1, 1)
    Kd, Vd = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    idx = torch.arange(S, device=dev)
    for i in range(steps):
        pos = torch.tensor(lengths, device=dev)
        c.append(Kd[idx, pos].unsqueeze(1).contiguous(), Vd[idx, pos].unsqueeze(1).contiguous())
        lengths = [n + 1 for n in lengths]
        if i in (0, B - 2, steps - 1):
            say("paged append", cid, i, lengths)
            assert c.check() == 0
            refs = refs_now()
            check_records(c, refs, lengths)
            check_placement(c)
            check_attention(torch, dev, c, refs, lengths, 4, 10 + i)


@pytest.mark.parametrize("bits,block", [(4, 64), (3, 128)])
def test_release_returns_pages_and_the_stream_is_reused(torch_dev, bits, block):
    torch, dev = torch_dev
    S, T = 3, 6 * block + 5
    K, V = make_kv("gauss", S, T, block, seed=5)
    c = paged(torch, dev, S, T + 8, 40, 2, bits, block, 1)
    say("paged release", bits, block)
    c.prefill(0, torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev))
    assert c.check() == 0
    owner = check_placement(c)
    held = sum(1 for s, _ in owner.values() if s == 1)
    free0 = c.free_pages()
    c.release(1)
    assert c.check() == 0
    assert c.lengths == [T, 0, T]
    assert c.free_pages() == free0 + held
    lengths = [T, 0, T]
    refs = [oracle_streams(K[s:s + 1], V[s:s + 1], bits, block, 1)[0] if n else None for s, n in enumerate(lengths)]
    check_records(c, refs, lengths)
    check_attention(torch, dev, c, refs, lengths, 1, 2)
    # the slot takes a new sequence of another length
    K2, V2 = make_kv("struct", 1, 2 * block + 40, block, seed=9)
    c.prefill(1, torch.from_numpy(K2).to(dev), torch.from_numpy(V2).to(dev))
    assert c.check() == 0
    lengths = [T, 2 * block + 40, T]
    refs[1] = oracle_streams(K2, V2, bits, block, 1)[0]
    check_records(c, refs, lengths)
    check_placement(c)
    check_attention(torch, dev, c, refs, lengths, 3, 4)


def test_pool_exhaustion_is_reported(torch_dev):
    torch, dev = torch_dev
    from decode_gemv_amd import _lib
    S, T, block = 2, 20 * 64, 64
    K, V = make_kv("gauss", S, T, block, seed=2)
    c = paged(torch, dev, S, T, 6, 1, 4, block, 1)          # one record per page, 6 pages
    say("paged exhaustion")
    c.prefill(0, torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev))
    assert c.check() == _lib.ECAPACITY
    assert c.lengths_dev.cpu().tolist() == [0, 0]            # no stream took the tokens


@pytest.mark.parametrize("G", [1, 4])
def test_equal_lengths_match_the_contiguous_cache_bit_for_bit(torch_dev, G):
    """Same tokens in both layouts: the launch divides the work the same way,
    so the outputs are identical, before and after decode steps."""
    torch, dev = torch_dev
    from decode_gemv_amd import PackedKVCache
    S, T, block, steps = 4, 700, 64, 12
    K, V = make_kv("gauss", S, T + steps, block, seed=8)
    Kd, Vd = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    a = PackedKVCache(S, T + steps, bits=4, block=block, permute=1, device=str(dev))
    a.compress(Kd[:, :T].contiguous(), Vd[:, :T].contiguous())
    b = paged(torch, dev, S, T + steps, 256, 4, 4, block, 1)
    b.prefill(0, Kd[:, :T].contiguous(), Vd[:, :T].contiguous())
    rng = np.random.default_rng(G)
    for i in range(steps + 1):
        q = torch.from_numpy(rng.standard_normal((S, G, 128)).astype(np.float16)).to(dev)
        if i % 4 == 0:
            say("paged vs contiguous", G, i)
            x, y = a.attention(q), b.attention(q)
            assert a.check() == 0 and b.check() == 0
            assert torch.equal(x, y), i
        if i < steps:
            kn, vn = Kd[:, T + i:T + i + 1].contiguous(), Vd[:, T + i:T + i + 1].contiguous()
            a.append(kn, vn)
            b.append(kn, vn)
