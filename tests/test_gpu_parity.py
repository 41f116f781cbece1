"""GPU parity: the HIP path against the fp64 oracle on small seeded inputs.

Bit-exact: records (padding included), offsets, permutation, tail staging,
decompressed ints and fp32 x_hat.  Floating point: rel-L2 <= 1e-4 per output
tensor (fp64 norms) for both GEMVs and the softmax helper.
"""

import numpy as np
import pytest

from gpu_common import say, make_kv, oracle_streams, rel_l2, worst_row_rel
import oracle
from oracle import stream as ostream, attention, unpack as ounpack

pytestmark = pytest.mark.gpu
TOL = 1e-4

CASES = [
    # id, bits, block, S, T, permute (0 identity, 1 greedy, 2 sort key), law
    ("b4B64-gauss", 4, 64, 3, 200, True, "gauss"),
    ("b4B64-struct", 4, 64, 2, 331, True, "struct"),
    ("b4B64-mixed", 4, 64, 2, 256, True, "mixed"),
    ("b2B64-bimodal", 2, 64, 2, 190, True, "bimodal"),
    ("b2B64-struct", 2, 64, 2, 97, True, "struct"),
    ("b3B64-struct", 3, 64, 2, 257, True, "struct"),
    ("b3B64-gauss", 3, 64, 2, 130, True, "gauss"),
    ("b4B128-gauss", 4, 128, 2, 300, True, "gauss"),
    ("b3B128-struct", 3, 128, 2, 390, True, "struct"),
    ("b2B128-mixed", 2, 128, 2, 129, True, "mixed"),
    ("b4B64-identity", 4, 64, 2, 150, False, "struct"),
    ("b4B64-sortkey-struct", 4, 64, 2, 331, 2, "struct"),
    ("b4B64-sortkey-gauss", 4, 64, 2, 200, 2, "gauss"),
    ("b3B128-sortkey-struct", 3, 128, 2, 390, 2, "struct"),
    ("b2B64-sortkey-mixed", 2, 64, 2, 190, 2, "mixed"),
    ("b4B64-one-token", 4, 64, 1, 1, True, "gauss"),
    ("b4B64-grid", 4, 64, 2, 64, True, "grid"),
    ("b3B64-subnormal", 3, 64, 2, 100, True, "subnormal"),
    # wide widths: two-byte header entries and byte containers
    ("b8B64-gauss", 8, 64, 3, 200, True, "gauss"),
    ("b5B64-struct", 5, 64, 2, 331, True, "struct"),
    ("b6B128-mixed", 6, 128, 2, 256, True, "mixed"),
    ("b7B64-sortkey-gauss", 7, 64, 2, 150, 2, "gauss"),
    ("b8B128-struct", 8, 128, 2, 300, True, "struct"),
    ("b5B64-identity-grid", 5, 64, 2, 97, False, "grid"),
    ("b6B64-subnormal", 6, 64, 2, 100, True, "subnormal"),
    ("b8B64-one-token", 8, 64, 1, 1, True, "gauss"),
]


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch, torch.device("cuda:0")


def gpu_cache(torch, dev, K, V, bits, block, permute, max_tokens=None, payload_order=0):
    from decode_gemv_amd import PackedKVCache
    S, T, D = K.shape
    c = PackedKVCache(S, max_tokens or T + 70, bits=bits, block=block, permute=permute, device=str(dev),
                      head_dim=D, payload_order=payload_order)
    c.compress(torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev))
    return c


def assert_state_equal(c, refs):
    """Bit-exact comparison of the whole packed state with the oracle streams."""
    T = c.n_tokens
    B = c.block
    nb = -(-T // B)
    for which in "KV":
        arena = c.arena(which).cpu().numpy()
        offs = c.offsets(which).cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        for s, ref in enumerate(refs):
            ro = ref.offsets(which)
            assert np.array_equal(offs[s, :nb + 1], ro), f"{which} offsets differ, stream {s}"
            got = arena[s, :ro[-1]].tobytes()
            exp = ref.arena(which)
            if got != exp:
                bad = next(i for i in range(len(exp)) if got[i] != exp[i])
                blk = int(np.searchsorted(ro, bad, side="right") - 1)
                raise AssertionError(f"{which} record bytes differ, stream {s}, block {blk}, "
                                     f"byte {bad - ro[blk]} of the record")
    perm = c.perm_table().cpu().numpy()
    for s, ref in enumerate(refs):
        assert np.array_equal(perm[s, :nb], ref.perm_table()), f"perm differs, stream {s}"
        nt = T % B
        tk = c.tail_k.view(c.n_streams, B, c.head_dim)[s, :nt].cpu().numpy()
        tv = c.tail_v.view(c.n_streams, B, c.head_dim)[s, :nt].cpu().numpy()
        assert np.array_equal(tk.view(np.uint16), ref.tail_k.view(np.uint16))
        assert np.array_equal(tv.view(np.uint16), ref.tail_v.view(np.uint16))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_encoder_and_decoder_bit_exact(torch_dev, case):
    torch, dev = torch_dev
    cid, bits, block, S, T, permute, law = case
    say("encode", cid)
    K, V = make_kv(law, S, T, block)
    refs = oracle_streams(K, V, bits, block, permute)
    c = gpu_cache(torch, dev, K, V, bits, block, permute)
    assert c.check() == 0
    assert_state_equal(c, refs)
    say("decompress", cid)
    for which, mode in (("K", 0), ("V", 0), ("K", 1), ("V", 1)):
        got = c.decompress(which, mode).cpu().numpy()
        assert c.check() == 0
        for s, ref in enumerate(refs):
            kh, vh, qk, qv = ostream.decode_stream(ref)
            if mode == 0:
                assert np.array_equal(got[s].astype(np.int64), qk if which == "K" else qv)
            else:
                exp = ostream.token_order(ref, kh if which == "K" else vh).astype(np.float32)
                assert np.array_equal(got[s].view(np.uint32), exp.view(np.uint32)), \
                    f"{which} x_hat not the correctly rounded fp32 of the exact value"


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("G", [1, 3, 4, 9])
def test_gemvs_within_tolerance(torch_dev, case, G):
    torch, dev = torch_dev
    cid, bits, block, S, T, permute, law = case
    K, V = make_kv(law, S, T, block)
    refs = oracle_streams(K, V, bits, block, permute)
    c = gpu_cache(torch, dev, K, V, bits, block, permute)
    rng = np.random.default_rng(G)
    q = rng.standard_normal((S, G, 128)).astype(np.float16)
    say("qk", cid, "G", G)
    scores = c.qk(torch.from_numpy(q).to(dev)).cpu().numpy()
    assert c.check() == 0
    ref_s = np.stack([attention.qk(q[s], ostream.decode_stream(refs[s])[0]) for s in range(S)])
    assert rel_l2(scores, ref_s) <= TOL and worst_row_rel(scores, ref_s) <= TOL, (rel_l2(scores, ref_s), worst_row_rel(scores, ref_s))
    # p: a softmax of the oracle scores, rounded to fp32 - the same input to both sides
    p = np.stack([attention.softmax(ref_s[s], 128) for s in range(S)]).astype(np.float32)
    say("pv", cid, "G", G)
    out = c.pv(torch.from_numpy(p).to(dev)).cpu().numpy()
    assert c.check() == 0
    ref_o = np.stack([attention.pv(p[s].astype(np.float64), ostream.decode_stream(refs[s])[1])
                      for s in range(S)])
    assert rel_l2(out, ref_o) <= TOL and worst_row_rel(out, ref_o) <= TOL, (rel_l2(out, ref_o), worst_row_rel(out, ref_o))


@pytest.mark.parametrize("rows,T,ld", [(5, 1000, 1000), (3, 65537, 65540), (2, 70001, 70003), (1, 4097, 4100)])
def test_softmax_helper(torch_dev, rows, T, ld):
    """Rows long enough for the unrolled loads, with a ragged tail, and a
    leading dimension that rules out vector loads."""
    torch, dev = torch_dev
    from decode_gemv_amd import softmax_rows
    rng = np.random.default_rng(T)
    x = (rng.standard_normal((rows, ld)) * 20).astype(np.float32)
    say("softmax", rows, T, ld)
    p = softmax_rows(torch.from_numpy(x).to(dev), T, 0.125).cpu().numpy()[:, :T]
    ref = np.stack([attention.softmax(r[:T].astype(np.float64) * 0.125 * np.sqrt(128), 128) for r in x])
    assert rel_l2(p, ref) <= TOL and worst_row_rel(p, ref) <= TOL
    assert np.all(np.abs(p.sum(1) - 1) < 1e-5)


def test_softmax_helper_in_place(torch_dev):
    """scores and p may be the same buffer (long rows included)."""
    torch, dev = torch_dev
    from decode_gemv_amd import softmax_rows
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((2, 131072)) * 20).astype(np.float32)
    say("softmax in place")
    xd = torch.from_numpy(x).to(dev)
    p = softmax_rows(xd, 131072, 0.125, out=xd).cpu().numpy()
    ref = np.stack([attention.softmax(r.astype(np.float64) * 0.125 * np.sqrt(128), 128) for r in x])
    assert rel_l2(p, ref) <= TOL and worst_row_rel(p, ref) <= TOL


@pytest.mark.parametrize("bits,block,law", [(4, 64, "mixed"), (2, 128, "struct"), (8, 64, "gauss"), (6, 128, "mixed")])
def test_stats_match_the_oracle_widths(torch_dev, bits, block, law):
    """Width histogram, payload words, runs and record bytes of the device
    cache equal those of the oracle's records."""
    torch, dev = torch_dev
    K, V = make_kv(law, 2, 3 * block + 17, block, seed=4)
    refs = oracle_streams(K, V, bits, block, True)
    c = gpu_cache(torch, dev, K, V, bits, block, True)
    say("stats", bits, block, law)
    st = c.stats()
    assert c.check() == 0
    cfg = oracle.Config(bits=bits, block=block)
    for which in "KV":
        hist = np.zeros(max(5, bits + 1), np.int64)
        words = runs = nbytes = 0
        for ref in refs:
            arena, off = ref.arena(which), ref.offsets(which)
            nbytes += int(off[-1])
            for j in range(len(off) - 1):
                n = ref.block_tokens(j)
                d = ounpack.decode_record(which, arena[off[j]:off[j + 1]], n, 128, block, 32, cfg.header_bytes)
                hist += np.bincount(d.w.ravel(), minlength=len(hist))[:len(hist)]
                words += int(d.w.sum())
                runs += d.w.size
        key = which.lower()
        assert st[f"{key}_width_hist"] == hist.tolist(), which
        assert st[f"{key}_words"] == words and st[f"{key}_runs"] == runs and st[f"{key}_bytes"] == nbytes


@pytest.mark.parametrize("bits,block,t0,steps,law,permute", [
    (3, 64, 60, 70, "gauss", 1), (4, 128, 0, 130, "gauss", 1), (2, 64, 64, 1, "gauss", 1),
    (4, 64, 30, 100, "struct", 2), (6, 64, 30, 70, "gauss", 1), (8, 128, 64, 65, "struct", 2)])
def test_append_matches_one_shot(torch_dev, bits, block, t0, steps, law, permute):
    torch, dev = torch_dev
    from decode_gemv_amd import PackedKVCache
    S = 2
    K, V = make_kv(law, S, t0 + steps + 5, block, seed=3)
    c = PackedKVCache(S, t0 + steps + 10, bits=bits, block=block, permute=permute, device=str(dev))
    Kd, Vd = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    say("append", bits, block, t0, steps, law, permute)
    if t0:
        c.compress(Kd[:, :t0].contiguous(), Vd[:, :t0].contiguous())
    for t in range(t0, t0 + steps):
        c.append(Kd[:, t:t + 1].contiguous(), Vd[:, t:t + 1].contiguous())
    # a multi-token append crossing a block boundary
    c.append(Kd[:, t0 + steps:].contiguous(), Vd[:, t0 + steps:].contiguous())
    assert c.check() == 0
    refs = oracle_streams(K, V, bits, block, permute)
    assert c.n_tokens == K.shape[1]
    assert_state_equal(c, refs)


def test_outputs_leave_the_leading_dimension_alone(torch_dev):
    torch, dev = torch_dev
    K, V = make_kv("gauss", 2, 100, 64)
    c = gpu_cache(torch, dev, K, V, 4, 64, True)
    q = torch.from_numpy(np.ones((2, 2, 128), np.float16)).to(dev)
    sc = torch.full((2, 2, 107), float("nan"), device=dev)
    say("ld canary")
    c.qk(q, sc)
    s = sc.cpu().numpy()
    assert np.all(np.isfinite(s[:, :, :100])) and np.all(np.isnan(s[:, :, 100:]))


def test_pv_is_bitwise_reproducible(torch_dev):
    torch, dev = torch_dev
    K, V = make_kv("gauss", 2, 1000, 64)
    c = gpu_cache(torch, dev, K, V, 4, 64, True)
    p = torch.rand(2, 1, 1000, device=dev)
    say("determinism")
    a = c.pv(p).clone()
    b = c.pv(p).clone()
    assert torch.equal(a, b)


def test_corrupt_header_is_reported_not_used(torch_dev):
    torch, dev = torch_dev
    K, V = make_kv("gauss", 1, 128, 64)
    c = gpu_cache(torch, dev, K, V, 4, 64, True)
    arena = c.arena("K")
    arena[0, 512 + 5] = 0x70          # width 7 > b: invalid
    q = torch.ones(1, 1, 128, dtype=torch.float16, device=dev)
    sc = torch.full((1, 1, 128), float("nan"), device=dev)
    say("corrupt header")
    c.qk(q, sc)
    from decode_gemv_amd import _lib
    assert c.check() == _lib.ECORRUPT
    s = sc.cpu().numpy()
    assert np.all(np.isnan(s[0, 0, :64])) and np.all(np.isfinite(s[0, 0, 64:]))
    assert c.check() == 0               # the latch was cleared


@pytest.mark.parametrize("bits,w,m", [(2, 2, 2), (2, 1, 3), (3, 3, 4), (3, 2, 9), (4, 4, 8), (4, 1, 15)],
                         ids=["b2-w2-m2", "b2-w1-m3", "b3-w3-m4", "b3-m-above-L", "b4-w4-m8", "b4-w1-m15"])
def test_corrupt_minimum_is_reported_not_used(torch_dev, bits, w, m):
    """One-byte header entries whose minimum leaves no room for the width
    (m + 2^(w-1) > 2^b - 1, or m > 2^b - 1): packkv_decompress rejects
    them, and so do the K GEMV, the V GEMV and fused attention - each
    latches ECORRUPT and takes nothing from that block."""
    torch, dev = torch_dev
    from decode_gemv_amd import _lib
    K, V = make_kv("gauss", 1, 128, 64)
    c = gpu_cache(torch, dev, K, V, bits, 64, True)
    rng = np.random.default_rng(bits)
    q = torch.from_numpy(rng.standard_normal((1, 1, 128)).astype(np.float16)).to(dev)
    p = torch.from_numpy(rng.random((1, 1, 128)).astype(np.float32)).to(dev)
    p0 = p.clone()
    p0[:, :, :64] = 0.0
    want_pv = c.pv(p0).clone()                   # block 0 weighted by zero
    assert c.check() == 0
    entry = (w << 4) | m
    say("corrupt minimum", bits, w, m)
    c.arena("K")[0, 512 + 5] = entry             # K header entry 5 of block 0
    sc = torch.full((1, 1, 128), float("nan"), device=dev)
    c.qk(q, sc)
    assert c.check() == _lib.ECORRUPT
    s = sc.cpu().numpy()
    assert np.all(np.isnan(s[0, 0, :64])) and np.all(np.isfinite(s[0, 0, 64:]))
    out = c.attention(q)
    assert c.check() == _lib.ECORRUPT
    assert torch.all(torch.isfinite(out))
    for which, mode in (("K", 0), ("K", 1)):
        c.decompress(which, mode)
        assert c.check() == _lib.ECORRUPT
    c.arena("V")[0, 256 + 5] = entry             # V header entry 5 of block 0
    got = c.pv(p)
    assert c.check() == _lib.ECORRUPT
    assert torch.equal(got, want_pv)
    assert c.check() == 0


@pytest.mark.parametrize("entry", [(7, None), (6, 40)], ids=["width-above-b", "minimum-leaves-no-room"])
def test_corrupt_wide_header_is_reported_not_used(torch_dev, entry):
    """b = 6 (two-byte entries): a width above b, or a minimum that leaves no
    room for its width (m + 2^(w-1) > 2^b - 1), latches ECORRUPT; the K
    GEMV writes nothing for that block and fused attention reports it."""
    torch, dev = torch_dev
    from decode_gemv_amd import _lib
    K, V = make_kv("gauss", 1, 128, 64)
    c = gpu_cache(torch, dev, K, V, 6, 64, True)
    w, m = entry
    arena = c.arena("K")
    arena[0, 512 + 2 * 5 + 1] = w                 # entry 5 of block 0: high byte w
    if m is not None:
        arena[0, 512 + 2 * 5] = m                 # low byte m
    q = torch.ones(1, 1, 128, dtype=torch.float16, device=dev)
    sc = torch.full((1, 1, 128), float("nan"), device=dev)
    say("corrupt wide header", w, m)
    c.qk(q, sc)
    assert c.check() == _lib.ECORRUPT
    s = sc.cpu().numpy()
    assert np.all(np.isnan(s[0, 0, :64])) and np.all(np.isfinite(s[0, 0, 64:]))
    c.attention(q)
    assert c.check() == _lib.ECORRUPT
    assert c.check() == 0


@pytest.mark.parametrize("payload", ["all-three", "random"])
def test_two_bit_slot_values_up_to_four(torch_dev, payload):
    """At 2 bits the K side turns container nibbles into floats as e2m1
    (fp4) codes, which are exact multiples of one step only up to 4.  A
    header entry that passes every check (w = 2, m = 1) lets an altered
    payload hold m + u = 4, the largest value such a record can carry; the K
    GEMV and fused attention must read those bytes as the oracle's record
    decoder does (records here are altered bytes, not encoder output)."""
    torch, dev = torch_dev
    D, B = 128, 64
    K, V = make_kv("gauss", 1, B, B)
    c = gpu_cache(torch, dev, K, V, 2, B, False)
    hdr = 4 * D                                   # K header after scale and zero
    pay = (hdr + 2 * D + 15) // 16 * 16           # two run rows of one-byte entries
    arena = c.arena("K")
    w_row0 = arena[0, hdr:hdr + D].cpu().numpy() >> 4
    full = np.nonzero(np.cumprod(w_row0 == 2))[0]  # channels after only full-width runs of row 0
    assert full.size >= 4, "gauss data at 2 bits: the first runs are at full width"
    ch = int(full[3])                              # run (0, ch) starts at word 2 * ch
    arena[0, hdr + ch] = (2 << 4) | 1
    rng = np.random.default_rng(7)
    words = np.full(8, 0xFF, np.uint8) if payload == "all-three" else rng.integers(0, 256, 8).astype(np.uint8)
    arena[0, pay + 8 * ch:pay + 8 * ch + 8] = torch.from_numpy(words).to(dev)
    koff = c.offsets("K").cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    voff = c.offsets("V").cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    kbuf = arena[0, koff[0, 0]:koff[0, 1]].cpu().numpy().tobytes()
    vbuf = c.arena("V")[0, voff[0, 0]:voff[0, 1]].cpu().numpy().tobytes()
    dk = ounpack.decode_record("K", kbuf, B, D, B, 32)
    dv = ounpack.decode_record("V", vbuf, B, D, B, 32)
    assert dk.q[:, ch].max() == 4 if payload == "all-three" else dk.q[:, ch].max() <= 4
    k_hat = dk.zero[None, :] + dk.scale[None, :] * dk.q          # slot order, fp64
    v_hat = dv.zero[:, None] + dv.scale[:, None] * dv.q
    qn = rng.standard_normal((1, 1, D)).astype(np.float16)
    q = torch.from_numpy(qn).to(dev)
    say("two-bit slot values up to four", payload, "channel", ch)
    sc = c.qk(q)
    assert c.check() == 0
    want = attention.qk(qn[0].astype(np.float64), k_hat)
    got = sc[0, :, :B].cpu().numpy()
    assert rel_l2(got, want) <= TOL and worst_row_rel(got, want) <= TOL
    out = c.attention(q)
    assert c.check() == 0
    want_o = attention.pv(attention.softmax(want, D), v_hat)
    got_o = out[0].cpu().numpy()
    assert rel_l2(got_o, want_o) <= TOL and worst_row_rel(got_o, want_o) <= TOL


@pytest.mark.parametrize("bad", ["negative", "nan", "inf"])
@pytest.mark.parametrize("bits,G", [(4, 1), (3, 4), (8, 1)])
def test_pv_rejects_weights_outside_its_domain(torch_dev, bad, bits, G):
    """The V GEMV takes p >= 0 and finite (softmax weights, which its 20-bit
    fixed point assumes): a block holding any other weight latches EINVAL
    and contributes nothing, so the output is that of p with the block's
    weights zeroed."""
    torch, dev = torch_dev
    from decode_gemv_amd import _lib
    K, V = make_kv("gauss", 2, 200, 64)
    c = gpu_cache(torch, dev, K, V, bits, 64, True)
    rng = np.random.default_rng(3)
    p = rng.random((2, G, 200)).astype(np.float32)
    p0 = p.copy()
    p0[1, :, 64:128] = 0.0                       # stream 1, block 1 zeroed
    p[1, G - 1, 70] = {"negative": -0.25, "nan": np.nan, "inf": np.inf}[bad]
    say("pv domain", bad, bits, G)
    want = c.pv(torch.from_numpy(p0).to(dev)).clone()
    assert c.check() == 0
    got = c.pv(torch.from_numpy(p).to(dev))
    assert c.check() == _lib.EINVAL
    assert torch.equal(got, want)
    assert c.check() == 0


@pytest.mark.parametrize("bad", [0x7C00, 0xFC00, 0x7E00])
def test_non_finite_input_latches_einval(torch_dev, bad):
    """Infinite or NaN fp16 inputs are outside the method: compress and
    append latch EINVAL; the other blocks' records are still exact."""
    torch, dev = torch_dev
    from decode_gemv_amd import _lib, PackedKVCache
    K, V = make_kv("gauss", 2, 150, 64)
    refs = oracle_streams(K[:, :128], V[:, :128], 4, 64)
    Kb, Vb = K.copy(), V.copy()
    Kb.view(np.uint16)[0, 140, 3] = bad          # in the partial last block
    say("non-finite", hex(bad))
    c = PackedKVCache(2, 300, bits=4, block=64, device=str(dev))
    c.compress(torch.from_numpy(Kb).to(dev), torch.from_numpy(Vb).to(dev))
    assert c.check() == _lib.EINVAL
    ko = c.offsets("K").cpu().numpy().astype(np.int64)
    for s, ref in enumerate(refs):                # the two closed blocks are untouched
        ro = ref.offsets("K")
        assert np.array_equal(ko[s, :3], ro)
        assert c.arena("K")[s, :int(ro[-1])].cpu().numpy().tobytes() == ref.arena("K")
    vnew = np.zeros((2, 1, 128), np.float16)
    vnew.view(np.uint16)[1, 0, 7] = bad
    c.append(torch.zeros(2, 1, 128, dtype=torch.float16, device=dev), torch.from_numpy(vnew).to(dev))
    assert c.check() == _lib.EINVAL
    assert c.check() == 0


@pytest.mark.parametrize("law", ["uniform", "one-hot", "peaked", "sparse-blocks", "wide-range"])
def test_pv_weight_laws(torch_dev, law):
    """V GEMV precision across weight distributions (fp64 oracle, rel-L2 <= 1e-4)."""
    torch, dev = torch_dev
    S, T = 2, 1000
    K, V = make_kv("gauss", S, T, 64)
    refs = oracle_streams(K, V, 4, 64)
    c = gpu_cache(torch, dev, K, V, 4, 64, True)
    rng = np.random.default_rng(11)
    if law == "uniform":
        p = np.full((S, 1, T), 1.0 / T)
    elif law == "one-hot":
        p = np.zeros((S, 1, T))
        p[:, 0, 517] = 1.0
    elif law == "peaked":
        z = rng.standard_normal((S, 1, T)) * 6
        p = np.exp(z - z.max(-1, keepdims=True))
        p /= p.sum(-1, keepdims=True)
    elif law == "sparse-blocks":        # whole blocks of zero weight
        p = rng.random((S, 1, T))
        p[:, :, 64:640] = 0.0
        p /= p.sum(-1, keepdims=True)
    else:                               # weights spanning ~30 orders of magnitude
        p = np.exp(rng.uniform(-70, 0, (S, 1, T)))
    p = p.astype(np.float32)
    say("pv law", law)
    out = c.pv(torch.from_numpy(p).to(dev)).cpu().numpy()
    assert c.check() == 0
    ref = np.stack([attention.pv(p[s].astype(np.float64), ostream.decode_stream(refs[s])[1]) for s in range(S)])
    assert rel_l2(out, ref) <= TOL and worst_row_rel(out, ref) <= TOL, (rel_l2(out, ref), worst_row_rel(out, ref))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("G", [1, 3, 4, 9])
def test_fused_attention_within_tolerance(torch_dev, case, G):
    """Fused K GEMV + softmax + V GEMV against the fp64 oracle's three steps."""
    torch, dev = torch_dev
    cid, bits, block, S, T, permute, law = case
    K, V = make_kv(law, S, T, block)
    refs = oracle_streams(K, V, bits, block, permute)
    c = gpu_cache(torch, dev, K, V, bits, block, permute)
    rng = np.random.default_rng(100 + G)
    q = (rng.standard_normal((S, G, 128)) * 2).astype(np.float16)
    say("attention", cid, "G", G)
    out = c.attention(torch.from_numpy(q).to(dev)).cpu().numpy()
    assert c.check() == 0
    ref = []
    for s in range(S):
        kh, vh, _, _ = ostream.decode_stream(refs[s])
        ref.append(attention.pv(attention.softmax(attention.qk(q[s], kh), 128), vh))
    ref = np.stack(ref)
    assert rel_l2(out, ref) <= TOL and worst_row_rel(out, ref) <= TOL, (rel_l2(out, ref), worst_row_rel(out, ref))


def test_fused_attention_is_bitwise_reproducible_and_reuses_its_workspace(torch_dev):
    torch, dev = torch_dev
    K, V = make_kv("gauss", 2, 1000, 64)
    c = gpu_cache(torch, dev, K, V, 4, 64, True)
    q = torch.from_numpy(np.random.default_rng(5).standard_normal((2, 4, 128)).astype(np.float16)).to(dev)
    say("attention determinism")
    a = c.attention(q).clone()
    b = c.attention(q).clone()
    assert torch.equal(a, b)
    # the per-stream counters are back at zero after every call
    ws = c.attention_workspace(4)
    tail = ws[-256:].view(torch.int32)[:2].cpu().numpy()
    assert np.all(tail == 0)


@pytest.mark.parametrize("bits,block,G,L", [(4, 64, 1, 3), (3, 128, 4, 2), (2, 64, 3, 35)])
def test_multi_cache_attention_matches_single_calls(torch_dev, bits, block, G, L):
    """One launch over L caches (35 takes two launches of at most 32) gives
    each cache's single-call result bit for bit, twice on one workspace; the
    first cache is also checked against the oracle."""
    torch, dev = torch_dev
    from decode_gemv_amd import attention_multi, attention_multi_workspace
    S, T = 2, 150
    caches, kvs = [], []
    for layer in range(L):
        K, V = make_kv("gauss", S, T, block, seed=100 + layer)
        kvs.append((K, V))
        caches.append(gpu_cache(torch, dev, K, V, bits, block, 1))
    rng = np.random.default_rng(L)
    q = rng.standard_normal((L, S, G, 128)).astype(np.float16)
    qd = torch.from_numpy(q).to(dev)
    say("attention multi", bits, block, G, L)
    ws = attention_multi_workspace(caches, G)
    single = torch.stack([c.attention(qd[i].contiguous()) for i, c in enumerate(caches)])
    for rep in range(2):
        out = attention_multi(caches, qd, workspace=ws)
        for c in caches:
            assert c.check() == 0
        assert torch.equal(out, single), f"repeat {rep}"
    refs = oracle_streams(*kvs[0], bits, block, 1)
    for s in range(S):
        kh, vh, _, _ = ostream.decode_stream(refs[s])
        ref = attention.pv(attention.softmax(attention.qk(q[0, s], kh), 128), vh)
        got = out[0, s].cpu().numpy()
        assert rel_l2(got, ref) <= TOL and worst_row_rel(got, ref) <= TOL


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 10 * 2**20 + 48, 70 * 2**20])
def test_stream_read_folds_every_word(torch_dev, nbytes):
    """The read-ceiling probe reads every word once: its XOR fold equals numpy's."""
    torch, dev = torch_dev
    from decode_gemv_amd import stream_read
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(dev)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    say("stream read", nbytes)
    stream_read(buf, sink)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host))
