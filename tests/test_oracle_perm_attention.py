"""Pins of the oracle's permutation, attention products, CR and append."""

import itertools

import numpy as np
import pytest

import kvsynth
from oracle import Config, perm, stream, attention, cr, record


def brute_groups(qk, qv, R):
    """Greedy grouping by exhaustive choice: at each step try every R-subset of
    the remaining tokens that contains the seed and keep the one whose sorted
    (distance, index) keys are lexicographically smallest."""
    feats = np.concatenate([qk, qv], axis=1)
    remaining = list(range(len(qk)))
    out = []
    while remaining:
        seed = remaining[0]
        key = {t: (int(np.abs(feats[t] - feats[seed]).sum()), t) for t in remaining}
        k = min(R, len(remaining))
        best = min((sorted(key[t] for t in sub) for sub in itertools.combinations(remaining, k)
                    if seed in sub))
        out.extend(t for _, t in best)
        remaining = [t for t in remaining if t not in {t for _, t in best}]
    return out


def test_greedy_order_matches_exhaustive_search():
    rng = np.random.default_rng(0)
    for trial in range(30):
        n = int(rng.integers(1, 9))
        qk = rng.integers(0, 4, (n, 3))
        qv = rng.integers(0, 4, (n, 2))
        assert perm.greedy_order(qk, qv, 2) == brute_groups(qk, qv, 2)
        assert perm.greedy_order(qk, qv, 3) == brute_groups(qk, qv, 3)


@pytest.mark.parametrize("n", [1, 17, 64])
def test_permutation_is_a_bijection_with_seed_first(n):
    rng = np.random.default_rng(n)
    qk = rng.integers(0, 16, (n, 128))
    qv = rng.integers(0, 16, (n, 128))
    order = perm.greedy_order(qk, qv, 32)
    assert sorted(order) == list(range(n))
    taken = set()
    for g in range(0, n, 32):
        assert order[g] == min(set(range(n)) - taken)
        taken |= set(order[g:g + 32])


def test_identity_fallback_and_switch():
    rng = np.random.default_rng(1)
    qk = rng.integers(0, 16, (64, 128))
    qv = rng.integers(0, 16, (64, 128))
    p = perm.block_permutation(qk, qv, 32, True)
    ident = list(range(64))
    assert perm.payload_words(qk, qv, p, 32) <= perm.payload_words(qk, qv, ident, 32)
    if list(p) != ident:
        assert perm.payload_words(qk, qv, p, 32) < perm.payload_words(qk, qv, ident, 32)
    assert list(perm.block_permutation(qk, qv, 32, False)) == ident


def test_grouping_recovers_clusters():
    """Shuffled clustered tokens: the grouping puts each cluster in one run."""
    k, v = kvsynth.structured_kv(64, 128, 64, 32, seed=4, noise=0.0)
    code = stream.encode_block(k, v, Config(bits=4, block=64))
    rows = k[code.perm].astype(np.float64)
    for g in (0, 32):
        assert np.all(rows[g:g + 32] == rows[g])
    assert record.run_widths(code.qk_slots, 32)[0].max() == 0


def test_sort_key_order_against_exhaustive_search():
    """Among all orders of a tiny block, exactly one has strictly increasing
    (total, index) pairs; the sort-key order must be that one."""
    rng = np.random.default_rng(11)
    for trial in range(40):
        n = int(rng.integers(1, 7))
        qk = rng.integers(0, 3, (n, 3))          # small values: many equal totals
        qv = rng.integers(0, 3, (n, 2))
        tot = [int(qk[t].sum() + qv[t].sum()) for t in range(n)]
        inc = [list(o) for o in itertools.permutations(range(n))
               if all((tot[o[i]], o[i]) < (tot[o[i + 1]], o[i + 1]) for i in range(n - 1))]
        assert len(inc) == 1
        assert perm.sort_key_order(qk, qv) == inc[0]


def test_sort_key_groups_clusters_with_distinct_totals():
    """Shuffled clusters whose quantised totals differ: sorting by the total
    puts each cluster in one run, every run has width 0, and the order is kept."""
    k, v = kvsynth.structured_kv(64, 128, 64, 32, seed=4, noise=0.0)
    cfg = Config(bits=4, block=64, permute=2)
    code = stream.encode_block(k, v, cfg)
    tot = code.qk_slots.sum(axis=1).astype(np.int64) + code.qv_slots.sum(axis=1)
    assert tot[0] != tot[32], "the two clusters must have different totals for this pin"
    rows = k[code.perm].astype(np.float64)
    for g in (0, 32):
        assert np.all(rows[g:g + 32] == rows[g])
    assert record.run_widths(code.qk_slots, 32)[0].max() == 0
    assert record.run_widths(code.qv_slots, 32)[0].max() == 0
    assert list(code.perm) != list(range(64))


def test_sort_key_falls_back_to_identity():
    """Identical tokens: no order is strictly smaller, so the identity stays;
    iid blocks: whatever is chosen is never larger than the identity."""
    qk = np.full((64, 128), 5)
    qv = np.full((64, 128), 9)
    assert list(perm.block_permutation(qk, qv, 32, 2)) == list(range(64))
    rng = np.random.default_rng(5)
    qk = rng.integers(0, 16, (64, 128))
    qv = rng.integers(0, 16, (64, 128))
    p = perm.block_permutation(qk, qv, 32, 2)
    assert perm.payload_words(qk, qv, p, 32) <= perm.payload_words(qk, qv, list(range(64)), 32)


def test_attention_is_unchanged_by_the_permutation():
    k, v = kvsynth.structured_kv(300, 128, 64, 32, seed=7)
    q = np.random.default_rng(2).standard_normal((2, 128)).astype(np.float16)
    outs = []
    for p in (1, 2, 0):
        c = stream.compress(k, v, Config(bits=4, block=64, permute=p))
        kh, vh, _, _ = stream.decode_stream(c)
        s = attention.qk(q, kh)
        outs.append(attention.pv(attention.softmax(s, 128), vh))
        # the dequantised rows are the same multiset: equal after un-permuting
        kt, vt = stream.token_order(c, kh), stream.token_order(c, vh)
        if p == 1:
            k1, v1 = kt, vt
        else:
            assert np.array_equal(kt, k1) and np.array_equal(vt, v1)
    assert attention.rel_l2(outs[0], outs[1]) < 1e-12
    assert attention.rel_l2(outs[0], outs[2]) < 1e-12


def test_gemv_definitions_against_loops():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((3, 8))
    K = rng.standard_normal((5, 8))
    V = rng.standard_normal((5, 8))
    s = attention.qk(q, K)
    for g in range(3):
        for t in range(5):
            assert abs(s[g, t] - sum(q[g, c] * K[t, c] for c in range(8))) < 1e-12
    p = attention.softmax(s, 8)
    o = attention.pv(p, V)
    for g in range(3):
        for c in range(8):
            assert abs(o[g, c] - sum(p[g, t] * V[t, c] for t in range(5))) < 1e-12
    onehot = np.zeros((1, 5))
    onehot[0, 3] = 1
    assert np.array_equal(attention.pv(onehot, V)[0], V[3])
    assert np.allclose(attention.qk(2 * q, K), 2 * s)


def test_softmax_properties():
    s = np.random.default_rng(4).standard_normal((4, 1000)) * 30
    p = attention.softmax(s, 128)
    assert np.all(np.abs(p.sum(-1) - 1) < 1e-14) and np.all(p >= 0)
    assert np.allclose(attention.softmax(s + 123.0, 128), p, rtol=1e-12, atol=0)
    one = attention.softmax(np.array([[0.0, 0.0]]), 128)
    assert np.all(one == 0.5)


@pytest.mark.parametrize("D,ratio", [(128, 2.0), (64, 3.0), (256, 5.0)])
def test_softmax_temperature_is_one_over_sqrt_head_dim(D, ratio):
    """Closed form: scores (0, sqrt(D) ln r) give weights 1/(1+r) and r/(1+r)
    exactly when the temperature is 1/sqrt(D); 1/D, no scaling or a fixed
    1/sqrt(128) would give other weights."""
    s = np.array([[0.0, np.sqrt(D) * np.log(ratio)]])
    p = attention.softmax(s, D)
    assert abs(p[0, 0] - 1.0 / (1.0 + ratio)) < 1e-14
    assert abs(p[0, 1] - ratio / (1.0 + ratio)) < 1e-14


@pytest.mark.parametrize("bits,block", [(4, 64), (2, 64), (3, 64), (4, 128), (5, 128), (8, 64)])
def test_cr_matches_closed_form_when_every_run_is_full_width(bits, block):
    """Construct blocks whose every run spans 0..L in every channel."""
    L = (1 << bits) - 1
    T = 4 * block
    rng = np.random.default_rng(bits)
    qk = rng.integers(0, L + 1, (T, 128))
    qk[::32] = 0
    qk[1::32] = L
    qv = rng.integers(0, L + 1, (T, 128))
    qv[:, 126], qv[:, 127] = 0, L          # every token spans 0..L
    qv[0::32], qv[1::32], qv[2::32], qv[3::32] = 0, L, 0, L
    qv[0::32, 5] = L                       # rows 0-3 of every run: each token
    qv[1::32, 5] = 0                       # still spans 0..L, and every
    qv[2::32, 6] = L                       # channel sees both 0 and L
    qv[3::32, 6] = 0
    c = stream.compress(qk.astype(np.float16), qv.astype(np.float16),
                        Config(bits=bits, block=block, permute=False))
    for which in "KV":
        r = cr.ratios(c, which)
        cf = cr.closed_form_full_width(which, bits, block, 32, 128)
        assert abs(r["cr_ideal"] - cf) < 1e-12
        assert abs(r["cr_phys"] - cf) < 1e-12     # all sections 16-byte aligned here
    assert abs(cr.closed_form_full_width("K", 4, 64, 32, 128) - 1024 / 304) < 1e-15
    # b = 8: 8 payload bits, 16/32 header bits (two-byte entries), 32/64 parameter bits
    assert abs(cr.closed_form_full_width("K", 8, 64, 32, 128) - 16 / 9) < 1e-15


@pytest.mark.parametrize("bits,block,k_rec,v_rec", [(4, 64, 4864, 4608), (3, 64, 3840, 3584),
                                                    (2, 64, 2816, 2560), (4, 128, 9216, 9216)])
def test_full_and_plain_quant_ratios_by_record_geometry(bits, block, k_rec, v_rec):
    """CR_full adds one permutation byte per token to the stored records, and
    plain b-bit quantisation stores T*D*b bits plus the same fp16 parameters.
    Blocks whose every run is at full width have records of the sizes the
    format's geometry gives (params + one header byte per run and channel +
    b words per run and channel): 4864 / 4608 bytes at b = 4, B = 64, etc.
    Both ratios are checked against those byte counts and against the
    printed plain-quantisation ratios 16 / (b + 32/B) (K) and 16 / (b + 32/D)
    (V): 3.556 / 3.765 at b = 4, B = 64; 6.400 / 7.111 at b = 2."""
    L = (1 << bits) - 1
    nb = 3
    T = nb * block
    t = np.arange(T)[:, None]
    c = np.arange(128)[None, :]
    # checkerboard of the two extremes: every K (block, channel) and every V
    # token spans 0..L, and every run holds both in every channel
    grid = np.where((t + c) % 2 == 0, 0.0, float(L)).astype(np.float16)
    cache = stream.compress(grid, grid, Config(bits=bits, block=block, permute=False))
    raw = 2 * T * 128
    for which, rec in (("K", k_rec), ("V", v_rec)):
        r = cr.ratios(cache, which)
        assert r["phys_bytes"] == nb * rec
        assert abs(r["cr_full"] - raw / (nb * rec + T)) < 1e-12
        params = 32 * 128 * nb if which == "K" else 32 * T
        assert abs(r["cr_plain_quant"] - 16 * T * 128 / (T * 128 * bits + params)) < 1e-12
    printed = {(4, 64): (3.556, 3.765), (3, 64): (4.571, 4.923), (2, 64): (6.400, 7.111), (4, 128): (3.765, 3.765)}
    pk, pv = printed[(bits, block)]
    assert abs(cr.ratios(cache, "K")["cr_plain_quant"] - pk) < 5e-4
    assert abs(cr.ratios(cache, "V")["cr_plain_quant"] - pv) < 5e-4


def test_plain_quant_ratio_does_not_depend_on_the_data():
    """Plain quantisation has no per-run width: its ratio depends only on T,
    D, b and the parameter count, whatever the values (ragged last block)."""
    w = kvsynth.WORKLOADS["llama7b-32k"]
    k, v = kvsynth.stream_kv(w, 5, tokens=200)
    c1 = stream.compress(k, v, Config(bits=4, block=64))
    ks, vs = kvsynth.structured_kv(200, 128, 64, 32, seed=9)
    c2 = stream.compress(ks, vs, Config(bits=4, block=64))
    for which in "KV":
        a, b = cr.ratios(c1, which)["cr_plain_quant"], cr.ratios(c2, which)["cr_plain_quant"]
        assert a == b
    # 4 blocks (the last holds 8 tokens): K params 4 * 128 * 32 bits, V 200 * 32
    assert abs(cr.ratios(c1, "K")["cr_plain_quant"] - 16 * 200 * 128 / (200 * 128 * 4 + 4 * 128 * 32)) < 1e-12
    assert abs(cr.ratios(c1, "V")["cr_plain_quant"] - 16 * 200 * 128 / (200 * 128 * 4 + 200 * 32)) < 1e-12


def test_cr_counts_the_bits_the_packer_writes():
    k, v = kvsynth.structured_kv(250, 128, 64, 32, seed=3)
    c = stream.compress(k, v, Config(bits=3, block=64))
    for which in "KV":
        r = cr.ratios(c, which)
        total = 0
        for j, b in enumerate(c.blocks):
            rec = b.k_record if which == "K" else b.v_record
            qs = b.qk_slots if which == "K" else b.qv_slots
            w, m = record.run_widths(qs, 32)
            payload = record.pack_payload(qs, w, m, 32, 4)
            par = 32 * 128 if which == "K" else 32 * len(b.perm)
            total += 8 * len(payload) + 8 * w.size + par
        assert r["ideal_bits"] == total


@pytest.mark.parametrize("t0,extra", [(0, 70), (50, 30), (64, 65), (130, 1)])
def test_append_equals_one_shot(t0, extra):
    cfg = Config(bits=3, block=64)
    w = kvsynth.WORKLOADS["append-64k"]
    k, v = kvsynth.stream_kv(w, 3, tokens=t0 + extra)
    if t0:
        c = stream.compress(k[:t0], v[:t0], cfg)
    else:
        c = stream.StreamCache(cfg, [], 0, k[:0], v[:0])
    c = stream.append(c, k[t0:], v[t0:])
    ref = stream.compress(k, v, cfg)
    assert c.n_tokens == ref.n_tokens
    for which in "KV":
        assert c.arena(which) == ref.arena(which)
        assert np.array_equal(c.offsets(which), ref.offsets(which))
    assert np.array_equal(c.perm_table(), ref.perm_table())
    assert np.array_equal(c.tail_k, ref.tail_k) and np.array_equal(c.tail_v, ref.tail_v)
