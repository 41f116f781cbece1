"""Full-size GPU parity: every measured workload at its real shape, in the
launch configuration bench.py times.

The oracle cannot follow a whole 256-stream cache in seconds, so each test
checks (1) one sampled stream completely - every record byte, the offsets,
the permutation and the tail, and its K-GEMV scores, V-GEMV output and fused
attention within rel-L2 1e-4 of the fp64 oracle (tensor and worst row) - and
(2) one sampled block of every stream, re-encoded by the oracle on its own (a
closed block depends only on its own tokens): its K and V record bytes, its
scores, and the stream's V-GEMV output for weights that are zero outside that
block (so the output is the block's product alone).  Every row also has to
satisfy what holds at any size (finite outputs, softmax rows summing to 1,
fused attention equal to the separate K GEMV -> softmax -> V GEMV).
"""

import concurrent.futures as cf

import numpy as np
import pytest

import kvsynth
import oracle
from gpu_common import say, rel_l2, worst_row_rel
from oracle import stream as ostream, attention

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch, torch.device("cuda:0")


def host_streams(w, tokens):
    """Seeded fp16 K, V of every stream, [S][tokens][D] each (host)."""
    S, D = w.streams, w.head_dim
    K = np.empty((S, tokens, D), np.float16)
    V = np.empty_like(K)
    with cf.ThreadPoolExecutor(16) as ex:
        for s, (k, v) in enumerate(ex.map(lambda i: kvsynth.stream_kv(w, i, tokens=tokens), range(S))):
            K[s], V[s] = k, v
    return K, V


def stream_state_equal(c, ref, s):
    """Bit-exact records, offsets, permutation and tail staging of stream s."""
    T, B = c.n_tokens, c.block
    nb = -(-T // B)
    for which in "KV":
        offs = c.offsets(which)[s, :nb + 1].cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        ro = ref.offsets(which)
        assert np.array_equal(offs, ro), f"{which} offsets of stream {s} differ"
        got = c.arena(which)[s, :int(ro[-1])].cpu().numpy().tobytes()
        assert got == ref.arena(which), f"{which} records of stream {s} differ"
    assert np.array_equal(c.perm_table()[s, :nb].cpu().numpy(), ref.perm_table())
    nt = T % B
    tk = c.tail_k.view(c.n_streams, B, 128)[s, :nt].cpu().numpy()
    assert np.array_equal(tk.view(np.uint16), ref.tail_k.view(np.uint16))


def check_offsets_all_streams(c, cfg):
    """Every stream: offsets start at 0, increase by a legal record size."""
    T, B = c.n_tokens, c.block
    nb = -(-T // B)
    nr_full = B // 32
    for which in "KV":
        offs = c.offsets(which)[:, :nb + 1].cpu().numpy().astype(np.int64) & 0xFFFFFFFF
        assert np.all(offs[:, 0] == 0)
        sizes = np.diff(offs, axis=1)
        params = 4 * 128 if which == "K" else 4 * B
        hdr = cfg.header_bytes * nr_full * 128             # one entry per (run, channel)
        lo = params + hdr                                  # header only (narrowest runs)
        hi = params + hdr + 16 + nr_full * 128 * 4 * cfg.bits
        assert np.all(sizes[:, :-1] >= lo) and np.all(sizes <= hi), f"{which} record sizes out of range"


def sampled_blocks(torch, dev, c, w, block_kv, cfg, scores, q, rng, closed=None):
    """One random closed block per stream, re-encoded by the oracle alone:
    its K and V record bytes, its scores, and the V GEMV of every stream
    against the oracle, with weights that are zero outside the stream's
    sampled block (the output is then that block's product alone).
    block_kv(s, j) gives the fp16 K, V of block j of stream s; closed: the
    blocks to sample from (default: every closed block)."""
    B = w.block
    S, G, T = w.streams, w.group, c.n_tokens
    closed = closed or range(T // B)
    ka = c.arena("K").cpu().numpy()
    va = c.arena("V").cpu().numpy()
    ko = c.offsets("K").cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    vo = c.offsets("V").cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    pick = [int(closed[int(rng.integers(len(closed)))]) for _ in range(S)]
    pw = rng.random((S, G, B)).astype(np.float32)
    p = np.zeros((S, G, T), np.float32)
    for s, j in enumerate(pick):
        p[s, :, j * B:(j + 1) * B] = pw[s]
    out = c.pv(torch.from_numpy(p).to(dev)).cpu().numpy()
    assert c.check() == 0
    worst_sc = worst_out = 0.0
    for s, j in enumerate(pick):
        kb, vb = block_kv(s, j)
        code = ostream.encode_block(kb, vb, cfg)
        assert ka[s, ko[s, j]:ko[s, j + 1]].tobytes() == code.k_record, f"K record ({s}, {j})"
        assert va[s, vo[s, j]:vo[s, j + 1]].tobytes() == code.v_record, f"V record ({s}, {j})"
        one = ostream.StreamCache(cfg, [code], B, kb[:0], vb[:0])
        kh, vh, _, _ = ostream.decode_stream(one)
        ref = attention.qk(q[s], kh)
        got = scores[s, :, j * B:(j + 1) * B]
        worst_sc = max(worst_sc, rel_l2(got, ref), worst_row_rel(got, ref))
        ref_o = attention.pv(pw[s].astype(np.float64), vh)
        worst_out = max(worst_out, rel_l2(out[s], ref_o), worst_row_rel(out[s], ref_o))
    assert worst_sc <= TOL, worst_sc
    assert worst_out <= TOL, worst_out


FULLSIZE = [("single-head-4k", 0), ("llama7b-32k", 0), ("gqa-128k", 0), ("2bit-16k", 0), ("8bit-16k", 0),
            # clustered tokens in the greedy order, with the K payload by
            # channel and width-sorted (payload order 1)
            ("struct-32k", 0), ("struct-32k", 1)]


@pytest.mark.parametrize("name,order", FULLSIZE, ids=[f"{n}-order{o}" for n, o in FULLSIZE])
def test_fullsize_workload(torch_dev, name, order):
    torch, dev = torch_dev
    from decode_gemv_amd import PackedKVCache, softmax_rows
    w = kvsynth.WORKLOADS[name]
    S, G, T, D = w.streams, w.group, w.tokens, w.head_dim
    cfg = oracle.Config(bits=w.bits, block=w.block, payload_order=order)
    say("fullsize", name, "order", order, "S", S, "T", T, "G", G)
    K, V = host_streams(w, T)
    c = PackedKVCache(S, T + 8, bits=w.bits, block=w.block, device=str(dev), payload_order=order)
    c.compress(torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev))
    assert c.check() == 0
    check_offsets_all_streams(c, cfg)
    q = np.stack([kvsynth.stream_q(w, s) for s in range(S)])
    say("fullsize gemvs", name)
    scores_d = c.qk(torch.from_numpy(q).to(dev))
    p_d = softmax_rows(scores_d, T, 1.0 / np.sqrt(D))
    out = c.pv(p_d).cpu().numpy()
    assert c.check() == 0
    scores = scores_d.cpu().numpy()
    p = p_d.cpu().numpy()
    assert np.all(np.isfinite(scores)) and np.all(np.isfinite(out))
    assert np.all(np.abs(p.sum(-1) - 1.0) < 1e-4)
    say("fullsize sampled blocks", name)
    sampled_blocks(torch, dev, c, w, lambda s_, j: (K[s_, j * w.block:(j + 1) * w.block],
                                                    V[s_, j * w.block:(j + 1) * w.block]),
                   cfg, scores, q, np.random.default_rng(7))
    s = S - 1                                   # the stream at the far end of the arenas
    say("fullsize oracle stream", name, s)
    ref = ostream.compress(K[s], V[s], cfg)
    stream_state_equal(c, ref, s)
    kh, vh, _, _ = ostream.decode_stream(ref)
    ref_sc = attention.qk(q[s], kh)
    assert rel_l2(scores[s], ref_sc) <= TOL and worst_row_rel(scores[s], ref_sc) <= TOL, \
        (rel_l2(scores[s], ref_sc), worst_row_rel(scores[s], ref_sc))
    ref_out = attention.pv(p[s].astype(np.float64), vh)
    assert rel_l2(out[s], ref_out) <= TOL and worst_row_rel(out[s], ref_out) <= TOL, \
        (rel_l2(out[s], ref_out), worst_row_rel(out[s], ref_out))
    say("fullsize fused attention", name)
    fused = c.attention(torch.from_numpy(q).to(dev)).cpu().numpy()
    assert c.check() == 0
    assert np.all(np.isfinite(fused))
    ref_att = attention.pv(attention.softmax(ref_sc, D), vh)
    assert rel_l2(fused[s], ref_att) <= TOL and worst_row_rel(fused[s], ref_att) <= TOL, \
        (rel_l2(fused[s], ref_att), worst_row_rel(fused[s], ref_att))
    # every stream: the fused path agrees with GEMV -> softmax -> GEMV, whose
    # K and V products were checked on every stream above
    assert rel_l2(fused, out) <= TOL and worst_row_rel(fused, out) <= TOL, (rel_l2(fused, out),
                                                                           worst_row_rel(fused, out))


def test_fullsize_streaming_append(torch_dev):
    """Prefill 65536 tokens, then 256 single-token appends over 256 streams;
    the sampled stream is checked against the oracle after steps 1, 64, 65
    and 256 (records, offsets, scores, V output)."""
    torch, dev = torch_dev
    from decode_gemv_amd import PackedKVCache, softmax_rows
    w = kvsynth.WORKLOADS["append-64k"]
    S, G, T0, D, n_app = w.streams, w.group, w.tokens, w.head_dim, w.append_steps
    cfg = oracle.Config(bits=w.bits, block=w.block)
    say("fullsize append", S, T0, n_app)
    K, V = host_streams(w, T0)
    c = PackedKVCache(S, T0 + n_app, bits=w.bits, block=w.block, device=str(dev))
    c.compress(torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev))
    assert c.check() == 0
    s = S - 1
    ref = ostream.compress(K[s], V[s], cfg)
    del K, V
    app_k = np.empty((S, n_app, D), np.float16)
    app_v = np.empty_like(app_k)
    for step in range(1, n_app + 1):
        new = [kvsynth.append_kv(w, i, step - 1) for i in range(S)]
        for i, (a_, b_) in enumerate(new):
            app_k[i, step - 1], app_v[i, step - 1] = a_[0], b_[0]
        kn = torch.from_numpy(np.stack([a for a, _ in new])).to(dev)
        vn = torch.from_numpy(np.stack([b for _, b in new])).to(dev)
        c.append(kn, vn)
        ostream.append(ref, *new[s])
        if step not in (1, 64, 65, n_app):
            continue
        say("append step", step)
        assert c.check() == 0
        T = c.n_tokens
        stream_state_equal(c, ref, s)
        q = np.stack([kvsynth.stream_q(w, i, step=step) for i in range(S)])
        scores_d = c.qk(torch.from_numpy(q).to(dev))
        p_d = softmax_rows(scores_d, T, 1.0 / np.sqrt(D))
        out = c.pv(p_d).cpu().numpy()
        assert c.check() == 0
        scores = scores_d.cpu().numpy()
        p = p_d.cpu().numpy()
        assert np.all(np.isfinite(scores)) and np.all(np.isfinite(out))
        kh, vh, _, _ = ostream.decode_stream(ref)
        ref_sc = attention.qk(q[s], kh)
        ref_out = attention.pv(p[s].astype(np.float64), vh)
        assert rel_l2(scores[s], ref_sc) <= TOL and worst_row_rel(scores[s], ref_sc) <= TOL
        assert rel_l2(out[s], ref_out) <= TOL and worst_row_rel(out[s], ref_out) <= TOL
        fused = c.attention(torch.from_numpy(q).to(dev)).cpu().numpy()
        assert c.check() == 0
        ref_att = attention.pv(attention.softmax(ref_sc, D), vh)
        assert rel_l2(fused[s], ref_att) <= TOL and worst_row_rel(fused[s], ref_att) <= TOL
        assert rel_l2(fused, out) <= TOL and worst_row_rel(fused, out) <= TOL
        if step == n_app:
            # every stream: one block closed by the appends, re-encoded by the
            # oracle from the appended tokens alone, with its scores and V GEMV
            say("append sampled blocks", step)
            B = w.block
            j0 = T0 // B
            sampled_blocks(torch, dev, c, w,
                           lambda s_, j: (app_k[s_, (j - j0) * B:(j - j0 + 1) * B],
                                          app_v[s_, (j - j0) * B:(j - j0 + 1) * B]),
                           cfg, scores, q, np.random.default_rng(step), closed=list(range(j0, T // B)))


def test_fullsize_paged_ragged(torch_dev):
    """The paged cache at the llama7b-32k shape with stream lengths spread from
    T down to T/4 (64 KiB pages, as bench.py times it): placement holds on
    every stream, one random closed block of every stream equals the oracle's
    encoding of that block alone, and the shortest stream is checked
    completely (records, permutation, tail, fused attention)."""
    torch, dev = torch_dev
    from decode_gemv_amd import PagedKVCache
    from gpu_common import check_placement
    w = kvsynth.WORKLOADS["llama7b-32k"]
    S, T, D, B = w.streams, w.tokens, w.head_dim, w.block
    cfg = oracle.Config(bits=w.bits, block=B)
    lens = [T - (3 * T // 4) * s // S for s in range(S)]
    say("fullsize paged ragged", S, T)
    K, V = host_streams(w, T)
    n_pages = sum(-(-L * 160 // 65536) + 3 for L in lens) + 16     # 148 B of records per token
    pc = PagedKVCache(S, T + 8, n_pages, page_bytes=65536, bits=w.bits, block=B, device=str(dev))
    Kd, Vd = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    for s, L in enumerate(lens):
        pc.prefill(s, Kd[s:s + 1, :L].contiguous(), Vd[s:s + 1, :L].contiguous())
    del Kd, Vd
    assert pc.check() == 0 and pc.lengths == lens
    check_placement(pc)
    say("fullsize paged sampled blocks")
    pool = pc.pool.cpu().numpy()
    (ks, kz), (vs, vz) = pc.tables()
    rng = np.random.default_rng(11)
    for s, L in enumerate(lens):
        j = int(rng.integers(L // B))
        code = ostream.encode_block(K[s, j * B:(j + 1) * B], V[s, j * B:(j + 1) * B], cfg)
        assert pool[ks[s, j]:ks[s, j] + kz[s, j]].tobytes() == code.k_record, f"K record ({s}, {j})"
        assert pool[vs[s, j]:vs[s, j] + vz[s, j]].tobytes() == code.v_record, f"V record ({s}, {j})"
    s = S - 1
    say("fullsize paged oracle stream", s, lens[s])
    ref = ostream.compress(K[s, :lens[s]], V[s, :lens[s]], cfg)
    ko, vo = ref.offsets("K"), ref.offsets("V")
    ka, va = ref.arena("K"), ref.arena("V")
    for j in range(len(ko) - 1):
        assert pool[ks[s, j]:ks[s, j] + kz[s, j]].tobytes() == ka[ko[j]:ko[j + 1]], f"K record {j}"
        assert pool[vs[s, j]:vs[s, j] + vz[s, j]].tobytes() == va[vo[j]:vo[j + 1]], f"V record {j}"
    nb = len(ko) - 1
    assert np.array_equal(pc.perm_table()[s, :nb].cpu().numpy(), ref.perm_table())
    q = np.stack([kvsynth.stream_q(w, i) for i in range(S)])
    fused = pc.attention(torch.from_numpy(q).to(dev)).cpu().numpy()
    assert pc.check() == 0
    assert np.all(np.isfinite(fused))
    kh, vh, _, _ = ostream.decode_stream(ref)
    want = attention.pv(attention.softmax(attention.qk(q[s], kh), D), vh)
    assert rel_l2(fused[s], want) <= TOL, rel_l2(fused[s], want)


def test_fullsize_paged_equals_contiguous(torch_dev):
    """Every stream at T tokens in both layouts at the llama7b-32k shape: fused
    attention through the block tables equals the contiguous cache's bit for
    bit on all 256 streams."""
    torch, dev = torch_dev
    from decode_gemv_amd import PackedKVCache, PagedKVCache
    w = kvsynth.WORKLOADS["llama7b-32k"]
    S, T = w.streams, w.tokens
    say("fullsize paged vs contiguous", S, T)
    K, V = host_streams(w, T)
    Kd, Vd = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    c = PackedKVCache(S, T + 8, bits=w.bits, block=w.block, device=str(dev))
    c.compress(Kd, Vd)
    pc = PagedKVCache(S, T + 8, S * (-(-T * 160 // 65536) + 3) + 16, page_bytes=65536, bits=w.bits,
                      block=w.block, device=str(dev))
    pc.prefill(0, Kd, Vd)
    del Kd, Vd
    assert c.check() == 0 and pc.check() == 0
    q = torch.from_numpy(np.stack([kvsynth.stream_q(w, i) for i in range(S)])).to(dev)
    x, y = c.attention(q), pc.attention(q)
    assert c.check() == 0 and pc.check() == 0
    assert torch.equal(x, y)
