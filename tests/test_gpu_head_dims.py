"""GPU parity at head_dim 64 and 256 (the oracle's other head dims).

For b in {2, 3, 4, 6, 8} and B in {64, 128}: the encoder's records,
offsets, permutation and tail staging are bit-exact with the fp64 oracle,
the decompressed ints and x_hat are exact, the K and V GEMVs and fused
attention are within rel-L2 1e-4 (tensor and worst row) with one and with
four queries per stream, and single-token appends give the one-shot bytes.
"""

import numpy as np
import pytest

from gpu_common import say, make_kv, oracle_streams, rel_l2, worst_row_rel
from oracle import stream as ostream, attention
from test_gpu_parity import assert_state_equal, gpu_cache

pytestmark = pytest.mark.gpu
TOL = 1e-4

CASES = [
    # D, bits, block, law, permute
    (64, 2, 64, "bimodal", 1), (64, 2, 128, "mixed", 1), (64, 3, 64, "struct", 1), (64, 4, 64, "gauss", 1),
    (64, 4, 128, "struct", 2), (64, 8, 64, "gauss", 1), (64, 8, 128, "mixed", 1), (64, 6, 64, "struct", 0),
    (256, 2, 64, "bimodal", 1), (256, 2, 128, "mixed", 1), (256, 3, 64, "struct", 1), (256, 4, 64, "gauss", 1),
    (256, 4, 128, "struct", 2), (256, 8, 64, "gauss", 1), (256, 8, 128, "mixed", 1), (256, 5, 128, "struct", 0),
]
IDS = [f"D{d}-b{b}-B{bl}-{law}-p{p}" for d, b, bl, law, p in CASES]


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch, torch.device("cuda:0")


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_head_dim_parity(torch_dev, case):
    torch, dev = torch_dev
    D, bits, block, law, permute = case
    S, T = 2, 3 * block + 37
    K, V = make_kv(law, S, T, block, seed=D + bits, D=D)
    refs = oracle_streams(K, V, bits, block, permute)
    say("head_dim encode", case)
    c = gpu_cache(torch, dev, K, V, bits, block, permute)
    assert c.check() == 0
    assert_state_equal(c, refs)
    decoded = [ostream.decode_stream(r) for r in refs]
    for which, mode in (("K", 0), ("V", 0), ("K", 1), ("V", 1)):
        got = c.decompress(which, mode).cpu().numpy()
        assert c.check() == 0
        for s, ref in enumerate(refs):
            kh, vh, qk, qv = decoded[s]
            if mode == 0:
                assert np.array_equal(got[s].astype(np.int64), qk if which == "K" else qv)
            else:
                exp = ostream.token_order(ref, kh if which == "K" else vh).astype(np.float32)
                assert np.array_equal(got[s].view(np.uint32), exp.view(np.uint32))
    for G in (1, 4):
        rng = np.random.default_rng(G + D)
        q = rng.standard_normal((S, G, D)).astype(np.float16)
        say("head_dim gemvs", case, "G", G)
        scores = c.qk(torch.from_numpy(q).to(dev)).cpu().numpy()
        assert c.check() == 0
        ref_s = np.stack([attention.qk(q[s], decoded[s][0]) for s in range(S)])
        assert rel_l2(scores, ref_s) <= TOL and worst_row_rel(scores, ref_s) <= TOL, \
            (rel_l2(scores, ref_s), worst_row_rel(scores, ref_s))
        p = np.stack([attention.softmax(ref_s[s], D) for s in range(S)]).astype(np.float32)
        out = c.pv(torch.from_numpy(p).to(dev)).cpu().numpy()
        assert c.check() == 0
        ref_o = np.stack([attention.pv(p[s].astype(np.float64), decoded[s][1]) for s in range(S)])
        assert rel_l2(out, ref_o) <= TOL and worst_row_rel(out, ref_o) <= TOL, \
            (rel_l2(out, ref_o), worst_row_rel(out, ref_o))
        att = c.attention(torch.from_numpy(q).to(dev)).cpu().numpy()
        assert c.check() == 0
        ref_a = np.stack([attention.pv(attention.softmax(ref_s[s], D), decoded[s][1]) for s in range(S)])
        assert rel_l2(att, ref_a) <= TOL and worst_row_rel(att, ref_a) <= TOL, \
            (rel_l2(att, ref_a), worst_row_rel(att, ref_a))


@pytest.mark.parametrize("D,bits,block", [(64, 3, 64), (256, 4, 128), (256, 8, 64)])
def test_head_dim_append_matches_one_shot(torch_dev, D, bits, block):
    torch, dev = torch_dev
    from decode_gemv_amd import PackedKVCache
    S, t0, steps = 2, block + 9, block + 5
    K, V = make_kv("gauss", S, t0 + steps, block, seed=7, D=D)
    c = PackedKVCache(S, t0 + steps + 4, bits=bits, block=block, device=str(dev), head_dim=D)
    Kd, Vd = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    say("head_dim append", D, bits, block)
    c.compress(Kd[:, :t0].contiguous(), Vd[:, :t0].contiguous())
    for t in range(t0, t0 + steps):
        c.append(Kd[:, t:t + 1].contiguous(), Vd[:, t:t + 1].contiguous())
    assert c.check() == 0
    assert_state_equal(c, oracle_streams(K, V, bits, block, True))

