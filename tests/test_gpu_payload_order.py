"""GPU parity of the width-sorted K payload (payload order 1): the encoder
writes the oracle's records byte for byte, the decoders read them back (ints
and x_hat bit-exact), and the K GEMV and fused attention over them stay
within rel-L2 1e-4 of the fp64 oracle.  The cases hold narrow runs (clustered
and half-constant data) so that rows of mixed widths are reordered, plus
full-width data, partial blocks and appends."""

import numpy as np
import pytest

from gpu_common import say, make_kv, oracle_streams, rel_l2, worst_row_rel
from oracle import stream as ostream, attention
from test_gpu_parity import assert_state_equal, gpu_cache

pytestmark = pytest.mark.gpu
TOL = 1e-4

CASES = [
    # id, bits, block, S, T, permute, law, head_dim
    ("b4B64-struct", 4, 64, 2, 331, 1, "struct", 128),
    ("b3B64-struct", 3, 64, 2, 257, 1, "struct", 128),
    ("b2B64-mixed", 2, 64, 2, 190, 1, "mixed", 128),
    ("b3B128-struct", 3, 128, 2, 390, 1, "struct", 128),
    ("b4B128-mixed", 4, 128, 2, 300, 1, "mixed", 128),
    ("b2B128-sortkey-struct", 2, 128, 2, 200, 2, "struct", 128),
    ("b4B64-gauss", 4, 64, 2, 200, 1, "gauss", 128),
    ("b4B64-identity-mixed", 4, 64, 2, 150, 0, "mixed", 128),
    ("b3B64-one-token", 3, 64, 1, 1, 1, "gauss", 128),
    ("b3B64-D64-mixed", 3, 64, 2, 170, 1, "mixed", 64),
    ("b4B128-D256-struct", 4, 128, 2, 300, 1, "struct", 256),
]


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch, torch.device("cuda:0")


def build(torch, dev, case):
    cid, bits, block, S, T, permute, law, D = case
    K, V = make_kv(law, S, T, block, D=D)
    refs = oracle_streams(K, V, bits, block, permute, payload_order=1)
    c = gpu_cache(torch, dev, K, V, bits, block, permute, payload_order=1)
    return K, V, refs, c


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_width_sorted_records_bit_exact(torch_dev, case):
    torch, dev = torch_dev
    say("wsorted encode", case[0])
    K, V, refs, c = build(torch, dev, case)
    assert c.check() == 0
    assert_state_equal(c, refs)
    for which, mode in (("K", 0), ("K", 1)):
        say("wsorted decompress", case[0], mode)
        got = c.decompress(which, mode).cpu().numpy()
        assert c.check() == 0
        for s, ref in enumerate(refs):
            kh, _, qk, _ = ostream.decode_stream(ref)
            if mode == 0:
                assert np.array_equal(got[s].astype(np.int64), qk)
            else:
                exp = ostream.token_order(ref, kh).astype(np.float32)
                assert np.array_equal(got[s].view(np.uint32), exp.view(np.uint32))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("G", [1, 4])
def test_width_sorted_qk_and_attention_within_tolerance(torch_dev, case, G):
    torch, dev = torch_dev
    K, V, refs, c = build(torch, dev, case)
    S, D = K.shape[0], K.shape[2]
    rng = np.random.default_rng(G)
    q = (rng.standard_normal((S, G, D)) * 2).astype(np.float16)
    qd = torch.from_numpy(q).to(dev)
    say("wsorted qk", case[0], "G", G)
    scores = c.qk(qd).cpu().numpy()
    assert c.check() == 0
    dec = [ostream.decode_stream(r) for r in refs]
    ref_s = np.stack([attention.qk(q[s], dec[s][0]) for s in range(S)])
    assert rel_l2(scores, ref_s) <= TOL and worst_row_rel(scores, ref_s) <= TOL, \
        (rel_l2(scores, ref_s), worst_row_rel(scores, ref_s))
    say("wsorted attention", case[0], "G", G)
    out = c.attention(qd).cpu().numpy()
    assert c.check() == 0
    ref = np.stack([attention.pv(attention.softmax(attention.qk(q[s], dec[s][0]), D), dec[s][1])
                    for s in range(S)])
    assert rel_l2(out, ref) <= TOL and worst_row_rel(out, ref) <= TOL, (rel_l2(out, ref), worst_row_rel(out, ref))


@pytest.mark.parametrize("bits,block,t0,steps,law", [(3, 64, 60, 70, "struct"), (4, 128, 0, 130, "mixed"),
                                                    (2, 64, 64, 1, "struct")])
def test_width_sorted_append_matches_one_shot(torch_dev, bits, block, t0, steps, law):
    torch, dev = torch_dev
    from decode_gemv_amd import PackedKVCache
    S = 2
    K, V = make_kv(law, S, t0 + steps + 5, block, seed=3)
    c = PackedKVCache(S, t0 + steps + 10, bits=bits, block=block, permute=1, device=str(dev), payload_order=1)
    Kd, Vd = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    say("wsorted append", bits, block, t0, steps, law)
    if t0:
        c.compress(Kd[:, :t0].contiguous(), Vd[:, :t0].contiguous())
    for t in range(t0, t0 + steps):
        c.append(Kd[:, t:t + 1].contiguous(), Vd[:, t:t + 1].contiguous())
    c.append(Kd[:, t0 + steps:].contiguous(), Vd[:, t0 + steps:].contiguous())
    assert c.check() == 0
    assert_state_equal(c, oracle_streams(K, V, bits, block, 1, payload_order=1))


def test_orders_give_the_same_attention(torch_dev):
    """The two payload orders hold the same ints; attention over them agrees
    within rounding (the K GEMV sums in the same order either way, so the
    scores are in fact identical)."""
    torch, dev = torch_dev
    K, V = make_kv("struct", 3, 500, 64, seed=6)
    a = gpu_cache(torch, dev, K, V, 3, 64, 1)
    b = gpu_cache(torch, dev, K, V, 3, 64, 1, payload_order=1)
    q = torch.from_numpy(np.random.default_rng(2).standard_normal((3, 1, 128)).astype(np.float16)).to(dev)
    say("wsorted vs channel order")
    assert torch.equal(a.qk(q), b.qk(q))
    assert torch.equal(a.attention(q), b.attention(q))
    assert a.check() == 0 and b.check() == 0
