"""packkv_attention_decode_noalloc (the entry point for callers that cannot
allocate): through the C ABI it gives packkv_attention_decode's output bit
for bit, on two calls in a row, the second with a smaller cache, and both
within rel-L2 1e-4 of the fp64 oracle; shapes past its scratch limit are
refused before any launch."""

import numpy as np
import pytest

from gpu_common import say, make_kv, oracle_streams, rel_l2, worst_row_rel
from oracle import stream as ostream, attention

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch, torch.device("cuda:0")


def _cache(torch, dev, S, T, bits, block, G, seed):
    from decode_gemv_amd import PackedKVCache
    K, V = make_kv("gauss", S, T, block, seed=seed)
    c = PackedKVCache(S, T + 8, bits=bits, block=block, device=str(dev))
    c.compress(torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev))
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S, G, 128)).astype(np.float16)
    return c, K, V, q


@pytest.mark.parametrize("first,second", [((6, 3000, 4, 64, 1), (2, 700, 4, 64, 1)),
                                          ((4, 2600, 3, 128, 4), (3, 300, 2, 64, 4))],
                         ids=["b4-G1", "mixed-G4"])
def test_noalloc_matches_workspace_entry_point(torch_dev, first, second):
    torch, dev = torch_dev
    for i, (S, T, bits, block, G) in enumerate((first, second)):
        say("noalloc call", i, S, T, bits, block, G)
        c, K, V, q = _cache(torch, dev, S, T, bits, block, G, seed=10 + i)
        qd = torch.from_numpy(q).to(dev)
        want = c.attention(qd).clone()
        out = torch.full((S, G, 128), float("nan"), dtype=torch.float32, device=dev)
        got = c.attention_noalloc(qd, out)
        assert c.check() == 0
        assert torch.equal(got, want), f"call {i}"
        refs = oracle_streams(K, V, bits, block, True)
        g = got.cpu().numpy()
        for s in range(S):
            kh, vh, _, _ = ostream.decode_stream(refs[s])
            ref = attention.pv(attention.softmax(attention.qk(q[s], kh), 128), vh)
            assert rel_l2(g[s], ref) <= TOL and worst_row_rel(g[s], ref) <= TOL


def test_noalloc_refuses_shapes_past_its_scratch(torch_dev):
    torch, dev = torch_dev
    from decode_gemv_amd import PackKVError, _lib
    # 2 streams of 100000 tokens with 64 queries: ~2 * 64 * 391 * 528 bytes of
    # partials, past 16 MiB
    S, T, G = 2, 100000, 64
    c, _, _, q = _cache(torch, dev, S, T, 4, 64, G, seed=3)
    out = torch.zeros(S, G, 128, dtype=torch.float32, device=dev)
    say("noalloc over the limit")
    with pytest.raises(PackKVError) as e:
        c.attention_noalloc(torch.from_numpy(q).to(dev), out)
    assert e.value.code == _lib.ECAPACITY
    assert c.check() == 0
