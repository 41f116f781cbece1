"""Checkpoint and resume: the packed cache is its whole state (both arenas,
offset tables, permutation, raw tail staging, token count).  A cache dumped
to host memory after prefill, restored into a new cache and appended to must
equal, bit for bit, a cache that was never interrupted, and decode attention
over the two must agree exactly."""

import numpy as np
import pytest

from gpu_common import say, make_kv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch, torch.device("cuda:0")


CASES = [(3, 64, 1, "gauss"), (2, 64, 1, "bimodal"), (4, 128, 2, "struct"), (8, 64, 1, "mixed"),
         (4, 64, 0, "gauss")]


@pytest.mark.parametrize("bits,block,permute,law", CASES, ids=[f"b{b}-B{B}-p{p}-{l}" for b, B, p, l in CASES])
def test_resume_equals_uninterrupted(torch_dev, bits, block, permute, law):
    torch, dev = torch_dev
    from decode_gemv_amd import PackedKVCache
    S, T0 = 3, 2 * block + 37                       # the prefill ends inside a block
    extra = block + 21                              # appends close that block and open another
    say("checkpoint", bits, block, permute, law)
    K, V = make_kv(law, S, T0 + extra, block, seed=11)
    kt, vt = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)

    def fresh():
        return PackedKVCache(S, T0 + extra + 8, bits=bits, block=block, permute=permute, device="cuda")

    a = fresh()
    a.compress(kt[:, :T0].contiguous(), vt[:, :T0].contiguous())
    b = fresh()
    b.compress(kt[:, :T0].contiguous(), vt[:, :T0].contiguous())
    state = b.state_dict()
    del b
    c = fresh()
    c.load_state_dict(state)
    assert c.n_tokens == T0
    for t in range(T0, T0 + extra):
        k1, v1 = kt[:, t:t + 1].contiguous(), vt[:, t:t + 1].contiguous()
        a.append(k1, v1)
        c.append(k1, v1)
    torch.cuda.synchronize()
    assert a.n_tokens == c.n_tokens == T0 + extra
    for name in ("k_arena", "v_arena", "k_off", "v_off", "perm", "tail_k", "tail_v"):
        x, y = getattr(a, name), getattr(c, name)
        assert torch.equal(x, y), f"{name} differs after resume"
    assert int(a.status.item()) == 0 and int(c.status.item()) == 0
    q = torch.from_numpy(np.random.default_rng(5).standard_normal((S, 1, 128)).astype(np.float16)).to(dev)
    oa, oc = a.attention(q), c.attention(q)
    torch.cuda.synchronize()
    assert torch.equal(oa, oc)


def test_state_of_another_configuration_is_refused(torch_dev):
    torch, dev = torch_dev
    from decode_gemv_amd import PackedKVCache
    a = PackedKVCache(2, 256, bits=4, block=64, device="cuda")
    b = PackedKVCache(2, 256, bits=3, block=64, device="cuda")
    with pytest.raises(ValueError):
        b.load_state_dict(a.state_dict())
