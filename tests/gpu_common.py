"""Helpers for the GPU parity tests: seeded inputs, oracle references, comparisons."""

import sys

import numpy as np

import kvsynth
import oracle
from oracle import stream as ostream


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def make_kv(law: str, S: int, T: int, block: int, seed: int = 0, D: int = 128):
    """fp16 K, V [S][T][D] for one of the small parity laws."""
    ks, vs = [], []
    for s in range(S):
        if law in ("gauss", "bimodal"):
            w = kvsynth.Workload("t", 1, S, 1, T, D, 4, block, law)
            k, v = kvsynth.stream_kv(w, s, seed=seed, tokens=T)
        elif law == "struct":
            k, v = kvsynth.structured_kv(T, D, block, 32, seed=seed + s)
        elif law == "mixed":            # half the channels nearly constant: narrow runs
            k, v = kvsynth.structured_kv(T, D, block, 32, seed=seed + s, noise=0.3, shuffle=False)
        elif law == "grid":             # values on an fp16 grid: exact dequantisation
            rng = np.random.default_rng([seed, s])
            k = (rng.integers(-60, 60, (T, D)) * 0.125).astype(np.float16)
            v = (rng.integers(-60, 60, (T, D)) * 0.0625).astype(np.float16)
        elif law == "subnormal":        # fp16 subnormals, signed zeros, tiny ranges
            rng = np.random.default_rng([seed, s, 7])
            bits = rng.integers(0, 0x0400, (2, T, D)).astype(np.uint16)
            bits |= (rng.random((2, T, D)) < 0.5).astype(np.uint16) << 15
            big = rng.random((2, T, D)) < 0.02             # a few normal values
            bits[big] = rng.integers(0x0400, 0x1400, int(big.sum())).astype(np.uint16)
            k, v = bits[0].view(np.float16), bits[1].view(np.float16)
        else:
            raise ValueError(law)
        ks.append(k)
        vs.append(v)
    return np.stack(ks), np.stack(vs)


def oracle_streams(K, V, bits, block, permute=True, payload_order=0):
    cfg = oracle.Config(head_dim=K.shape[2], bits=bits, block=block, permute=permute,
                        payload_order=payload_order)
    return [ostream.compress(K[s], V[s], cfg) for s in range(K.shape[0])]


def rel_l2(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


def worst_row_rel(y, ref):
    y = np.asarray(y, np.float64).reshape(-1, y.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    num = np.linalg.norm(y - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-300)
    return float((num / den).max())


def check_placement(c):
    """Every record of a closed block lies inside one page; a page belongs to
    one stream and holds only K or only V records; open blocks sit in their
    stream's tail slots; nothing overlaps; the free count is what the streams
    do not hold."""
    (ks, kz), (vs, vz) = c.tables()
    slot, page = int(c.sizes.slot_bytes), c.page_bytes
    tail0 = c.n_pages * page
    spans, owner = [], {}
    for s, n in enumerate(c.lengths):
        nfull, nb = n // c.block, -(-n // c.block)
        for j in range(nb):
            for st, sz, which in ((ks[s, j], kz[s, j], 0), (vs[s, j], vz[s, j], 1)):
                assert sz >= 16 and sz % 16 == 0
                if j < nfull:
                    p = st // page
                    assert p < c.n_pages and (st + sz - 1) // page == p, f"record straddles a page, stream {s}"
                    assert owner.setdefault(p, (s, which)) == (s, which), f"page {p} shared"
                else:
                    assert st == tail0 + (2 * s + which) * slot, f"open block not in its tail slot, stream {s}"
                    assert sz <= slot
                spans.append((st, st + sz))
    spans.sort()
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0, "records overlap"
    assert c.free_pages() == c.n_pages - len(owner)
    return owner
