"""Pins of the run-length study (oracle/cr.py): at the format's run length it
reproduces the ideal bits counted from the stored records, and two limits
have closed forms.
"""

import numpy as np
import pytest

import kvsynth
import oracle
from oracle import cr, stream as ostream


def streams(law, T, block, seed):
    if law == "struct":
        return kvsynth.structured_kv(T, 128, block, 32, seed=seed)
    w = kvsynth.Workload("t", 1, 1, 1, T, 128, 4, block, "gauss")
    return kvsynth.stream_kv(w, 0, seed=seed, tokens=T)


@pytest.mark.parametrize("law,bits,block,permute,T", [("struct", 4, 64, 1, 200), ("gauss", 3, 128, 2, 300),
                                                      ("struct", 2, 64, 0, 97)])
def test_run_32_matches_the_records(law, bits, block, permute, T):
    k, v = streams(law, T, block, 3)
    cache = ostream.compress(k, v, oracle.Config(bits=bits, block=block, permute=permute))
    kb, vb = cr.run_length_bits(k, v, bits, block, permute, 32)
    assert kb == cr.ratios(cache, "K")["ideal_bits"]
    assert vb == cr.ratios(cache, "V")["ideal_bits"]


def test_run_of_one_slot_has_no_payload():
    # every run holds one value: width 0, only headers and parameters remain
    k, v = streams("gauss", 130, 64, 5)
    kb, vb = cr.run_length_bits(k, v, 4, 64, 1, 1)
    n, D, nb = 130, 128, 3
    assert kb == 8 * n * D + 32 * D * nb
    assert vb == 8 * n * D + 32 * n


@pytest.mark.parametrize("bits,block", [(4, 64), (2, 128), (6, 64)])
def test_run_of_a_whole_block_is_the_full_width_closed_form(bits, block):
    # K is quantised per channel over the block, so a run spanning the block
    # holds both 0 and 2^b - 1 in every non-constant channel: width b
    rng = np.random.default_rng(bits)
    k = rng.standard_normal((4 * block, 128)).astype(np.float16)
    v = rng.standard_normal((4 * block, 128)).astype(np.float16)
    kb, _ = cr.run_length_bits(k, v, bits, block, 1, block)
    per_value = kb / k.size
    assert per_value == pytest.approx(16 / cr.closed_form_full_width("K", bits, block, block, 128), rel=1e-12)
