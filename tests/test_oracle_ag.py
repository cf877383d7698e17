"""Pins of the oracle's all-gather layout (rank r's contribution to the
gradient of every gathered key row, "Hybrid / Hierarchical Context Parallel
Skill", Implementation Map: "all_gather" communication type):

* summed over all ranks, the contributions are the gradient of the whole
  packed attention (every query row), computed in one call;
* restricted to shard s's rows they are the ring share's part for shard s;
* rows of keys that no query of the rank reaches (and padding rows) are 0.
"""
import math

import numpy as np
import pytest

from context_packed_attention_amd import synth
from oracle import cp_attn_oracle as O

CASES = [
    ("ag-ragged-cp2-d16", [37, 5, 64, 8], [40, 8, 64, 8], 2, 4, 2, 16),
    ("ag-ragged-cp3-d16-gqa", [60, 1, 25, 0], [60, 12, 30, 6], 3, 6, 2, 16),
    ("ag-tiny-cp4-d8-pad", [5, 9, 1], [8, 16, 8], 4, 2, 1, 8),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gathered_gradients(case):
    name, L, P, cp, hq, hkv, d = case
    bt = synth.make_batch(name, 31, L, P, hq, hkv, d)
    scale = 1.0 / math.sqrt(d)
    f = O.bf16_to_f64
    full = O.attention(f(bt.q), f(bt.k), f(bt.v), f(bt.do), bt.cu, bt.cup, scale)
    sum_dk = np.zeros_like(full[3])
    sum_dv = np.zeros_like(full[4])
    valid = O.valid_mask(bt.cu, bt.cup)
    rank_of, _ = O.owner_map(bt.cu, bt.cup, cp)
    seq = np.searchsorted(bt.cup, np.arange(bt.total_rows), side="right") - 1
    for r in range(cp):
        res = O.share(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale)
        sum_dk += res["dk_full"]
        sum_dv += res["dv_full"]
        for s in range(cp):
            rows = O.shard_rows(bt.cu, bt.cup, cp, s)
            assert np.array_equal(res["dk_full"][rows], res["dk_parts"][s])
            assert np.array_equal(res["dv_full"][rows], res["dv_parts"][s])
        # last position of rank r's queries in every sequence
        last = np.full(bt.cu.size - 1, -1)
        for g in np.nonzero((rank_of == r) & valid)[0]:
            last[seq[g]] = max(last[seq[g]], g)
        unreached = ~valid | (np.arange(bt.total_rows) > last[seq])
        assert not res["dk_full"][unreached].any() and not res["dv_full"][unreached].any()
    np.testing.assert_allclose(sum_dk, full[3], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sum_dv, full[4], rtol=0, atol=1e-12)
    assert np.abs(full[3]).max() > 0.01  # the identity is not vacuous
