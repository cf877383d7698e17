"""The pair count the benchmark derives from the device tables equals the
oracle's count of causal pairs of the rank's share."""
import numpy as np
import pytest

from context_packed_attention_amd import api, synth
from oracle import cp_attn_oracle as O
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_step_pairs_match_oracle(cfg):
    w = synth.workload(cfg)
    L = w["lengths"]
    P = L if w["max_pad"] is None else synth.draw_padded_lengths(w["seed"], L, w["max_pad"], 2 * w["cp"])
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    cup = np.concatenate([[0], np.cumsum(P)]).astype(np.int32)
    for r in w["ranks"]:
        m = api.cp_attn_rank_metadata(H.dev_i32(cu), H.dev_i32(cup), w["cp"], r, -1, int(cup[-1]) // w["cp"])
        got = sum(api.step_pairs(m))
        ref = O.flops_share(cu, cup, w["cp"], r, w["hq"], w["d"])["pairs"]
        assert got == ref, (cfg, r, got, ref)
        m.close()
