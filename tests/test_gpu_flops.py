"""The pair count the benchmark derives from the device tables equals the
oracle's count of causal pairs of the rank's share; the matrix-unit
calibration the benchmark reports beside it gives a plausible rate."""
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


def test_mfma_calibration_within_the_published_peak():
    # the matrix-unit calibration kernel: a positive rate that cannot exceed
    # the device's published dense bf16 peak (2.5 PFLOP/s) by more than timing
    # noise, and a doubled chain length takes about twice as long
    import torch
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    api.cp_attn_mfma_probe(1000, sink)  # warm up
    ms1, tf1 = api.cp_attn_mfma_probe(20000, sink)
    ms2, tf2 = api.cp_attn_mfma_probe(40000, sink)
    H.log(f"[mfma probe] {tf1:.1f} / {tf2:.1f} TFLOP/s ({ms1:.3f} / {ms2:.3f} ms)")
    assert 0 < tf1 <= 2600 and 0 < tf2 <= 2600
    assert 1.6 < ms2 / ms1 < 2.4
    assert float(sink[0]) == 0.0
