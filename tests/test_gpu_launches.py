"""Launch sequence checks (through the library's event timing, which counts
every launch per kernel):

* ring completeness: one forward kernel, one dK/dV and one dQ kernel per ring
  step, and either CP-1 pairwise merges or (steps run concurrently) one merge
  of all step partials (a CP path that silently drops ring steps runs fast with
  wrong gradients - "Hybrid / Hierarchical Context Parallel Skill", Pitfalls);
* the padding decision by value gives the same launch sequence for an
  aliased, NULL or distinct-equal cu_seqlens_padded;
* tail zeroing is launched only when the local tensors have rows past the
  valid end.
"""
import math

import pytest

from context_packed_attention_amd import api, synth
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _launches(bt, cp, r, tail=0, cup="copy"):
    db = H.DeviceBatch(bt)
    meta, loc = H.local_inputs(db, cp, r, tail=tail, cup=cup)
    scale = 1.0 / math.sqrt(bt.d)
    import torch
    torch.cuda.synchronize()
    api.cp_attn_timing_enable(True)
    out, lse = H.run_fwd(meta, loc, bt, scale)
    H.run_bwd(meta, loc, bt, scale, out, lse)
    torch.cuda.synchronize()
    api.cp_attn_timing_enable(False)
    t = api.cp_attn_timing_read()
    meta.close()
    return {k: v[1] for k, v in t.items()}


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_ring_completeness(cfg):
    bt, w = synth.make_workload(cfg)
    cp = w["cp"]
    for r in range(cp):
        n = _launches(bt, cp, r)
        H.log(f"[launch] cfg{cfg} rank {r}: {n}")
        assert n["fwd_step"] == cp and n["bwd_dkdv"] == cp and n["bwd_dq"] == cp
        if "lse_merge_all" in n:
            assert n["lse_merge_all"] == 1 and "lse_merge" not in n and cp > 1
        else:
            assert n["lse_merge"] == max(1, cp - 1)
        assert n["bwd_pre"] == 1 and n["dq_finalize"] == 1
        assert "tail_zero" not in n


def test_same_launches_for_alias_null_copy():
    bt, w = synth.make_workload(2)
    seqs = [_launches(bt, w["cp"], 1, cup=c) for c in ("copy", "alias", "null")]
    assert seqs[0] == seqs[1] == seqs[2]


def test_tail_zero_gated():
    bt, w = synth.make_workload(1)
    assert "tail_zero" not in _launches(bt, 2, 0, tail=0)
    assert _launches(bt, 2, 0, tail=37)["tail_zero"] == 1
