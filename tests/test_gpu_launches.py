"""Launch sequence checks (through the library's event timing, which counts
every launch per kernel):

* ring completeness: one forward kernel per ring step, each step folding its
  partial into the accumulator in its own epilogue, or (short steps) one
  fused launch whose blocks run through every step; the backward runs every
  step's dK/dV in one launch and every step's dQ in one launch (a CP path
  that silently drops ring steps runs fast with wrong gradients - "Hybrid /
  Hierarchical Context Parallel Skill", Pitfalls; the parity tests compare
  every step's dK/dV part and the dQ summed over all steps);
* the padding decision by value gives the same launch sequence for an
  aliased, NULL or distinct-equal cu_seqlens_padded, and for an asserted
  pad_hint that agrees with the values;
* tail zeroing is launched only when the local tensors have rows past the
  valid end.
"""
import math

import pytest

from context_packed_attention_amd import api, synth
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _launches(bt, cp, r, tail=0, cup="copy", pad_hint=-1):
    db = H.DeviceBatch(bt)
    meta, loc = H.local_inputs(db, cp, r, tail=tail, cup=cup, pad_hint=pad_hint)
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


def meta_valid_rows(bt, cp, r):
    from oracle import cp_attn_oracle as O
    return int(O.valid_mask(bt.cu, bt.cup)[O.shard_rows(bt.cu, bt.cup, cp, r)].sum())


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_ring_completeness(cfg):
    bt, w = synth.make_workload(cfg)
    cp = w["cp"]
    for r in range(cp):
        n = _launches(bt, cp, r)
        H.log(f"[launch] cfg{cfg} rank {r}: {n}")
        # in order: one launch per ring step; short steps: one fused launch
        if "fwd_fused" in n:
            assert n["fwd_fused"] == 1 and "fwd_step" not in n and cp > 1
        else:
            assert n["fwd_step"] == cp
        assert n["bwd_dkdv"] == 1 and n["bwd_dq"] == 1
        # padding rows of out / LSE get their own small launch, only when present
        assert n.get("pad_rows", 0) == int(meta_valid_rows(bt, cp, r) < bt.total_rows // cp)
        assert n["bwd_pre"] == 1
        assert n.get("dq_pad_rows", 0) == int(meta_valid_rows(bt, cp, r) < bt.total_rows // cp)
        assert "tail_zero" not in n


def test_same_launches_for_alias_null_copy():
    bt, w = synth.make_workload(2)
    seqs = [_launches(bt, w["cp"], 1, cup=c) for c in ("copy", "alias", "null")]
    assert seqs[0] == seqs[1] == seqs[2]


@pytest.mark.parametrize("cfg,hint", [(2, 0), (3, 1)])
def test_same_launches_for_pad_hint(cfg, hint):
    # an asserted hint that agrees with the values takes the path the
    # value-based decision (-1) takes
    bt, w = synth.make_workload(cfg)
    assert _launches(bt, w["cp"], 1, pad_hint=hint) == _launches(bt, w["cp"], 1, pad_hint=-1)


def test_tail_zero_gated():
    bt, w = synth.make_workload(1)
    assert "tail_zero" not in _launches(bt, 2, 0, tail=0)
    assert _launches(bt, 2, 0, tail=37)["tail_zero"] == 1
