"""The in-order forward on a padded pack large enough to take it (the launch
plan is chosen by size: these steps are too long to run concurrently): each
ring step folds its partial into the accumulator in its own epilogue, the
causal step last writing the bf16 output, and padding rows get their own
launch. Sampled rows (valid and padding) of out / LSE / dQ against the oracle,
exact dK / dV of late key rows, padding rows exactly 0 / -inf, and the launch
plan itself. Both ranks, so both step orders (a second-chunk step first, a
first-chunk step first) are covered."""
import math

import numpy as np
import pytest

from context_packed_attention_amd import api, synth
from oracle import cp_attn_oracle as O
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

LENGTHS = [3000, 1500, 3800, 5]
PADDED = [3008, 1600, 3804, 8]   # multiples of 2 * CP, with padding in three slots
CP, HQ, HKV, D = 2, 64, 8, 64


@pytest.mark.parametrize("rank", [0, 1])
def test_in_order_forward_with_padding(rank):
    import torch
    bt = synth.make_batch("inorder-padded", 17, LENGTHS, PADDED, HQ, HKV, D)
    scale = 1.0 / math.sqrt(D)
    db = H.DeviceBatch(bt)
    meta, loc = H.local_inputs(db, CP, rank)
    tl = loc["t_local"]
    torch.cuda.synchronize()
    api.cp_attn_timing_enable(True)
    out, lse = H.run_fwd(meta, loc, bt, scale)
    dq, dks, dvs = H.run_bwd(meta, loc, bt, scale, out, lse)
    torch.cuda.synchronize()
    api.cp_attn_timing_enable(False)
    n = {k: v[1] for k, v in api.cp_attn_timing_read().items()}
    H.log(f"[inorder] rank {rank} launches {n}")
    assert n["fwd_step"] == CP and "fwd_fused" not in n and n.get("pad_rows") == 1

    own = O.shard_rows(bt.cu, bt.cup, CP, rank)
    valid = O.valid_mask(bt.cu, bt.cup)[own]
    assert (~valid).any()
    outb = H.bf16_to_np(out)[:tl]
    lsen = lse.cpu().numpy()[:, :tl]
    assert not outb[~valid].any() and np.isneginf(lsen[:, ~valid]).all(), "padding rows must be 0 / -inf"

    rng = np.random.default_rng(3 + rank)
    slot_end = (np.asarray(bt.cup[1:], dtype=np.int64) // CP)
    fixed = np.concatenate([[0, 1, 127, 128], slot_end - 1, slot_end - 2, np.nonzero(~valid)[0][:4]])
    rows = np.unique(np.concatenate([fixed, rng.integers(0, tl, 24)]))
    heads = [0, 7, 31, HQ - 1]
    o_ref, l_ref, dq_ref = O.share_rows(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, CP, rank, scale, rows, heads,
                                        want_dq=True)
    H.compare_bf16("out", outb[rows][:, heads], o_ref)
    H.compare_lse("lse", lsen[heads][:, rows], l_ref)
    H.compare_bf16("dq", H.bf16_to_np(dq)[:tl][rows][:, heads], dq_ref)
    keys = np.unique(np.concatenate([slot_end - k for k in range(1, 7)]))
    keys = keys[(keys >= 0) & (keys < tl)]
    dk_ref, dv_ref = O.share_keys_dkdv(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, CP, rank, scale, rank, keys, [0, HKV - 1])
    H.compare_bf16("dk rows", H.bf16_to_np(dks[rank])[keys][:, [0, HKV - 1]], dk_ref)
    H.compare_bf16("dv rows", H.bf16_to_np(dvs[rank])[keys][:, [0, HKV - 1]], dv_ref)
    meta.close()
