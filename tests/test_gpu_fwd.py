"""Forward of a rank's share on the GPU vs the fp64 oracle: bf16 out within
max-abs 2e-2 and relative L2 1e-2, LSE within 1e-3 * max(1, |lse|), padding
rows exactly 0 / -inf."""
import math

import numpy as np
import pytest

from context_packed_attention_amd import synth
from oracle import cp_attn_oracle as O
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

SMALL = [
    # name, lengths, padded, cp, hq, hkv, d
    ("one-seq-cp1-d128", [300], [304], 1, 2, 1, 128),
    ("ragged-cp2-d64", [257, 31, 640, 8], [264, 32, 640, 8], 2, 4, 2, 64),
    ("ragged-cp3-d128-gqa", [600, 1, 250, 0], [600, 12, 252, 6], 3, 8, 2, 128),
    ("long-cp4-d128", [1800, 500], [1808, 504], 4, 4, 4, 128),
    ("tiny-cp4-d64-pad", [5, 9, 1], [8, 16, 8], 4, 2, 2, 64),
    # one long sequence among many short ones: the single-launch forward's
    # work list, ordered by each item's keys over all ring steps, starts with
    # the long sequence's last query tiles
    ("mixed-cp2-d128", [2048] + [64] * 40, [2048] + [64] * 40, 2, 2, 2, 128),
]


def _check_fwd(bt, cp, ranks, tail=0, cup="copy"):
    db = H.DeviceBatch(bt)
    scale = 1.0 / math.sqrt(bt.d)
    for r in ranks:
        H.log(f"[fwd] {bt.name} cp={cp} rank={r} hq={bt.hq} hkv={bt.hkv} d={bt.d} tail={tail}")
        meta, loc = H.local_inputs(db, cp, r, tail=tail, cup=cup)
        out, lse = H.run_fwd(meta, loc, bt, scale)
        ref = O.share(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale, want_grad=False)
        sd = O.share_rounding_sd(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale)
        tl = loc["t_local"]
        ob = H.bf16_to_np(out)
        start = len(H.BAR_LOG)
        st = H.compare_bf16("out", ob[:tl], ref["out"], sd=sd["out"])
        H.annotate_ideal(start, bt, cp, r, scale, {"out": (ref["out"], "out", None)})
        lt = lse.cpu().numpy()
        sl = H.compare_lse("lse", lt[:, :tl], ref["lse"])
        rows = O.shard_rows(bt.cu, bt.cup, cp, r)
        pad = ~O.valid_mask(bt.cu, bt.cup)[rows]
        assert not ob[:tl][pad].any(), "padding rows of out must be 0"
        if tail:  # rows past T_local untouched
            assert (H.bf16_bits_to_f64(ob[tl:]) == 7.0).all()
            assert (lt[:, tl:] == 7.0).all()
        H.log(f"    out {st}  lse {sl}")
        meta.close()


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_fwd_small(case):
    name, L, P, cp, hq, hkv, d = case
    bt = synth.make_batch(name, 17, L, P, hq, hkv, d)
    _check_fwd(bt, cp, range(cp), tail=5)


def test_fwd_cfg1_both_ranks():
    bt, w = synth.make_workload(1)
    _check_fwd(bt, w["cp"], w["ranks"])


@pytest.mark.parametrize("cup", ["alias", "null"])
def test_fwd_cfg1_alias_and_null(cup):
    bt, w = synth.make_workload(1)
    _check_fwd(bt, w["cp"], [1], cup=cup)


def test_fwd_cfg2():
    bt, w = synth.make_workload(2)
    _check_fwd(bt, w["cp"], w["ranks"])


def test_fwd_cfg3_all_ranks():
    bt, w = synth.make_workload(3)
    _check_fwd(bt, w["cp"], range(w["cp"]))
