"""Backward of a rank's share on the GPU vs the fp64 oracle: dQ and every
dK/dV part within max-abs 2e-2 and relative L2 1e-2; padding rows and rows
outside a step's key range exactly 0; the gradient tail [T_local, t_alloc)
zeroed only when it exists."""
import math

import numpy as np
import pytest

from context_packed_attention_amd import synth
from oracle import cp_attn_oracle as O
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

SMALL = [
    ("one-seq-cp1-d128", [300], [304], 1, 2, 1, 128),
    ("ragged-cp2-d64", [257, 31, 640, 8], [264, 32, 640, 8], 2, 4, 2, 64),
    ("ragged-cp3-d128-gqa", [600, 1, 250, 0], [600, 12, 252, 6], 3, 8, 2, 128),
    ("long-cp4-d128", [1800, 500], [1808, 504], 4, 4, 4, 128),
    ("tiny-cp4-d64-pad", [5, 9, 1], [8, 16, 8], 4, 2, 2, 64),
]


def _check_bwd(bt, cp, ranks, tail=0):
    db = H.DeviceBatch(bt)
    scale = 1.0 / math.sqrt(bt.d)
    for r in ranks:
        H.log(f"[bwd] {bt.name} cp={cp} rank={r} hq={bt.hq} hkv={bt.hkv} d={bt.d} tail={tail}")
        meta, loc = H.local_inputs(db, cp, r, tail=tail)
        out, lse = H.run_fwd(meta, loc, bt, scale)
        dq, dks, dvs = H.run_bwd(meta, loc, bt, scale, out, lse)
        ref = O.share(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale, want_grad=True)
        sd = O.share_rounding_sd(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale)
        tl = loc["t_local"]
        start = len(H.BAR_LOG)
        H.compare_bf16("out", H.bf16_to_np(out)[:tl], ref["out"], sd=sd["out"])
        dqb = H.bf16_to_np(dq)
        st = H.compare_bf16("dq", dqb[:tl], ref["dq"], sd=sd["dq"])
        rows_r = O.shard_rows(bt.cu, bt.cup, cp, r)
        pad_r = ~O.valid_mask(bt.cu, bt.cup)[rows_r]
        assert not dqb[:tl][pad_r].any(), "dq padding rows must be exactly 0"
        for s in range(cp):
            dkb = H.bf16_to_np(dks[s])
            dvb = H.bf16_to_np(dvs[s])
            a = H.compare_bf16(f"dk[{s}]", dkb[:tl], ref["dk_parts"][s], sd=sd["dk_parts"][s])
            b = H.compare_bf16(f"dv[{s}]", dvb[:tl], ref["dv_parts"][s], sd=sd["dv_parts"][s])
            zero_rows = np.all(ref["dk_parts"][s] == 0, axis=(1, 2)) & np.all(ref["dv_parts"][s] == 0, axis=(1, 2))
            assert not dkb[:tl][zero_rows].any() and not dvb[:tl][zero_rows].any(), \
                f"part {s}: rows no query of this rank reaches must be exactly 0"
            H.log(f"    part {s}: dk {a['max_abs']:.2e}/{a['rel_l2']:.2e} dv {b['max_abs']:.2e}/{b['rel_l2']:.2e}")
            if tail:
                assert not dkb[tl:].any() and not dvb[tl:].any()
        if tail:
            assert not dqb[tl:].any(), "dq tail rows must be zeroed"
        H.log(f"    dq {st}")
        refs = {"out": (ref["out"], "out", None), "dq": (ref["dq"], "dq", None)}
        for s in range(cp):
            refs[f"dk[{s}]"] = (ref["dk_parts"][s], "dk_parts", s)
            refs[f"dv[{s}]"] = (ref["dv_parts"][s], "dv_parts", s)
        H.annotate_ideal(start, bt, cp, r, scale, refs)
        meta.close()


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_bwd_small(case):
    name, L, P, cp, hq, hkv, d = case
    bt = synth.make_batch(name, 23, L, P, hq, hkv, d)
    _check_bwd(bt, cp, range(cp), tail=37)


def test_bwd_cfg1_both_ranks():
    bt, w = synth.make_workload(1)
    _check_bwd(bt, w["cp"], w["ranks"])


def test_bwd_cfg2():
    bt, w = synth.make_workload(2)
    _check_bwd(bt, w["cp"], w["ranks"])


def test_bwd_cfg3_all_ranks():
    bt, w = synth.make_workload(3)
    _check_bwd(bt, w["cp"], range(w["cp"]))
