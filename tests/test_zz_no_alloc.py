"""The allocation-free backward (cp_attn_bwd_noalloc: its per-row scratch in
a fixed device array instead of a caller's workspace) against cp_attn_bwd on
the same inputs: bit for bit (the same kernels in the same order), on two
calls in a row, the second on a smaller share, into garbage-prefilled
outputs; and a share whose scratch would not fit is refused before any
launch."""
import math

import numpy as np
import pytest

from context_packed_attention_amd import api, synth
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _pair(bt, cp, r, tail):
    import torch
    db = H.DeviceBatch(bt)
    meta, loc = H.local_inputs(db, cp, r, tail=tail)
    scale = 1.0 / math.sqrt(bt.d)
    H.log(f"[noalloc] {bt.name} cp={cp} rank={r} hq={bt.hq} tail={tail}")
    out, lse = H.run_fwd(meta, loc, bt, scale)
    dq_a, dks_a, dvs_a = H.run_bwd(meta, loc, bt, scale, out, lse)
    dq_b = torch.full_like(dq_a, 9.0)
    dks_b = [torch.full_like(x, -3.0) for x in dks_a]
    dvs_b = [torch.full_like(x, 11.0) for x in dvs_a]
    api.cp_attn_bwd_noalloc(meta, loc["q"], loc["k"], loc["v"], out, lse, loc["do"], bt.hq, bt.hkv, bt.d, scale, 1,
                            dq_b, dks_b, dvs_b)
    torch.cuda.synchronize()
    same = lambda a, b: torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert same(dq_a, dq_b), "dq differs"
    for s in range(cp):
        assert same(dks_a[s], dks_b[s]) and same(dvs_a[s], dvs_b[s]), f"part {s} differs"
    meta.close()


def test_matches_workspace_backward_twice_second_smaller():
    bt, w = synth.make_workload(2)      # 16K pack, CP = 4, rank 1, 32 heads
    _pair(bt, w["cp"], 1, tail=0)
    bt1, w1 = synth.make_workload(1)    # the tiny pack, CP = 2: a smaller share next
    _pair(bt1, w1["cp"], 0, tail=5)


def test_oversize_share_refused():
    import torch
    cp, hq, hkv, d = 2, 64, 8, 128
    T = 2 * 131072
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    meta = api.cp_attn_rank_metadata(cu, None, cp, 0, -1, T // cp)
    tl = T // cp
    assert 8 * hq * tl > 32 << 20
    e = lambda h: torch.empty((tl, h, d), dtype=torch.bfloat16, device="cuda")
    q, out, do, dq = e(hq), e(hq), e(hq), e(hq)
    lse = torch.empty((hq, tl), dtype=torch.float32, device="cuda")
    ks, vs = [e(hkv) for _ in range(cp)], [e(hkv) for _ in range(cp)]
    dks, dvs = [e(hkv) for _ in range(cp)], [e(hkv) for _ in range(cp)]
    with pytest.raises(api.CpAttnError) as err:
        api.cp_attn_bwd_noalloc(meta, q, ks, vs, out, lse, do, hq, hkv, d, 0.0884, 1, dq, dks, dvs)
    assert err.value.status == 4 and "allocation-free" in str(err.value)
    meta.close()
