"""HIP-graph capture of a rank share (cp_attn_graph_*): the metadata is built
once, the forward and backward launches are captured, and every replay must
equal the eager calls bit for bit (the kernels are deterministic: no atomics,
fixed reduction order). Replays are checked one by one with eager work and
synchronisations between them, again after the inputs change in place, and
the graph must hold exactly the eager launch sequence ("[PyTorch][Attention]
THD P2P context-parallel regression ...", "Expected behavior": padding
metadata that is safe under graph capture). The first replay and the replay
after the inputs change are also compared with the fp64 oracle (all heads of
the tiny pack; two KV heads and their query-head groups of the larger packs,
whose heads are independent problems)."""
import copy
import math

import numpy as np
import pytest

from context_packed_attention_amd import api, synth
from oracle import cp_attn_oracle as O
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _same(name, a, b):
    import torch
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b), f"{name} differs from the eager result"


def _sub_heads(bt, kv_heads):
    """The batch restricted to some KV heads and their query-head groups."""
    group = bt.hq // bt.hkv
    qh = [g * group + j for g in kv_heads for j in range(group)]
    sub = copy.copy(bt)
    sub.q, sub.do = bt.q[:, qh], bt.do[:, qh]
    sub.k, sub.v = bt.k[:, kv_heads], bt.v[:, kv_heads]
    sub.hq, sub.hkv = len(qh), len(kv_heads)
    return sub, qh


def _vs_oracle(tag, bt, cp, rank, scale, tl, res):
    out, lse, dq, dks, dvs = res
    kv_heads = list(range(bt.hkv)) if bt.hkv * (bt.hq // bt.hkv) <= 4 else sorted({0, bt.hkv - 1})
    sub, qh = _sub_heads(bt, kv_heads)
    H.log(f"[graph] {tag}: oracle on kv heads {kv_heads}")
    ref = O.share(sub.q, sub.k, sub.v, sub.do, sub.cu, sub.cup, cp, rank, scale)
    sd = O.share_rounding_sd(sub.q, sub.k, sub.v, sub.do, sub.cu, sub.cup, cp, rank, scale)
    H.compare_bf16(f"{tag} out", H.bf16_to_np(out)[:tl][:, qh], ref["out"], sd=sd["out"])
    H.compare_lse(f"{tag} lse", lse.cpu().numpy()[qh][:, :tl], ref["lse"])
    H.compare_bf16(f"{tag} dq", H.bf16_to_np(dq)[:tl][:, qh], ref["dq"], sd=sd["dq"])
    for s in range(cp):
        H.compare_bf16(f"{tag} dk[{s}]", H.bf16_to_np(dks[s])[:tl][:, kv_heads], ref["dk_parts"][s],
                       sd=sd["dk_parts"][s])
        H.compare_bf16(f"{tag} dv[{s}]", H.bf16_to_np(dvs[s])[:tl][:, kv_heads], ref["dv_parts"][s],
                       sd=sd["dv_parts"][s])


# the padded pack of test_gpu_inorder: long enough for the in-order launch plan
INORDER = ([3000, 1500, 3800, 5], [3008, 1600, 3804, 8], 2, 64, 8, 64)


@pytest.mark.parametrize("cfg,rank,tail", [(2, 1, 0), (3, 0, 0), (1, 1, 37), ("inorder", 1, 0)])
def test_graph_replays_match_eager(cfg, rank, tail):
    import torch
    if cfg == "inorder":
        L, P, cp, hq, hkv, d = INORDER
        bt = synth.make_batch("inorder-padded", 17, L, P, hq, hkv, d)
    else:
        bt, w = synth.make_workload(cfg)
        cp = w["cp"]
    H.log(f"[graph] cfg{cfg} rank {rank} tail {tail}")
    db = H.DeviceBatch(bt)
    meta, loc = H.local_inputs(db, cp, rank, tail=tail)
    scale = 1.0 / math.sqrt(bt.d)
    tl = loc["t_local"]

    def eager():
        torch.cuda.synchronize()
        api.cp_attn_timing_enable(True)
        out, lse = H.run_fwd(meta, loc, bt, scale)
        dq, dks, dvs = H.run_bwd(meta, loc, bt, scale, out, lse)
        torch.cuda.synchronize()
        api.cp_attn_timing_enable(False)
        n = sum(v[1] for v in api.cp_attn_timing_read().values())
        return (out, lse, dq, dks, dvs), n

    ref, n_eager = eager()
    out = torch.full_like(ref[0], 3.0)
    lse = torch.full_like(ref[1], 3.0)
    dq = torch.full_like(ref[2], 3.0)
    dks = [torch.full_like(x, 3.0) for x in ref[3]]
    dvs = [torch.full_like(x, 3.0) for x in ref[4]]
    wsf = torch.empty(api.cp_attn_workspace_bytes(meta, bt.hq, bt.hkv, bt.d, 0), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(api.cp_attn_workspace_bytes(meta, bt.hq, bt.hkv, bt.d, 1), dtype=torch.uint8, device="cuda")
    g = api.cp_attn_graph_capture(meta, 3, loc["q"], loc["k"], loc["v"], bt.hq, bt.hkv, bt.d, scale, 1, out, lse,
                                  loc["do"], dq, dks, dvs, wsf, wsb)
    H.log(f"[graph] {g.kernels} kernels captured, {n_eager} eager launches")
    assert g.kernels == n_eager

    def check(r):
        _same("out", out[:tl], r[0][:tl])
        _same("lse", lse[:, :tl], r[1][:, :tl])
        _same("dq", dq, r[2])
        for s in range(cp):
            _same(f"dk[{s}]", dks[s], r[3][s])
            _same(f"dv[{s}]", dvs[s], r[4][s])

    for rep in range(3):
        for t in [out, lse, dq, *dks, *dvs]:
            t.fill_(5.0)  # eager work between replays
        torch.cuda.synchronize()
        g.launch()
        torch.cuda.synchronize()
        check(ref)
        H.log(f"[graph] replay {rep} matches")
        if rep == 0:
            _vs_oracle("replay 0", bt, cp, rank, scale, tl, (out, lse, dq, dks, dvs))
    # the graph reads its inputs' current contents
    loc["q"].mul_(0.5)
    loc["do"].mul_(-1.0)
    ref2, _ = eager()
    g.launch()
    torch.cuda.synchronize()
    check(ref2)
    assert not torch.equal(ref2[2].view(torch.int16), ref[2].view(torch.int16))
    # the oracle on the changed inputs (halving and negating are exact in bf16)
    bt2 = copy.copy(bt)
    bt2.q = synth.f32_to_bf16_bits((O.bf16_to_f64(bt.q) * 0.5).astype(np.float32))
    bt2.do = bt.do ^ np.uint16(0x8000)
    _vs_oracle("changed inputs", bt2, cp, rank, scale, tl, (out, lse, dq, dks, dvs))
    g.close()
    meta.close()


def test_graph_capture_rejects_bad_arguments():
    import torch
    bt, w = synth.make_workload(1)
    db = H.DeviceBatch(bt)
    meta, loc = H.local_inputs(db, 2, 0)
    out = torch.empty((loc["t_alloc"], bt.hq, bt.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((bt.hq, loc["t_alloc"]), dtype=torch.float32, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(api.CpAttnError) as e:
        api.cp_attn_graph_capture(meta, 1, loc["q"], loc["k"], loc["v"], bt.hq, bt.hkv, bt.d, 0.125, 1, out, lse,
                                  ws_fwd=small)
    assert e.value.status == 4  # workspace too small, found while capturing; no graph is left
    with pytest.raises(api.CpAttnError):
        api.cp_attn_graph_capture(meta, 4, loc["q"], loc["k"], loc["v"], bt.hq, bt.hkv, bt.d, 0.125, 1, out, lse)
    # the device still works after a failed capture
    o2, l2 = H.run_fwd(meta, loc, bt, 0.125)
    torch.cuda.synchronize()
    assert torch.isfinite(o2.float()).all()
    meta.close()
