"""All-gather share on the GPU (cp_attn_ag_fwd / cp_attn_ag_bwd): the rank's
queries against the gathered K/V, and its contribution to the gradient of
every gathered key row ("Hybrid / Hierarchical Context Parallel Skill",
Implementation Map: the "all_gather" communication type).

* out / LSE / dQ are bit-identical to the ring share's, and each shard's rows
  of the gathered dK / dV are bit-identical to the ring share's part for that
  shard (same kernels, same data);
* the gathered dK / dV match the fp64 oracle to the bf16 bar, every row
  [0, cu_seqlens_padded[B]) is written (no garbage left), and rows past it
  are untouched.
"""
import math

import numpy as np
import pytest

from context_packed_attention_amd import api, synth
from oracle import cp_attn_oracle as O
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

CASES = [
    ("ag-ragged-cp2-d64", [257, 31, 640, 8], [264, 32, 640, 8], 2, 4, 2, 64, 0),
    ("ag-ragged-cp3-d128-gqa", [600, 1, 250, 0], [600, 12, 252, 6], 3, 8, 2, 128, 37),
    ("ag-tiny-cp4-d64-pad", [5, 9, 1], [8, 16, 8], 4, 2, 2, 64, 0),
    ("ag-long-cp4-d128", [1800, 500], [1808, 504], 4, 4, 4, 128, 0),
    ("ag-cp1-d128", [300, 77], [304, 80], 1, 2, 1, 128, 5),
]


def _run_ag(meta, db, loc, bt, scale, extra_rows=16):
    import torch
    t_alloc = loc["t_alloc"]
    T = bt.total_rows
    out = torch.full((t_alloc, bt.hq, bt.d), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((bt.hq, t_alloc), 7.0, dtype=torch.float32, device="cuda")
    wsf = torch.empty(api.cp_attn_ag_workspace_bytes(meta, bt.hq, bt.hkv, bt.d, 0), dtype=torch.uint8, device="cuda")
    api.cp_attn_ag_fwd(meta, loc["q"], db.k, db.v, bt.hq, bt.hkv, bt.d, scale, 1, out, lse, wsf)
    dq = torch.full((t_alloc, bt.hq, bt.d), 5.0, dtype=torch.bfloat16, device="cuda")
    dk = torch.full((T + extra_rows, bt.hkv, bt.d), 5.0, dtype=torch.bfloat16, device="cuda")
    dv = torch.full((T + extra_rows, bt.hkv, bt.d), 5.0, dtype=torch.bfloat16, device="cuda")
    wsb = torch.empty(api.cp_attn_ag_workspace_bytes(meta, bt.hq, bt.hkv, bt.d, 1), dtype=torch.uint8, device="cuda")
    api.cp_attn_ag_bwd(meta, loc["q"], db.k, db.v, out, lse, loc["do"], bt.hq, bt.hkv, bt.d, scale, 1, dq, dk, dv,
                       wsb)
    return out, lse, dq, dk, dv


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ag_share(case):
    import torch
    name, L, P, cp, hq, hkv, d, tail = case
    bt = synth.make_batch(name, 29, L, P, hq, hkv, d)
    scale = 1.0 / math.sqrt(d)
    db = H.DeviceBatch(bt)
    T = bt.total_rows
    for r in range(cp):
        H.log(f"[ag] {name} cp={cp} rank={r} tail={tail}")
        meta, loc = H.local_inputs(db, cp, r, tail=tail)
        tl = loc["t_local"]
        out, lse = H.run_fwd(meta, loc, bt, scale)
        dq, dks, dvs = H.run_bwd(meta, loc, bt, scale, out, lse)
        a_out, a_lse, a_dq, a_dk, a_dv = _run_ag(meta, db, loc, bt, scale)
        torch.cuda.synchronize()
        assert torch.equal(a_out[:tl].view(torch.int16), out[:tl].view(torch.int16))
        assert torch.equal(a_lse[:, :tl], lse[:, :tl])
        assert torch.equal(a_dq.view(torch.int16), dq.view(torch.int16))
        dkf = H.bf16_to_np(a_dk)
        dvf = H.bf16_to_np(a_dv)
        for s in range(cp):
            rows = O.shard_rows(bt.cu, bt.cup, cp, s)
            assert np.array_equal(dkf[rows], H.bf16_to_np(dks[s])[:tl]), f"dk rows of shard {s}"
            assert np.array_equal(dvf[rows], H.bf16_to_np(dvs[s])[:tl]), f"dv rows of shard {s}"
        five = np.uint16(0x40A0)  # bf16 5.0: the fill past the gathered rows
        assert (dkf[T:] == five).all() and (dvf[T:] == five).all(), "rows past the gathered tensor must be untouched"
        ref = O.share(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale, want_grad=True)
        sd = O.share_rounding_sd(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale)
        a = H.compare_bf16("dk_full", dkf[:T], ref["dk_full"], sd=sd["dk_full"])
        b = H.compare_bf16("dv_full", dvf[:T], ref["dv_full"], sd=sd["dv_full"])
        zero = np.all(ref["dk_full"] == 0, axis=(1, 2)) & np.all(ref["dv_full"] == 0, axis=(1, 2))
        assert not dkf[:T][zero].any() and not dvf[:T][zero].any(), "unreached and padding key rows must be 0"
        H.log(f"    dk_full {a['max_abs']:.2e}/{a['rel_l2']:.2e} dv_full {b['max_abs']:.2e}/{b['rel_l2']:.2e}")
        meta.close()


def test_ag_argument_errors():
    import torch
    bt = synth.make_batch("ag-err", 3, [64], [64], 2, 2, 64)
    db = H.DeviceBatch(bt)
    meta, loc = H.local_inputs(db, 2, 0)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    out = torch.empty((loc["t_alloc"], 2, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((2, loc["t_alloc"]), dtype=torch.float32, device="cuda")
    with pytest.raises(api.CpAttnError) as e:
        api.cp_attn_ag_fwd(meta, loc["q"], db.k, db.v, 2, 2, 64, 0.125, 1, out, lse, small)
    assert e.value.status == 4  # workspace too small
    ws = torch.empty(api.cp_attn_ag_workspace_bytes(meta, 2, 2, 64, 0), dtype=torch.uint8, device="cuda")
    n = db.k.numel()
    buf = torch.empty(n + 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(api.CpAttnError):
        api.cp_attn_ag_fwd(meta, loc["q"], buf[1:1 + n], db.v, 2, 2, 64, 0.125, 1, out, lse, ws)  # misaligned K
    with pytest.raises(ValueError):
        api.cp_attn_ag_fwd(meta, loc["q"], db.k[:-1], db.v, 2, 2, 64, 0.125, 1, out, lse, ws)  # K too short
    meta.close()


def test_ag_graph_capture_replays():
    """The all-gather calls only launch kernels: captured into a HIP graph
    (torch's stream capture) every replay equals the eager result bit for bit,
    with eager work between replays."""
    import torch
    bt = synth.make_batch("ag-graph", 41, [700, 333, 64], [704, 336, 64], 4, 2, 128)
    cp, r = 2, 1
    scale = 1.0 / math.sqrt(bt.d)
    db = H.DeviceBatch(bt)
    meta, loc = H.local_inputs(db, cp, r)
    ref = _run_ag(meta, db, loc, bt, scale, extra_rows=0)
    torch.cuda.synchronize()
    t_alloc, T = loc["t_alloc"], bt.total_rows
    out = torch.zeros_like(ref[0])
    lse = torch.zeros_like(ref[1])
    dq = torch.zeros_like(ref[2])
    dk = torch.zeros((T, bt.hkv, bt.d), dtype=torch.bfloat16, device="cuda")
    dv = torch.zeros_like(dk)
    wsf = torch.empty(api.cp_attn_ag_workspace_bytes(meta, bt.hq, bt.hkv, bt.d, 0), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(api.cp_attn_ag_workspace_bytes(meta, bt.hq, bt.hkv, bt.d, 1), dtype=torch.uint8, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            api.cp_attn_ag_fwd(meta, loc["q"], db.k, db.v, bt.hq, bt.hkv, bt.d, scale, 1, out, lse, wsf, stream=s)
            api.cp_attn_ag_bwd(meta, loc["q"], db.k, db.v, out, lse, loc["do"], bt.hq, bt.hkv, bt.d, scale, 1, dq, dk,
                               dv, wsb, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    tl = loc["t_local"]
    for rep in range(3):
        for t in (out, lse, dq, dk, dv):
            t.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out[:tl].view(torch.int16), ref[0][:tl].view(torch.int16)), rep
        assert torch.equal(lse[:, :tl], ref[1][:, :tl]), rep
        assert torch.equal(dq.view(torch.int16), ref[2].view(torch.int16)), rep
        assert torch.equal(dk.view(torch.int16), ref[3].view(torch.int16)), rep
        assert torch.equal(dv.view(torch.int16), ref[4].view(torch.int16)), rep
        H.log(f"[ag graph] replay {rep} matches")
    del g
    meta.close()
