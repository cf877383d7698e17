"""The hierarchical front end's all-to-all on the GPU (cp_attn_a2a_*):

* bit-exact against the oracle's permutation, both directions, for several
  (a2a, p2p) sizes and ragged / padded / empty-sequence packs, with garbage
  in rows the call must not read or write past;
* a whole hierarchical share ("Hybrid / Hierarchical Context Parallel Skill",
  "Enablement"; [a2a, p2p] = [2, 2], GQA): CP-level shards -> all-to-all ->
  the p2p-level share's forward and backward on each head group -> the
  inverse all-to-all. Out, LSE and dQ match the oracle's p2p-level share of
  that head group, and the dQ brought back matches the oracle's CP-level dQ
  of every CP rank (all heads)."""
import math

import numpy as np
import pytest

from context_packed_attention_amd import api, synth
from oracle import cp_attn_oracle as O
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _dev16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda")


def _host16(t):
    return t.cpu().numpy().view(np.uint16)


def _pack(rng, B, cp, max_mult):
    P = [2 * cp * int(rng.integers(0, max_mult + 1)) for _ in range(B)]
    L = [int(rng.integers(0, p + 1)) for p in P]
    return np.concatenate([[0], np.cumsum(L)]).astype(np.int32), np.concatenate([[0], np.cumsum(P)]).astype(np.int32)


@pytest.mark.parametrize("A,P,d", [(2, 1, 128), (2, 2, 128), (4, 2, 64), (4, 1, 128), (2, 4, 64), (8, 2, 128)])
def test_a2a_bit_exact(A, P, d):
    import torch
    rng = np.random.default_rng(1000 * A + 10 * P + d)
    cp = A * P
    heads = 2 * A
    for trial in range(2):
        cu, cup = _pack(rng, int(rng.integers(1, 8)), cp, 12)
        T = int(cup[-1])
        tl = T // cp
        X = rng.integers(0, 1 << 16, size=(T, heads, d), dtype=np.uint32).astype(np.uint16)
        m = api.cp_attn_rank_metadata(H.dev_i32(cu), H.dev_i32(cup), cp, 0, -1, tl + 3)
        H.log(f"[a2a] A={A} P={P} d={d} B={len(cu) - 1} T_local={tl}")
        for p in range(P):
            xs = [O.gather_shard(X, cu, cup, cp, p * A + a) for a in range(A)]
            ins = []
            for x in xs:
                t = torch.full((tl + 3, heads, d), 0x7bc0, dtype=torch.int16, device="cuda")
                t[:tl] = _dev16(x)
                ins.append(t)
            outs = [torch.full((A * tl + 2, heads // A, d), 0x1234, dtype=torch.int16, device="cuda") for _ in range(A)]
            api.cp_attn_a2a_seq_to_head(m, A, p, heads, d * 2, ins, outs)
            torch.cuda.synchronize()
            ref = O.a2a_seq_to_head(xs, cup, cp, A, p)
            for a in range(A):
                got = _host16(outs[a])
                assert np.array_equal(got[:A * tl], ref[a]), (p, a)
                assert (got[A * tl:] == 0x1234).all(), "rows past A * T_local must be untouched"
            backs = [torch.full((tl + 3, heads, d), 0x4321, dtype=torch.int16, device="cuda") for _ in range(A)]
            api.cp_attn_a2a_head_to_seq(m, A, p, heads, d * 2, outs, backs)
            torch.cuda.synchronize()
            inv = O.a2a_head_to_seq(ref, cup, cp, A, p)
            for a in range(A):
                got = _host16(backs[a])
                assert np.array_equal(got[:tl], xs[a]) and np.array_equal(got[:tl], inv[a]), (p, a)
                assert (got[tl:] == 0x4321).all(), "rows past T_local must be untouched"
        m.close()


def test_hierarchical_share_end_to_end():
    import torch
    A, P = 2, 2
    cp = A * P
    hq, hkv, d = 8, 4, 128
    L = [600, 200, 0, 1000]
    Pd = [608, 200, 8, 1000]
    bt = synth.make_batch("hier-a2a2-p2p2", 41, L, Pd, hq, hkv, d)
    scale = 1.0 / math.sqrt(d)
    db = H.DeviceBatch(bt)
    T = int(bt.cup[-1])
    tl_cp, tl_p = T // cp, T // P
    m_cp = api.cp_attn_rank_metadata(db.cu, db.cup, cp, 0, -1, tl_cp)

    def cp_shard(src, h, c):
        dst = torch.zeros((tl_cp, h, d), dtype=torch.bfloat16, device="cuda")
        api.cp_attn_shard_gather(m_cp, c, src, dst, h * d * 2)
        return dst

    # head-split p2p-level tensors: split[name][p][a'] = [tl_p, h/A, d]
    split = {}
    for name, src, h in (("q", db.q, hq), ("k", db.k, hkv), ("v", db.v, hkv), ("do", db.do, hq)):
        split[name] = []
        for p in range(P):
            ins = [cp_shard(src, h, p * A + a) for a in range(A)]
            outs = [torch.empty((A * tl_cp, h // A, d), dtype=torch.bfloat16, device="cuda") for _ in range(A)]
            api.cp_attn_a2a_seq_to_head(m_cp, A, p, h, d * 2, ins, outs)
            split[name].append(outs)
    torch.cuda.synchronize()
    hq_l, hkv_l = hq // A, hkv // A
    for p in range(P):
        m_p = api.cp_attn_rank_metadata(db.cu, db.cup, P, p, -1, tl_p)
        dq_heads = []
        for a in range(A):
            H.log(f"[hier] p2p rank {p} head group {a}")
            loc = {"q": split["q"][p][a], "do": split["do"][p][a], "k": [split["k"][s][a] for s in range(P)],
                   "v": [split["v"][s][a] for s in range(P)], "t_alloc": tl_p, "t_local": tl_p}
            sub = synth.PackedBatch(name="sub", seed=bt.seed, cu=bt.cu, cup=bt.cup, hq=hq_l, hkv=hkv_l, d=d,
                                    q=bt.q[:, a * hq_l:(a + 1) * hq_l], k=bt.k[:, a * hkv_l:(a + 1) * hkv_l],
                                    v=bt.v[:, a * hkv_l:(a + 1) * hkv_l], do=bt.do[:, a * hq_l:(a + 1) * hq_l])
            out, lse = H.run_fwd(m_p, loc, sub, scale)
            dq, dks, dvs = H.run_bwd(m_p, loc, sub, scale, out, lse)
            ref = O.share(sub.q, sub.k, sub.v, sub.do, bt.cu, bt.cup, P, p, scale, want_grad=True)
            H.compare_bf16("out", H.bf16_to_np(out), ref["out"])
            H.compare_lse("lse", lse.cpu().numpy(), ref["lse"])
            H.compare_bf16("dq", H.bf16_to_np(dq), ref["dq"])
            dq_heads.append(dq)
        # dQ back to the sequence split: CP ranks p*A + a, all heads
        backs = [torch.empty((tl_cp, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(A)]
        api.cp_attn_a2a_head_to_seq(m_cp, A, p, hq, d * 2, dq_heads, backs)
        torch.cuda.synchronize()
        for a in range(A):
            c = p * A + a
            ref_c = O.share(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, c, scale, want_grad=True)
            st = H.compare_bf16(f"dq cp rank {c}", H.bf16_to_np(backs[a]), ref_c["dq"])
            H.log(f"    CP rank {c} dq {st['max_abs']:.2e} / {st['rel_l2']:.2e}")
        m_p.close()
    m_cp.close()


def test_hierarchical_step_full_pack_sampled():
    """The whole a2a+p2p step of a2a group 0 on the 64K hierarchical pack
    (the benchmark's --hier workload: [2, 2], 32 heads before the split),
    end to end through both all-to-alls; sampled rows of the CP-level out,
    LSE and dQ of CP ranks 0 and 1, and the CP-level dK / dV of late key rows
    of their own shards (the contribution of the group's queries), against
    the oracle's CP = 4 shares."""
    import torch
    A, P = 2, 2
    cp = A * P
    w = synth.workload(5)
    L = w["lengths"]
    H_, d = 2 * w["hq"], w["d"]
    hs = H_ // A
    bt = synth.make_batch("pack64k-hier-32heads", 1005, L, L, H_, H_, d)
    scale = 1.0 / math.sqrt(d)
    db = H.DeviceBatch(bt)
    T = int(bt.cup[-1])
    tl_cp, tl_p = T // cp, T // P
    m_cp = api.cp_attn_rank_metadata(db.cu, db.cup, cp, 0, -1, tl_cp)

    def cp_shard(src, c):
        dst = torch.zeros((tl_cp, H_, d), dtype=torch.bfloat16, device="cuda")
        api.cp_attn_shard_gather(m_cp, c, src, dst, H_ * d * 2)
        return dst

    def split(src, p):
        outs = [torch.empty((tl_p, hs, d), dtype=torch.bfloat16, device="cuda") for _ in range(A)]
        api.cp_attn_a2a_seq_to_head(m_cp, A, p, H_, d * 2, [cp_shard(src, p * A + a) for a in range(A)], outs)
        return outs

    H.log("[hier-full] all-to-all of Q, K, V, dO")
    q_h, do_h = split(db.q, 0), split(db.do, 0)
    k_h = [split(db.k, p) for p in range(P)]
    v_h = [split(db.v, p) for p in range(P)]
    m_p = api.cp_attn_rank_metadata(db.cu, db.cup, P, 0, -1, tl_p)
    outs, lses, dqs, dks, dvs = [], [], [], [], []
    for a in range(A):
        H.log(f"[hier-full] p2p share of head group {a}")
        loc = {"q": q_h[a], "do": do_h[a], "k": [k_h[s][a] for s in range(P)], "v": [v_h[s][a] for s in range(P)],
               "t_alloc": tl_p, "t_local": tl_p}
        sub = synth.PackedBatch(name="sub", seed=0, cu=bt.cu, cup=bt.cup, hq=hs, hkv=hs, d=d, q=None, k=None,
                                v=None, do=None)
        out, lse = H.run_fwd(m_p, loc, sub, scale)
        dq, dk, dv = H.run_bwd(m_p, loc, sub, scale, out, lse)
        outs.append(out)
        lses.append(lse)
        dqs.append(dq)
        dks.append(dk[0])
        dvs.append(dv[0])
    back = {}
    for name, src in (("out", outs), ("dq", dqs), ("dk", dks), ("dv", dvs)):
        back[name] = [torch.empty((tl_cp, H_, d), dtype=torch.bfloat16, device="cuda") for _ in range(A)]
        api.cp_attn_a2a_head_to_seq(m_cp, A, 0, H_, d * 2, src, back[name])
    torch.cuda.synchronize()
    # LSE back to the sequence split by the oracle's own permutation of
    # [rows, heads] arrays (the LSE planes are [heads, rows] on the device)
    lse_cp = O.a2a_head_to_seq([l.cpu().numpy().T.copy() for l in lses], bt.cup, cp, A, 0)
    rng = np.random.default_rng(5)
    heads = [0, 7, 16, 31]
    for a in range(A):
        c = a  # CP rank of group 0, a2a rank a
        rows = np.unique(np.concatenate([[0, 1, tl_cp // 2, tl_cp - 1], rng.integers(0, tl_cp, 12)]))
        H.log(f"[hier-full] CP rank {c}: oracle on {rows.size} rows x {len(heads)} heads")
        o, l, dq = O.share_rows(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, c, scale, rows, heads, want_dq=True)
        H.compare_bf16(f"out cp{c}", H.bf16_to_np(back["out"][a])[rows][:, heads], o)
        H.compare_lse(f"lse cp{c}", lse_cp[a][rows][:, heads].T, l)
        H.compare_bf16(f"dq cp{c}", H.bf16_to_np(back["dq"][a])[rows][:, heads], dq)
        # the own shard's dK / dV: both CP ranks' queries of the group contribute
        keys = np.arange(tl_cp - 3, tl_cp)
        kvh = [3, 30]
        ref_k = ref_v = 0
        for r in range(A):
            k_, v_ = O.share_keys_dkdv(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale, c, keys, kvh)
            ref_k, ref_v = ref_k + k_, ref_v + v_
        H.compare_bf16(f"dk cp{c}", H.bf16_to_np(back["dk"][a])[keys][:, kvh], ref_k)
        H.compare_bf16(f"dv cp{c}", H.bf16_to_np(back["dv"][a])[keys][:, kvh], ref_v)
    m_p.close()
    m_cp.close()
