"""A share whose local tensors reach 2 GiB: one 262144-token sequence, CP = 2,
rank 0, 64 query heads and 8 KV heads of 128 (the local Q, dO, out and dQ are
2 GiB each, the forward workspace 8 GiB). The tile copies address every
tensor through buffer resources rebased on each tile in 64-bit arithmetic.
Inputs are drawn on the device from fixed seeds and copied to the host only
where the oracle reads them: out / LSE / dQ on sampled rows, and exact dK / dV
on the last key rows of the rank's own shard (only the sequence's last
queries reach them)."""
import math

import numpy as np
import pytest

from context_packed_attention_amd import api, synth
from oracle import cp_attn_oracle as O
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_share_past_2gib():
    import torch
    T, cp, r, hq, hkv, d = 262144, 2, 0, 64, 8, 128
    tl = T // cp
    scale = 1.0 / math.sqrt(d)
    cu = np.array([0, T], dtype=np.int32)
    H.log(f"[big] T={T} cp={cp} rank={r} hq={hq} hkv={hkv}: local Q {tl * hq * d * 2 / 2**30:.2f} GiB")
    gq = synth.device_normal_bf16((T, hq, d), 51)
    gk = synth.device_normal_bf16((T, hkv, d), 52)
    gv = synth.device_normal_bf16((T, hkv, d), 53)
    gdo = synth.device_normal_bf16((T, hq, d), 54)
    meta = api.cp_attn_rank_metadata(H.dev_i32(cu), H.dev_i32(cu.copy()), cp, r, -1, tl)

    def gather(src, h, s):
        dst = torch.empty((tl, h, d), dtype=torch.bfloat16, device="cuda")
        api.cp_attn_shard_gather(meta, s, src, dst, h * d * 2)
        return dst

    loc = {"q": gather(gq, hq, r), "do": gather(gdo, hq, r), "k": [gather(gk, hkv, s) for s in range(cp)],
           "v": [gather(gv, hkv, s) for s in range(cp)], "t_alloc": tl, "t_local": tl}
    # host copies of what the oracle reads: every key / value, and the query
    # rows it evaluates
    own = O.shard_rows(cu, cu, cp, r)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, tl // 2 - 1, tl // 2, tl - 2, tl - 1], rng.integers(0, tl, 8)]))
    keys = np.arange(tl - 4, tl)                       # local rows of the rank's own shard
    reach = np.arange(int(own[keys[0]]), T)            # global query positions at or after them
    need = np.unique(np.concatenate([own[rows], reach]))
    qh = np.zeros((T, hq, d), dtype=np.uint16)
    doh = np.zeros((T, hq, d), dtype=np.uint16)
    idx = torch.from_numpy(need).to("cuda")
    qh[need] = _bits(gq.index_select(0, idx))
    doh[need] = _bits(gdo.index_select(0, idx))
    kh, vh = _bits(gk), _bits(gv)
    del gq, gdo, gk, gv
    torch.cuda.empty_cache()
    H.log("[big] GPU fwd + bwd")
    bt = synth.PackedBatch(name="big", seed=51, cu=cu, cup=cu.copy(), hq=hq, hkv=hkv, d=d, q=qh, k=kh, v=vh, do=doh)
    out, lse = H.run_fwd(meta, loc, bt, scale)
    dq, dks, dvs = H.run_bwd(meta, loc, bt, scale, out, lse)
    torch.cuda.synchronize()
    heads = [0, 17, 63]
    H.log(f"[big] oracle: {rows.size} rows x {len(heads)} heads")
    o, l, dqr = O.share_rows(qh, kh, vh, doh, cu, cu, cp, r, scale, rows, heads, want_dq=True)
    ridx = torch.from_numpy(rows).to("cuda")
    H.compare_bf16("out", _bits(out.index_select(0, ridx)[:, heads]), o)
    H.compare_lse("lse", lse[heads][:, ridx].cpu().numpy(), l)
    H.compare_bf16("dq", _bits(dq.index_select(0, ridx)[:, heads]), dqr)
    H.log(f"[big] oracle: dK / dV of {keys.size} key rows")
    dk, dv = O.share_keys_dkdv(qh, kh, vh, doh, cu, cu, cp, r, scale, r, keys, [0, hkv - 1])
    kidx = torch.from_numpy(keys).to("cuda")
    H.compare_bf16("dk", _bits(dks[r].index_select(0, kidx)[:, [0, hkv - 1]]), dk)
    H.compare_bf16("dv", _bits(dvs[r].index_select(0, kidx)[:, [0, hkv - 1]]), dv)
    meta.close()


def test_work_lists_past_sort_cap():
    """One 600000-token sequence at CP = 1 (one head of 64): 4688 forward and
    4688 dK/dV work items in the step, more than the device sorts (lists of
    up to 4096 items are ordered heaviest first, longer ones keep each
    sequence's last tile first). Every item must still run exactly once: out /
    LSE / dQ on sampled rows against the oracle, exact dK / dV of the last key
    rows, and over all key rows the sums sum_j dV_j = sum_p dO_p and
    sum_j dK_j = 0 (softmax rows sum to one and are shift invariant)."""
    import torch
    T, cp, r, hq, hkv, d = 600000, 1, 0, 1, 1, 64
    scale = 1.0 / math.sqrt(d)
    cu = np.array([0, T], dtype=np.int32)
    meta = api.cp_attn_rank_metadata(H.dev_i32(cu), H.dev_i32(cu.copy()), cp, r, -1, T)
    s = meta.summary
    H.log(f"[long lists] T={T}: {int(s.tiles_fwd[0])} forward and {int(s.tiles_dkdv[0])} dK/dV work items")
    assert int(s.tiles_fwd[0]) > 4096 and int(s.tiles_dkdv[0]) > 4096
    g = {nm: synth.device_normal_bf16((T, h, d), seed) for nm, h, seed in
         (("q", hq, 61), ("k", hkv, 62), ("v", hkv, 63), ("do", hq, 64))}
    loc = {"q": g["q"], "do": g["do"], "k": [g["k"]], "v": [g["v"]], "t_alloc": T, "t_local": T}
    host = {nm: _bits(t) for nm, t in g.items()}
    bt = synth.PackedBatch(name="long-lists", seed=61, cu=cu, cup=cu.copy(), hq=hq, hkv=hkv, d=d, **host)
    out, lse = H.run_fwd(meta, loc, bt, scale)
    dq, dks, dvs = H.run_bwd(meta, loc, bt, scale, out, lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 4095 * 128, 4096 * 128 + 5, T // 2, T - 2, T - 1],
                                     rng.integers(0, T, 12)]))
    H.log(f"[long lists] oracle: {rows.size} rows")
    o, l, dqr = O.share_rows(host["q"], host["k"], host["v"], host["do"], cu, cu, cp, r, scale, rows, [0],
                             want_dq=True)
    ridx = torch.from_numpy(rows).to("cuda")
    H.compare_bf16("out", _bits(out.index_select(0, ridx)[:, [0]]), o)
    H.compare_lse("lse", lse[[0]][:, ridx].cpu().numpy(), l)
    H.compare_bf16("dq", _bits(dq.index_select(0, ridx)[:, [0]]), dqr)
    keys = np.arange(T - 6, T)
    dk, dv = O.share_keys_dkdv(host["q"], host["k"], host["v"], host["do"], cu, cu, cp, r, scale, r, keys, [0])
    kidx = torch.from_numpy(keys).to("cuda")
    H.compare_bf16("dk", _bits(dks[0].index_select(0, kidx)[:, [0]]), dk)
    H.compare_bf16("dv", _bits(dvs[0].index_select(0, kidx)[:, [0]]), dv)
    f = H.bf16_bits_to_f64
    sum_dv = f(_bits(dvs[0]))[:, 0].sum(axis=0)
    ref_dv = f(host["do"])[:, 0].sum(axis=0)
    assert np.abs(sum_dv - ref_dv).max() <= 1e-3 * np.sqrt((ref_dv ** 2).sum()) + 0.05
    dk_all = f(_bits(dks[0]))[:, 0]
    # sum_j dK_j vanishes up to the rounding of D = <dO, out> (bf16 out) and of
    # each dK row: bound as in the full-size identities
    e = 2.0 ** -8 * np.abs(f(host["do"])[:, 0] * f(_bits(out))[:, 0]).sum(axis=-1)
    std = scale * np.sqrt(((f(host["q"])[:, 0] ** 2) * (e ** 2)[:, None]).sum(axis=0))
    rnd = 2.0 ** -9 * np.sqrt((dk_all ** 2).sum(axis=0))
    assert (np.abs(dk_all.sum(axis=0)) / (6 * std + 8 * rnd + 1e-6)).max() <= 1.0
    meta.close()


def test_kv_shard_past_2gib():
    """One 262144-token sequence at CP = 1 with 32 KV heads of 128: each K / V
    shard spans 2^31 bytes, so the forward and dQ kernels take their 64-bit
    tile addressing (shorter key ranges use 32-bit offsets). Sampled out /
    LSE / dQ rows and the last key rows' dK / dV against the oracle."""
    import torch
    T, cp, r, hq, hkv, d = 262144, 1, 0, 32, 32, 128
    scale = 1.0 / math.sqrt(d)
    cu = np.array([0, T], dtype=np.int32)
    assert T * hkv * d * 2 >= 2 ** 31
    H.log(f"[big kv] T={T} hq={hq} hkv={hkv}: K shard {T * hkv * d * 2 / 2**30:.2f} GiB")
    meta = api.cp_attn_rank_metadata(H.dev_i32(cu), H.dev_i32(cu.copy()), cp, r, -1, T)
    g = {nm: synth.device_normal_bf16((T, h, d), seed) for nm, h, seed in
         (("q", hq, 71), ("k", hkv, 72), ("v", hkv, 73), ("do", hq, 74))}
    loc = {"q": g["q"], "do": g["do"], "k": [g["k"]], "v": [g["v"]], "t_alloc": T, "t_local": T}
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 127, T // 2, T - 2, T - 1], rng.integers(T - 4096, T, 4)]))
    heads = [0, 31]
    keys = np.arange(T - 4, T)
    # host copies of what the oracle reads: every key / value row of the
    # checked heads' KV heads, the sampled query rows and the rows after the
    # first checked key
    need = np.unique(np.concatenate([rows, np.arange(keys[0], T)]))
    qh = np.zeros((T, hq, d), dtype=np.uint16)
    doh = np.zeros((T, hq, d), dtype=np.uint16)
    idx = torch.from_numpy(need).to("cuda")
    qh[need] = _bits(g["q"].index_select(0, idx))
    doh[need] = _bits(g["do"].index_select(0, idx))
    kh, vh = _bits(g["k"]), _bits(g["v"])
    bt = synth.PackedBatch(name="big-kv", seed=71, cu=cu, cup=cu.copy(), hq=hq, hkv=hkv, d=d, q=qh, k=kh, v=vh, do=doh)
    H.log("[big kv] GPU fwd + bwd")
    out, lse = H.run_fwd(meta, loc, bt, scale)
    dq, dks, dvs = H.run_bwd(meta, loc, bt, scale, out, lse)
    torch.cuda.synchronize()
    H.log(f"[big kv] oracle: {rows.size} rows x {len(heads)} heads")
    o, l, dqr = O.share_rows(qh, kh, vh, doh, cu, cu, cp, r, scale, rows, heads, want_dq=True)
    ridx = torch.from_numpy(rows).to("cuda")
    H.compare_bf16("out", _bits(out.index_select(0, ridx)[:, heads]), o)
    H.compare_lse("lse", lse[heads][:, ridx].cpu().numpy(), l)
    H.compare_bf16("dq", _bits(dq.index_select(0, ridx)[:, heads]), dqr)
    H.log(f"[big kv] oracle: dK / dV of {keys.size} key rows")
    dk, dv = O.share_keys_dkdv(qh, kh, vh, doh, cu, cu, cp, r, scale, r, keys, [0, hkv - 1])
    kidx = torch.from_numpy(keys).to("cuda")
    H.compare_bf16("dk", _bits(dks[0].index_select(0, kidx)[:, [0, hkv - 1]]), dk)
    H.compare_bf16("dv", _bits(dvs[0].index_select(0, kidx)[:, [0, hkv - 1]]), dv)
    meta.close()
