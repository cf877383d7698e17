"""Parity at the full sizes the benchmark runs (the 131072-token GQA share and
the 64K hierarchical-pack share), in the same launch configuration.

The whole share is too large for the oracle, so: out / LSE / dQ are checked on
sampled rows (each row one full softmax row of the oracle), and for every row
of one KV head's query heads the LSE and the out and dQ rows projected on a
fixed unit vector against stored oracle values, and that KV head's dK and dV
rows projected the same way on every key row of every part; dK / dV element by
element on key rows at the start, middle and end of every source shard's part
(so every ring step's launch, the causal one included, and key rows that all
of the rank's queries reach), against values the oracle's two-pass helper
computed once (tests/golden/make_fullsize_dkdv.py writes them, with a digest
of the inputs they depend on); exactly on key rows that few of the rank's
queries reach, computed here; every part's rows that no query of the rank
reaches must be exactly zero; and four identities that hold at any size tie
all rows of all parts together:
  sum_j dV_j = sum_p dO_p            (softmax rows sum to one)
  sum_j dK_j = 0                     (softmax is shift invariant)
  sum_p <dQ_p, Q_p> = sum_j <dK_j, K_j>   (both equal scale * sum dS_pj s_pj)
  sum_p <dO_p, out_p> = sum_j <dV_j, V_j>
each per KV head, summed over the query heads of its group.
"""
import math
import os

import numpy as np
import pytest

from context_packed_attention_amd import synth
from oracle import cp_attn_oracle as O
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _run(cfg):
    bt, w = synth.make_workload(cfg)
    r = w["ranks"][-1]
    cp = w["cp"]
    scale = 1.0 / math.sqrt(bt.d)
    H.log(f"[full] {bt.name} cp={cp} rank={r}: GPU fwd+bwd")
    db = H.DeviceBatch(bt)
    meta, loc = H.local_inputs(db, cp, r)
    out, lse = H.run_fwd(meta, loc, bt, scale)
    dq, dks, dvs = H.run_bwd(meta, loc, bt, scale, out, lse)
    res = {"out": H.bf16_to_np(out), "lse": lse.cpu().numpy(), "dq": H.bf16_to_np(dq),
           "dk": [H.bf16_to_np(x) for x in dks], "dv": [H.bf16_to_np(x) for x in dvs],
           "q": H.bf16_to_np(loc["q"]), "do": H.bf16_to_np(loc["do"]),
           "k": [H.bf16_to_np(x) for x in loc["k"]], "v": [H.bf16_to_np(x) for x in loc["v"]]}
    meta.close()
    del db
    return bt, w, r, scale, res


def _sample_rows(T_local, n, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 127, 128, T_local // 2 - 1, T_local // 2, T_local // 2 + 1, T_local - 2, T_local - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, T_local, n)]))


@pytest.fixture(scope="module", params=[4, 5], ids=["single131072-gqa-cp4", "pack64k-hier2x2-p2p"])
def full(request):
    return _run(request.param)


def test_sampled_rows_out_lse_dq(full):
    bt, w, r, scale, res = full
    T_local = bt.total_rows // w["cp"]
    rows = _sample_rows(T_local, 24, 7)
    heads = sorted({0, bt.hq - 1, bt.hq // 2, 3 % bt.hq})
    H.log(f"[full] oracle rows={rows.size} heads={heads}")
    o, l, dq = O.share_rows(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, w["cp"], r, scale, rows, heads, want_dq=True)
    H.compare_bf16("out", res["out"][rows][:, heads], o)
    H.compare_lse("lse", res["lse"][heads][:, rows], l)
    H.compare_bf16("dq", res["dq"][rows][:, heads], dq)


def test_exact_key_rows_and_zero_rows(full):
    bt, w, r, scale, res = full
    cp = w["cp"]
    T_local = bt.total_rows // cp
    own_rows = O.shard_rows(bt.cu, bt.cup, cp, r)
    # the last few local rows of the rank's last sequence: few queries reach them
    keys = np.arange(T_local - 12, T_local)
    kvh = [0, bt.hkv - 1]
    H.log(f"[full] oracle dK/dV for {keys.size} key rows")
    dk, dv = O.share_keys_dkdv(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale, r, keys, kvh)
    H.compare_bf16("dk rows", res["dk"][r][keys][:, kvh], dk)
    H.compare_bf16("dv rows", res["dv"][r][keys][:, kvh], dv)
    # rows of each part that no query of this rank reaches are exactly zero
    rank_of, _ = O.owner_map(bt.cu, bt.cup, cp)
    seq = np.searchsorted(bt.cup, np.arange(bt.total_rows), side="right") - 1
    valid = O.valid_mask(bt.cu, bt.cup)
    last_q = np.full(bt.cu.size - 1, -1)
    for g in np.nonzero((rank_of == r) & valid)[0]:
        last_q[seq[g]] = max(last_q[seq[g]], g)
    for s in range(cp):
        rows = O.shard_rows(bt.cu, bt.cup, cp, s)
        unreached = ~valid[rows] | (rows > last_q[seq[rows]])
        assert not res["dk"][s][unreached].any() and not res["dv"][s][unreached].any(), s


FIXTURE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fullsize_dkdv.npz")


def test_dkdv_every_shard_vs_oracle_fixture(full):
    """Key rows at the start, middle and end of every source shard's part
    (both chunks), one KV head, element by element with the rounding model's
    per-element standard deviation."""
    from tests.golden.make_fullsize_dkdv import input_digest
    bt, w, r, scale, res = full
    cfg = 4 if bt.hkv != bt.hq else 5
    fx = np.load(FIXTURE, allow_pickle=False)
    pre = f"w{cfg}_"
    cp, rank, g = (int(x) for x in fx[pre + "meta"])
    assert (cp, rank) == (w["cp"], r)
    assert str(fx[pre + "digest"]) == input_digest(bt, g), "fixture is stale: rerun tests/golden/make_fullsize_dkdv.py"
    for s in range(cp):
        rows = fx[pre + f"s{s}_rows"]
        H.log(f"[full] shard {s}: {rows.size} key rows vs the fixture (kv head {g})")
        a = H.compare_bf16(f"dk[{s}] rows", res["dk"][s][rows][:, g], fx[pre + f"s{s}_dk"], sd=fx[pre + f"s{s}_dk_sd"])
        b = H.compare_bf16(f"dv[{s}] rows", res["dv"][s][rows][:, g], fx[pre + f"s{s}_dv"], sd=fx[pre + f"s{s}_dv_sd"])
        H.log(f"    dk max {a['max_abs']:.2e} (max |ref| {a['max_ref']:.3f}), dv max {b['max_abs']:.2e} "
              f"(max |ref| {b['max_ref']:.3f})")


def test_lse_every_row_vs_oracle_fixture(full):
    """The LSE of every query row of the rank for one KV head's query heads,
    against the oracle's values stored beside the dK / dV fixture."""
    from tests.golden.make_fullsize_dkdv import input_digest
    bt, w, r, scale, res = full
    cfg = 4 if bt.hkv != bt.hq else 5
    fx = np.load(FIXTURE, allow_pickle=False)
    pre = f"w{cfg}_"
    cp, rank, g = (int(x) for x in fx[pre + "meta"])
    assert (cp, rank) == (w["cp"], r)
    assert str(fx[pre + "digest"]) == input_digest(bt, g), "fixture is stale: rerun tests/golden/make_fullsize_dkdv.py"
    group = bt.hq // bt.hkv
    heads = list(range(g * group, (g + 1) * group))
    rows = fx[pre + "lse_rows"]
    H.log(f"[full] LSE of {rows.size} rows x {group} heads vs the fixture")
    H.compare_lse("lse every row", res["lse"][heads][:, rows], fx[pre + "lse"].astype(np.float64))


def test_out_dq_every_row_projected_vs_oracle_fixture(full):
    """The output and query gradient of every query row of the rank for one
    KV head's query heads, projected on the stored unit vector of each head,
    against the oracle's exact projections. Bar: the bf16 rounding of the
    row's own elements (at most 2^-8 of each, weighted by |u_d|) plus six of
    the rounding model's deviations of the projection (P rounded before
    P V, dS before dS K, D formed from the rounded output), plus 1e-5 of the
    row's norm for fp32 accumulation."""
    bt, w, r, scale, res = full
    cfg = 4 if bt.hkv != bt.hq else 5
    fx = np.load(FIXTURE, allow_pickle=False)
    pre = f"w{cfg}_"
    cp, rank, g = (int(x) for x in fx[pre + "meta"])
    group = bt.hq // bt.hkv
    heads = list(range(g * group, (g + 1) * group))
    rows = fx[pre + "lse_rows"]
    u = fx[pre + "proj_u"]
    for name, key in (("out", "out_proj"), ("dq", "dq_proj")):
        got = H.bf16_bits_to_f64(res[name][rows][:, heads])  # [n, group, D]
        ref, sd = fx[pre + key].astype(np.float64), fx[pre + key + "_sd"].astype(np.float64)
        worst = 0.0
        for jh in range(group):
            gp = got[:, jh] @ u[jh]
            tol = 2.0 ** -8 * (np.abs(got[:, jh]) @ np.abs(u[jh])) + 6.0 * sd[jh] + \
                1e-5 * np.linalg.norm(got[:, jh], axis=1) + 1e-7
            ratio = np.abs(gp - ref[jh]) / tol
            worst = max(worst, float(ratio.max()))
            bad = np.nonzero(ratio > 1.0)[0]
            assert bad.size == 0, (f"{name} head {heads[jh]}: {bad.size} rows over the bar, first local row "
                                   f"{int(rows[bad[0]])}: {gp[bad[0]]:.6g} vs {ref[jh, bad[0]]:.6g}")
        H.log(f"[full] {name} projected on every row ({rows.size} x {group}): worst / bar {worst:.3f}")


def test_dkdv_every_key_row_projected_vs_oracle_fixture(full):
    """The rank's dK and dV of every valid key row of one KV head, in every
    source shard's part, projected on the stored unit vectors, against the
    oracle's exact projections (bar as for out / dQ: the elements' own bf16
    rounding, six of the rounding model's deviations of the projection, 1e-5
    of the row's norm)."""
    bt, w, r, scale, res = full
    cfg = 4 if bt.hkv != bt.hq else 5
    fx = np.load(FIXTURE, allow_pickle=False)
    pre = f"w{cfg}_"
    cp, rank, g = (int(x) for x in fx[pre + "meta"])
    keys = np.nonzero(O.valid_mask(bt.cu, bt.cup))[0]
    owner, local = O.owner_map(bt.cu, bt.cup, cp)
    uk = fx[pre + "key_u"]
    for name, j in (("dk", 0), ("dv", 1)):
        got = np.zeros((keys.size, bt.d))
        for s in range(cp):
            m = owner[keys] == s
            got[m] = H.bf16_bits_to_f64(res[name][s][local[keys[m]], g])
        gp = got @ uk[j]
        ref = fx[pre + name + "_proj"].astype(np.float64)
        sd = fx[pre + name + "_proj_sd"].astype(np.float64)
        tol = 2.0 ** -8 * (np.abs(got) @ np.abs(uk[j])) + 6.0 * sd + 1e-5 * np.linalg.norm(got, axis=1) + 1e-7
        ratio = np.abs(gp - ref) / tol
        bad = np.nonzero(ratio > 1.0)[0]
        assert bad.size == 0, (f"{name}: {bad.size} key rows over the bar, first global row {int(keys[bad[0]])}: "
                               f"{gp[bad[0]]:.6g} vs {ref[bad[0]]:.6g}")
        H.log(f"[full] {name} projected on every key row ({keys.size}, {cp} parts): worst / bar {ratio.max():.3f}")


def _tol(vals):
    return 1e-3 * np.sqrt((vals ** 2).sum()) + 1e-6


def test_gradient_identities(full):
    bt, w, r, scale, res = full
    cp = w["cp"]
    group = bt.hq // bt.hkv
    f = H.bf16_bits_to_f64
    q = f(res["q"])
    do = f(res["do"])
    dq = f(res["dq"])
    out = f(res["out"])
    own = O.shard_rows(bt.cu, bt.cup, cp, r)
    valid_q = O.valid_mask(bt.cu, bt.cup)[own]
    for g in range(bt.hkv):
        hs = slice(g * group, (g + 1) * group)
        sum_dv = sum(f(res["dv"][s][:, g]).sum(axis=0) for s in range(cp))
        ref_dv = do[valid_q, hs].sum(axis=(0, 1))
        err = np.abs(sum_dv - ref_dv).max()
        assert err <= _tol(ref_dv) + 0.05, (g, err)
        # sum_j dS_pj vanishes only up to the rounding of D_p = <dO_p, out_p>
        # (taken from the bf16 output): e_p ~ 2^-8 * sum_d |dO out|, so the
        # d-th component of sum_j dK_j is a random sum with standard deviation
        # scale * sqrt(sum_p Q_pd^2 e_p^2), plus the bf16 rounding of the dK rows.
        sum_dk = sum(f(res["dk"][s][:, g]).sum(axis=0) for s in range(cp))
        e = 2.0 ** -8 * np.abs(do[valid_q, hs] * out[valid_q, hs]).sum(axis=-1)        # [rows, group]
        std = scale * np.sqrt(((q[valid_q, hs] ** 2) * (e ** 2)[..., None]).sum(axis=(0, 1)))
        rnd = 2.0 ** -9 * np.sqrt(sum((f(res["dk"][s][:, g]) ** 2).sum(axis=0) for s in range(cp)))
        worst = float((np.abs(sum_dk) / (6 * std + 8 * rnd + 1e-6)).max())
        assert worst <= 1.0, (g, float(np.abs(sum_dk).max()), worst)
        lhs = float((dq[valid_q, hs] * q[valid_q, hs]).sum())
        rhs = sum(float((f(res["dk"][s][:, g]) * f(res["k"][s][:, g])).sum()) for s in range(cp))
        mag = math.sqrt(float((dq[valid_q, hs] ** 2).sum()) * float((q[valid_q, hs] ** 2).sum()))
        assert abs(lhs - rhs) <= 1e-3 * mag + 1e-3, (g, lhs, rhs)
        lhs2 = float((do[valid_q, hs] * out[valid_q, hs]).sum())
        rhs2 = sum(float((f(res["dv"][s][:, g]) * f(res["v"][s][:, g])).sum()) for s in range(cp))
        mag2 = math.sqrt(float((do[valid_q, hs] ** 2).sum()) * float((out[valid_q, hs] ** 2).sum()))
        assert abs(lhs2 - rhs2) <= 1e-3 * mag2 + 1e-3, (g, lhs2, rhs2)
