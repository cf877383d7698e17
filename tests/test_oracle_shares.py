"""All-ranks invariants of the oracle's rank shares, and planted mistakes.

Concatenating every rank's out / lse / dQ reproduces the unsharded result, and
summing every rank's dK/dV part for shard s reproduces shard s of the unsharded
dK/dV (float64, to 1e-12). A second group of tests plants plausible mistakes
in a copy of the oracle and checks that some pin catches each one.
"""
import importlib.util
import os
import sys

import numpy as np
import pytest

from oracle import cp_attn_oracle as O
from context_packed_attention_amd import synth

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "cp_attn_oracle.py")


def _random_batch(seed, cp, B, hq, hkv, d, pad=True):
    rng = np.random.default_rng(seed)
    L, P = [], []
    for _ in range(B):
        c = int(rng.integers(1, 5))
        Pb = 2 * cp * c
        L.append(int(rng.integers(0, Pb + 1)) if pad else Pb)
        P.append(Pb)
    return synth.make_batch("t", seed, L, P, hq, hkv, d)


@pytest.mark.parametrize("cp", [1, 2, 3, 4])
@pytest.mark.parametrize("pad", [False, True])
def test_all_ranks_reassemble_unsharded(cp, pad):
    bt = _random_batch(10 * cp + pad, cp, 3, 4, 2, 8, pad)
    scale = 1 / np.sqrt(8)
    q, k, v, do = (O.bf16_to_f64(x) for x in (bt.q, bt.k, bt.v, bt.do))
    full = O.attention(q, k, v, do, bt.cu, bt.cup, scale)
    T = bt.total_rows
    out = np.zeros_like(full[0])
    lse = np.full_like(full[1], -np.inf)
    dq = np.zeros_like(full[2])
    dk_sum = [np.zeros((T // cp, 2, 8)) for _ in range(cp)]
    dv_sum = [np.zeros((T // cp, 2, 8)) for _ in range(cp)]
    for r in range(cp):
        sh = O.share(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale)
        rows = O.shard_rows(bt.cu, bt.cup, cp, r)
        out[rows] = sh["out"]
        lse[:, rows] = sh["lse"]
        dq[rows] = sh["dq"]
        for s in range(cp):
            dk_sum[s] += sh["dk_parts"][s]
            dv_sum[s] += sh["dv_parts"][s]
    np.testing.assert_allclose(out, full[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isfinite(lse), np.isfinite(full[1]))
    f = np.isfinite(lse)
    np.testing.assert_allclose(lse[f], full[1][f], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dq, full[2], rtol=1e-12, atol=1e-12)
    for s in range(cp):
        np.testing.assert_allclose(dk_sum[s], O.gather_shard(full[3], bt.cu, bt.cup, cp, s), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dv_sum[s], O.gather_shard(full[4], bt.cu, bt.cup, cp, s), rtol=1e-12, atol=1e-12)


def test_share_padding_rows_zero():
    bt = _random_batch(77, 2, 3, 2, 2, 8, True)
    sh = O.share(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, 2, 1, 0.35)
    rows = O.shard_rows(bt.cu, bt.cup, 2, 1)
    pad = ~O.valid_mask(bt.cu, bt.cup)[rows]
    assert not sh["out"][pad].any() and not sh["dq"][pad].any()
    assert np.isneginf(sh["lse"][:, pad]).all()
    for s in range(2):
        padk = ~O.valid_mask(bt.cu, bt.cup)[O.shard_rows(bt.cu, bt.cup, 2, s)]
        assert not sh["dk_parts"][s][padk].any() and not sh["dv_parts"][s][padk].any()


def test_sampled_rows_match_full_share():
    bt = _random_batch(5, 2, 3, 4, 2, 8, True)
    sh = O.share(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, 2, 0, 0.3)
    rows = np.arange(bt.total_rows // 2)
    o, l = O.share_rows_forward(bt.q, bt.k, bt.v, bt.cu, bt.cup, 2, 0, 0.3, rows, [0, 3])
    np.testing.assert_allclose(o, sh["out"][:, [0, 3]], rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isfinite(l), np.isfinite(sh["lse"][[0, 3]]))
    dq = O.share_rows_dq(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, 2, 0, 0.3, rows, [1, 2])
    np.testing.assert_allclose(dq, sh["dq"][:, [1, 2]], rtol=1e-12, atol=1e-12)


def test_flop_count_closed_form():
    """No padding: the rank's causal pairs are sum_b L_b (L_b + 1) / 2 / CP
    when chunks are paired r with 2CP-1-r (load balance)."""
    cu = np.array([0, 64, 192, 256])
    for cp in (1, 2, 4):
        for r in range(cp):
            f = O.flops_share(cu, cu.copy(), cp, r, 2, 64)
            assert f["pairs"] * cp == sum(L * (L + 1) // 2 for L in (64, 128, 64))
    f = O.flops_share(cu, cu.copy(), 2, 0, 2, 64)
    assert f["pairs"] == 6208 and f["total"] == 14 * 64 * 2 * 6208


# ---------------------------------------------------------------- planted mistakes

def _mutant(old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, old
    name = f"_oracle_mutant_{abs(hash(old)) % 10**8}"
    spec = importlib.util.spec_from_loader(name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src.replace(old, new), name, "exec"), mod.__dict__)
    return mod


MUTATIONS = [
    ("causal mask off", "allowed = np.arange(L)[None, :] <= pos[:, None]",
     "allowed = np.arange(L)[None, :] < L"),
    ("diagonal dropped", "allowed = np.arange(L)[None, :] <= pos[:, None]",
     "allowed = np.arange(L)[None, :] < np.maximum(pos[:, None], 1)"),
    ("D term dropped", "ds = p * (dp - dcoef[:, None])", "ds = p * dp"),
    ("dK scale dropped", "dk = scale * (ds.T @ qh)", "dk = ds.T @ qh"),
    ("unnormalised weights", "p = np.exp(s - lse[:, None])", "p = np.exp(s - m[:, None])"),
    ("gqa map", "g = h // group", "g = h % hkv"),
    ("wrong chunk pairing", "rank[g] = 2 * cp - 1 - k", "rank[g] = k - cp"),
    ("lse sign", "lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))",
     "lse = m - np.log(np.exp(s - m[:, None]).sum(axis=1))"),
]


def _pins_pass(mod):
    """Run a subset of the pins against a (possibly mutated) oracle module."""
    import tests.test_oracle_attention as TA
    import tests.test_oracle_meta as TM
    saved = (TA.O, TM.O)
    TA.O = mod
    TM.O = mod
    try:
        for case in TM._cases():
            TM.test_handworked_fixture(case)
        TM.test_step_tables_cover_exactly_the_causal_pairs(3)
        for args in TA.CASES:
            TA.test_forward_vs_dense_brute_force(*args)
            TA.test_forward_backward_vs_torch(*args)
        TA.test_closed_form_single_token_sequences()
    except AssertionError:
        return False
    finally:
        TA.O, TM.O = saved
    return True


def test_unmutated_oracle_passes_pins():
    assert _pins_pass(O)


@pytest.mark.parametrize("label,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(label, old, new):
    assert not _pins_pass(_mutant(old, new)), label


def test_key_rows_match_full_share():
    bt = _random_batch(9, 2, 3, 4, 2, 8, True)
    scale = 0.33
    for r in range(2):
        sh = O.share(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, 2, r, scale)
        for s in range(2):
            keys = np.arange(bt.total_rows // 2)
            dk, dv = O.share_keys_dkdv(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, 2, r, scale, s, keys, [0, 1])
            np.testing.assert_allclose(dk, sh["dk_parts"][s], rtol=1e-11, atol=1e-11)
            np.testing.assert_allclose(dv, sh["dv_parts"][s], rtol=1e-11, atol=1e-11)


def test_dropped_ring_steps_would_fail_parity():
    """A share computed from the rank's own shard only (every ring step after
    the first dropped) is far outside the parity tolerance on the tiny pack,
    so the GPU parity tests detect a path that skips the exchange."""
    bt, w = synth.make_workload(1)
    scale = 1 / np.sqrt(bt.d)
    for r in (0, 1):
        full = O.share(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, 2, r, scale)
        rows = O.shard_rows(bt.cu, bt.cup, 2, r)
        md = O.rank_metadata(bt.cu, bt.cup, 2, r)
        cu_loc = md[f"cu_full_{r}"]
        sub = lambda x: O.bf16_to_f64(x[rows])
        own = O.attention(sub(bt.q), sub(bt.k), sub(bt.v), sub(bt.do), cu_loc, md["cu_padded_local"], scale)
        assert np.abs(own[0] - full["out"]).max() > 0.2
        assert np.abs(own[2] - full["dq"]).max() > 0.2


@pytest.mark.parametrize("cp,hq,hkv,pad,seed", [(1, 4, 1, False, 31), (2, 4, 2, True, 32), (3, 6, 2, True, 33),
                                                 (4, 8, 2, False, 34)])
def test_two_pass_key_rows_match_full_share(cp, hq, hkv, pad, seed):
    """The two-pass dK / dV (first pass: every rank row's lse and D; second:
    chosen key rows) reproduces every row of every shard's part of the full
    share, and its standard deviation the rounding model's, on packs with
    GQA, padding and several ranks."""
    bt = _random_batch(seed, cp, 3, hq, hkv, 8, pad)
    scale = 0.31
    T_local = bt.total_rows // cp
    for r in range(cp):
        sh = O.share(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale)
        sd = O.share_rounding_sd(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale)
        for g in range(hkv):
            # a small batch limit forces the first pass to split its rows
            stats = O.group_row_stats(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale, g, max_elems=40)
            for s in range(cp):
                keys = np.arange(T_local)
                dk, dv, dks, dvs = O.share_keys_dkdv_two_pass(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r,
                                                              scale, s, keys, g, stats=stats)
                np.testing.assert_allclose(dk, sh["dk_parts"][s][:, g], rtol=1e-11, atol=1e-12)
                np.testing.assert_allclose(dv, sh["dv_parts"][s][:, g], rtol=1e-11, atol=1e-12)
                np.testing.assert_allclose(dks, sd["dk_parts"][s][:, g], rtol=1e-9, atol=1e-15)
                np.testing.assert_allclose(dvs, sd["dv_parts"][s][:, g], rtol=1e-9, atol=1e-15)


def test_two_pass_stats_are_the_rows_softmax():
    """First-pass lse equals the share's LSE on every rank row, and D the
    inner product of dO with the share's output."""
    bt = _random_batch(41, 2, 3, 4, 2, 8, True)
    scale = 0.4
    sh = O.share(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, 2, 1, scale)
    own = O.shard_rows(bt.cu, bt.cup, 2, 1)
    loc = {int(g): i for i, g in enumerate(own)}
    for g in range(2):
        st = O.group_row_stats(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, 2, 1, scale, g)
        idx = np.array([loc[int(x)] for x in st["rows"]])
        valid = O.valid_mask(bt.cu, bt.cup)[own]
        assert valid[idx].all() and idx.size == int(valid.sum())
        for jh, h in enumerate(range(2 * g, 2 * g + 2)):
            np.testing.assert_allclose(st["lse"][jh], sh["lse"][h, idx], rtol=1e-12, atol=1e-12)
            dref = (O.bf16_to_f64(bt.do[st["rows"], h]) * sh["out"][idx, h]).sum(axis=1)
            np.testing.assert_allclose(st["dcoef"][jh], dref, rtol=1e-10, atol=1e-12)


def test_row_projections_match_full_share():
    """With projection vectors, the first pass's projected output and query
    gradient of every rank row equal the full share's rows projected on the
    same vectors, and along unit basis vectors its projected deviations are
    the rounding model's per-element deviations (share_rounding_sd, computed
    element by element on its own)."""
    bt = _random_batch(43, 2, 3, 4, 2, 8, True)
    scale, cp, r = 0.4, 2, 1
    sh = O.share(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale)
    sd = O.share_rounding_sd(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale)
    own = O.shard_rows(bt.cu, bt.cup, cp, r)
    loc = {int(g): i for i, g in enumerate(own)}
    rng = np.random.default_rng(5)
    for g in range(2):
        u = rng.standard_normal((2, 8))
        st = O.group_row_stats(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale, g, max_elems=40, proj=u)
        idx = np.array([loc[int(x)] for x in st["rows"]])
        for jh, h in enumerate(range(2 * g, 2 * g + 2)):
            np.testing.assert_allclose(st["out_proj"][jh], sh["out"][idx, h] @ u[jh], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(st["dq_proj"][jh], sh["dq"][idx, h] @ u[jh], rtol=1e-10, atol=1e-12)
        for d in range(8):
            e = np.zeros((2, 8))
            e[:, d] = 1.0
            sb = O.group_row_stats(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale, g, proj=e)
            for jh, h in enumerate(range(2 * g, 2 * g + 2)):
                np.testing.assert_allclose(sb["out_proj_sd"][jh], sd["out"][idx, h, d], rtol=1e-9, atol=1e-15)
                np.testing.assert_allclose(sb["dq_proj_sd"][jh], sd["dq"][idx, h, d], rtol=1e-9, atol=1e-15)


@pytest.mark.parametrize("cp,hq,hkv,pad,seed", [(2, 4, 2, True, 51), (3, 6, 2, False, 52), (1, 2, 1, True, 53)])
def test_key_projections_match_full_share(cp, hq, hkv, pad, seed):
    """The blocked second pass's projected dK / dV of every key row equal the
    full share's dK / dV (global order) projected on the same vectors, with
    blocks small enough to split every sequence; along unit basis vectors its
    deviations are the per-element rounding model's."""
    bt = _random_batch(seed, cp, 3, hq, hkv, 8, pad)
    scale = 0.35
    rng = np.random.default_rng(seed)
    valid = O.valid_mask(bt.cu, bt.cup)
    for r in range(cp):
        sh = O.share(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale)
        sd = O.share_rounding_sd(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale)
        for g in range(hkv):
            st = O.group_row_stats(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale, g)
            u, v = rng.standard_normal(8), rng.standard_normal(8)
            kp = O.group_key_projections(st, bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, scale, u, v, max_elems=7)
            rows = kp["key_rows"]
            assert np.array_equal(rows, np.nonzero(valid)[0])
            np.testing.assert_allclose(kp["dk_proj"], sh["dk_full"][rows, g] @ u, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(kp["dv_proj"], sh["dv_full"][rows, g] @ v, rtol=1e-10, atol=1e-12)
            for d in (0, 5):
                e = np.zeros(8)
                e[d] = 1.0
                kb = O.group_key_projections(st, bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, scale, e, e, max_elems=7)
                np.testing.assert_allclose(kb["dk_proj_sd"], sd["dk_full"][rows, g, d], rtol=1e-9, atol=1e-15)
                np.testing.assert_allclose(kb["dv_proj_sd"], sd["dv_full"][rows, g, d], rtol=1e-9, atol=1e-15)
