"""The full-size dK / dV fixture (tests/golden/fullsize_dkdv.npz) still
matches the seeded input generator (digest of the inputs its values depend
on), and its values agree with the oracle's one-pass key-row routine on the
key rows that routine computes cheaply (those few of the rank's queries
reach), an independent path to the same numbers; its every-row LSE and
projected out / dQ agree with the oracle's single-row routine on sampled
rows and cover every valid local row of the rank once."""
import math
import os

import numpy as np
import pytest

from context_packed_attention_amd import synth
from oracle import cp_attn_oracle as O
from tests.golden.make_fullsize_dkdv import OUT, input_digest


@pytest.mark.parametrize("cfg", [4, 5])
def test_fixture_matches_generator_and_one_pass_oracle(cfg):
    assert os.path.exists(OUT)
    fx = np.load(OUT, allow_pickle=False)
    bt, w = synth.make_workload(cfg)
    pre = f"w{cfg}_"
    cp, r, g = (int(x) for x in fx[pre + "meta"])
    assert (cp, r) == (w["cp"], w["ranks"][-1]) and 0 <= g < bt.hkv
    assert str(fx[pre + "digest"]) == input_digest(bt, g)
    scale = 1.0 / math.sqrt(bt.d)
    t_local = bt.total_rows // cp
    rows = fx[pre + f"s{r}_rows"]
    late = rows[rows >= t_local - 2]
    assert late.size == 2
    sel = np.searchsorted(rows, late)
    dk, dv = O.share_keys_dkdv(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale, r, late, [g])
    np.testing.assert_allclose(fx[pre + f"s{r}_dk"][sel], dk[:, 0], rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(fx[pre + f"s{r}_dv"][sel], dv[:, 0], rtol=1e-5, atol=1e-7)
    # every part has start, middle and end rows, and finite values
    for s in range(cp):
        rs = fx[pre + f"s{s}_rows"]
        assert rs[0] == 0 and rs[-1] == t_local - 1 and (t_local // 2) in rs
        for name in ("dk", "dv", "dk_sd", "dv_sd"):
            a = fx[pre + f"s{s}_{name}"]
            assert a.shape == (rs.size, bt.d) and np.isfinite(a).all()


@pytest.mark.parametrize("cfg", [4, 5])
def test_fixture_lse_rows(cfg):
    fx = np.load(OUT, allow_pickle=False)
    bt, w = synth.make_workload(cfg)
    pre = f"w{cfg}_"
    cp, r, g = (int(x) for x in fx[pre + "meta"])
    group = bt.hq // bt.hkv
    rows, lse = fx[pre + "lse_rows"], fx[pre + "lse"]
    t_local = bt.total_rows // cp
    valid = O.valid_mask(bt.cu, bt.cup)[O.shard_rows(bt.cu, bt.cup, cp, r)]
    assert np.array_equal(np.sort(rows), np.nonzero(valid)[0]) and lse.shape == (group, rows.size)
    pick = np.random.default_rng(9).choice(rows.size, 6, replace=False)
    heads = list(range(g * group, (g + 1) * group))
    o, l, dq = O.share_rows(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, 1.0 / math.sqrt(bt.d), rows[pick], heads,
                            want_dq=True)
    np.testing.assert_allclose(lse[:, pick], l, rtol=1e-6, atol=1e-5)
    assert rows.max() < t_local
    # every row's projected out / dQ: the oracle's single-row routine on the
    # sampled rows, projected on the stored unit vectors
    u = fx[pre + "proj_u"]
    assert u.shape == (group, bt.d) and np.allclose(np.linalg.norm(u, axis=1), 1.0)
    for name, ref in (("out_proj", o), ("dq_proj", dq)):
        a = fx[pre + name]
        assert a.shape == lse.shape and np.isfinite(a).all()
        want = np.stack([ref[:, jh] @ u[jh] for jh in range(group)])
        np.testing.assert_allclose(a[:, pick], want, rtol=1e-5, atol=1e-7)
        sd = fx[pre + name + "_sd"]
        assert sd.shape == lse.shape and np.isfinite(sd).all() and (sd >= 0).all()


@pytest.mark.parametrize("cfg", [4, 5])
def test_fixture_key_projections(cfg):
    """Every valid key row's projected dK / dV: one value per key row in
    global order, and on the last key rows (few queries reach them) the
    oracle's one-pass key-row routine projected on the stored vectors."""
    fx = np.load(OUT, allow_pickle=False)
    bt, w = synth.make_workload(cfg)
    pre = f"w{cfg}_"
    cp, r, g = (int(x) for x in fx[pre + "meta"])
    keys = np.nonzero(O.valid_mask(bt.cu, bt.cup))[0]
    uk = fx[pre + "key_u"]
    assert uk.shape == (2, bt.d) and np.allclose(np.linalg.norm(uk, axis=1), 1.0)
    for nm in ("dk_proj", "dv_proj", "dk_proj_sd", "dv_proj_sd"):
        a = fx[pre + nm]
        assert a.shape == keys.shape and np.isfinite(a).all()
    # the rank's own shard's last local key rows (local order = global
    # positions the owner map sends there)
    t_local = bt.total_rows // cp
    late = np.array([t_local - 2, t_local - 1])
    dk, dv = O.share_keys_dkdv(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, 1.0 / math.sqrt(bt.d), r, late, [g])
    glob = O.shard_rows(bt.cu, bt.cup, cp, r)[late]
    at = np.searchsorted(keys, glob)
    assert np.array_equal(keys[at], glob)
    np.testing.assert_allclose(fx[pre + "dk_proj"][at], dk[:, 0] @ uk[0], rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(fx[pre + "dv_proj"][at], dv[:, 0] @ uk[1], rtol=1e-5, atol=1e-7)
