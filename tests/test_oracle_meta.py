"""Pins of the oracle's sharding map and per-rank metadata (CPU only).

The pins do not come from the oracle itself: a hand-worked fixture, brute-force
counting over an explicit row-owner map, closed forms for unpadded packs, and a
brute-force enumeration of which (query, key) pairs each ring step must cover.
"""
import json
import os

import numpy as np
import pytest

from oracle import cp_attn_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "meta_handworked.json")


def _ranges(spec):
    out = []
    for part in spec.split(","):
        a, b = part.split("-")
        out.extend(range(int(a), int(b) + 1))
    return out


def _cases():
    with open(GOLD) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_handworked_fixture(case):
    cu = np.array(case["cu"], dtype=np.int32)
    cup = np.array(case["cup"], dtype=np.int32)
    cp = case["cp"]
    for s, sh in case["shards"].items():
        assert list(O.shard_rows(cu, cup, cp, int(s))) == _ranges(sh["rows"])
    for r, steps in case["ranks"].items():
        md = O.rank_metadata(cu, cup, cp, int(r))
        assert md["t_local"] == case["t_local"]
        assert md["pad_between_seqs"] == case["pad_between_seqs"]
        assert list(md["chunk"]) == case["chunk"]
        assert list(md["cu_padded_local"]) == case["cu_padded_local"]
        assert list(md["cu_padded_half"]) == case["cu_padded_half"]
        for s, sh in case["shards"].items():
            assert list(md[f"cu_full_{s}"]) == sh["cu_full"]
            assert list(md[f"cu_first_{s}"]) == sh["cu_first"]
            assert list(md[f"cu_second_{s}"]) == sh["cu_second"]
        for i, st in enumerate(steps):
            got = md["steps"][i]
            for key in ("kind", "src"):
                assert got[key] == st[key]
            for key in ("q_start", "q_len", "kv_start", "kv_len"):
                assert list(got[key]) == st[key], (r, i, key)


def _random_pack(rng, B, cp, max_chunk=6, pad=True):
    L, P = [], []
    for _ in range(B):
        c = int(rng.integers(0, max_chunk + 1))
        Pb = 2 * cp * c
        Lb = int(rng.integers(0, Pb + 1)) if pad else Pb
        L.append(Lb)
        P.append(Pb)
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    cup = np.concatenate([[0], np.cumsum(P)]).astype(np.int32)
    return cu, cup


@pytest.mark.parametrize("cp", [1, 2, 3, 4, 5])
def test_valid_counts_by_brute_force(cp):
    """Clamp formula vs counting rows of the explicit owner map."""
    rng = np.random.default_rng(7 + cp)
    for _ in range(6):
        cu, cup = _random_pack(rng, int(rng.integers(1, 6)), cp)
        owner, local = O.owner_map(cu, cup, cp)
        valid = O.valid_mask(cu, cup)
        seq = np.searchsorted(cup, np.arange(cup[-1]), side="right") - 1
        for r in range(cp):
            md = O.rank_metadata(cu, cup, cp, r)
            for s in range(cp):
                first = np.diff(md[f"cu_first_{s}"])
                second = np.diff(md[f"cu_second_{s}"])
                full = np.diff(md[f"cu_full_{s}"])
                for b in range(cu.size - 1):
                    rows = np.nonzero((owner == s) & (seq == b))[0]
                    lrow = local[rows] - cup[b] // cp
                    c = (cup[b + 1] - cup[b]) // (2 * cp)
                    n_first = int((valid[rows] & (lrow < c)).sum())
                    n_second = int((valid[rows] & (lrow >= c)).sum())
                    assert first[b] == n_first and second[b] == n_second
                    assert full[b] == n_first + n_second
            # every valid row is held by exactly one rank
        tot = sum(np.diff(O.rank_metadata(cu, cup, cp, 0)[f"cu_full_{s}"]) for s in range(cp))
        assert list(tot) == list(np.diff(cu))


@pytest.mark.parametrize("cp", [1, 2, 4, 8])
def test_unpadded_closed_form(cp):
    """No padding: every table is cu/CP or cu/(2CP)."""
    rng = np.random.default_rng(cp)
    cu, cup = _random_pack(rng, 7, cp, pad=False)
    cup = cup.copy()  # distinct, value-equal
    for r in range(cp):
        md = O.rank_metadata(cu, cup, cp, r)
        assert md["pad_between_seqs"] == 0
        for s in range(cp):
            assert list(md[f"cu_full_{s}"]) == list(cu // cp)
            assert list(md[f"cu_first_{s}"]) == list(cu // (2 * cp))
            assert list(md[f"cu_second_{s}"]) == list(cu // (2 * cp))


def test_padding_decision_by_value_not_identity():
    cu = np.array([0, 128], dtype=np.int32)
    same = cu
    copy = cu.copy()
    assert copy is not cu and np.array_equal(copy, cu)
    a = O.rank_metadata(cu, same, 4, 1)
    b = O.rank_metadata(cu, copy, 4, 1)
    assert a["pad_between_seqs"] == b["pad_between_seqs"] == 0
    padded = np.array([0, 136], dtype=np.int32)
    assert O.rank_metadata(cu, padded, 4, 1)["pad_between_seqs"] == 1


@pytest.mark.parametrize("cp", [1, 2, 3, 4])
def test_step_tables_cover_exactly_the_causal_pairs(cp):
    """Brute force: for every step, the (query row, key row) pairs the step's
    table describes equal the causal pairs between this rank's valid query rows
    and the source shard's valid key rows."""
    rng = np.random.default_rng(100 + cp)
    for _ in range(4):
        cu, cup = _random_pack(rng, int(rng.integers(1, 4)), cp, max_chunk=4)
        valid = O.valid_mask(cu, cup)
        for r in range(cp):
            md = O.rank_metadata(cu, cup, cp, r)
            qrows = O.shard_rows(cu, cup, cp, r)
            seen = set()
            for st in md["steps"]:
                s = st["src"]
                krows = O.shard_rows(cu, cup, cp, s)
                want = set()
                for tq, gq in enumerate(qrows):
                    for tk, gk in enumerate(krows):
                        same_seq = np.searchsorted(cup, gq, side="right") == np.searchsorted(cup, gk, side="right")
                        if valid[gq] and valid[gk] and same_seq and gk <= gq:
                            want.add((tq, tk))
                got = set()
                for b in range(cu.size - 1):
                    for tq in range(st["q_start"][b], st["q_start"][b] + st["q_len"][b]):
                        for tk in range(st["kv_start"][b], st["kv_start"][b] + st["kv_len"][b]):
                            if st["kind"] != 0 or tk <= tq:
                                got.add((tq, tk))
                assert got == want, (cp, r, st["kind"], s)
                seen |= {(s, p) for p in got}
            # all steps together: each (shard, pair) once, one step per shard
            assert len({st["src"] for st in md["steps"]}) == cp


@pytest.mark.parametrize("bad", [
    dict(cu=[1, 8], cup=[1, 8], cp=1),
    dict(cu=[0, 8, 4], cup=[0, 8, 16], cp=1),
    dict(cu=[0, 9], cup=[0, 8], cp=1),
    dict(cu=[0, 6], cup=[0, 6], cp=2),
    dict(cu=[0, 8], cup=[0, 8], cp=0),
])
def test_validation_rejects(bad):
    with pytest.raises(O.OracleError):
        O.rank_metadata(np.array(bad["cu"]), np.array(bad["cup"]), bad["cp"], 0)
