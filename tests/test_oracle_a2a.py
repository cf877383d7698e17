"""Pins for the oracle's hierarchical (a2a + p2p) all-to-all permutation.

The main pin ties it to two independently defined shard maps: sharding a
global packed tensor at CP = A * P and then applying group p's all-to-all must
give the p2p-level shard of rank p (sharding the same tensor at CP = P),
split by heads across the group ("Hybrid / Hierarchical Context Parallel
Skill", "Enablement": CP = a2a size x p2p size, lengths divisible by 2*CP).
Also: the inverse undoes it, A = 1 is the identity, invalid sizes raise, and
a planted mistake (the mirrored chunks taken in the wrong order) fails the
main pin."""
import numpy as np
import pytest

from oracle import cp_attn_oracle as O


def _pack(rng, B, cp, max_mult=6, empty_ok=True):
    P = [2 * cp * int(rng.integers(0 if empty_ok else 1, max_mult + 1)) for _ in range(B)]
    L = [int(rng.integers(0, p + 1)) for p in P]
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
    cup = np.concatenate([[0], np.cumsum(P)]).astype(np.int64)
    return cu, cup


CASES = [(2, 1), (2, 2), (4, 2), (2, 4), (3, 2), (8, 1), (4, 4)]


@pytest.mark.parametrize("A,P", CASES)
def test_a2a_equals_p2p_level_shard_split_by_heads(A, P):
    rng = np.random.default_rng(100 * A + P)
    cp = A * P
    H = 2 * A
    for trial in range(3):
        cu, cup = _pack(rng, int(rng.integers(1, 7)), cp)
        T = int(cup[-1])
        X = rng.integers(-1000, 1000, size=(T, H, 3)).astype(np.int64)
        for p in range(P):
            xs = [O.gather_shard(X, cu, cup, cp, p * A + a) for a in range(A)]
            ys = O.a2a_seq_to_head(xs, cup, cp, A, p)
            want = O.gather_shard(X, cu, cup, P, p)
            hs = H // A
            for a in range(A):
                assert np.array_equal(ys[a], want[:, a * hs:(a + 1) * hs]), (A, P, p, a)
            back = O.a2a_head_to_seq(ys, cup, cp, A, p)
            for a in range(A):
                assert np.array_equal(back[a], xs[a]), (A, P, p, a)


def test_a2a_of_one_is_identity():
    rng = np.random.default_rng(5)
    cu, cup = _pack(rng, 4, 3)
    X = rng.integers(-9, 9, size=(int(cup[-1]), 2, 4))
    for r in range(3):
        x = O.gather_shard(X, cu, cup, 3, r)
        (y,) = O.a2a_seq_to_head([x], cup, 3, 1, r)
        assert np.array_equal(y, x)


def test_a2a_rejects_invalid_sizes():
    cup = np.array([0, 16, 48])
    xs = [np.zeros((12, 4, 1))] * 2
    with pytest.raises(O.OracleError):
        O.a2a_seq_to_head(xs, cup, 4, 3, 0)  # cp not a multiple of A
    with pytest.raises(O.OracleError):
        O.a2a_seq_to_head(xs, cup, 4, 2, 2)  # p2p rank out of range
    with pytest.raises(O.OracleError):
        O.a2a_seq_to_head(xs, np.array([0, 12]), 4, 2, 0)  # 12 % (2*4) != 0
    with pytest.raises(O.OracleError):
        O.a2a_seq_to_head([np.zeros((12, 3, 1))] * 2, cup, 4, 2, 0)  # heads % A != 0


def test_planted_mirror_order_mistake_is_caught():
    """The mirrored chunks taken from CP rank pA + j instead of pA + A-1-j."""
    def wrong(xs, cup, cp, A, p):
        H = xs[0].shape[1]
        T_local = int(cup[-1]) // cp
        rows = np.zeros((A * T_local,) + xs[0].shape[1:], dtype=xs[0].dtype)
        for base_cp, base_p, c in O._a2a_slots(cup, cp, A, p):
            for j in range(A):
                rows[base_p + j * c: base_p + (j + 1) * c] = xs[j][base_cp: base_cp + c]
                rows[base_p + (A + j) * c: base_p + (A + j + 1) * c] = xs[j][base_cp + c: base_cp + 2 * c]
        hs = H // A
        return [rows[:, a * hs:(a + 1) * hs] for a in range(A)]

    rng = np.random.default_rng(9)
    A, P = 2, 2
    cp = A * P
    cu, cup = _pack(rng, 3, cp, empty_ok=False)
    X = rng.integers(-1000, 1000, size=(int(cup[-1]), 2 * A, 2))
    xs = [O.gather_shard(X, cu, cup, cp, a) for a in range(A)]
    want = O.gather_shard(X, cu, cup, P, 0)
    ok = O.a2a_seq_to_head(xs, cup, cp, A, 0)
    bad = wrong(xs, cup, cp, A, 0)
    assert np.array_equal(ok[0], want[:, :2])
    assert not np.array_equal(bad[0], want[:, :2])
