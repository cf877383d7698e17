"""The host-summary metadata path (cp_attn_rank_metadata_host) validates its
inputs on the host before touching a GPU, so its answers are checked here on
the CPU against the oracle's statement of the layout's rules (cu[0] = cup[0]
= 0, both non-decreasing, L_b <= P_b, P_b divisible by 2*CP: page "Hybrid /
Hierarchical Context Parallel Skill", section "Enablement"), plus the padding
hint (page "[PyTorch][Attention] THD P2P context-parallel regression ...",
"Expected behavior": the decision is taken from values) and t_alloc.
Valid inputs get past validation and stop at the first device call (no GPU
here): status HIP, never a validation status."""
import numpy as np
import pytest

from context_packed_attention_amd import _lib, api
from oracle import cp_attn_oracle as O


def _status(cu, cup, cp, rank, hint, t_alloc):
    try:
        api.cp_attn_rank_metadata_host(cu, cup, cp, rank, hint, t_alloc, stream=0)
    except api.CpAttnError as e:
        return e.status, str(e)
    return 0, ""


def _expected(cu, cup, cp, rank, hint, t_alloc):
    cup_v = cu if cup is None else cup
    try:
        O.validate(cu, cup_v, cp, rank)
    except O.OracleError:
        return {_lib.ERR_INVALID_ARG}  # a broken rule outranks a hint mismatch
    if int(cup_v[-1]) // cp > t_alloc:
        return {_lib.ERR_INVALID_ARG}
    pad = int(not np.array_equal(np.asarray(cu), np.asarray(cup_v)))
    if hint >= 0 and hint != pad:
        return {_lib.ERR_HINT_MISMATCH}
    return {_lib.ERR_HIP}  # valid: the first device call fails on a machine without a GPU


def _cases():
    rng = np.random.default_rng(5)
    out = []
    for n in range(300):
        cp = int(rng.integers(1, 9))
        B = int(rng.integers(1, 12))
        P = [2 * cp * int(rng.integers(0, 20)) for _ in range(B)]
        L = [int(rng.integers(0, p + 1)) for p in P]
        kind = n % 6
        if kind == 1:      # a padded length not divisible by 2*CP
            P[rng.integers(0, B)] += int(rng.integers(1, 2 * cp)) if cp > 1 else 0
        elif kind == 2:    # a valid length above its padded length
            b = int(rng.integers(0, B))
            L[b] = P[b] + 1
        cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
        cup = np.concatenate([[0], np.cumsum(P)]).astype(np.int32)
        if kind == 3:      # decreasing
            cu[-1] = cu[-2] - 1 if B > 1 else -1
        if kind == 4:      # does not start at 0
            cup = cup + 2 * cp
        t_alloc = int(cup[-1]) // cp + int(rng.integers(-3, 4)) * (kind == 5)
        hint = int(rng.integers(-1, 2))
        out.append((cu, None if (kind == 0 and n % 12 == 0) else cup, cp, int(rng.integers(0, cp)), hint,
                    max(t_alloc, 0)))
    return out


def test_validation_matches_the_oracle_rules():
    seen = set()
    for cu, cup, cp, rank, hint, t_alloc in _cases():
        st, msg = _status(cu, cup, cp, rank, hint, t_alloc)
        exp = _expected(cu, cup, cp, rank, hint, t_alloc)
        assert st in exp, (cu.tolist(), None if cup is None else cup.tolist(), cp, rank, hint, t_alloc, st, msg)
        seen.add(st)
    assert {_lib.ERR_INVALID_ARG, _lib.ERR_HINT_MISMATCH, _lib.ERR_HIP} <= seen


@pytest.mark.parametrize("cu,cup,hint,t_alloc,status,words", [
    ([0, 4096], [0, 4104], 0, 1026, 3, "pad_hint"),
    ([0, 4096], None, 1, 1024, 3, "pad_hint"),
    ([0, 4090], [0, 4090], -1, 1024, 1, "divisible"),
    ([0, 4096], [0, 4096], -1, 1000, 1, "t_alloc"),
    ([0, 4096, 4000], [0, 4096, 4000], -1, 2048, 1, "non-decreasing"),
    ([0, 4200], [0, 4096], -1, 1024, 1, "exceeds"),
    ([8, 4096], [8, 4096], -1, 1024, 1, "start at 0"),
])
def test_messages_name_the_rule(cu, cup, hint, t_alloc, status, words):
    st, msg = _status(np.array(cu, np.int32), None if cup is None else np.array(cup, np.int32), 4, 1, hint, t_alloc)
    assert st == status and words in msg, msg


def test_too_many_sequences_for_the_host_path():
    B = 256
    cu = np.arange(B + 1, dtype=np.int32) * 8
    st, msg = _status(cu, cu, 4, 0, -1, int(cu[-1]) // 4)
    assert st == _lib.ERR_UNSUPPORTED and "cp_attn_rank_metadata" in msg
