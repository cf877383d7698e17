"""Seeded random shares against the oracle, forward and backward, every rank:
CP 1..8, head_dim 64 / 128, GQA ratios 1..8, ragged packs with empty and
one-token sequences, inter-sequence padding or none, with and without a row
tail. Same bars as the other parity tests."""
import numpy as np
import pytest

from context_packed_attention_amd import synth
from tests import test_gpu_bwd as TB
from tests import test_gpu_fwd as TF

pytestmark = pytest.mark.gpu


def _case(i):
    rng = np.random.default_rng(7000 + i)
    cp = int(rng.choice([1, 2, 3, 4, 5, 8]))
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 7))
    unit = 2 * cp
    L, P = [], []
    for _ in range(B):
        kind = rng.random()
        Lb = 0 if kind < 0.1 else (1 if kind < 0.2 else int(rng.integers(2, 700)))
        pad = int(rng.integers(0, 40)) if rng.random() < 0.5 else 0
        L.append(Lb)
        P.append(((Lb + pad + unit - 1) // unit) * unit)
    tail = int(rng.choice([0, 0, 9]))
    return f"rand{i}-cp{cp}-d{d}-h{hq}x{hkv}", L, P, cp, hq, hkv, d, tail


CASES = [_case(i) for i in range(16)]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_random_share(case):
    name, L, P, cp, hq, hkv, d, tail = case
    bt = synth.make_batch(name, 61, L, P, hq, hkv, d)
    TF._check_fwd(bt, cp, range(cp), tail=tail)
    TB._check_bwd(bt, cp, range(cp), tail=tail)
