"""Edge cases of a rank share against the fp64 oracle, forward (out, LSE) and
backward (dQ, every dK/dV part), every rank: the largest ring (CP = 16), a
CP = 8 ragged pack, a pack with no valid token at all (every output row is
padding: out, dQ, dK, dV exactly 0 and LSE -inf), many one-token sequences,
a GQA group of 8 query heads per KV head, and (forward) scores spread over
hundreds of nats (Q and K scaled by 16, exact in bf16: the online softmax's
running max must be the true row max, or exp2 overflows). Tolerances as in the other
parity tests (bf16 max-abs 2e-2 or two ulps, relative L2 1e-2; LSE 1e-3
relative)."""
import numpy as np
import pytest

from context_packed_attention_amd import synth
from oracle import cp_attn_oracle as O
from tests import test_gpu_bwd as TB
from tests import test_gpu_fwd as TF

pytestmark = pytest.mark.gpu


def _ragged(seed, B, lo, hi, mult):
    rng = np.random.default_rng(seed)
    L = [int(x) for x in rng.integers(lo, hi, B)]
    P = [((x + mult - 1) // mult) * mult if x else mult * int(rng.integers(0, 2)) for x in L]
    return L, P


CASES = [
    # name, lengths, padded, cp, hq, hkv, d
    ("cp16-max-d64", [100, 33, 0, 250], [128, 64, 32, 256], 16, 2, 2, 64),
    ("cp8-ragged-d64",) + tuple(_ragged(5, 9, 0, 300, 16)) + (8, 2, 1, 64),
    ("all-padding-cp2", [0, 0, 0], [16, 32, 4], 2, 2, 1, 128),
    ("one-token-seqs-cp4", [1] * 24, [8] * 24, 4, 4, 4, 128),
    ("gqa8-cp2-d128", [700, 300], [700, 300], 2, 8, 1, 128),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_edge_fwd_bwd(case):
    name, L, P, cp, hq, hkv, d = case
    bt = synth.make_batch(name, 29, L, P, hq, hkv, d)
    TF._check_fwd(bt, cp, range(cp))
    TB._check_bwd(bt, cp, range(cp), tail=5)


def test_large_scores_fwd():
    """Forward only: the running max is a forward concern. (With the softmax
    this close to one-hot, dS = P (dP - D) is a difference of nearly equal
    numbers and D can only be formed from the bf16 out the backward
    receives, so the backward's error there is set by that rounding, not by
    the kernels.)"""
    L, P = [900, 130], [904, 136]
    bt = synth.make_batch("large-scores-cp2", 31, L, P, 4, 2, 128)
    for name in ("q", "k"):
        x = O.bf16_to_f64(getattr(bt, name)) * 16.0  # a power of two: exact in bf16
        setattr(bt, name, synth.f32_to_bf16_bits(x.astype(np.float32)))
    TF._check_fwd(bt, 2, range(2))
