"""Pin for the bf16 comparison bar of the GPU parity tests
(tests/gpu_harness.py::compare_bf16): |got - ref| <= max(2e-2, 2 ulp(ref)).

The interface fixes three roundings that no implementation of it can avoid:
the backward receives the forward's output in bf16, so D = rowsum(dO * out)
sees a rounded out; P and dS enter the dV / dK / dQ contractions as bf16
matrix-core operands; and the gradients are stored in bf16. Here a result
that takes exactly those roundings and nothing else is computed in fp64 from
the plain definition, on a pack whose gradients accumulate over a GQA group of
8 query heads, and compared with the exact gradients:

* below |ref| = 2 it stays within the stated 2e-2, so the bar there is 2e-2;
* at |ref| >= 2 it passes one bf16 ulp, so a one-ulp bar would fail every
  implementation, and it stays within two ulps, the bar used there.
"""
import math

import numpy as np

from context_packed_attention_amd import synth
from oracle import cp_attn_oracle as O


def _round_bf16(x):
    bits = synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    return O.bf16_to_f64(bits)


def _ulp(x):
    return 2.0 ** (np.floor(np.log2(np.maximum(np.abs(x), 1e-300))) - 7)


def _forced_rounding_errors():
    L, hq, hkv, d = [700, 300], 8, 1, 128
    bt = synth.make_batch("gqa8-cp2-d128", 29, L, L, hq, hkv, d)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = (O.bf16_to_f64(x) for x in (bt.q, bt.k, bt.v, bt.do))
    ref, got = [], []
    for b, n in enumerate(L):
        s0 = int(bt.cup[b])
        K, V = k[s0:s0 + n, 0], v[s0:s0 + n, 0]
        dk_e, dv_e, dk_r, dv_r = (np.zeros((n, d)) for _ in range(4))
        for h in range(hq):
            Q, dO = q[s0:s0 + n, h], do[s0:s0 + n, h]
            S = scale * (Q @ K.T)
            S[np.triu_indices(n, 1)] = -np.inf
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            out = P @ V
            dP = dO @ V.T
            dS = P * (dP - (dO * out).sum(axis=1, keepdims=True))
            dS_r = _round_bf16(P * (dP - (dO * _round_bf16(out)).sum(axis=1, keepdims=True)))
            dq_e, dq_r = scale * (dS @ K), scale * (dS_r @ K)
            ref.append(dq_e)
            got.append(_round_bf16(dq_r))
            dk_e += scale * (dS.T @ Q)
            dk_r += scale * (dS_r.T @ Q)
            dv_e += P.T @ dO
            dv_r += _round_bf16(P).T @ dO
        ref += [dk_e, dv_e]
        got += [_round_bf16(dk_r), _round_bf16(dv_r)]
    ref = np.concatenate([r.ravel() for r in ref])
    got = np.concatenate([g.ravel() for g in got])
    return ref, np.abs(got - ref)


def test_forced_roundings_need_two_ulps_above_two_and_fit_2e_2_below():
    ref, err = _forced_rounding_errors()
    small = np.abs(ref) < 2
    assert small.any() and (~small).any()
    assert err[small].max() <= 2e-2
    over = err[~small] / _ulp(ref[~small])
    assert over.max() > 1.0, "a one-ulp bar would already hold; the two-ulp allowance is not needed"
    assert over.max() <= 2.0
