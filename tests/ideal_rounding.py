"""An ideal bf16 implementation of a rank's share, for judging the GPU's
rounding error (test infrastructure, not the method): float64 throughout,
except for the roundings the interface forces on any implementation:

* the unnormalised probabilities enter P V as a bf16 matrix operand, and the
  output is stored in bf16;
* D = rowsum(dO * out) is formed from that bf16 output;
* P enters P^T dO and dS = P (dP - D) enters dS K and dS^T Q as bf16
  operands;
* every result is stored in bf16.

Where the GPU exceeds the flat max-abs 2e-2 on some element, the parity tests
record this implementation's figures on the same inputs beside the GPU's.
"""
from __future__ import annotations

import numpy as np

from context_packed_attention_amd import synth
from oracle import cp_attn_oracle as O


def round_bf16(x):
    bits = synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    return O.bf16_to_f64(bits)


def ideal_share(bt, cp: int, r: int, scale: float, p_offset: float = 0.0) -> dict:
    """Rank r's share (out, dq in r's local layout; dk / dv parts per source
    shard) with only the forced roundings. ``p_offset`` shifts the exponent
    of the unnormalised probabilities (every row's P~ multiplied by
    e^p_offset before its bf16 rounding): any such scaling is an equally valid
    implementation and gives another realisation of the same roundings."""
    q, k, v, do = (O.bf16_to_f64(x) for x in (bt.q, bt.k, bt.v, bt.do))
    T, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    rank_of, _ = O.owner_map(bt.cu, bt.cup, cp)
    out = np.zeros((T, hq, d))
    dq = np.zeros((T, hq, d))
    dk = np.zeros((T, hkv, d))
    dv = np.zeros((T, hkv, d))
    for b in range(bt.cu.size - 1):
        s0, n = int(bt.cup[b]), int(bt.cu[b + 1] - bt.cu[b])
        pos = np.nonzero(rank_of[s0:s0 + n] == r)[0]
        if pos.size == 0:
            continue
        for h in range(hq):
            g = h // group
            K, V = k[s0:s0 + n, g], v[s0:s0 + n, g]
            Q, dO = q[s0 + pos, h], do[s0 + pos, h]
            S = scale * (Q @ K.T)
            S = np.where(np.arange(n)[None, :] <= pos[:, None], S, -np.inf)
            Pt = np.exp(S - S.max(axis=1, keepdims=True) + p_offset)
            lsum = Pt.sum(axis=1, keepdims=True)
            out_b = round_bf16((round_bf16(Pt) @ V) / lsum)
            P = Pt / lsum
            dS_b = round_bf16(P * (dO @ V.T - (dO * out_b).sum(axis=1, keepdims=True)))
            out[s0 + pos, h] = out_b
            dq[s0 + pos, h] = round_bf16(scale * (dS_b @ K))
            dk[s0:s0 + n, g] += scale * (dS_b.T @ Q)
            dv[s0:s0 + n, g] += round_bf16(P).T @ dO
    dk = round_bf16(dk)
    dv = round_bf16(dv)
    own = O.shard_rows(bt.cu, bt.cup, cp, r)
    return {"out": out[own], "dq": dq[own],
            "dk_parts": [dk[O.shard_rows(bt.cu, bt.cup, cp, s)] for s in range(cp)],
            "dv_parts": [dv[O.shard_rows(bt.cu, bt.cup, cp, s)] for s in range(cp)]}


def flat_figures(got: np.ndarray, ref: np.ndarray) -> dict:
    err = np.abs(got - ref)
    small = np.abs(ref) < 2.0
    return {"n_over_2e-2": int((err > 2e-2).sum()), "max_abs": float(err.max()) if err.size else 0.0,
            "n_over_2e-2_ref_lt_2": int((err[small] > 2e-2).sum()),
            "max_abs_ref_lt_2": float(err[small].max()) if small.any() else 0.0}
