"""Pins of the oracle's attention forward and backward (CPU only).

Pins: a dense brute force over an explicit mask of the whole pack; torch's
float64 CPU attention routine (out and LSE) and autograd through torch's
attention; central finite differences; closed forms (Q = 0, one-token
sequences); exact zeros on padding rows.
"""
import numpy as np
import pytest
import torch

from oracle import cp_attn_oracle as O


def _pack(rng, lengths, padded, hq, hkv, d, garbage=1000.0):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cup = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    T = int(cup[-1])
    q = rng.standard_normal((T, hq, d))
    k = rng.standard_normal((T, hkv, d))
    v = rng.standard_normal((T, hkv, d))
    do = rng.standard_normal((T, hq, d))
    valid = O.valid_mask(cu, cup)
    for x in (q, k, v, do):
        x[~valid] = garbage * rng.standard_normal(x[~valid].shape)
    return cu, cup, q, k, v, do


def _dense_brute_force(q, k, v, cu, cup, scale):
    """Whole pack as one attention with an explicit T x T mask:
    allowed[p, j] = same sequence, both valid, j <= p."""
    T, hq, d = q.shape
    group = hq // k.shape[1]
    valid = O.valid_mask(cu, cup)
    seq = np.searchsorted(cup, np.arange(T), side="right")
    allowed = (seq[:, None] == seq[None, :]) & valid[:, None] & valid[None, :] \
        & (np.arange(T)[None, :] <= np.arange(T)[:, None])
    out = np.zeros_like(q)
    lse = np.full((hq, T), -np.inf)
    for h in range(hq):
        for p in range(T):
            if not valid[p]:
                continue
            w = [np.exp(scale * float(q[p, h] @ k[j, h // group])) if allowed[p, j] else 0.0
                 for j in range(T)]
            z = float(np.sum(w))
            lse[h, p] = np.log(z)
            out[p, h] = sum(wj * v[j, h // group] for wj, j in zip(w, range(T)) if wj) / z
    return out, lse


CASES = [
    ("unpadded", [8, 4, 12], [8, 4, 12], 2, 2, 4),
    ("padded-gqa", [5, 0, 7, 1], [8, 4, 8, 4], 4, 2, 4),
]


@pytest.mark.parametrize("name,lengths,padded,hq,hkv,d", CASES)
def test_forward_vs_dense_brute_force(name, lengths, padded, hq, hkv, d):
    rng = np.random.default_rng(1)
    cu, cup, q, k, v, do = _pack(rng, lengths, padded, hq, hkv, d, garbage=3.0)
    scale = 1 / np.sqrt(d)
    out, lse = O.attention(q, k, v, do, cu, cup, scale, want_grad=False)
    bo, bl = _dense_brute_force(q, k, v, cu, cup, scale)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(bl))
    fin = np.isfinite(bl)
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=1e-12, atol=1e-12)


def _torch_reference(q, k, v, do, cu, cup, scale):
    """Per sequence: torch's fp64 CPU attention (out, LSE) and autograd grads."""
    T, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    out = np.zeros_like(q)
    lse = np.full((hq, T), -np.inf)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(cu.size - 1):
        a = int(cup[b])
        L = int(cu[b + 1] - cu[b])
        if L == 0:
            continue
        tq = torch.tensor(q[a:a + L]).permute(1, 0, 2)[None].contiguous()
        tk = torch.tensor(k[a:a + L]).permute(1, 0, 2)[None].contiguous()
        tv = torch.tensor(v[a:a + L]).permute(1, 0, 2)[None].contiguous()
        tk_r = tk.repeat_interleave(group, dim=1)
        tv_r = tv.repeat_interleave(group, dim=1)
        o, l = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
            tq, tk_r, tv_r, 0.0, True, scale=scale)[:2]
        out[a:a + L] = o[0].permute(1, 0, 2).numpy()
        lse[:, a:a + L] = l[0].numpy()
        tq.requires_grad_(True)
        tk.requires_grad_(True)
        tv.requires_grad_(True)
        o2 = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.repeat_interleave(group, dim=1), tv.repeat_interleave(group, dim=1),
            is_causal=True, scale=scale)
        tdo = torch.tensor(do[a:a + L]).permute(1, 0, 2)[None]
        (o2 * tdo).sum().backward()
        dq[a:a + L] = tq.grad[0].permute(1, 0, 2).numpy()
        dk[a:a + L] = tk.grad[0].permute(1, 0, 2).numpy()
        dv[a:a + L] = tv.grad[0].permute(1, 0, 2).numpy()
    return out, lse, dq, dk, dv


@pytest.mark.parametrize("name,lengths,padded,hq,hkv,d", CASES + [
    ("longer-gqa", [96, 40, 64], [104, 48, 64], 8, 2, 16),
])
def test_forward_backward_vs_torch(name, lengths, padded, hq, hkv, d):
    rng = np.random.default_rng(2)
    cu, cup, q, k, v, do = _pack(rng, lengths, padded, hq, hkv, d)
    scale = 1 / np.sqrt(d)
    out, lse, dq, dk, dv = O.attention(q, k, v, do, cu, cup, scale)
    ro, rl, rdq, rdk, rdv = _torch_reference(q, k, v, do, cu, cup, scale)
    np.testing.assert_allclose(out, ro, rtol=1e-11, atol=1e-11)
    fin = np.isfinite(rl)
    np.testing.assert_array_equal(np.isfinite(lse), fin)
    np.testing.assert_allclose(lse[fin], rl[fin], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dq, rdq, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dk, rdk, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dv, rdv, rtol=1e-10, atol=1e-10)
    # padding rows: exact zeros / -inf
    valid = O.valid_mask(cu, cup)
    for g in (out, dq, dk, dv):
        assert not g[~valid].any()
    assert np.all(np.isneginf(lse[:, ~valid]))


def test_backward_finite_differences():
    """Central differences of L = sum(dO * out) against the analytic gradient."""
    rng = np.random.default_rng(3)
    cu, cup, q, k, v, do = _pack(rng, [6, 3], [8, 4], 4, 2, 3, garbage=5.0)
    scale = 0.7
    _, _, dq, dk, dv = O.attention(q, k, v, do, cu, cup, scale)

    def loss(q_, k_, v_):
        o, _ = O.attention(q_, k_, v_, do, cu, cup, scale, want_grad=False)
        return float((o * do).sum())

    h = 1e-6
    valid = O.valid_mask(cu, cup)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp = x.copy()
            xm = x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name] = xp
            args_m[name] = xm
            fd = (loss(**{f"{a}_": b for a, b in args_p.items()}) -
                  loss(**{f"{a}_": b for a, b in args_m.items()})) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-7 * max(1.0, abs(g[idx])), (name, idx, fd, g[idx], valid[idx[0]])


def test_closed_form_zero_queries():
    """Q = 0: every visible key has weight 1, so lse_p = log(p + 1) and out_p is
    the mean of V over positions 0..p."""
    rng = np.random.default_rng(4)
    cu, cup, q, k, v, do = _pack(rng, [9, 16], [12, 16], 2, 1, 5)
    q[:] = 0.0
    out, lse = O.attention(q, k, v, do, cu, cup, 0.3, want_grad=False)
    for b in range(2):
        a = int(cup[b])
        L = int(cu[b + 1] - cu[b])
        for p in range(L):
            for h in range(2):
                assert abs(lse[h, a + p] - np.log(p + 1)) < 1e-13
                np.testing.assert_allclose(out[a + p, h], v[a:a + p + 1, 0].mean(axis=0), rtol=1e-13, atol=1e-13)


def test_closed_form_single_token_sequences():
    """L_b = 1: out = V_0, lse = scale * <q, k>, dQ = dK = 0, dV = dO (summed
    over the query heads that share the KV head)."""
    rng = np.random.default_rng(5)
    cu, cup, q, k, v, do = _pack(rng, [1, 1, 1], [4, 4, 4], 4, 2, 6)
    scale = 0.41
    out, lse, dq, dk, dv = O.attention(q, k, v, do, cu, cup, scale)
    for b in range(3):
        a = int(cup[b])
        for h in range(4):
            g = h // 2
            np.testing.assert_allclose(out[a, h], v[a, g], rtol=0, atol=0)
            assert abs(lse[h, a] - scale * float(q[a, h] @ k[a, g])) < 1e-14
        # dS = P (dP - D) with P = 1 and dP = D up to summation order
        assert np.abs(dq[a]).max() < 1e-13 and np.abs(dk[a]).max() < 1e-13
        np.testing.assert_allclose(dv[a, 0], do[a, 0] + do[a, 1], rtol=1e-15)
        np.testing.assert_allclose(dv[a, 1], do[a, 2] + do[a, 3], rtol=1e-15)


def test_lse_gradient_is_softmax_average_of_keys():
    """d lse_p / d q_p = scale * sum_j P_pj K_j, i.e. scale * out_p with V := K.
    Central differences of the oracle's lse against its own out with V = K
    tie the LSE's normalisation to the attention weights."""
    rng = np.random.default_rng(6)
    cu, cup, q, k, v, do = _pack(rng, [7], [8], 1, 1, 4)
    scale = 0.8
    out_k, _ = O.attention(q, k, k, do, cu, cup, scale, want_grad=False)
    h = 1e-6
    for p in range(7):
        for dd in range(4):
            qp = q.copy()
            qm = q.copy()
            qp[p, 0, dd] += h
            qm[p, 0, dd] -= h
            _, lp = O.attention(qp, k, v, do, cu, cup, scale, want_grad=False)
            _, lm = O.attention(qm, k, v, do, cu, cup, scale, want_grad=False)
            fd = (lp[0, p] - lm[0, p]) / (2 * h)
            assert abs(fd - scale * out_k[p, 0, dd]) < 1e-8
