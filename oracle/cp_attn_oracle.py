"""fp64 CPU oracle for one context-parallel rank's share of packed causal attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module. The product path never
does; it shares no code with this file.

What is computed is the plain definition, written out slowly in float64 numpy:

* Packed ("thd") layout with inter-sequence padding, the per-rank
  sequence-length metadata and the value-based padding decision: page "[PyTorch]
  [Attention] THD P2P context-parallel regression when padded cu_seqlens are
  value-equal but not object-identical", sections "Describe the bug" and
  "Expected behavior".
* Load-balanced sharding into 2*CP chunks per sequence, rank r holding chunks r
  and 2*CP-1-r: the divisibility rule is on page "Hybrid / Hierarchical Context
  Parallel Skill", section "Enablement"; the chunk assignment itself is the
  standard zig-zag reading (the pages do not spell it out).
* Causal softmax attention forward (out, natural-log LSE) and its exact
  gradient: not on the pages; the textbook definition.
* The hierarchical (a2a + p2p) front end's all-to-all of one a2a group, as a
  row / head permutation: page "Hybrid / Hierarchical Context Parallel Skill",
  sections "Enablement" and "Implementation Map" (CP = a2a size x p2p size);
  the rank numbering inside the group is a reading, stated where it is coded.
* The all-gather variant's layout of a rank's dK/dV contribution (every key row
  of the packed batch in global order): the same page, section "Implementation
  Map", names "all_gather" among the communication types; the layout is a
  reading (the rank holds the gathered K/V).

Readings taken where the pages are silent (each is listed in the design notes):
padding sits at the end of each sequence's padded slot; valid rows fill the
2*CP chunks in order; LSE is natural log, laid out [heads, rows]; padding rows
get out = 0, lse = -inf and zero gradients; query head h uses KV head
h // (Hq / Hkv); the dK/dV "part" for shard s is the contribution of this
rank's query rows only.

Parity is pinned by the "not gpu" tests: brute force over an explicit mask of
the whole pack, torch's fp64 CPU attention routine (out and LSE) and autograd,
central finite differences, closed forms and the all-ranks invariants (the
gathered-layout contributions of all ranks sum to the whole pack's gradient); the
all-to-all by the identity "CP-level shards, then the group's all-to-all =
the p2p-level shard, split by heads" and its inverse.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


class OracleError(ValueError):
    pass


# ---------------------------------------------------------------------------
# inputs
# ---------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def validate(cu, cup, cp: int, rank: int | None = None):
    """Argument rules of the packed CP layout.

    cu[0] = cup[0] = 0, both non-decreasing, 0 <= L_b <= P_b, and every padded
    length divisible by 2*CP (page "Hybrid / Hierarchical Context Parallel
    Skill", section "Enablement": sequence length must divide by 2*CP).
    """
    cu = np.asarray(cu, dtype=np.int64)
    cup = np.asarray(cup, dtype=np.int64)
    if cp < 1:
        raise OracleError("cp_size must be >= 1")
    if rank is not None and not (0 <= rank < cp):
        raise OracleError("cp_rank out of range")
    if cu.ndim != 1 or cup.shape != cu.shape or cu.size < 1:
        raise OracleError("cu_seqlens and cu_seqlens_padded must be [B+1]")
    if cu[0] != 0 or cup[0] != 0:
        raise OracleError("cu_seqlens must start at 0")
    L = np.diff(cu)
    P = np.diff(cup)
    if (L < 0).any() or (P < 0).any():
        raise OracleError("cu_seqlens must be non-decreasing")
    if (L > P).any():
        raise OracleError("valid length exceeds padded length")
    if (P % (2 * cp)).any():
        raise OracleError("padded length not divisible by 2*cp")
    return cu, cup


# ---------------------------------------------------------------------------
# sharding (where each global row goes)
# ---------------------------------------------------------------------------

def owner_map(cu, cup, cp: int):
    """For every global row: (owning rank, local row on that rank).

    Sequence b's padded slot [cup[b], cup[b+1]) is cut into 2*CP chunks of
    c_b = P_b / (2*CP) rows. Chunk k belongs to rank k if k < CP and to rank
    2*CP-1-k otherwise; on its rank the two chunks are stored in increasing
    chunk order, the sequence's pair of chunks starting at local row
    cup[b] / CP.
    """
    cu, cup = validate(cu, cup, cp)
    T = int(cup[-1])
    rank = np.empty(T, dtype=np.int64)
    local = np.empty(T, dtype=np.int64)
    for b in range(cup.size - 1):
        P = int(cup[b + 1] - cup[b])
        c = P // (2 * cp)
        for q in range(P):
            k = q // c
            o = q % c
            g = int(cup[b]) + q
            if k < cp:
                rank[g] = k
                local[g] = int(cup[b]) // cp + o
            else:
                rank[g] = 2 * cp - 1 - k
                local[g] = int(cup[b]) // cp + c + o
    return rank, local


def shard_rows(cu, cup, cp: int, s: int) -> np.ndarray:
    """Global row index held at each local row of rank (= shard) s."""
    rank, local = owner_map(cu, cup, cp)
    T_local = int(cup[-1]) // cp
    rows = np.full(T_local, -1, dtype=np.int64)
    sel = np.nonzero(rank == s)[0]
    rows[local[sel]] = sel
    if (rows < 0).any():
        raise OracleError("owner map does not cover every local row")
    return rows


def valid_mask(cu, cup) -> np.ndarray:
    """True for global rows holding a real token (not a padding slot)."""
    cu = np.asarray(cu, dtype=np.int64)
    cup = np.asarray(cup, dtype=np.int64)
    m = np.zeros(int(cup[-1]), dtype=bool)
    for b in range(cu.size - 1):
        m[cup[b]:cup[b] + (cu[b + 1] - cu[b])] = True
    return m


def gather_shard(x: np.ndarray, cu, cup, cp: int, s: int) -> np.ndarray:
    """Rows of a global packed array that rank s holds, in its local order."""
    return x[shard_rows(cu, cup, cp, s)]


# ---------------------------------------------------------------------------
# hierarchical (a2a + p2p) front end: the all-to-all of one a2a group
# ---------------------------------------------------------------------------
# Page "Hybrid / Hierarchical Context Parallel Skill", sections "Enablement"
# and "Implementation Map": CP = a2a size x p2p size, sequence lengths divide
# by 2*CP. Reading (the pages do not spell out the numbering): the a2a groups
# are runs of consecutive CP ranks, CP rank c = p * A + a for p2p rank p and
# a2a rank a. The group's CP chunks {pA .. pA+A-1} and their mirrors are then
# exactly the p2p-level chunks p and 2P-1-p (a p2p-level chunk is A
# consecutive CP-level chunks), and the all-to-all trades the sequence split
# inside the group for a head split: a2a rank a' ends with heads
# [a' H/A, (a'+1) H/A) of the p2p rank's rows.

def _a2a_slots(cup, cp: int, a2a: int, p: int):
    """(sequence start in CP-local rows, in p2p-local rows, CP chunk rows)."""
    cup = np.asarray(cup, dtype=np.int64)
    if cp % a2a:
        raise OracleError("cp must be a multiple of the a2a size")
    P = cp // a2a
    if not 0 <= p < P:
        raise OracleError("p2p rank out of range")
    for b in range(cup.size - 1):
        if (cup[b + 1] - cup[b]) % (2 * cp):
            raise OracleError("padded lengths must divide by 2*CP")
        yield int(cup[b]) // cp, int(cup[b]) // P, int(cup[b + 1] - cup[b]) // (2 * cp)


def a2a_seq_to_head(xs, cup, cp: int, a2a: int, p: int):
    """All-to-all of a2a group p. xs[a] holds the CP-local rows of CP rank
    p*A + a, all heads, [>= T_local, H, ...]. Returns A arrays: entry a' holds
    heads [a' H/A, (a'+1) H/A) of p2p rank p's local rows (per sequence, CP
    chunks pA, .., pA+A-1 and then their mirrors 2CP-1-(pA+A-1), .., 2CP-1-pA),
    [A * T_local, H/A, ...]."""
    A = a2a
    H = xs[0].shape[1]
    if H % A:
        raise OracleError("heads must divide by the a2a size")
    T_local = int(np.asarray(cup)[-1]) // cp
    rows = np.zeros((A * T_local,) + xs[0].shape[1:], dtype=xs[0].dtype)
    for base_cp, base_p, c in _a2a_slots(cup, cp, A, p):
        for j in range(A):
            # first half: CP chunk pA + j = first chunk of CP rank pA + j
            rows[base_p + j * c: base_p + (j + 1) * c] = xs[j][base_cp: base_cp + c]
            # second half: CP chunk 2CP-1-(pA+A-1-j) = second chunk of CP rank pA + A-1-j
            rows[base_p + (A + j) * c: base_p + (A + j + 1) * c] = xs[A - 1 - j][base_cp + c: base_cp + 2 * c]
    hs = H // A
    return [rows[:, a * hs:(a + 1) * hs].copy() for a in range(A)]


def a2a_head_to_seq(ys, cup, cp: int, a2a: int, p: int):
    """The inverse all-to-all (gradients back to the sequence split): ys[a']
    holds heads a' of p2p rank p's local rows, [A * T_local, H/A, ...];
    returns A arrays [T_local, H, ...], entry a = CP rank p*A + a."""
    A = a2a
    hs = ys[0].shape[1]
    T_local = int(np.asarray(cup)[-1]) // cp
    full = np.concatenate(ys, axis=1)  # [A T_local, H, ...], heads in a2a-rank order
    xs = [np.zeros((T_local,) + full.shape[1:], dtype=full.dtype) for _ in range(A)]
    for base_cp, base_p, c in _a2a_slots(cup, cp, A, p):
        for j in range(A):
            xs[j][base_cp: base_cp + c] = full[base_p + j * c: base_p + (j + 1) * c]
            xs[A - 1 - j][base_cp + c: base_cp + 2 * c] = full[base_p + (A + j) * c: base_p + (A + j + 1) * c]
    del hs
    return xs


# ---------------------------------------------------------------------------
# per-rank metadata (integers, exact)
# ---------------------------------------------------------------------------

def _chunk_valid(L: int, c: int, k: int) -> int:
    """Valid rows in chunk k of a sequence with L valid rows and chunk size c:
    valid tokens fill the chunks in order, so this is clamp(L - k*c, 0, c)."""
    return max(0, min(c, L - k * c))


def step_kind(cp: int, r: int, i: int) -> tuple[int, int]:
    """(kind, source shard) of ring step i on rank r.

    The shard arriving at step i comes from rank s = (r - i) mod CP. Local rows
    are [chunk r | chunk 2CP-1-r] with increasing global position, so:
    kind 0 (i == 0): own shard, plain causal mask on local rows;
    kind 1 (s < r): all query rows see only chunk s (the first half of shard s),
        with no mask (chunk s precedes both query chunks, chunk 2CP-1-s follows);
    kind 2 (s > r): only the second query chunk sees all of shard s, with no mask.
    """
    s = (r - i) % cp
    if i == 0:
        return 0, s
    return (1 if s < r else 2), s


def rank_metadata(cu, cup, cp: int, r: int, t_alloc: int | None = None) -> dict:
    """Per-rank sequence tables of rank r (all int64 numpy arrays).

    The inter-sequence padding decision is taken from the values of the two
    cumulative-length arrays, never from whether they are the same object
    (page "[PyTorch][Attention] THD P2P context-parallel regression ...",
    sections "Describe the bug" and "Expected behavior").
    """
    cu, cup = validate(cu, cup, cp, r)
    B = cu.size - 1
    L = np.diff(cu)
    P = np.diff(cup)
    c = P // (2 * cp)
    T_local = int(cup[-1]) // cp
    md = {
        "B": B, "cp": cp, "rank": r, "t_local": T_local,
        "pad_between_seqs": int(bool((cu != cup).any())),
        "has_tail": int(t_alloc is not None and t_alloc > T_local),
        "chunk": c.copy(),
        "cu_padded_local": cup // cp,
        "cu_padded_half": cup // (2 * cp),
    }

    def excl_cumsum(x):
        out = np.zeros(B + 1, dtype=np.int64)
        out[1:] = np.cumsum(x)
        return out

    first, second = {}, {}
    for s in range(cp):
        f = np.array([_chunk_valid(int(L[b]), int(c[b]), s) for b in range(B)], dtype=np.int64)
        sc = np.array([_chunk_valid(int(L[b]), int(c[b]), 2 * cp - 1 - s) for b in range(B)], dtype=np.int64)
        first[s], second[s] = f, sc
        md[f"cu_full_{s}"] = excl_cumsum(f + sc)
        md[f"cu_first_{s}"] = excl_cumsum(f)
        md[f"cu_second_{s}"] = excl_cumsum(sc)
    base = cup[:-1] // cp
    steps = []
    for i in range(cp):
        kind, s = step_kind(cp, r, i)
        q_start = base + (c if kind == 2 else 0)
        q_len = second[r] if kind == 2 else first[r] + second[r]
        kv_start = base.copy()
        kv_len = first[s] if kind == 1 else first[s] + second[s]
        steps.append({"kind": kind, "src": s, "q_start": q_start, "q_len": q_len,
                      "kv_start": kv_start, "kv_len": kv_len})
    md["steps"] = steps
    return md


# ---------------------------------------------------------------------------
# attention (plain definition, float64)
# ---------------------------------------------------------------------------

def _attend_sequence(qh, kh, vh, doh, pos, scale, want_grad):
    """One sequence, one query head.

    qh: [n, D] queries at in-sequence positions ``pos`` (int array, length n);
    kh, vh: [L, D] keys/values of the whole sequence; doh: [n, D] or None.
    Query at position p sees keys j <= p.
    Returns out [n, D], lse [n] and, if asked, (dq [n, D], dk [L, D], dv [L, D]).
    """
    L = kh.shape[0]
    s = scale * (qh @ kh.T)                                   # [n, L]
    allowed = np.arange(L)[None, :] <= pos[:, None]
    s = np.where(allowed, s, NEG_INF)
    m = s.max(axis=1)
    lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    p = np.exp(s - lse[:, None])                              # 0 where masked
    out = p @ vh
    if not want_grad:
        return out, lse, None
    dp = doh @ vh.T                                           # [n, L]
    dcoef = (doh * out).sum(axis=1)                           # D_p = <dO_p, out_p>
    ds = p * (dp - dcoef[:, None])
    dq = scale * (ds @ kh)
    dk = scale * (ds.T @ qh)
    dv = p.T @ doh
    return out, lse, (dq, dk, dv)


def attention(q, k, v, do, cu, cup, scale, query_mask=None, want_grad=True,
              max_elems: int = 1 << 25):
    """Packed causal attention over global rows, float64.

    q, k, v, do are float64 global packed arrays ([T, Hq, D], [T, Hkv, D],
    [T, Hkv, D], [T, Hq, D]). Only the query rows where ``query_mask`` is True
    (default: all valid rows) are computed; keys are every valid row of the
    same sequence at or before the query. The gradient is that of
    sum(do * out) over the selected query rows, so dK/dV collect only those
    rows' contributions.

    Returns out [T, Hq, D] (0 outside the selection), lse [Hq, T] (-inf
    outside), and if ``want_grad``: dq [T, Hq, D], dk, dv [T, Hkv, D].
    Query rows are processed in batches of at most ``max_elems`` scores; this
    splits only the outer loop, every row's sums stay whole.
    """
    cu = np.asarray(cu, dtype=np.int64)
    cup = np.asarray(cup, dtype=np.int64)
    T, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise OracleError("Hq must be a multiple of Hkv")
    group = hq // hkv
    vm = valid_mask(cu, cup)
    if query_mask is None:
        query_mask = vm
    query_mask = query_mask & vm
    out = np.zeros((T, hq, d))
    lse = np.full((hq, T), NEG_INF)
    if want_grad:
        dq = np.zeros((T, hq, d))
        dk = np.zeros((T, hkv, d))
        dv = np.zeros((T, hkv, d))
    for b in range(cu.size - 1):
        base = int(cup[b])
        Lb = int(cu[b + 1] - cu[b])
        if Lb == 0:
            continue
        rows = np.nonzero(query_mask[base:base + Lb])[0]     # in-sequence positions
        if rows.size == 0:
            continue
        step = max(1, max_elems // Lb)
        for h in range(hq):
            g = h // group
            kh = k[base:base + Lb, g]
            vh = v[base:base + Lb, g]
            for a in range(0, rows.size, step):
                pos = rows[a:a + step]
                o, l, gr = _attend_sequence(q[base + pos, h], kh, vh,
                                            do[base + pos, h] if want_grad else None,
                                            pos, scale, want_grad)
                out[base + pos, h] = o
                lse[h, base + pos] = l
                if want_grad:
                    dq[base + pos, h] = gr[0]
                    dk[base:base + Lb, g] += gr[1]
                    dv[base:base + Lb, g] += gr[2]
    if want_grad:
        return out, lse, dq, dk, dv
    return out, lse


def share(q_bits, k_bits, v_bits, do_bits, cu, cup, cp: int, r: int, scale: float,
          want_grad: bool = True):
    """Rank r's share: its query rows against every key, in r's local layout.

    Returns a dict with out [T_local, Hq, D], lse [Hq, T_local], and if asked
    dq [T_local, Hq, D] and dk_parts / dv_parts: a list over source shards s of
    [T_local, Hkv, D] arrays, the contribution of r's query rows to the
    gradient of shard s's keys and values, in shard s's local layout; plus
    dk_full / dv_full [T, Hkv, D]: the same contribution for every key row of
    the packed batch in its global order (the all-gather variant's layout:
    rank r holds the gathered K/V, page "Hybrid / Hierarchical Context
    Parallel Skill", section "Implementation Map", names "all_gather" as a
    communication type).
    Inputs are bf16 bit arrays in the global packed layout.
    """
    cu, cup = validate(cu, cup, cp, r)
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(k_bits)
    v = bf16_to_f64(v_bits)
    do = bf16_to_f64(do_bits) if want_grad else None
    rank_of, _ = owner_map(cu, cup, cp)
    res = attention(q, k, v, do if want_grad else np.zeros_like(q), cu, cup, scale,
                    query_mask=(rank_of == r), want_grad=want_grad)
    own = shard_rows(cu, cup, cp, r)
    outd = {"out": res[0][own], "lse": res[1][:, own]}
    if want_grad:
        outd["dq"] = res[2][own]
        outd["dk_parts"] = [res[3][shard_rows(cu, cup, cp, s)] for s in range(cp)]
        outd["dv_parts"] = [res[4][shard_rows(cu, cup, cp, s)] for s in range(cp)]
        outd["dk_full"] = res[3]
        outd["dv_full"] = res[4]
    return outd


BF16_UNIT_ROUNDOFF = 2.0 ** -8   # round-to-nearest-even, 8-bit significand


def share_rounding_sd(q_bits, k_bits, v_bits, do_bits, cu, cup, cp: int, r: int, scale: float):
    """Tolerance model for comparing a bf16 implementation with this oracle
    (not part of the method): the standard deviation, per element of rank r's
    share, of the error that three roundings forced by the interface induce,
    each taken as an independent unbiased relative error of variance u^2 / 3
    (u = 2^-8, bf16):

    * P enters the P V and P^T dO contractions as a bf16 matrix operand;
    * dS = P (dP - D) enters dS K and dS^T Q as a bf16 operand;
    * D = rowsum(dO * out) is formed from the output the backward receives,
      which carries its own bf16 rounding and that of P in P V, so D_i
      carries var_D = u^2/3 (sum_d dO_id^2 out_id^2 + sum_j P_ij^2 dP_ij^2);
      it reaches dQ_i through -scale D_i sum_j P_ij K_j (one error per row)
      and dK_j through -scale sum_i P_ij D_i Q_i (independent per row i).

    Returns {"out", "dq": [T_local, Hq, D], "dk_parts", "dv_parts": lists of
    [T_local, Hkv, D]} in rank r's / shard s's local layouts, and "dk_full",
    "dv_full" [T, Hkv, D] in the global order (0 where an element is not
    computed).
    """
    cu, cup = validate(cu, cup, cp, r)
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(k_bits)
    v = bf16_to_f64(v_bits)
    do = bf16_to_f64(do_bits)
    T, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    c = BF16_UNIT_ROUNDOFF ** 2 / 3.0
    rank_of, _ = owner_map(cu, cup, cp)
    var_out = np.zeros((T, hq, d))
    var_dq = np.zeros((T, hq, d))
    var_dk = np.zeros((T, hkv, d))
    var_dv = np.zeros((T, hkv, d))
    for b in range(cu.size - 1):
        base = int(cup[b])
        Lb = int(cu[b + 1] - cu[b])
        pos = np.nonzero(rank_of[base:base + Lb] == r)[0]
        if pos.size == 0:
            continue
        for h in range(hq):
            kvh = h // group
            K, V = k[base:base + Lb, kvh], v[base:base + Lb, kvh]
            Q, dO = q[base + pos, h], do[base + pos, h]
            S = scale * (Q @ K.T)
            S = np.where(np.arange(Lb)[None, :] <= pos[:, None], S, NEG_INF)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            out = P @ V
            dP = dO @ V.T
            dS = P * (dP - (dO * out).sum(axis=1, keepdims=True))
            var_D = c * (((dO * out) ** 2).sum(axis=1) + ((P * dP) ** 2).sum(axis=1))
            var_out[base + pos, h] = c * ((P ** 2) @ (V ** 2))
            var_dq[base + pos, h] = c * scale ** 2 * ((dS ** 2) @ (K ** 2)) + \
                scale ** 2 * var_D[:, None] * (P @ K) ** 2
            var_dk[base:base + Lb, kvh] += c * scale ** 2 * ((dS ** 2).T @ (Q ** 2)) + \
                scale ** 2 * (P ** 2).T @ (var_D[:, None] * Q ** 2)
            var_dv[base:base + Lb, kvh] += c * ((P ** 2).T @ (dO ** 2))
    own = shard_rows(cu, cup, cp, r)
    return {"out": np.sqrt(var_out[own]), "dq": np.sqrt(var_dq[own]),
            "dk_parts": [np.sqrt(var_dk[shard_rows(cu, cup, cp, s)]) for s in range(cp)],
            "dv_parts": [np.sqrt(var_dv[shard_rows(cu, cup, cp, s)]) for s in range(cp)],
            "dk_full": np.sqrt(var_dk), "dv_full": np.sqrt(var_dv)}


class _HeadCache:
    """float64 copies of one KV head's keys and values, converted on first use."""

    def __init__(self, k_bits, v_bits):
        self.k_bits, self.v_bits = k_bits, v_bits
        self.g = None

    def get(self, g):
        if self.g != g:
            self.k = bf16_to_f64(self.k_bits[:, g])
            self.v = bf16_to_f64(self.v_bits[:, g])
            self.g = g
        return self.k, self.v


def _row_position(cu, cup, g_row):
    """(sequence, in-sequence position) of a global row, or None for padding."""
    b = int(np.searchsorted(np.asarray(cup), g_row, side="right") - 1)
    p = g_row - int(cup[b])
    if p >= int(cu[b + 1] - cu[b]):
        return None
    return b, p


def share_rows(q_bits, k_bits, v_bits, do_bits, cu, cup, cp: int, r: int, scale: float,
               local_rows, heads, want_dq: bool = False):
    """out, lse (and dQ) of selected local rows / heads of rank r's share.

    Each (row, head) is one full softmax row over the keys 0..p of its
    sequence, computed on its own, so single entries of a large share can be
    checked without computing the whole share. dQ_p needs only row p's
    softmax and D_p = <dO_p, out_p>.
    Returns out [n_rows, n_heads, D], lse [n_heads, n_rows] and dq (or None).
    """
    cu, cup = validate(cu, cup, cp, r)
    own = shard_rows(cu, cup, cp, r)
    hq = q_bits.shape[1]
    group = hq // k_bits.shape[1]
    d = q_bits.shape[2]
    local_rows = np.asarray(local_rows, dtype=np.int64)
    heads = list(heads)
    out = np.zeros((local_rows.size, len(heads), d))
    lse = np.full((len(heads), local_rows.size), NEG_INF)
    dq = np.zeros((local_rows.size, len(heads), d)) if want_dq else None
    cache = _HeadCache(k_bits, v_bits)
    order = sorted(range(len(heads)), key=lambda j: heads[j] // group)
    for j in order:
        h = heads[j]
        kf, vf = cache.get(h // group)
        for i, t in enumerate(local_rows):
            g_row = int(own[t])
            pos = _row_position(cu, cup, g_row)
            if pos is None:
                continue
            b, p = pos
            base = int(cup[b])
            qh = bf16_to_f64(q_bits[g_row, h])[None, :]
            doh = bf16_to_f64(do_bits[g_row, h])[None, :] if want_dq else None
            o, l, gr = _attend_sequence(qh, kf[base:base + p + 1], vf[base:base + p + 1], doh,
                                        np.array([p]), scale, want_dq)
            out[i, j] = o[0]
            lse[j, i] = l[0]
            if want_dq:
                dq[i, j] = gr[0][0]
    return out, lse, dq


def share_rows_forward(q_bits, k_bits, v_bits, cu, cup, cp: int, r: int, scale: float, local_rows, heads):
    """out [n_rows, n_heads, D] and lse [n_heads, n_rows] of selected rows."""
    o, l, _ = share_rows(q_bits, k_bits, v_bits, None, cu, cup, cp, r, scale, local_rows, heads)
    return o, l


def share_rows_dq(q_bits, k_bits, v_bits, do_bits, cu, cup, cp: int, r: int, scale: float, local_rows, heads):
    """dQ [n_rows, n_heads, D] of selected rows."""
    return share_rows(q_bits, k_bits, v_bits, do_bits, cu, cup, cp, r, scale, local_rows, heads, True)[2]


def share_keys_dkdv(q_bits, k_bits, v_bits, do_bits, cu, cup, cp: int, r: int, scale: float,
                    shard: int, key_local_rows, kv_heads):
    """Exact dK / dV rows of shard `shard`'s part of rank r's share, for the
    selected local key rows and KV heads: the sum over rank r's valid query
    rows p at or after the key, and over the query heads of the KV group, of
    scale * dS_pj * Q_p and P_pj * dO_p. Every query row needs its own full
    softmax row (for lse_p and D_p), so this is cheap only for keys that few
    of the rank's queries reach (e.g. the last rows of a sequence).
    Returns dk, dv: [n_keys, n_kv_heads, D].
    """
    cu, cup = validate(cu, cup, cp, r)
    rank_of, _ = owner_map(cu, cup, cp)
    krows = shard_rows(cu, cup, cp, shard)
    hq = q_bits.shape[1]
    hkv = k_bits.shape[1]
    group = hq // hkv
    d = q_bits.shape[2]
    key_local_rows = np.asarray(key_local_rows, dtype=np.int64)
    dk = np.zeros((key_local_rows.size, len(kv_heads), d))
    dv = np.zeros((key_local_rows.size, len(kv_heads), d))
    cache = _HeadCache(k_bits, v_bits)
    for jg, g in enumerate(kv_heads):
        kf, vf = cache.get(g)
        for i, t in enumerate(key_local_rows):
            gk = int(krows[t])
            pos = _row_position(cu, cup, gk)
            if pos is None:
                continue
            b, pk = pos
            base = int(cup[b])
            L = int(cu[b + 1] - cu[b])
            for p in range(pk, L):
                if rank_of[base + p] != r:
                    continue
                for h in range(g * group, (g + 1) * group):
                    qh = bf16_to_f64(q_bits[base + p, h])[None, :]
                    doh = bf16_to_f64(do_bits[base + p, h])[None, :]
                    o, l, _ = _attend_sequence(qh, kf[base:base + p + 1], vf[base:base + p + 1], None,
                                               np.array([p]), scale, False)
                    s_pj = scale * float(qh[0] @ kf[base + pk])
                    p_pj = np.exp(s_pj - l[0])
                    dp = float(doh[0] @ vf[base + pk])
                    dcoef = float(doh[0] @ o[0])
                    ds = p_pj * (dp - dcoef)
                    dk[i, jg] += scale * ds * qh[0]
                    dv[i, jg] += p_pj * doh[0]
    return dk, dv


def group_row_stats(q_bits, k_bits, v_bits, do_bits, cu, cup, cp: int, r: int, scale: float, kv_head: int,
                    max_elems: int = 1 << 24, proj=None) -> dict:
    """First pass of the exact dK / dV of chosen key rows at any size: for
    every valid query row p that rank r owns and every query head h of KV
    group ``kv_head``, the row's softmax statistics

        lse_{p,h} = log sum_{j <= p} exp(s_pj),   s_pj = scale <Q_p,h, K_j>
        D_{p,h}   = <dO_p,h, out_p,h>,            out_p,h = sum_j P_pj V_j

    with the exact float64 out, and (for the comparison tolerance, not the
    method) var_D_{p,h} = sum_d (dO out)^2 + sum_j (P_pj dP_pj)^2, the sum the
    rounding model of share_rounding_sd needs.

    With ``proj`` (float64 [group, D], one vector u_h per query head of the
    group) it also returns, per row, the projections of the row's exact
    output and query gradient on u_h,

        out_proj_{p,h} = <out_p,h, u_h>,   dq_proj_{p,h} = <dQ_p,h, u_h>,
        dQ_p,h = scale sum_{j <= p} dS_pj K_j,   dS_pj = P_pj (dP_pj - D_p,h),

    and, for the comparison tolerance only (not the method), the standard
    deviations "out_proj_sd" and "dq_proj_sd" of those projections under the
    rounding model of share_rounding_sd (P rounded before P V, dS before
    dS K, D formed from the rounded output), taken along u_h: with u_h a
    unit basis vector e_d they are that model's per-element deviations.

    Each softmax row is whole (keys 0..p of its sequence); the rows are only
    processed in batches of at most ``max_elems`` scores. Returns a dict with
    "rows" (global query rows, int64 [n]), "seq", "pos" (sequence and
    in-sequence position of each), and [group, n] float64 arrays "lse",
    "dcoef", "var_d_terms" (and the four projection arrays with ``proj``).
    """
    cu, cup = validate(cu, cup, cp, r)
    hq = q_bits.shape[1]
    hkv = k_bits.shape[1]
    if hq % hkv:
        raise OracleError("Hq must be a multiple of Hkv")
    group = hq // hkv
    rank_of, _ = owner_map(cu, cup, cp)
    rows, seq, pos = [], [], []
    for b in range(cu.size - 1):
        base = int(cup[b])
        Lb = int(cu[b + 1] - cu[b])
        p = np.nonzero(rank_of[base:base + Lb] == r)[0]
        rows.append(base + p)
        seq.append(np.full(p.size, b))
        pos.append(p)
    rows = np.concatenate(rows) if rows else np.zeros(0, np.int64)
    seq = np.concatenate(seq) if seq else np.zeros(0, np.int64)
    pos = np.concatenate(pos) if pos else np.zeros(0, np.int64)
    n = rows.size
    lse = np.full((group, n), NEG_INF)
    dcoef = np.zeros((group, n))
    var_terms = np.zeros((group, n))
    pnames = ("out_proj", "dq_proj", "out_proj_sd", "dq_proj_sd")
    c_rnd = BF16_UNIT_ROUNDOFF ** 2 / 3.0
    pj = {nm: np.zeros((group, n)) for nm in pnames} if proj is not None else None
    kf = bf16_to_f64(k_bits[:, kv_head])
    vf = bf16_to_f64(v_bits[:, kv_head])
    for jh, h in enumerate(range(kv_head * group, (kv_head + 1) * group)):
        i = 0
        while i < n:
            # a batch of rows of one sequence whose score block stays small
            b = seq[i]
            base = int(cup[b])
            j = i
            while j < n and seq[j] == b and (j - i + 1) * (int(pos[j]) + 1) <= max_elems:
                j += 1
            j = max(j, i + 1)
            p = pos[i:j]
            nk = int(p.max()) + 1
            K, V = kf[base:base + nk], vf[base:base + nk]
            Q = bf16_to_f64(q_bits[base + p, h])
            dO = bf16_to_f64(do_bits[base + p, h])
            s = scale * (Q @ K.T)
            s = np.where(np.arange(nk)[None, :] <= p[:, None], s, NEG_INF)
            m = s.max(axis=1)
            l = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
            P = np.exp(s - l[:, None])
            out = P @ V
            dP = dO @ V.T
            lse[jh, i:j] = l
            dcoef[jh, i:j] = (dO * out).sum(axis=1)
            var_terms[jh, i:j] = ((dO * out) ** 2).sum(axis=1) + ((P * dP) ** 2).sum(axis=1)
            if pj is not None:
                u = np.asarray(proj[jh], dtype=np.float64)
                Ku, Vu = K @ u, V @ u
                dS = P * (dP - dcoef[jh, i:j][:, None])
                pj["out_proj"][jh, i:j] = out @ u
                pj["dq_proj"][jh, i:j] = scale * (dS @ Ku)
                var_D = c_rnd * var_terms[jh, i:j]
                pj["out_proj_sd"][jh, i:j] = np.sqrt(c_rnd * ((P ** 2) @ (Vu ** 2)))
                pj["dq_proj_sd"][jh, i:j] = np.sqrt(c_rnd * scale ** 2 * ((dS ** 2) @ (Ku ** 2)) +
                                                    scale ** 2 * var_D * (P @ Ku) ** 2)
            i = j
    res = {"rows": rows, "seq": seq, "pos": pos, "kv_head": kv_head, "group": group,
           "lse": lse, "dcoef": dcoef, "var_d_terms": var_terms}
    if pj is not None:
        res.update(pj)
    return res


def keys_dkdv_from_stats(stats: dict, q_bits, k_bits, v_bits, do_bits, cu, cup, scale: float, key_rows):
    """Second pass: exact dK / dV of the given global key rows (of the stats'
    KV head), from the first pass's per-row lse and D. For key j at position
    k of sequence b:

        dV_j = sum_{p, h} P_pj dO_p,h,   dK_j = scale sum_{p, h} dS_pj Q_p,h
        P_pj = exp(s_pj - lse_p,h),      dS_pj = P_pj (<dO_p,h, V_j> - D_p,h)

    over the stats' query rows p of sequence b at positions >= k and the
    group's query heads h. Padding key rows get 0. Also returns the rounding
    model's standard deviation of each element (as share_rounding_sd).
    Returns dk, dv, dk_sd, dv_sd: [n_keys, D].
    """
    cu = np.asarray(cu, dtype=np.int64)
    cup = np.asarray(cup, dtype=np.int64)
    key_rows = np.asarray(key_rows, dtype=np.int64)
    g, group = stats["kv_head"], stats["group"]
    d = q_bits.shape[2]
    c = BF16_UNIT_ROUNDOFF ** 2 / 3.0
    dk = np.zeros((key_rows.size, d))
    dv = np.zeros((key_rows.size, d))
    var_dk = np.zeros((key_rows.size, d))
    var_dv = np.zeros((key_rows.size, d))
    for i, gk in enumerate(key_rows):
        posk = _row_position(cu, cup, int(gk))
        if posk is None:
            continue
        b, pk = posk
        sel = np.nonzero((stats["seq"] == b) & (stats["pos"] >= pk))[0]
        if sel.size == 0:
            continue
        kj = bf16_to_f64(k_bits[gk, g])
        vj = bf16_to_f64(v_bits[gk, g])
        for jh, h in enumerate(range(g * group, (g + 1) * group)):
            Q = bf16_to_f64(q_bits[stats["rows"][sel], h])
            dO = bf16_to_f64(do_bits[stats["rows"][sel], h])
            P = np.exp(scale * (Q @ kj) - stats["lse"][jh, sel])
            dS = P * (dO @ vj - stats["dcoef"][jh, sel])
            dk[i] += scale * (dS @ Q)
            dv[i] += P @ dO
            var_D = c * stats["var_d_terms"][jh, sel]
            var_dk[i] += c * scale ** 2 * ((dS ** 2) @ (Q ** 2)) + scale ** 2 * ((P ** 2) * var_D) @ (Q ** 2)
            var_dv[i] += c * ((P ** 2) @ (dO ** 2))
    return dk, dv, np.sqrt(var_dk), np.sqrt(var_dv)


def group_key_projections(stats: dict, q_bits, k_bits, v_bits, do_bits, cu, cup, scale: float, u_dk, u_dv,
                          max_elems: int = 1 << 24) -> dict:
    """Second pass over every key row at once, projected: for every valid
    global key row j of the stats' KV head, the rank's contribution to dK_j
    and dV_j (the same sums as keys_dkdv_from_stats) projected on the unit
    vectors u_dk and u_dv,

        dk_proj_j = <dK_j, u_dk>,   dv_proj_j = <dV_j, u_dv>,

    and, for the comparison tolerance only, their standard deviations under
    the rounding model of share_rounding_sd taken along u_dk / u_dv (with a
    unit basis vector: that model's per-element deviations). Keys are taken
    in blocks so that each block's score matrix stays below ``max_elems``.
    Returns {"key_rows": global rows [n], "dk_proj", "dv_proj",
    "dk_proj_sd", "dv_proj_sd": [n]}; key rows no query of the rank reaches
    get 0.
    """
    cu = np.asarray(cu, dtype=np.int64)
    cup = np.asarray(cup, dtype=np.int64)
    g, group = stats["kv_head"], stats["group"]
    u_dk = np.asarray(u_dk, dtype=np.float64)
    u_dv = np.asarray(u_dv, dtype=np.float64)
    c = BF16_UNIT_ROUNDOFF ** 2 / 3.0
    keys, dkp, dvp, vdk, vdv = [], [], [], [], []
    for b in range(cu.size - 1):
        base = int(cup[b])
        Lb = int(cu[b + 1] - cu[b])
        if Lb == 0:
            continue
        sel = np.nonzero(stats["seq"] == b)[0]
        kf = bf16_to_f64(k_bits[base:base + Lb, g])
        vf = bf16_to_f64(v_bits[base:base + Lb, g])
        acc = np.zeros((4, Lb))  # dk_proj, dv_proj, var_dk_proj, var_dv_proj
        if sel.size:
            pos = stats["pos"][sel]
            heads = []
            for jh, h in enumerate(range(g * group, (g + 1) * group)):
                Q = bf16_to_f64(q_bits[stats["rows"][sel], h])
                dO = bf16_to_f64(do_bits[stats["rows"][sel], h])
                heads.append((Q, dO, Q @ u_dk, dO @ u_dv, stats["lse"][jh, sel], stats["dcoef"][jh, sel],
                              c * stats["var_d_terms"][jh, sel]))
            kb = max(1, min(Lb, max_elems // max(1, sel.size)))
            for k0 in range(0, Lb, kb):
                k1 = min(Lb, k0 + kb)
                rq = pos >= k0  # query rows that reach some key of the block
                if not rq.any():
                    continue
                mask = pos[rq][:, None] >= np.arange(k0, k1)[None, :]
                K, V = kf[k0:k1], vf[k0:k1]
                for Q, dO, Qu, dOu, lse, dco, vD in heads:
                    S = scale * (Q[rq] @ K.T)
                    P = np.where(mask, np.exp(S - lse[rq][:, None]), 0.0)
                    dS = P * (dO[rq] @ V.T - dco[rq][:, None])
                    acc[0, k0:k1] += scale * (Qu[rq] @ dS)
                    acc[1, k0:k1] += dOu[rq] @ P
                    acc[2, k0:k1] += c * scale ** 2 * ((Qu[rq] ** 2) @ (dS ** 2)) + \
                        scale ** 2 * ((vD[rq] * Qu[rq] ** 2) @ (P ** 2))
                    acc[3, k0:k1] += c * ((dOu[rq] ** 2) @ (P ** 2))
        keys.append(base + np.arange(Lb))
        dkp.append(acc[0])
        dvp.append(acc[1])
        vdk.append(acc[2])
        vdv.append(acc[3])
    cat = (lambda xs: np.concatenate(xs) if xs else np.zeros(0))
    return {"key_rows": cat(keys).astype(np.int64), "dk_proj": cat(dkp), "dv_proj": cat(dvp),
            "dk_proj_sd": np.sqrt(cat(vdk)), "dv_proj_sd": np.sqrt(cat(vdv))}


def share_keys_dkdv_two_pass(q_bits, k_bits, v_bits, do_bits, cu, cup, cp: int, r: int, scale: float,
                             shard: int, key_local_rows, kv_head: int, stats: dict | None = None):
    """dK / dV rows of shard `shard`'s part of rank r's share for the selected
    local key rows of one KV head, by the two passes above (the same values
    as share_keys_dkdv, at a cost that does not grow with how many queries
    reach a key). ``stats`` may hold a first pass already computed for this
    rank and KV head. Returns dk, dv, dk_sd, dv_sd: [n_keys, D]."""
    if stats is None:
        stats = group_row_stats(q_bits, k_bits, v_bits, do_bits, cu, cup, cp, r, scale, kv_head)
    krows = shard_rows(cu, cup, cp, shard)[np.asarray(key_local_rows, dtype=np.int64)]
    return keys_dkdv_from_stats(stats, q_bits, k_bits, v_bits, do_bits, cu, cup, scale, krows)


def flops_share(cu, cup, cp: int, r: int, hq: int, d: int) -> dict:
    """Algorithmic work of rank r's share: causal (query, key) pairs over valid
    rows (diagonal included) and the flop counts 4*D per pair per query head
    (forward) and 10*D (backward)."""
    cu, cup = validate(cu, cup, cp, r)
    rank_of, _ = owner_map(cu, cup, cp)
    vm = valid_mask(cu, cup)
    pairs = 0
    for b in range(cu.size - 1):
        base = int(cup[b])
        Lb = int(cu[b + 1] - cu[b])
        pos = np.nonzero((rank_of[base:base + Lb] == r) & vm[base:base + Lb])[0]
        pairs += int((pos + 1).sum())
    return {"pairs": pairs, "fwd": 4 * d * hq * pairs, "bwd": 10 * d * hq * pairs,
            "total": 14 * d * hq * pairs}
