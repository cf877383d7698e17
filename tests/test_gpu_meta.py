"""Device metadata builder vs the oracle: integer tables bit-exact, the padding
decision taken from values (aliased / NULL / distinct-equal padded
cu_seqlens all give identical tables), and device-side argument checks. The
host-summary path (cp_attn_rank_metadata_host) must give the same tables,
summary, statuses and messages, and the same forward / backward bits."""
import numpy as np
import pytest

from context_packed_attention_amd import api, synth
from oracle import cp_attn_oracle as O
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def _compare(md_gpu, md_ref):
    for key in ("B", "cp", "rank", "pad_between_seqs", "t_local", "has_tail"):
        assert md_gpu[key] == md_ref[key], key
    for key in ("chunk", "cu_padded_local", "cu_padded_half"):
        assert list(md_gpu[key]) == [int(x) for x in md_ref[key]], key
    for s in range(md_ref["cp"]):
        for k in ("full", "first", "second"):
            assert list(md_gpu[f"cu_{k}_{s}"]) == [int(x) for x in md_ref[f"cu_{k}_{s}"]], (k, s)
    for i, (g, r) in enumerate(zip(md_gpu["steps"], md_ref["steps"])):
        assert g["kind"] == r["kind"] and g["src"] == r["src"], i
        for k in ("q_start", "q_len", "kv_start", "kv_len"):
            assert list(g[k]) == [int(x) for x in r[k]], (i, k)


def _packs():
    out = []
    for cfg in (1, 2, 3, 4, 5):
        w = synth.workload(cfg)
        L = w["lengths"]
        P = L if w["max_pad"] is None else synth.draw_padded_lengths(w["seed"], L, w["max_pad"], 2 * w["cp"])
        out.append((f"cfg{cfg}", L, P, w["cp"]))
    rng = np.random.default_rng(11)
    for cp in (1, 2, 3, 4, 8):
        for j in range(3):
            B = int(rng.integers(1, 40))
            P = [2 * cp * int(rng.integers(0, 50)) for _ in range(B)]
            L = [int(rng.integers(0, p + 1)) for p in P]
            out.append((f"rand-cp{cp}-{j}", L, P, cp))
    return out


@pytest.mark.parametrize("name,L,P,cp", _packs(), ids=[p[0] for p in _packs()])
def test_metadata_bit_exact(name, L, P, cp):
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    cup = np.concatenate([[0], np.cumsum(P)]).astype(np.int32)
    H.log(f"[meta] {name} B={len(L)} cp={cp}")
    dcu, dcup = H.dev_i32(cu), H.dev_i32(cup)
    for r in range(cp):
        for tail in (0, 37):
            T_local = int(cup[-1]) // cp
            m = api.cp_attn_rank_metadata(dcu, dcup, cp, r, -1, T_local + tail)
            got = H.parse_export(m.export())
            ref = O.rank_metadata(cu, cup, cp, r, T_local + tail)
            _compare(got, ref)
            s = m.summary
            assert s.has_tail == (1 if tail else 0)
            assert s.valid_rows == int(np.diff(ref[f"cu_full_{r}"]).sum())
            mh = api.cp_attn_rank_metadata_host(cu, cup, cp, r, -1, T_local + tail)
            assert np.array_equal(mh.export(), m.export())
            assert _summary(mh) == _summary(m)
            mh.close()
            m.close()


def _summary(m):
    s = m.summary
    cp = int(s.cp_size)
    return (int(s.B), cp, int(s.cp_rank), int(s.pad_between_seqs), int(s.t_local), int(s.has_tail), int(s.t_alloc),
            int(s.valid_rows), list(s.step_kind)[:cp], list(s.step_src)[:cp], list(s.tiles_fwd)[:cp],
            list(s.tiles_dkdv)[:cp])


def test_padding_decision_by_value_not_identity():
    """Same tensor, distinct value-equal copy, NULL, explicit hint 0: all the
    same tables and pad_between_seqs = 0; real padding gives 1."""
    cu = np.array([0, 4096], dtype=np.int32)
    dcu = H.dev_i32(cu)
    dcopy = dcu.clone()
    assert dcopy.data_ptr() != dcu.data_ptr()
    exports = []
    for cup_arg, hint in ((dcu, -1), (dcopy, -1), (None, -1), (dcopy, 0), (dcu, 0)):
        m = api.cp_attn_rank_metadata(dcu, cup_arg, 4, 1, hint, 1024)
        assert m.summary.pad_between_seqs == 0
        exports.append(m.export())
        m.close()
    for e in exports[1:]:
        assert np.array_equal(e, exports[0])
    padded = H.dev_i32([0, 4104])
    m = api.cp_attn_rank_metadata(dcu, padded, 4, 1, -1, 1026)
    assert m.summary.pad_between_seqs == 1
    m.close()
    m = api.cp_attn_rank_metadata(dcu, padded, 4, 1, 1, 1026)
    assert m.summary.pad_between_seqs == 1
    m.close()


@pytest.mark.parametrize("cu,cup,hint,t_alloc,status", [
    ([0, 4096], [0, 4104], 0, 1026, 3),      # hint says no padding, values disagree
    ([0, 4096], None, 1, 1024, 3),           # hint says padding, there is none
    ([0, 4090], [0, 4090], -1, 1024, 1),     # not divisible by 2*CP
    ([0, 4096], [0, 4096], -1, 1000, 1),     # t_alloc < T_local
    ([0, 4096, 4000], [0, 4096, 4000], -1, 2048, 1),  # decreasing
    ([0, 4200], [0, 4096], -1, 1024, 1),     # valid longer than padded
    ([8, 4096], [8, 4096], -1, 1024, 1),     # does not start at 0
])
def test_device_side_validation(cu, cup, hint, t_alloc, status):
    dcu = H.dev_i32(cu)
    dcup = H.dev_i32(cup) if cup is not None else None
    with pytest.raises(api.CpAttnError) as ei:
        api.cp_attn_rank_metadata(dcu, dcup, 4, 1, hint, t_alloc)
    assert ei.value.status == status
    with pytest.raises(api.CpAttnError) as eh:
        api.cp_attn_rank_metadata_host(cu, cup, 4, 1, hint, t_alloc)
    assert eh.value.status == status and str(eh.value) == str(ei.value).replace(
        "cp_attn_rank_metadata", "cp_attn_rank_metadata_host")


@pytest.mark.parametrize("cfg,rank,tail", [(3, 1, 0), (1, 0, 37)])
def test_host_path_same_results(cfg, rank, tail):
    """Forward and backward with the host-path handle equal those with the
    device-path handle bit for bit (the 16K padded pack; the tiny pack with a
    tail)."""
    import math
    import torch
    bt, w = synth.make_workload(cfg)
    cp = w["cp"]
    db = H.DeviceBatch(bt)
    meta, loc = H.local_inputs(db, cp, rank, tail=tail)
    scale = 1.0 / math.sqrt(bt.d)
    res = []
    for host in (False, True):
        if host:
            m = api.cp_attn_rank_metadata_host(bt.cu, bt.cup, cp, rank, -1, loc["t_alloc"])
        else:
            m = meta
        out, lse = H.run_fwd(m, loc, bt, scale)
        dq, dks, dvs = H.run_bwd(m, loc, bt, scale, out, lse)
        torch.cuda.synchronize()
        res.append([out, lse, dq, *dks, *dvs])
        if host:
            m.close()
    for a, b in zip(*res):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    meta.close()


def test_shard_gather_matches_oracle_map():
    bt = synth.make_batch("g", 5, [40, 0, 13, 64], [48, 16, 16, 64], 3, 1, 64)
    db = H.DeviceBatch(bt)
    for cp in (1, 2, 4):
        for s in range(cp):
            meta, loc = H.local_inputs(db, cp, s)
            rows = O.shard_rows(bt.cu, bt.cup, cp, s)
            assert np.array_equal(H.bf16_to_np(loc["q"]), bt.q[rows])
            assert np.array_equal(H.bf16_to_np(loc["k"][s]), bt.k[rows])
            meta.close()
