"""Write fullsize_dkdv.npz: exact dK / dV of sampled key rows of every source
shard's part, at the two full-size shares the benchmark runs (the 131072-token
GQA share, CP = 4, rank 2, and the 64K hierarchical pack's p2p share, CP = 2,
rank 0), for one KV head each, and the exact LSE of every query row of the
rank for that KV head's query heads (a by-product of the first pass), with
every such row's output and query gradient projected on a seeded unit
vector per head and the rounding model's deviation of each projection, and
the rank's dK / dV of every valid key row (all source shards) projected the
same way.

Calls only the oracle (its two-pass key-row helper) and the seeded input
generator; nothing comes from the HIP path. The inputs the values depend on
(that KV head's K / V and its group's Q / dO, and the sequence tables) are
hashed into the file, so a test reading it can tell that it still matches
the generator. Run from the repository root:

    python tests/golden/make_fullsize_dkdv.py
"""
import hashlib
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from context_packed_attention_amd import synth  # noqa: E402
from oracle import cp_attn_oracle as O  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fullsize_dkdv.npz")


def key_rows(t_local: int, cu, cup, cp: int, shard: int) -> np.ndarray:
    """Start, middle and end of the part, both chunk halves of the first and
    last sequence slots, and a few seeded rows."""
    half = t_local // 2
    fixed = [0, 1, 31, 32, 127, half // 2, half - 1, half, half + 1, half + half // 2, t_local - 2, t_local - 1]
    slot = np.asarray(cup) // cp
    chunk = np.diff(np.asarray(cup)) // (2 * cp)
    for b in (0, len(chunk) - 1):
        fixed += [int(slot[b]), int(slot[b] + chunk[b]), int(slot[b] + chunk[b] - 1)]
    rng = np.random.default_rng(1000 + shard)
    fixed += list(rng.integers(0, t_local, 4))
    return np.unique(np.clip(np.array(fixed, dtype=np.int64), 0, t_local - 1))


def input_digest(bt, kv_head: int) -> str:
    group = bt.hq // bt.hkv
    hs = slice(kv_head * group, (kv_head + 1) * group)
    h = hashlib.sha256()
    for a in (np.asarray(bt.cu, np.int64), np.asarray(bt.cup, np.int64), bt.q[:, hs], bt.do[:, hs],
              bt.k[:, kv_head], bt.v[:, kv_head]):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def main():
    arrays = {}
    for cfg in (4, 5):
        bt, w = synth.make_workload(cfg)
        cp, r = w["cp"], w["ranks"][-1]
        g = bt.hkv - 1
        scale = 1.0 / math.sqrt(bt.d)
        t0 = time.time()
        group = bt.hq // bt.hkv
        u = np.random.default_rng(7000 + cfg).standard_normal((group, bt.d))
        u /= np.linalg.norm(u, axis=1, keepdims=True)
        stats = O.group_row_stats(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale, g, proj=u)
        print(f"{bt.name}: first pass over {stats['rows'].size} rows x {stats['group']} heads "
              f"in {time.time() - t0:.1f} s", flush=True)
        t_local = bt.total_rows // cp
        pre = f"w{cfg}_"
        arrays[pre + "meta"] = np.array([cp, r, g], dtype=np.int64)
        arrays[pre + "digest"] = np.array(input_digest(bt, g))
        # every valid query row's LSE for the group's heads, at the rank's local rows
        _, local = O.owner_map(bt.cu, bt.cup, cp)
        arrays[pre + "lse_rows"] = local[stats["rows"]].astype(np.int32)
        arrays[pre + "lse"] = stats["lse"].astype(np.float32)
        # every such row's out and dQ projected on u (one vector per head)
        arrays[pre + "proj_u"] = u
        for nm in ("out_proj", "dq_proj", "out_proj_sd", "dq_proj_sd"):
            arrays[pre + nm] = stats[nm].astype(np.float32)
        # every valid key row's dK / dV (global order), projected
        uk = np.random.default_rng(7100 + cfg).standard_normal((2, bt.d))
        uk /= np.linalg.norm(uk, axis=1, keepdims=True)
        t1 = time.time()
        kp = O.group_key_projections(stats, bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, scale, uk[0], uk[1])
        print(f"{bt.name}: projected dK / dV of {kp['key_rows'].size} key rows in {time.time() - t1:.1f} s", flush=True)
        assert np.array_equal(kp["key_rows"], np.nonzero(O.valid_mask(bt.cu, bt.cup))[0])
        arrays[pre + "key_u"] = uk
        for nm in ("dk_proj", "dv_proj"):
            arrays[pre + nm] = kp[nm].astype(np.float32)
        for nm in ("dk_proj_sd", "dv_proj_sd"):
            arrays[pre + nm] = kp[nm].astype(np.float16)
        for s in range(cp):
            rows = key_rows(t_local, bt.cu, bt.cup, cp, s)
            dk, dv, dks, dvs = O.share_keys_dkdv_two_pass(bt.q, bt.k, bt.v, bt.do, bt.cu, bt.cup, cp, r, scale,
                                                          s, rows, g, stats=stats)
            arrays[pre + f"s{s}_rows"] = rows
            # float32 keeps ~7 significant digits, far below any comparison bar
            for name, a in (("dk", dk), ("dv", dv), ("dk_sd", dks), ("dv_sd", dvs)):
                arrays[pre + f"s{s}_{name}"] = a.astype(np.float32)
            print(f"  shard {s}: {rows.size} key rows, max |dk| {np.abs(dk).max():.4f}, "
                  f"max |dv| {np.abs(dv).max():.4f}", flush=True)
    np.savez_compressed(OUT, **arrays)
    print("wrote", OUT, os.path.getsize(OUT), "bytes")


if __name__ == "__main__":
    main()
