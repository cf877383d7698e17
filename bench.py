#!/usr/bin/env python3
"""Benchmark: one CP rank's share of packed-THD causal ring attention, fwd+bwd.

One step = the whole hot path over one batch: the per-rank metadata build,
the forward (one flash kernel per ring step, each folding its partial into the
accumulator through the LSE merge, or for short shares one launch over every
step) and the backward (D preprocess, one dK/dV launch over every step, one
dQ launch, tail zeroing when a tail exists). Beside it, the forward + backward captured once as a HIP graph is
timed against the same calls made eagerly (the "graph" object). Inputs are seeded synthetic bf16 tensors already resident in
HBM. The reported value is algorithmic TFLOP/s: 14 * D * Hq * causal pairs of
the share per step (4 forward + 10 backward), divided by the measured time.

Prints one JSON line. Only one GPU is used; --gpus above 1 exits.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0

# HBM bytes per launch of a kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE
# counters scaled by a plain copy's readings; a file under profiles/ holds the
# figure with the SHA-256 of the kernel sources it was taken on, and the
# figure is dropped once those sources change
TRAFFIC_SOURCES = ("context_packed_attention_amd/csrc/bwd.hip", "context_packed_attention_amd/csrc/fwd.hip",
                   "context_packed_attention_amd/csrc/kern_common.h", "context_packed_attention_amd/csrc/internal.h",
                   "context_packed_attention_amd/csrc/meta.hip")


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary, or None when there is none or the sources changed."""
    import re
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel sources sha256: `([0-9a-f]{64})`", text)
    row = re.search(r"^\| " + re.escape(kernel) + r" \|[^\n]*\| ([0-9]+) \|\s*$", text, re.M)
    if not sha or not row or sha.group(1) != kernel_sources_sha256():
        return None
    return int(row.group(1))


# algorithmic flops per causal pair per query head, in units of head_dim
ALGO_FLOPS_PER_PAIR = {"fwd_step": 4, "fwd_fused": 4, "bwd_dkdv": 8, "bwd_dq": 2}
EXEC_FLOPS_PER_PAIR = {"fwd_step": 4, "fwd_fused": 4, "bwd_dkdv": 8, "bwd_dq": 6}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4,
                    help="1..5: tiny / 16K pack / padded 16K pack / 131072-token GQA / 64K hierarchical pack")
    ap.add_argument("--cpu-sample-stride", type=int, default=128,
                    help="oracle baseline: every Nth query row of the share (0 = skip the baseline)")
    ap.add_argument("--a2a", action="store_true",
                    help="only time the hierarchical front end's all-to-all (sequence split -> head split and back) "
                         "on the 64K hierarchical pack, [a2a, p2p] = [2, 2], Q of 32 heads, and exit")
    ap.add_argument("--hier", action="store_true",
                    help="time one whole a2a+p2p step of an a2a group on the 64K hierarchical pack "
                         "([a2a, p2p] = [2, 2], CP = 4, 32 heads before the head split): sequence -> head "
                         "all-to-all of Q, K, V (and dO), the p2p-level share of each head group, forward and "
                         "backward, and the head -> sequence all-to-all of out, dQ and the own shard's dK / dV; "
                         "print one JSON line and exit")
    ap.add_argument("--all-gather", action="store_true",
                    help="time the all-gather share of the selected workload instead (gathered K/V in, the rank's "
                         "contribution to every gathered dK/dV row out) and exit")
    ap.add_argument("--tail", type=int, default=0, metavar="ROWS",
                    help="allocate the rank-local tensors ROWS rows past the valid end (the gradients' tail "
                         "is then zeroed by one extra launch, whose HBM rate the kernel entry reports)")
    ap.add_argument("--pad-hint-abba", action="store_true",
                    help="only run the padding-decision A/B on the 16K pack (cu_seqlens_padded a distinct, "
                         "value-equal copy): steps with pad_hint -1 and 0 alternate in A B B A blocks of --steps "
                         "steps, repeated three times; print both step times and launch sequences and exit")
    ap.add_argument("--phases", type=float, default=0.0, metavar="SECONDS",
                    help="only run the power / clock phases on the selected workload and exit: the matrix-unit "
                         "calibration, the forward alone and the backward alone, each back to back for SECONDS, "
                         "with amd-smi sampled in the background (socket power, per-XCD graphics clocks)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times and exit "
                         "(the known-size reference for the HBM byte counters)")
    return ap.parse_args()


class SmiSampler:
    """Background sampling of the GPU's socket power and per-XCD graphics
    clocks through the amd-smi command-line tool (one call at a time)."""

    def __init__(self):
        import threading
        self.samples = []
        self.stop = threading.Event()
        self.th = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        import subprocess
        while not self.stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-p", "--json"], capture_output=True,
                                   text=True, timeout=10)
                t = time.time()
                o = json.loads(r.stdout)
                g = o["gpu_data"][0] if isinstance(o, dict) else o[0]
                clk = [g["clock"][f"gfx_{x}"]["clk"]["value"] for x in range(8) if f"gfx_{x}" in g["clock"]]
                self.samples.append((t, float(g["power"]["socket_power"]["value"]), [float(c) for c in clk]))
            except Exception:
                time.sleep(0.2)

    def __enter__(self):
        self.th.start()
        return self

    def __exit__(self, *a):
        self.stop.set()
        self.th.join(timeout=15)

    def between(self, t0, t1):
        """Mean power and per-XCD clocks of the samples inside [t0, t1] (the
        first 0.5 s left out: the tool reports with some lag)."""
        sel = [x for x in self.samples if t0 + 0.5 <= x[0] <= t1]
        if not sel:
            return None
        n = len(sel[0][2])
        clk = [sum(x[2][i] for x in sel) / len(sel) for i in range(n)]
        return {"samples": len(sel), "socket_power_w": round(sum(x[1] for x in sel) / len(sel), 1),
                "gfx_mhz_mean": round(sum(clk) / n, 1), "gfx_mhz_per_xcd": [round(c) for c in clk]}


def power_phases(seconds, fwd, bwd, probe, flops_fwd, flops_bwd):
    """Each phase back to back for `seconds`: its rate and, from amd-smi, the
    socket power and graphics clocks it ran at."""
    import torch
    out = {}
    with SmiSampler() as smi:
        time.sleep(1.0)
        for name, fn, flops in (("mfma_calibration", probe, None), ("forward", fwd, flops_fwd),
                                ("backward", bwd, flops_bwd)):
            torch.cuda.synchronize()
            t0 = time.time()
            n, tf = 0, []
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            while time.time() - t0 < seconds:
                r = fn()
                if flops is None:
                    tf.append(r)
                n += 1
                if n % 4 == 0:
                    torch.cuda.synchronize()
            e1.record()
            torch.cuda.synchronize()
            t1 = time.time()
            ms = e0.elapsed_time(e1) / n
            rate = (sorted(tf)[len(tf) // 2] if flops is None else flops / (ms * 1e-3) / 1e12)
            out[name] = {"launches": n, "ms_each": round(ms, 3), "tflops": round(rate, 1), "smi": smi.between(t0, t1)}
            log(f"[phases] {name}: {n} calls, {ms:.3f} ms each, {rate:.1f} TFLOP/s, {out[name]['smi']}")
            time.sleep(1.0)
    return out


def copy_calibration(mib):
    """A plain copy kernel of known size: reads and writes mib MiB per launch."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 3}), flush=True)


def cpu_baseline(batch, w, rank, scale, stride):
    """The fp64 oracle, as it stands, on a bounded sample of the same share:
    every `stride`-th local query row of the rank, all heads, forward and
    backward (its dK/dV contributions included)."""
    import numpy as np
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    from oracle import cp_attn_oracle as O
    cp = w["cp"]
    own = O.shard_rows(batch.cu, batch.cup, cp, rank)
    valid = O.valid_mask(batch.cu, batch.cup)
    rows = own[::stride]
    rows = rows[valid[rows]]
    T = batch.total_rows

    def lazy(bits, sel):
        a = np.zeros(bits.shape, dtype=np.float64)
        a[sel] = O.bf16_to_f64(bits[sel])
        return a

    q = lazy(batch.q, rows)
    do = lazy(batch.do, rows)
    k = O.bf16_to_f64(batch.k)
    v = O.bf16_to_f64(batch.v)
    mask = np.zeros(T, dtype=bool)
    mask[rows] = True
    seq = np.searchsorted(batch.cup, rows, side="right") - 1
    pairs = int(sum(int(r - batch.cup[b]) + 1 for r, b in zip(rows, seq)))
    flops = 14 * batch.d * batch.hq * pairs
    t0 = time.perf_counter()
    O.attention(q, k, v, do, batch.cu, batch.cup, scale, query_mask=mask, want_grad=True)
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows.size} of {own.size} local query rows (every {stride}th), all {batch.hq} heads, "
                      f"fp64 fwd+bwd, {pairs} causal pairs, {dt:.1f} s on {threads} BLAS threads "
                      f"({os.cpu_count()} host cpus visible)",
            "seconds": dt}


def a2a_bench(args):
    """The all-to-all of one a2a group on the 64K hierarchical pack: 65536
    padded tokens, CP = 4 as [a2a, p2p] = [2, 2], 32 heads of 128 bf16 (the
    query tensor before the head split). HBM-bound: every byte is read once
    and written once."""
    import numpy as np
    import torch
    from context_packed_attention_amd import api, synth
    w = synth.workload(5)
    A, P = 2, 2
    cp = A * P
    L = w["lengths"]
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    heads, d = 2 * w["hq"], w["d"]
    T = int(cu[-1])
    tl = T // cp
    dcu = torch.tensor(cu, dtype=torch.int32, device="cuda")
    m = api.cp_attn_rank_metadata(dcu, None, cp, 0, -1, tl)
    ins = [torch.randn((tl, heads, d), device="cuda").to(torch.bfloat16) for _ in range(A)]
    outs = [torch.empty((A * tl, heads // A, d), dtype=torch.bfloat16, device="cuda") for _ in range(A)]
    backs = [torch.empty_like(x) for x in ins]
    stream = torch.cuda.current_stream()
    moved = 2 * A * tl * heads * d * 2  # bytes read + written per call

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    fwd_ms = timed(lambda: api.cp_attn_a2a_seq_to_head(m, A, 0, heads, d * 2, ins, outs, stream=stream))
    inv_ms = timed(lambda: api.cp_attn_a2a_head_to_seq(m, A, 0, heads, d * 2, outs, backs, stream=stream))
    ok = all(torch.equal(x.view(torch.int16), y.view(torch.int16)) for x, y in zip(ins, backs))
    m.close()
    gbs = moved / (fwd_ms * 1e-3) / 1e9
    line = {
        "metric": "hierarchical a2a permutation (sequence split -> head split), GB/s on 1 MI355X",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(fwd_ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (N(0,1) bf16)",
        "config": {"workload": w["name"] + "-a2a", "cp_size": cp, "a2a_size": A, "p2p_size": P, "heads": heads,
                   "head_dim": d, "t_local": tl, "bytes_per_call": moved},
        "inverse": {"ms": round(inv_ms, 5), "GB/s": round(moved / (inv_ms * 1e-3) / 1e9, 1), "round_trip_exact": ok},
        "roofline": {"kernel": "a2a_seq_to_head", "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }
    print(json.dumps(line), flush=True)


def hier_bench(args):
    """One a2a+p2p step of a2a group p = 0 on the 64K hierarchical pack, all
    on one GPU: both a2a ranks' work (CP ranks 0 and 1, head groups 0 and 1).
    The K / V of the p2p ring's other shard arrive over the ring in a real
    run (the other group's all-to-all makes them), so they are inputs here,
    head-split already; likewise that shard's dK / dV parts leave over the
    ring. Timed: seq -> head of Q, K, V, the forward share of each head
    group, head -> seq of out; seq -> head of dO, the backward share of each
    head group, head -> seq of dQ, dK and dV of the own shard."""
    import numpy as np
    import torch
    from context_packed_attention_amd import api, synth
    w = synth.workload(5)
    A, P = 2, 2
    cp = A * P
    L = w["lengths"]
    cu = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    H, d = 2 * w["hq"], w["d"]  # heads before the split (query and key / value alike)
    hs = H // A
    T = int(cu[-1])
    tl_cp, tl_p = T // cp, T // P
    scale = 1.0 / math.sqrt(d)
    dcu = torch.tensor(cu, dtype=torch.int32, device="cuda")
    dcup = dcu.clone()
    m_cp = api.cp_attn_rank_metadata(dcu, dcup, cp, 0, -1, tl_cp)
    m_p = api.cp_attn_rank_metadata(dcu, dcup, P, 0, -1, tl_p)
    pairs = sum(api.step_pairs(m_p))
    flops_step = A * 14 * d * hs * pairs
    nd = synth.device_normal_bf16
    # CP-level rows of CP ranks 0 and 1, all heads
    q_cp = [nd((tl_cp, H, d), 50 + a) for a in range(A)]
    k_cp = [nd((tl_cp, H, d), 60 + a) for a in range(A)]
    v_cp = [nd((tl_cp, H, d), 70 + a) for a in range(A)]
    do_cp = [nd((tl_cp, H, d), 80 + a) for a in range(A)]
    # the ring's other shard (p2p rank 1), per head group
    k_s1 = [nd((tl_p, hs, d), 90 + a) for a in range(A)]
    v_s1 = [nd((tl_p, hs, d), 95 + a) for a in range(A)]
    e = lambda shape: torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    q_h, k_h, v_h, do_h = ([e((tl_p, hs, d)) for _ in range(A)] for _ in range(4))
    out_h, dq_h = [e((tl_p, hs, d)) for _ in range(A)], [e((tl_p, hs, d)) for _ in range(A)]
    lse_h = [torch.empty((hs, tl_p), dtype=torch.float32, device="cuda") for _ in range(A)]
    dk_h = [[e((tl_p, hs, d)) for _ in range(P)] for _ in range(A)]
    dv_h = [[e((tl_p, hs, d)) for _ in range(P)] for _ in range(A)]
    out_cp, dq_cp, dk_cp, dv_cp = ([e((tl_cp, H, d)) for _ in range(A)] for _ in range(4))
    ws_f = torch.empty(api.cp_attn_workspace_bytes(m_p, hs, hs, d, 0), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(api.cp_attn_workspace_bytes(m_p, hs, hs, d, 1), dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream()
    s2h = lambda ins, outs: api.cp_attn_a2a_seq_to_head(m_cp, A, 0, H, d * 2, ins, outs, stream=st)
    h2s = lambda ins, outs: api.cp_attn_a2a_head_to_seq(m_cp, A, 0, H, d * 2, ins, outs, stream=st)

    def step():
        s2h(q_cp, q_h)
        s2h(k_cp, k_h)
        s2h(v_cp, v_h)
        for a in range(A):
            api.cp_attn_fwd(m_p, q_h[a], [k_h[a], k_s1[a]], [v_h[a], v_s1[a]], hs, hs, d, scale, 1, out_h[a],
                            lse_h[a], ws_f, stream=st)
        h2s(out_h, out_cp)
        s2h(do_cp, do_h)
        for a in range(A):
            api.cp_attn_bwd(m_p, q_h[a], [k_h[a], k_s1[a]], [v_h[a], v_s1[a]], out_h[a], lse_h[a], do_h[a], hs, hs,
                            d, scale, 1, dq_h[a], dk_h[a], dv_h[a], ws_b, stream=st)
        h2s(dq_h, dq_cp)
        h2s([dk_h[a][0] for a in range(A)], dk_cp)
        h2s([dv_h[a][0] for a in range(A)], dv_cp)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    api.cp_attn_timing_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.steps):
        step()
    e1.record(st)
    torch.cuda.synchronize()
    api.cp_attn_timing_enable(False)
    per_kernel = api.cp_attn_timing_read()
    ms = e0.elapsed_time(e1) / args.steps
    tflops = flops_step / (ms * 1e-3) / 1e12
    perm_bytes = 2 * A * tl_cp * H * d * 2  # one all-to-all call reads and writes this
    kernels = {}
    for name, (kms, n) in per_kernel.items():
        ent = {"launches_per_step": n / args.steps, "ms_per_step": kms / args.steps, "avg_launch_ms": kms / n}
        if name in ALGO_FLOPS_PER_PAIR:
            ent["algo_tflops"] = ALGO_FLOPS_PER_PAIR[name] * d * hs * pairs * A * args.steps / (kms * 1e-3) / 1e12
        if name.startswith("a2a_"):
            ent["algo_GBps"] = perm_bytes * n / (kms * 1e-3) / 1e9
        kernels[name] = ent
    dom = max(per_kernel.items(), key=lambda kv: kv[1][0])[0]
    dms, dn = per_kernel[dom]
    roof = {"kernel": dom, "bound": "mfma", "unit": "TFLOP/s", "peak": BF16_PEAK_TFLOPS, "traffic": None}
    if dom in ALGO_FLOPS_PER_PAIR:
        per_launch = ALGO_FLOPS_PER_PAIR[dom] * d * hs * pairs * A * args.steps / dn
        roof.update({"achieved": round(per_launch / (dms / dn * 1e-3) / 1e12, 2), "algo_flops_per_launch": per_launch,
                     "avg_launch_ms": dms / dn})
        roof["frac"] = round(roof["achieved"] / BF16_PEAK_TFLOPS, 4)
    a2a_ms = sum(v["ms_per_step"] for k, v in kernels.items() if k.startswith("a2a_"))
    log(f"[bench] hierarchical step {ms:.3f} ms, {tflops:.1f} TFLOP/s; all-to-all {a2a_ms:.3f} ms of it")
    line = {
        "metric": "attention fwd+bwd TFLOP/s per CP-rank share (1 MI355X), % of bf16 MFMA peak",
        "value": round(tflops, 3), "unit": "TFLOP/s", "pct_of_bf16_peak": round(100.0 * tflops / BF16_PEAK_TFLOPS, 2),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, drawn on the device)",
        "config": {"workload": w["name"] + "-a2a+p2p-step", "a2a_size": A, "p2p_size": P, "cp_size": cp,
                   "heads_before_split": H, "heads_per_group": hs, "head_dim": d, "tokens": T,
                   "p2p_t_local": tl_p, "pairs_per_group": pairs, "flops_per_step": flops_step,
                   "parallelism": "one a2a group's step (both a2a ranks) on one GPU"},
        "all_to_all_ms_per_step": round(a2a_ms, 4), "all_to_all_bytes_per_call": perm_bytes,
        "kernels": kernels, "roofline": roof,
    }
    m_cp.close()
    m_p.close()
    print(json.dumps(line), flush=True)


def ag_bench(args):
    """All-gather share of the selected workload: the rank's queries against
    the gathered K/V (metadata build + forward + backward per step), the same
    attention pairs as the ring share plus the shard-view gather and the
    dK/dV scatter."""
    import numpy as np
    import torch
    from context_packed_attention_amd import api, synth
    w = synth.workload(args.workload)
    rank = w["ranks"][-1] if args.workload != 1 else 0
    batch, _ = synth.make_workload(args.workload)
    cp, hq, hkv, d = w["cp"], w["hq"], w["hkv"], w["d"]
    scale = 1.0 / math.sqrt(d)

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)

    cu = torch.tensor(batch.cu, dtype=torch.int32, device="cuda")
    cup = torch.tensor(batch.cup, dtype=torch.int32, device="cuda")
    T = batch.total_rows
    t_alloc = T // cp
    meta = api.cp_attn_rank_metadata(cu, cup, cp, rank, -1, t_alloc)
    gq, gdo = dev_bf16(batch.q), dev_bf16(batch.do)
    k_full, v_full = dev_bf16(batch.k), dev_bf16(batch.v)
    q = torch.empty((t_alloc, hq, d), dtype=torch.bfloat16, device="cuda")
    do = torch.empty_like(q)
    api.cp_attn_shard_gather(meta, rank, gq, q, hq * d * 2)
    api.cp_attn_shard_gather(meta, rank, gdo, do, hq * d * 2)
    del gq, gdo
    out = torch.empty_like(q)
    lse = torch.empty((hq, t_alloc), dtype=torch.float32, device="cuda")
    dq = torch.empty_like(q)
    dk_full = torch.empty_like(k_full)
    dv_full = torch.empty_like(v_full)
    ws_f = torch.empty(api.cp_attn_ag_workspace_bytes(meta, hq, hkv, d, 0), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(api.cp_attn_ag_workspace_bytes(meta, hq, hkv, d, 1), dtype=torch.uint8, device="cuda")
    pairs = sum(api.step_pairs(meta))
    meta.close()
    stream = torch.cuda.current_stream()

    def one_step():
        m = api.cp_attn_rank_metadata(cu, cup, cp, rank, -1, t_alloc, stream=stream)
        api.cp_attn_ag_fwd(m, q, k_full, v_full, hq, hkv, d, scale, 1, out, lse, ws_f, stream=stream)
        api.cp_attn_ag_bwd(m, q, k_full, v_full, out, lse, do, hq, hkv, d, scale, 1, dq, dk_full, dv_full, ws_b,
                           stream=stream)
        return m

    held = [one_step() for _ in range(args.warmup)]
    torch.cuda.synchronize()
    for m in held:
        m.close()
    held = []
    api.cp_attn_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        held.append(one_step())
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    api.cp_attn_timing_enable(False)
    per_kernel = api.cp_attn_timing_read()
    for m in held:
        m.close()
    ms = (t1 - t0) * 1e3 / args.steps
    tflops = 14 * d * hq * pairs / (ms * 1e-3) / 1e12
    kernels = {k: {"launches_per_step": v[1] / args.steps, "ms_per_step": v[0] / args.steps}
               for k, v in per_kernel.items()}
    line = {
        "metric": "all-gather CP share: attention fwd+bwd TFLOP/s (1 MI355X)",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16 Q/K/V/dO)",
        "config": {"workload": w["name"] + "-allgather", "cp_size": cp, "cp_rank": rank, "hq": hq, "hkv": hkv,
                   "head_dim": d, "gathered_rows": T, "pairs": pairs},
        "kernels": kernels,
    }
    print(json.dumps(line), flush=True)


def abba_bench(args):
    """The padding decision's cost, after the pages' own experiment ("[PyTorch]
    [Attention] THD P2P context-parallel regression when padded cu_seqlens are
    value-equal but not object-identical", Describe the bug: the same batch run
    with value-equal cu_seqlens_padded as a copy and as the same object took
    different paths and times). Here the decision is made on the device from
    values: pad_hint -1 (decide from the values) and 0 (the caller asserts no
    padding) must give the same launch sequence and the same step time within
    noise. Steps alternate in A B B A blocks so a drift of the clock or the
    box's load falls on both sides alike."""
    import numpy as np
    import torch
    from context_packed_attention_amd import api, synth
    w = synth.workload(2)
    rank = w["ranks"][-1]
    batch, _ = synth.make_workload(2)
    cp, hq, hkv, d = w["cp"], w["hq"], w["hkv"], w["d"]
    scale = 1.0 / math.sqrt(d)

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)

    cu = torch.tensor(batch.cu, dtype=torch.int32, device="cuda")
    cup = torch.tensor(batch.cup, dtype=torch.int32, device="cuda")  # distinct tensor, equal values
    t_alloc = int(batch.cup[-1]) // cp
    meta = api.cp_attn_rank_metadata(cu, cup, cp, rank, -1, t_alloc)
    gq, gk, gv, gdo = (dev_bf16(x) for x in (batch.q, batch.k, batch.v, batch.do))

    def gather(src, h, s):
        dst = torch.empty((t_alloc, h, d), dtype=torch.bfloat16, device="cuda")
        api.cp_attn_shard_gather(meta, s, src, dst, h * d * 2)
        return dst

    q, do = gather(gq, hq, rank), gather(gdo, hq, rank)
    ks = [gather(gk, hkv, s) for s in range(cp)]
    vs = [gather(gv, hkv, s) for s in range(cp)]
    out = torch.empty_like(q)
    lse = torch.empty((hq, t_alloc), dtype=torch.float32, device="cuda")
    dq = torch.empty_like(q)
    dks = [torch.empty_like(x) for x in ks]
    dvs = [torch.empty_like(x) for x in vs]
    ws_f = torch.empty(api.cp_attn_workspace_bytes(meta, hq, hkv, d, 0), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(api.cp_attn_workspace_bytes(meta, hq, hkv, d, 1), dtype=torch.uint8, device="cuda")
    pairs = sum(api.step_pairs(meta))
    meta.close()
    stream = torch.cuda.current_stream()

    def block(hint, n, record):
        held = []
        api.cp_attn_timing_enable(record)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            m = api.cp_attn_rank_metadata(cu, cup, cp, rank, hint, t_alloc, stream=stream)
            api.cp_attn_fwd(m, q, ks, vs, hq, hkv, d, scale, 1, out, lse, ws_f, stream=stream)
            api.cp_attn_bwd(m, q, ks, vs, out, lse, do, hq, hkv, d, scale, 1, dq, dks, dvs, ws_b, stream=stream)
            held.append(m)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) * 1e3 / n
        api.cp_attn_timing_enable(False)
        launches = {k: v[1] / n for k, v in api.cp_attn_timing_read().items()} if record else None
        for m in held:
            m.close()
        return dt, launches

    hints = {"A": -1, "B": 0}
    for h in hints.values():
        block(h, args.warmup, False)
    launches = {k: block(h, 1, True)[1] for k, h in hints.items()}
    times = {"A": [], "B": []}
    order = "ABBA" * 3
    for k in order:
        times[k].append(block(hints[k], args.steps, False)[0])
    ma, mb = float(np.mean(times["A"])), float(np.mean(times["B"]))
    spread = float(np.std(times["A"] + times["B"]) / np.mean(times["A"] + times["B"]))
    line = {
        "metric": "padding decision A/B on the 16K pack: ms per step with pad_hint -1 vs 0 (1 MI355X)",
        "value": round(ma, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ma, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16 Q/K/V/dO)",
        "config": {"workload": w["name"], "cp_size": cp, "cp_rank": rank, "hq": hq, "hkv": hkv, "head_dim": d,
                   "pairs": pairs, "order": order, "steps_per_block": args.steps,
                   "cu_seqlens_padded": "distinct tensor, value-equal"},
        "hint_auto_ms": round(ma, 4), "hint_zero_ms": round(mb, 4), "ratio": round(ma / mb, 4),
        "block_spread": round(spread, 4), "blocks_ms": {k: [round(x, 4) for x in v] for k, v in times.items()},
        "same_launches": launches["A"] == launches["B"], "launches_per_step": launches["A"],
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (one rank's share played on one MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from context_packed_attention_amd import api, synth
    from context_packed_attention_amd import _lib

    _lib.load()  # raises if the HIP library was not built
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)
    torch.cuda.set_device(0)
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return
    if args.a2a:
        a2a_bench(args)
        return
    if args.all_gather:
        ag_bench(args)
        return
    if args.hier:
        hier_bench(args)
        return
    if args.pad_hint_abba:
        abba_bench(args)
        return
    w = synth.workload(args.workload)
    rank = w["ranks"][-1] if args.workload != 1 else 0
    log(f"[bench] drawing inputs for {w['name']}")
    t0 = time.time()
    batch, _ = synth.make_workload(args.workload)
    log(f"[bench] inputs drawn in {time.time() - t0:.1f} s (T={batch.total_rows})")
    cp, hq, hkv, d = w["cp"], w["hq"], w["hkv"], w["d"]
    scale = 1.0 / math.sqrt(d)

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)

    cu = torch.tensor(batch.cu, dtype=torch.int32, device="cuda")
    cup = torch.tensor(batch.cup, dtype=torch.int32, device="cuda")   # distinct, value-equal when unpadded
    T_local = int(batch.cup[-1]) // cp
    t_alloc = T_local + max(0, args.tail)
    meta = api.cp_attn_rank_metadata(cu, cup, cp, rank, -1, t_alloc)
    gq, gk, gv, gdo = (dev_bf16(x) for x in (batch.q, batch.k, batch.v, batch.do))

    def gather(src, h, s):
        dst = torch.empty((t_alloc, h, d), dtype=torch.bfloat16, device="cuda")
        api.cp_attn_shard_gather(meta, s, src, dst, h * d * 2)
        return dst

    q = gather(gq, hq, rank)
    do = gather(gdo, hq, rank)
    ks = [gather(gk, hkv, s) for s in range(cp)]
    vs = [gather(gv, hkv, s) for s in range(cp)]
    del gq, gk, gv, gdo
    out = torch.empty((t_alloc, hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((hq, t_alloc), dtype=torch.float32, device="cuda")
    dq = torch.empty_like(q)
    dks = [torch.empty_like(x) for x in ks]
    dvs = [torch.empty_like(x) for x in vs]
    ws_f = torch.empty(api.cp_attn_workspace_bytes(meta, hq, hkv, d, 0), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(api.cp_attn_workspace_bytes(meta, hq, hkv, d, 1), dtype=torch.uint8, device="cuda")
    step_pairs = api.step_pairs(meta)
    pairs = sum(step_pairs)
    flops_step = 14 * d * hq * pairs
    valid_rows = int(meta.summary.valid_rows)
    stream = torch.cuda.current_stream()
    if args.phases > 0:
        sink = torch.zeros(1, dtype=torch.float32, device="cuda")
        res = power_phases(
            args.phases,
            lambda: api.cp_attn_fwd(meta, q, ks, vs, hq, hkv, d, scale, 1, out, lse, ws_f, stream=stream),
            lambda: api.cp_attn_bwd(meta, q, ks, vs, out, lse, do, hq, hkv, d, scale, 1, dq, dks, dvs, ws_b,
                                    stream=stream),
            lambda: api.cp_attn_mfma_probe(100000, sink, stream=stream)[1],
            4 * d * hq * pairs, 10 * d * hq * pairs)
        print(json.dumps({"workload": w["name"], "phases": res}), flush=True)
        meta.close()
        return
    meta.close()

    # host-side cost of one metadata build on an idle device (it ends in the
    # library's single synchronisation)
    torch.cuda.synchronize()
    meta_ms = []
    for _ in range(5):
        t = time.perf_counter()
        m = api.cp_attn_rank_metadata(cu, cup, cp, rank, -1, t_alloc, stream=stream)
        meta_ms.append((time.perf_counter() - t) * 1e3)
        m.close()

    # A step = this batch's metadata, forward and backward. The metadata comes
    # from the host copies of cu_seqlens (the batch's lengths are on the host,
    # where a data loader makes them) through the path that needs no host
    # synchronisation, on a second stream (default priority), one step ahead:
    # the next batch's tables are built while this one computes, and an event
    # orders its forward after them, as a data loader feeding a training loop
    # would. Every one of the K steps still builds its metadata inside the
    # timed region. Packs of more sequences than the host path carries use the
    # device path, in line. The in-line host-path and device-path step times
    # are reported beside it.
    cu_h = np.asarray(batch.cu, dtype=np.int32)
    cup_h = np.asarray(batch.cup, dtype=np.int32)
    host_meta = len(cu_h) - 1 <= 255
    meta_stream = torch.cuda.Stream()

    def make_meta(host, strm=None):
        strm = stream if strm is None else strm
        if host:
            return api.cp_attn_rank_metadata_host(cu_h, cup_h, cp, rank, -1, t_alloc, stream=strm)
        return api.cp_attn_rank_metadata(cu, cup, cp, rank, -1, t_alloc, stream=strm)

    def fwd_bwd(m):
        api.cp_attn_fwd(m, q, ks, vs, hq, hkv, d, scale, 1, out, lse, ws_f, stream=stream)
        api.cp_attn_bwd(m, q, ks, vs, out, lse, do, hq, hkv, d, scale, 1, dq, dks, dvs, ws_b, stream=stream)

    def run_pass(n, held, how):
        """how: 'pipelined' (host path, one step ahead), 'host' or 'device' (in line)."""
        if how != "pipelined":
            for _ in range(n):
                m = make_meta(how == "host")
                fwd_bwd(m)
                held.append(m)
            return
        m = make_meta(True, meta_stream)
        ev = torch.cuda.Event()
        ev.record(meta_stream)
        for k in range(n):
            stream.wait_event(ev)
            fwd_bwd(m)
            held.append(m)
            if k + 1 < n:
                m = make_meta(True, meta_stream)
                ev = torch.cuda.Event()
                ev.record(meta_stream)

    def timed_pass(how):
        held = []
        torch.cuda.synchronize()
        t = time.perf_counter()
        run_pass(args.steps, held, how)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t
        for m in held:
            m.close()
        return t, t + dt

    main_how = "pipelined" if host_meta else "device"
    log(f"[bench] warmup {args.warmup}")
    held = []
    run_pass(args.warmup, held, main_how)
    # the passes hold every step's handle until they end; the library pools
    # the handles' device buffers, so K of them are built and freed here first
    # (untimed), as a training loop's first steps would
    held += [make_meta(host_meta) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for m in held:
        m.close()
    held.clear()
    # per-kernel times: the same K steps with an event pair around every
    # launch (kept out of the timed pass: on short packs the events cost
    # several percent of a step)
    api.cp_attn_timing_enable(True)
    torch.cuda.synchronize()
    run_pass(args.steps, held, main_how)
    torch.cuda.synchronize()
    api.cp_attn_timing_enable(False)
    per_kernel = api.cp_attn_timing_read()
    for m in held:
        m.close()
    held.clear()
    # the same steps with the metadata built in line: device path (one host
    # wait per step), and host path
    a, b = timed_pass("device")
    device_meta_ms = (b - a) * 1e3 / args.steps
    inline_host_ms = None
    if host_meta:
        a, b = timed_pass("host")
        inline_host_ms = (b - a) * 1e3 / args.steps
    # the timed pass, last: the passes above keep the GPU busy before it
    log(f"[bench] timing {args.steps} steps")
    t0, t1 = timed_pass(main_how)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tflops = flops_step / (ms_per_step * 1e-3) / 1e12
    log(f"[bench] {ms_per_step:.3f} ms/step, {tflops:.1f} TFLOP/s")

    # algorithmic HBM bytes per launch of the HBM-bound kernels: bwd_pre reads
    # dO and out (bf16) and the LSE and writes two fp32 planes; dq_pad_rows
    # writes the padding rows of dQ; tail_zero writes the tail rows of dQ and
    # of every dK / dV part
    hbm_bytes = {"bwd_pre": T_local * hq * (4 * d + 12), "dq_pad_rows": (T_local - valid_rows) * hq * 2 * d,
                 "tail_zero": 2 * (t_alloc - T_local) * (hq + 2 * cp * hkv) * d}
    kernels = {}
    for name, (ms, n) in per_kernel.items():
        entry = {"launches_per_step": n / args.steps, "ms_per_step": ms / args.steps, "avg_launch_ms": ms / n}
        if name in ALGO_FLOPS_PER_PAIR:
            fl = ALGO_FLOPS_PER_PAIR[name] * d * hq * pairs * args.steps
            entry["algo_tflops"] = fl / (ms * 1e-3) / 1e12
            entry["exec_tflops"] = EXEC_FLOPS_PER_PAIR[name] * d * hq * pairs * args.steps / (ms * 1e-3) / 1e12
        if name in hbm_bytes:
            entry["algo_bytes_per_launch"] = hbm_bytes[name]
            entry["algo_GBps"] = hbm_bytes[name] * n / (ms * 1e-3) / 1e9
        kernels[name] = entry
    dom = max(per_kernel.items(), key=lambda kv: kv[1][0])[0]
    dom_ms, dom_n = per_kernel[dom]
    if dom in ALGO_FLOPS_PER_PAIR:
        per_launch = ALGO_FLOPS_PER_PAIR[dom] * d * hq * pairs * args.steps / dom_n
        achieved = per_launch / (dom_ms / dom_n * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(dom, w["name"]),
                "algo_flops_per_launch": per_launch, "avg_launch_ms": dom_ms / dom_n,
                "timing": "HIP event pair around every launch on its own stream, over a second pass of the "
                          "same timed steps"}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": None, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": None, "traffic": None}

    # the share as one HIP graph launch: metadata built once per batch, then
    # the captured forward + backward replayed; eager fwd + bwd (no timing
    # events) timed beside it on the same buffers
    gmeta = api.cp_attn_rank_metadata(cu, cup, cp, rank, -1, t_alloc, stream=stream)
    graph = api.cp_attn_graph_capture(gmeta, 3, q, ks, vs, hq, hkv, d, scale, 1, out, lse, do, dq, dks, dvs,
                                      ws_f, ws_b)

    def timed(fn, n):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3 / n

    def eager_fwd_bwd():
        api.cp_attn_fwd(gmeta, q, ks, vs, hq, hkv, d, scale, 1, out, lse, ws_f, stream=stream)
        api.cp_attn_bwd(gmeta, q, ks, vs, out, lse, do, hq, hkv, d, scale, 1, dq, dks, dvs, ws_b, stream=stream)

    for _ in range(max(1, args.warmup)):
        graph.launch(stream)
    eager_ms = timed(eager_fwd_bwd, args.steps)
    graph_ms = timed(lambda: graph.launch(stream), args.steps)
    graph_info = {"kernels_per_launch": graph.kernels, "eager_fwd_bwd_ms": round(eager_ms, 4),
                  "graph_fwd_bwd_ms": round(graph_ms, 4), "saving_ms": round(eager_ms - graph_ms, 4)}
    log(f"[bench] fwd+bwd eager {eager_ms:.3f} ms, one graph launch {graph_ms:.3f} ms ({graph.kernels} kernels)")
    graph.close()
    gmeta.close()

    # attainable matrix-unit rate on this device: the library's calibration
    # kernel (nothing but independent MFMA chains on toggling pseudo-random
    # operands), sustained: 40 back-to-back launches (about 0.6 s, long
    # enough for the power limit to set the clock), the median of the last 20
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    probes = [api.cp_attn_mfma_probe(100000, sink, stream=stream) for _ in range(40)]
    attainable = float(np.median([tf for _, tf in probes[20:]]))
    log(f"[bench] matrix-unit calibration: {attainable:.1f} TFLOP/s attainable")
    if roof.get("bound") == "mfma":
        roof["attainable_peak"] = round(attainable, 1)
        roof["frac_of_attainable"] = round(roof["achieved"] / attainable, 4)

    cpu = None
    if args.cpu_sample_stride > 0:
        log("[bench] oracle CPU baseline")
        cpu = cpu_baseline(batch, w, rank, scale, args.cpu_sample_stride)
        log(f"[bench] oracle: {cpu['value'] * 1e3:.2f} GFLOP/s ({cpu['seconds']:.1f} s)")

    line = {
        "metric": "attention fwd+bwd TFLOP/s per CP-rank share (1 MI355X), % of bf16 MFMA peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "pct_of_bf16_peak": round(100.0 * tflops / BF16_PEAK_TFLOPS, 2),
        "pct_of_attainable": round(100.0 * tflops / attainable, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V/dO)",
        "config": {"workload": w["name"], "cp_size": cp, "cp_rank": rank, "tokens": batch.total_rows,
                   "t_local": T_local, "hq": hq, "hkv": hkv, "head_dim": d, "causal": True,
                   "pairs": pairs, "step_pairs": step_pairs, "flops_per_step": flops_step, "t_alloc": t_alloc,
                   "parallelism": "one CP rank's share, all ring steps on one GPU"},
        "metadata_call_ms": round(sorted(meta_ms)[len(meta_ms) // 2], 4),
        "metadata": ("host copies of cu_seqlens, no host synchronisation, built on a second stream one step "
                     "ahead" if host_meta else "device path, in line") + "; built every step inside the timed region",
        "ms_per_step_host_metadata_inline": None if inline_host_ms is None else round(inline_host_ms, 4),
        "ms_per_step_device_metadata": round(device_meta_ms, 4),
        "kernels": kernels,
        "roofline": roof,
        "graph": graph_info,
        "mfma_calibration": {"attainable_tflops": round(attainable, 1),
                             "launch_ms_first_last": [round(probes[0][0], 3), round(probes[-1][0], 3)],
                             "kernel": "independent v_mfma_f32_32x32x16_bf16 chains on rotating pseudo-random "
                                       "bf16 operands, 8 per SIMD, no memory traffic; median of launches 21-40 "
                                       "of 40 back to back"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
