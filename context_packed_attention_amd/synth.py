"""Seeded synthetic inputs for packed variable-length ("thd") attention.

This module only draws numbers: sequence lengths, padding amounts and the
bf16 tensors Q, K, V and dO of a packed batch, in *global* packed layout
(sequence b's valid tokens at rows [cup[b], cup[b] + L_b), padding slots up to
cup[b+1]). It holds none of the attention arithmetic and none of the
context-parallel sharding: both the fp64 oracle and the HIP path take its
output as their input.

Recipe (the pages name no dataset; these workloads stand in for the
unnamed training run of "THD P2P context-parallel regression when padded
cu_seqlens are value-equal but not object-identical", "Steps/Code to
reproduce bug", and for the "128K length with CP4" regime of "thd format is
not supported with hierarchical CP implementation yet"):

* lengths: multiples of 8 drawn uniformly from [lo, hi] until the running sum
  reaches the total; the last length is then cut so the sum equals the total
  exactly (it may fall below lo, down to 8).
* padding: pad_b uniform in {0..max_pad}; P_b = ceil((L_b + pad_b) / m) * m
  with m = 2 * CP, so every padded length is divisible by 2 * CP.
* values: i.i.d. N(0, 1) drawn as float32 and rounded to bf16 with
  round-to-nearest-even. Padding slots hold "garbage" N(0, 1) * 1000 (bf16),
  so any leak of a padding row into a valid result is far above tolerance.

Every tensor is drawn in blocks of ``BLOCK_ROWS`` rows; block j of tensor
``tid`` comes from ``numpy.random.default_rng([seed, tid, j])``. Any row range
can therefore be regenerated on its own and blocks can be drawn in parallel.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

BLOCK_ROWS = 2048

# stream ids of numpy.random.default_rng([seed, id, ...])
_SID_LENGTHS = 100
_SID_PADS = 101
_TID = {"q": 0, "k": 1, "v": 2, "do": 3}
_GARBAGE_TID_OFFSET = 10
GARBAGE_SCALE = 1000.0


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits (uint16) to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_lengths(seed: int, total: int, lo: int, hi: int, mult: int = 8) -> list[int]:
    """Multiples of ``mult`` uniform in [lo, hi] until the sum reaches ``total``;
    the last one is cut so the lengths sum to ``total`` exactly."""
    rng = np.random.default_rng([seed, _SID_LENGTHS])
    lens: list[int] = []
    s = 0
    while s < total:
        L = int(rng.integers(lo // mult, hi // mult + 1)) * mult
        if s + L > total:
            L = total - s
        lens.append(L)
        s += L
    return lens


def draw_padded_lengths(seed: int, lengths: list[int], max_pad: int, mult: int) -> list[int]:
    """P_b = ceil((L_b + pad_b) / mult) * mult with pad_b uniform in {0..max_pad}."""
    rng = np.random.default_rng([seed, _SID_PADS])
    pads = rng.integers(0, max_pad + 1, size=len(lengths))
    return [int(-(-(L + int(p)) // mult) * mult) for L, p in zip(lengths, pads)]


def _draw_rows(seed: int, tid: int, r0: int, r1: int, row_shape: tuple, scale: float = 1.0) -> np.ndarray:
    """Rows [r0, r1) of tensor ``tid`` as bf16 bits, block by block."""
    out = np.empty((r1 - r0,) + tuple(row_shape), dtype=np.uint16)
    width = int(np.prod(row_shape))
    jobs = []
    j0, j1 = r0 // BLOCK_ROWS, (r1 - 1) // BLOCK_ROWS if r1 > r0 else -1

    def one(j):
        rng = np.random.default_rng([seed, tid, j])
        blk = rng.standard_normal((BLOCK_ROWS, width), dtype=np.float32)
        if scale != 1.0:
            blk *= np.float32(scale)
        a, b = max(r0, j * BLOCK_ROWS), min(r1, (j + 1) * BLOCK_ROWS)
        out[a - r0:b - r0] = f32_to_bf16_bits(blk[a - j * BLOCK_ROWS:b - j * BLOCK_ROWS]).reshape((b - a,) + tuple(row_shape))

    workers = max(1, min(16, os.cpu_count() or 1))
    if j1 - j0 + 1 <= 2:
        for j in range(j0, j1 + 1):
            one(j)
    else:
        with _cf.ThreadPoolExecutor(workers) as ex:
            jobs = [ex.submit(one, j) for j in range(j0, j1 + 1)]
            for f in jobs:
                f.result()
    return out


@dataclass
class PackedBatch:
    """A packed batch in global layout. Tensors are bf16 bits (uint16)."""
    name: str
    seed: int
    cu: np.ndarray            # int32 [B+1], cumulative valid lengths
    cup: np.ndarray           # int32 [B+1], cumulative padded lengths (a distinct array)
    hq: int
    hkv: int
    d: int
    q: np.ndarray             # uint16 [T, hq, d]
    k: np.ndarray             # uint16 [T, hkv, d]
    v: np.ndarray             # uint16 [T, hkv, d]
    do: np.ndarray            # uint16 [T, hq, d]
    extra: dict = field(default_factory=dict)

    @property
    def total_rows(self) -> int:
        return int(self.cup[-1])


def make_batch(name: str, seed: int, lengths, padded, hq: int, hkv: int, d: int,
               garbage_scale: float | None = GARBAGE_SCALE) -> PackedBatch:
    """Draw Q, K, V, dO for the given lengths; padding rows get garbage."""
    lengths = [int(x) for x in lengths]
    padded = [int(x) for x in padded]
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    cup = np.zeros(len(padded) + 1, dtype=np.int32)
    cup[1:] = np.cumsum(padded)
    T = int(cup[-1])
    tensors = {}
    for nm, h in (("q", hq), ("k", hkv), ("v", hkv), ("do", hq)):
        t = _draw_rows(seed, _TID[nm], 0, T, (h, d))
        if garbage_scale is not None and any(P > L for L, P in zip(lengths, padded)):
            for b, (L, P) in enumerate(zip(lengths, padded)):
                if P > L:
                    a = int(cup[b]) + L
                    e = int(cup[b + 1])
                    t[a:e] = _draw_rows(seed, _TID[nm] + _GARBAGE_TID_OFFSET, a, e, (h, d), garbage_scale)
        tensors[nm] = t
    return PackedBatch(name, seed, cu, cup.copy(), hq, hkv, d, **tensors)


# The five workloads: (name, seed, cp, ranks, builder)
def workload(cfg: int) -> dict:
    """Shapes and shares of the five standard workloads (1-based index)."""
    if cfg == 1:
        return dict(name="tiny-3seq-cp2", seed=1001, cp=2, ranks=[0, 1], hq=2, hkv=2, d=64,
                    lengths=[64, 128, 64], max_pad=None)
    if cfg == 2:
        return dict(name="pack16k-cp4", seed=1002, cp=4, ranks=[1], hq=32, hkv=32, d=128,
                    lengths=draw_lengths(1002, 16384, 512, 4096), max_pad=None)
    if cfg == 3:
        # the same lengths as the 16K pack, then padding drawn from this seed
        return dict(name="pack16k-padded-cp4", seed=1003, cp=4, ranks=[1], hq=32, hkv=32, d=128,
                    lengths=draw_lengths(1002, 16384, 512, 4096), max_pad=64)
    if cfg == 4:
        return dict(name="single131072-gqa-cp4", seed=1004, cp=4, ranks=[2], hq=32, hkv=8, d=128,
                    lengths=[131072], max_pad=None)
    if cfg == 5:
        return dict(name="pack64k-hier2x2-p2p", seed=1005, cp=2, ranks=[0], hq=16, hkv=16, d=128,
                    lengths=draw_lengths(1005, 65536, 2048, 16384), max_pad=None)
    raise ValueError(f"unknown workload {cfg}")


def make_workload(cfg: int) -> tuple[PackedBatch, dict]:
    w = workload(cfg)
    lengths = w["lengths"]
    if w["max_pad"] is None:
        padded = list(lengths)
    else:
        padded = draw_padded_lengths(w["seed"], lengths, w["max_pad"], 2 * w["cp"])
    batch = make_batch(w["name"], w["seed"], lengths, padded, w["hq"], w["hkv"], w["d"])
    return batch, w


def device_normal_bf16(shape, seed: int):
    """Seeded N(0, 1) bf16 tensor drawn directly on the current GPU (for
    shapes too large to draw and upload from the host); the same seed and
    shape give the same tensor."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, device="cuda", dtype=torch.bfloat16)
