"""Pin of the oracle's only input conversion, bf16 bit patterns -> float64.

Every oracle input passes through ``bf16_to_f64``, and the tolerance model
calls it on both sides, so a mistake there would show only as a GPU parity
failure blamed on the kernels. It is checked here against an independent
implementation (torch's bfloat16 -> float64 conversion on the CPU) on all
65,536 bit patterns, and against values fixed by the bfloat16 format
(1 sign, 8 exponent, 7 fraction bits; the upper half of an IEEE binary32).
"""
import math

import numpy as np
import torch

from oracle import cp_attn_oracle as O


def test_all_bit_patterns_match_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.bf16_to_f64(bits)
    assert got.dtype == np.float64 and got.shape == bits.shape
    want = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    assert np.array_equal(nan_g, nan_w)
    assert np.array_equal(got[~nan_g], want[~nan_w])
    # signed zeros and infinities keep their signs
    assert np.array_equal(np.signbit(got[~nan_g]), np.signbit(want[~nan_w]))
    # 2 * 127 * 128 finite nonzero normal patterns, 2 * 127 subnormals, 2 zeros,
    # 2 infinities, 2 * 127 NaNs
    assert int(nan_g.sum()) == 2 * 127
    assert int(np.isinf(got).sum()) == 2


def test_fixed_values_of_the_format():
    cases = {
        0x3F80: 1.0, 0xC000: -2.0, 0x4049: 3.140625, 0x3F00: 0.5, 0x0000: 0.0,
        0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,     # largest finite
        0x0080: 2.0 ** -126,                    # smallest normal
        0x0001: 2.0 ** -133,                    # smallest subnormal
        0x7F80: math.inf, 0xFF80: -math.inf,
    }
    got = O.bf16_to_f64(np.array(list(cases), dtype=np.uint16))
    for (b, v), g in zip(cases.items(), got):
        assert g == v, (hex(b), g, v)
    neg0 = O.bf16_to_f64(np.array([0x8000], dtype=np.uint16))[0]
    assert neg0 == 0.0 and math.copysign(1.0, neg0) == -1.0
    nan = O.bf16_to_f64(np.array([0x7FC1, 0xFFC0, 0x7F81], dtype=np.uint16))
    assert np.isnan(nan).all()


def test_round_trip_of_exactly_representable_values():
    # integers up to 256 and their negatives are exact in bf16 (8 significant bits)
    vals = np.concatenate([np.arange(-256, 257), [2.0 ** e for e in range(-126, 128)]]).astype(np.float64)
    bits = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(O.bf16_to_f64(bits), vals)
