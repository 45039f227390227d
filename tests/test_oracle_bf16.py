"""Pins for the oracle's bf16 codec (CPU only).

The pages fix no number format; bf16 storage is the reading taken here.  The codec is
pinned to (a) hand-derived cases of the format's definition (tests/golden/bf16_cases.txt),
(b) a brute-force nearest-value search with exact rational arithmetic, (c) torch's
float32 -> bfloat16 conversion on float32 inputs and (d) a round trip over all patterns.
"""
import bisect
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bf16_cases.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        x, bits = line.split()
        rows.append((float.fromhex(x), int(bits, 16)))
    return rows


def test_golden_cases():
    rows = _golden()
    assert len(rows) >= 15
    x = np.array([r[0] for r in rows])
    want = np.array([r[1] for r in rows], dtype=np.uint16)
    got = bf16.f64_to_bits(x)
    for xi, g, w in zip(x, got, want):
        assert g == w, f"{xi.hex()}: got {g:#06x} want {w:#06x}"


# All finite non-negative bf16 values, ascending, as exact floats.
_POS = bf16.bits_to_f64(np.arange(0x0000, 0x7F80, dtype=np.uint16))
_POS_LIST = [float(v) for v in _POS]


def _brute(x):
    """Nearest bf16 to x by exact comparison with its two neighbours; ties to even."""
    a = abs(x)
    top = Fraction(2) ** 128  # first value past the largest finite (the inf encoding's place)
    i = bisect.bisect_right(_POS_LIST, a) - 1  # _POS[i] <= a
    lo = Fraction(_POS_LIST[i])
    lo_bits = i
    if i + 1 < len(_POS_LIST):
        hi = Fraction(_POS_LIST[i + 1])
    else:
        hi = top
    hi_bits = i + 1
    fa = Fraction(a)
    if fa == lo:
        bits = lo_bits
    else:
        dl, dh = fa - lo, hi - fa
        if dl < dh:
            bits = lo_bits
        elif dh < dl:
            bits = hi_bits
        else:
            bits = lo_bits if lo_bits % 2 == 0 else hi_bits
    if x < 0 or (x == 0 and np.signbit(x)):
        bits |= 0x8000
    return bits


def test_brute_force_random_and_edges():
    rng = np.random.default_rng(1234)
    xs = []
    # log-uniform magnitudes over the whole bf16 range incl. subnormals
    e = rng.uniform(-136, 128, 3000)
    xs += list(rng.choice([-1.0, 1.0], 3000) * 2.0 ** e)
    # midpoints between neighbouring bf16 values and their float64 neighbours
    idx = rng.integers(0, len(_POS_LIST) - 1, 1500)
    for i in idx:
        m = (_POS_LIST[i] + _POS_LIST[i + 1]) / 2.0  # exact in float64
        xs += [m, np.nextafter(m, np.inf), np.nextafter(m, -np.inf), -m]
    xs += [0.0, -0.0]
    xs = np.array(xs, dtype=np.float64)
    got = bf16.f64_to_bits(xs)
    for x, g in zip(xs, got):
        assert int(g) == _brute(float(x)), float(x).hex()


def test_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(7)
    x32 = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),   # float32 subnormals
        (rng.standard_normal(20000) * 1e37).astype(np.float32),
    ])
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16.f64_to_bits(x32.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_trip_all_patterns():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    v = bf16.bits_to_f64(bits)
    keep = ~np.isnan(v)
    assert np.array_equal(bf16.f64_to_bits(v[keep]), bits[keep])
    assert np.all(np.isnan(v[~keep]))


def test_overflow_and_specials():
    got = bf16.f64_to_bits(np.array([1e39, -1e39, np.inf, -np.inf, np.nan]))
    assert list(got[:4]) == [0x7F80, 0xFF80, 0x7F80, 0xFF80]
    assert got[4] & 0x7F80 == 0x7F80 and got[4] & 0x7F


@pytest.mark.parametrize("x", [1.0, -3.5, 0.15625, 2.0 ** -130])
def test_bits_to_f64_exact(x):
    # values exactly representable in bf16 come back unchanged
    assert bf16.bits_to_f64(bf16.f64_to_bits(np.array([x])))[0] == x
