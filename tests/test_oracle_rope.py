"""Pins for the oracle's 3D RoPE (CPU only).

The pages say RoPE covers time, height and width and give no formula; the readings
(interleaved pairs, 22/21/21 split in t/h/w order, per-axis frequencies base^(-j/P),
counter-clockwise rotation, absolute frame index) are pinned by closed forms written
independently here, so a wrong sign, split, offset, exponent or position fails.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16, rope3d

GH, GW, PAIRS, BASE = 30, 52, (22, 21, 21), 10000.0
D = 128
N = GH * GW
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rope_closed_form.txt")


def _unit_token(t, r, c, p):
    """A block starting at frame t whose last token sits at (t, r, c), dim 2p = 1."""
    i = r * GW + c
    x = np.zeros((i + 1, 1, D))
    x[i, 0, 2 * p] = 1.0
    return x, i


def test_golden_closed_forms():
    n = 0
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        t, r, c, p, y0, y1 = line.split()
        t, r, c, p = int(t), int(r), int(c), int(p)
        x, i = _unit_token(t, r, c, p)
        y = rope3d.rope_exact(x, t, GH, GW, PAIRS, BASE)[i, 0]
        assert y[2 * p] == pytest.approx(float(y0), abs=1e-13)
        assert y[2 * p + 1] == pytest.approx(float(y1), abs=1e-13)
        others = np.delete(y, [2 * p, 2 * p + 1])
        assert np.all(others == 0.0)
        n += 1
    assert n >= 8


def test_positions_frame_major_row_major():
    t, r, c = rope3d.token_positions(7, 3 * N, GH, GW)
    assert (t[0], r[0], c[0]) == (7, 0, 0)
    assert (t[GW], r[GW], c[GW]) == (7, 1, 0)
    assert (t[N - 1], r[N - 1], c[N - 1]) == (7, GH - 1, GW - 1)
    assert (t[N], r[N], c[N]) == (8, 0, 0)
    assert (t[2 * N + 5 * GW + 3], r[2 * N + 5 * GW + 3], c[2 * N + 5 * GW + 3]) == (9, 5, 3)


def test_positions_with_token_offset():
    # a block cut out of the frame sequence at token N-2 of frame 7
    t, r, c = rope3d.token_positions(7, 5, GH, GW, tok0=N - 2)
    got = list(zip(t.tolist(), r.tolist(), c.tolist()))
    assert got == [(7, GH - 1, GW - 2), (7, GH - 1, GW - 1), (8, 0, 0), (8, 0, 1), (8, 0, 2)]
    with pytest.raises(ValueError):
        rope3d.token_positions(7, 5, GH, GW, tok0=N)


def _complex_axis(z, pos, n_pairs):
    """Independent 1-D RoPE: pair j of the axis times exp(i pos 10000^(-j/P))."""
    j = np.arange(n_pairs)
    w = np.power(10000.0, -j / n_pairs)
    return z * np.exp(1j * pos * w)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_each_axis_is_a_1d_rope(axis):
    rng = np.random.default_rng(axis)
    off = [0, PAIRS[0], PAIRS[0] + PAIRS[1]][axis]
    P = PAIRS[axis]
    for pos in [1, 3, 17, 29]:
        t, r, c = [(pos, 0, 0), (0, pos, 0), (0, 0, pos % GW)][axis]
        posv = [t, r, c][axis]
        x = rng.standard_normal((r * GW + c + 1, 2, D))
        i = r * GW + c
        y = rope3d.rope_exact(x, t, GH, GW, PAIRS, BASE)[i]
        z = x[i, :, 0::2] + 1j * x[i, :, 1::2]
        want = z.copy()
        want[:, off:off + P] = _complex_axis(z[:, off:off + P], posv, P)
        got = y[:, 0::2] + 1j * y[:, 1::2]
        assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_norm_preserved_per_pair():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3 * N, 2, D))
    y = rope3d.rope_exact(x, 11, GH, GW, PAIRS, BASE)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.allclose(nx, ny, rtol=1e-13, atol=0)


def test_relative_position_property():
    """q^(p+d) . k^(p'+d) == q^(p) . k^(p'): the score sees only the (t,h,w) offset."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal(D)
    k = rng.standard_normal(D)

    def rot(vec, t, r, c):
        x = np.zeros((r * GW + c + 1, 1, D))
        x[-1, 0] = vec
        return rope3d.rope_exact(x, t, GH, GW, PAIRS, BASE)[-1, 0]

    for (p, pp, d) in [((2, 3, 4), (5, 10, 20), (7, 6, 9)),
                       ((0, 0, 0), (1, 1, 1), (40, 20, 30)),
                       ((9, 12, 40), (3, 2, 1), (100, 3, 5))]:
        a = rot(q, *p) @ rot(k, *pp)
        b = rot(q, p[0] + d[0], p[1] + d[1], p[2] + d[2]) @ rot(k, pp[0] + d[0], pp[1] + d[1], pp[2] + d[2])
        assert a == pytest.approx(b, rel=1e-11, abs=1e-11)
    # and it does depend on the offset
    assert abs(rot(q, 0, 0, 0) @ rot(k, 1, 0, 0) - rot(q, 0, 0, 0) @ rot(k, 0, 0, 0)) > 1e-3


def test_spec_within_one_ulp_of_exact():
    rng = np.random.default_rng(5)
    xb = bf16.f64_to_bits(rng.standard_normal((2 * N, 3, D)))
    spec = bf16.bits_to_f64(rope3d.rope_spec_bits(xb, 20, GH, GW, PAIRS, BASE))
    exact = rope3d.rope_exact(bf16.bits_to_f64(xb), 20, GH, GW, PAIRS, BASE)
    _, E = np.frexp(np.abs(exact))
    ulp = np.ldexp(1.0, np.maximum(E - 1, -126) - 7)
    # float32 tables move each term by at most 2^-24 relative; then one bf16 rounding
    x = bf16.bits_to_f64(xb)
    mag = np.empty_like(x)
    mag[..., 0::2] = np.abs(x[..., 0::2]) + np.abs(x[..., 1::2])
    mag[..., 1::2] = mag[..., 0::2]
    assert np.all(np.abs(spec - exact) <= ulp + mag * 2.0 ** -24)
    # away from cancellation it is within one bf16 ulp of the exact rotation
    big = np.abs(exact) > mag * 2.0 ** -8
    assert np.all(np.abs(spec - exact)[big] <= ulp[big])
    # and the two actually differ somewhere (spec is rounded)
    assert np.any(spec != exact)


def _nearest_bf16_fraction(v):
    """bf16 bits nearest to the Fraction v (ties to even), by search over neighbours."""
    f = float(v)  # correctly rounded; start near it
    b = int(bf16.f64_to_bits(np.array([f]))[0])
    cands = [(b + d) & 0xFFFF for d in (-1, 0, 1)]
    best = None
    for cb in cands:
        cv = bf16.bits_to_f64(np.array([cb], dtype=np.uint16))[0]
        if not np.isfinite(cv):
            continue
        dist = abs(Fraction(cv) - v)
        key = (dist, cb & 1)
        if best is None or key < best[0]:
            best = (key, cb)
    return best[1]


def test_spec_bits_against_rational_arithmetic():
    """Recompute the spec for sampled elements with Fractions: float32 tables, exact
    products, one float64 rounding of the sum, then nearest bf16."""
    rng = np.random.default_rng(6)
    L = 2 * N
    t0 = 3
    xb = bf16.f64_to_bits(rng.standard_normal((L, 2, D)))
    got = rope3d.rope_spec_bits(xb, t0, GH, GW, PAIRS, BASE)
    x = bf16.bits_to_f64(xb)
    offs = [0, 22, 43]
    for _ in range(400):
        i = int(rng.integers(L))
        h = int(rng.integers(2))
        p = int(rng.integers(64))
        t, r, c = t0 + i // N, (i % N) // GW, i % GW
        a = 0 if p < 22 else (1 if p < 43 else 2)
        j = p - offs[a]
        P = PAIRS[a]
        pos = [t, r, c][a]
        th = float(pos) * (BASE ** (-(j / P)))
        c32 = Fraction(float(np.float32(math.cos(th))))
        s32 = Fraction(float(np.float32(math.sin(th))))
        x0 = Fraction(float(x[i, h, 2 * p]))
        x1 = Fraction(float(x[i, h, 2 * p + 1]))
        y0 = Fraction(float(x0 * c32 - x1 * s32))  # float() rounds the exact value once
        y1 = Fraction(float(x0 * s32 + x1 * c32))
        assert got[i, h, 2 * p] == _nearest_bf16_fraction(y0)
        assert got[i, h, 2 * p + 1] == _nearest_bf16_fraction(y1)


def test_spec_uses_the_float32_tables():
    """The specification rotates with float32-rounded cos/sin (the device's tables), not
    float64 ones.  The two choices round an element to different bf16 values only about
    once in 2^16 elements, so this pin scans a 3.2 M-element block for every element where
    they differ and checks the specification there with rational arithmetic."""
    rng = np.random.default_rng(9)
    L, H, t0 = 4 * N, 4, 37
    xb = bf16.f64_to_bits(rng.standard_normal((L, H, D)))
    x = bf16.bits_to_f64(xb)
    got = rope3d.rope_spec_bits(xb, t0, GH, GW, PAIRS, BASE)
    # cos/sin written out here: pair j of an axis with P pairs turns by pos * BASE^(-j/P)
    i = np.arange(L)
    axes = [(t0 + i // N, PAIRS[0]), ((i % N) // GW, PAIRS[1]), (i % GW, PAIRS[2])]
    c64, s64 = [], []
    for pos, P in axes:
        table = {int(p): [(math.cos(float(p) * BASE ** (-(j / P))), math.sin(float(p) * BASE ** (-(j / P))))
                          for j in range(P)] for p in np.unique(pos)}
        c64.append(np.array([[cs[0] for cs in table[int(p)]] for p in pos]))
        s64.append(np.array([[cs[1] for cs in table[int(p)]] for p in pos]))
    c64, s64 = np.concatenate(c64, axis=1)[:, None, :], np.concatenate(s64, axis=1)[:, None, :]
    c32, s32 = c64.astype(np.float32).astype(np.float64), s64.astype(np.float32).astype(np.float64)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    cand = []
    for k, (f32_val, f64_val) in enumerate([(x0 * c32 - x1 * s32, x0 * c64 - x1 * s64),
                                            (x0 * s32 + x1 * c32, x0 * s64 + x1 * c64)]):
        differ = bf16.f64_to_bits(f32_val) != bf16.f64_to_bits(f64_val)
        cand += [(a, b, cc, k) for a, b, cc in zip(*np.nonzero(differ))]
    assert len(cand) >= 10, len(cand)
    for a, b, p, k in cand:
        fc, fs = Fraction(float(c32[a, 0, p])), Fraction(float(s32[a, 0, p]))
        f0, f1 = Fraction(float(x0[a, b, p])), Fraction(float(x1[a, b, p]))
        exact = f0 * fc - f1 * fs if k == 0 else f0 * fs + f1 * fc
        assert got[a, b, 2 * p + k] == _nearest_bf16_fraction(Fraction(float(exact)))


def test_absolute_frame_index_is_used():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((N, 1, D))
    a = rope3d.rope_exact(x, 0, GH, GW, PAIRS, BASE)
    b = rope3d.rope_exact(x, 1000, GH, GW, PAIRS, BASE)
    # time dims differ, row/col dims identical
    assert not np.allclose(a[:, :, :44], b[:, :, :44])
    assert np.array_equal(a[:, :, 44:], b[:, :, 44:])
