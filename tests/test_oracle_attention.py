"""Pins for the oracle's window attention (CPU only).

Closed forms (q = 0 gives the mean of V; constant V; one key returns its V row),
invariants (rows of the softmax sum to 1, key-order and global time-shift invariance),
a pure-Python brute force on a tiny case with RoPE written out by hand, and torch's
scaled_dot_product_attention in float64 on the oracle's rotated q/k.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, rope3d

# Tiny geometry: 6x8 grid (48 tokens per frame), 12 heads of 128, pairs 22/21/21.
GH, GW, PAIRS, BASE, H, D = 6, 8, (22, 21, 21), 10000.0, 12, 128
N = GH * GW


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_softmax_rows_sum_to_one():
    s = _rand((64, 300), 1) * 20
    p = attention.softmax_rows(s)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(p >= 0)


def test_attend_head_uses_the_normalised_weights():
    """attend_head is the softmax weights (the pinned helper above) applied to V: with
    V = I the output is the weight matrix itself, so its rows sum to 1."""
    qh, kh = _rand((40, D), 4), _rand((D, D), 5)
    o = attention.attend_head(qh, kh, np.eye(D), 1.0 / math.sqrt(D))
    assert np.allclose(o.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(o >= 0)
    assert np.allclose(o, attention.softmax_rows((qh @ kh.T) / math.sqrt(D)), rtol=0, atol=1e-15)


def test_zero_query_gives_mean_of_values():
    q = np.zeros((3 * N, H, D))
    k = _rand((5 * N, H, D), 2)
    v = _rand((5 * N, H, D), 3)
    o = attention.window_attention(q, 2, k, v, 0, GH, GW, PAIRS, BASE)
    want = v.mean(axis=0)
    assert np.allclose(o, want[None], rtol=0, atol=1e-14)


def test_constant_values_give_constant():
    q = _rand((2 * N, H, D), 4)
    k = _rand((4 * N, H, D), 5)
    v = np.broadcast_to(_rand((1, H, D), 6), (4 * N, H, D))
    o = attention.window_attention(q, 5, k, v, 3, GH, GW, PAIRS, BASE)
    assert np.allclose(o, v[:1], rtol=0, atol=1e-13)


def test_single_key_returns_its_value():
    # a 1x1 grid: one token per frame, one context frame -> one key
    q = _rand((3, 2, D), 7)
    k = _rand((1, 2, D), 8)
    v = _rand((1, 2, D), 9)
    o = attention.window_attention(q, 4, k, v, 4, 1, 1, PAIRS, BASE)
    assert np.allclose(o, v[:1], rtol=0, atol=1e-15)


def test_key_order_invariance():
    rng = np.random.default_rng(10)
    qh = rng.standard_normal((40, D))
    kh = rng.standard_normal((200, D))
    vh = rng.standard_normal((200, D))
    perm = rng.permutation(200)
    a = attention.attend_head(qh, kh, vh, 0.1)
    b = attention.attend_head(qh, kh[perm], vh[perm], 0.1)
    assert np.allclose(a, b, rtol=0, atol=1e-13)


def test_global_time_shift_invariance():
    q = _rand((3 * N, H, D), 11)
    k = _rand((5 * N, H, D), 12)
    v = _rand((5 * N, H, D), 13)
    a = attention.window_attention(q, 2, k, v, 0, GH, GW, PAIRS, BASE)
    b = attention.window_attention(q, 1002, k, v, 1000, GH, GW, PAIRS, BASE)
    assert np.allclose(a, b, rtol=0, atol=1e-11)
    # a relative shift does change the result
    c = attention.window_attention(q, 3, k, v, 0, GH, GW, PAIRS, BASE)
    assert not np.allclose(a, c, atol=1e-3)


def test_rows_subset_matches_full():
    q = _rand((3 * N, H, D), 14)
    k = _rand((5 * N, H, D), 15)
    v = _rand((5 * N, H, D), 16)
    full = attention.window_attention(q, 2, k, v, 0, GH, GW, PAIRS, BASE, block=37)
    rows = np.array([0, 1, 47, 48, 100, 143])
    sub = attention.window_attention(q, 2, k, v, 0, GH, GW, PAIRS, BASE, rows=rows, workers=1)
    assert np.allclose(full[rows], sub, rtol=0, atol=1e-15)


def _brute(q, q_t0, k, v, ctx_t0, gh, gw, pairs, base, q_tok0=0):
    """Pure-Python loops: RoPE pair by pair from the formulas, then softmax attention.
    Query token i sits at token q_tok0 + i counted from the start of frame q_t0."""
    n = gh * gw

    def pos(t0, i):
        return (t0 + i // n, (i % n) // gw, i % gw)

    def rot(x, p3):
        out = list(x)
        pair = 0
        for axis, P in enumerate(pairs):
            for j in range(P):
                th = p3[axis] * base ** (-j / P)
                a, b = x[2 * pair], x[2 * pair + 1]
                out[2 * pair] = a * math.cos(th) - b * math.sin(th)
                out[2 * pair + 1] = a * math.sin(th) + b * math.cos(th)
                pair += 1
        return out

    Lq, Hh, Dd = q.shape
    Lk = k.shape[0]
    o = np.zeros((Lq, Hh, Dd))
    for h in range(Hh):
        kr = [rot(list(k[j, h]), pos(ctx_t0, j)) for j in range(Lk)]
        for i in range(Lq):
            qr = rot(list(q[i, h]), pos(q_t0, q_tok0 + i))
            s = [sum(qr[d] * kr[j][d] for d in range(Dd)) / math.sqrt(Dd) for j in range(Lk)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for d in range(Dd):
                o[i, h, d] = sum(e[j] * v[j, h, d] for j in range(Lk)) / z
    return o


def test_brute_force_tiny():
    # 2x3 grid, 2 heads, head_dim 12 with pairs 2/2/2; q frames 3..4, context frames 1..4
    gh, gw, pairs = 2, 3, (2, 2, 2)
    n = gh * gw
    q = _rand((2 * n, 2, 12), 17)
    k = _rand((4 * n, 2, 12), 18)
    v = _rand((4 * n, 2, 12), 19)
    o = attention.window_attention(q, 3, k, v, 1, gh, gw, pairs, BASE, workers=1)
    want = _brute(q, 3, k, v, 1, gh, gw, pairs, BASE)
    assert np.allclose(o, want, rtol=0, atol=1e-13)


def test_brute_force_token_offset():
    # a query block starting at token 4 of frame 3 (of 6) and running into frame 4
    gh, gw, pairs = 2, 3, (2, 2, 2)
    n = gh * gw
    q = _rand((5, 2, 12), 27)
    k = _rand((4 * n, 2, 12), 28)
    v = _rand((4 * n, 2, 12), 29)
    o = attention.window_attention(q, 3, k, v, 1, gh, gw, pairs, BASE, workers=1, q_tok0=4)
    want = _brute(q, 3, k, v, 1, gh, gw, pairs, BASE, q_tok0=4)
    assert np.allclose(o, want, rtol=0, atol=1e-13)


def test_token_offset_rows_equal_whole_frame_rows():
    # rows are independent: a block cut at token 29 of frame 2 gives the same rows as
    # the whole frames 2..4 it was cut from
    q = _rand((3 * N, H, D), 30)
    k = _rand((5 * N, H, D), 31)
    v = _rand((5 * N, H, D), 32)
    full = attention.window_attention(q, 2, k, v, 0, GH, GW, PAIRS, BASE)
    part = attention.window_attention(q[29:29 + 70], 2, k, v, 0, GH, GW, PAIRS, BASE, q_tok0=29)
    assert np.allclose(full[29:29 + 70], part, rtol=0, atol=1e-15)
    # and a block starting in a later frame is the same as one at offset tok0 + N
    late = attention.window_attention(q[N + 5:N + 40], 3, k, v, 0, GH, GW, PAIRS, BASE, q_tok0=5)
    assert np.allclose(full[N + 5:N + 40], late, rtol=0, atol=1e-15)


def test_brute_force_full_head_dim():
    # the real head_dim/pair split on a 2x2 grid, a few tokens
    gh, gw = 2, 2
    q = _rand((4, 1, D), 20)
    k = _rand((8, 1, D), 21)
    v = _rand((8, 1, D), 22)
    o = attention.window_attention(q, 7, k, v, 6, gh, gw, PAIRS, BASE, workers=1)
    want = _brute(q, 7, k, v, 6, gh, gw, PAIRS, BASE)
    assert np.allclose(o, want, rtol=0, atol=1e-13)


def test_matches_torch_sdpa_float64():
    q = _rand((3 * N, H, D), 23)
    k = _rand((5 * N, H, D), 24)
    v = _rand((5 * N, H, D), 25)
    o = attention.window_attention(q, 2, k, v, 0, GH, GW, PAIRS, BASE)
    qh = rope3d.rope_exact(q, 2, GH, GW, PAIRS, BASE)
    kh = rope3d.rope_exact(k, 0, GH, GW, PAIRS, BASE)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))  # [H, L, D]
    ref = torch.nn.functional.scaled_dot_product_attention(t(qh), t(kh), t(v))
    assert np.allclose(o, ref.numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_explicit_scale_is_used():
    q = _rand((N, 2, D), 26)
    k = _rand((2 * N, 2, D), 27)
    v = _rand((2 * N, 2, D), 28)
    a = attention.window_attention(q, 1, k, v, 0, GH, GW, PAIRS, BASE, scale=1 / math.sqrt(D))
    b = attention.window_attention(q, 1, k, v, 0, GH, GW, PAIRS, BASE)
    c = attention.window_attention(q, 1, k, v, 0, GH, GW, PAIRS, BASE, scale=0.5)
    assert np.array_equal(a, b)
    assert not np.allclose(a, c, atol=1e-3)
