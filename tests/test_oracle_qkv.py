"""Pins of oracle.qkv (the QKV projection feeding the cache) against brute force,
closed forms and the already pinned RoPE and bf16 oracles."""
import itertools

import numpy as np
import pytest

from oracle import bf16, qkv, rope3d


def _bits(a):
    return bf16.f64_to_bits(np.asarray(a, dtype=np.float64))


def test_brute_force_integer_inputs():
    # small integers are exact in bf16 and every sum is exact in float64
    rng = np.random.default_rng(1)
    H, D, L = 2, 4, 5
    C = H * D
    x = rng.integers(-3, 4, size=(L, C))
    w = rng.integers(-3, 4, size=(3 * C, C))
    q, k, v = qkv.project(_bits(x), _bits(w), H, D)
    want = np.zeros((L, 3 * C))
    for i, j in itertools.product(range(L), range(3 * C)):
        want[i, j] = sum(int(x[i, c]) * int(w[j, c]) for c in range(C))
    assert np.array_equal(q.reshape(L, C), want[:, :C])
    assert np.array_equal(k.reshape(L, C), want[:, C:2 * C])
    assert np.array_equal(v.reshape(L, C), want[:, 2 * C:])


def test_block_order_q_then_k_then_v():
    H, D = 2, 4
    C = H * D
    x = np.random.default_rng(2).standard_normal((6, C))
    xb = _bits(x)
    eye = np.eye(C)
    q, k, v = qkv.project(xb, _bits(np.vstack([eye, 2 * eye, -eye])), H, D)
    xv = bf16.bits_to_f64(xb).reshape(6, H, D)
    assert np.array_equal(q, xv)
    assert np.array_equal(k, 2 * xv)
    assert np.array_equal(v, -xv)


def test_feature_index_is_head_major():
    # output feature j of each block reads input feature perm[j]; [L, H, D] views put
    # feature h*D + d at [:, h, d]
    H, D = 3, 4
    C = H * D
    perm = (5 * np.arange(C) + 3) % C
    w = np.zeros((3 * C, C))
    for blk in range(3):
        w[blk * C + np.arange(C), perm] = blk + 1
    x = np.random.default_rng(3).standard_normal((4, C))
    xb = _bits(x)
    xv = bf16.bits_to_f64(xb)
    outs = qkv.project(xb, _bits(w), H, D)
    for blk, o in enumerate(outs):
        for h, d in itertools.product(range(H), range(D)):
            assert np.array_equal(o[:, h, d], (blk + 1) * xv[:, perm[h * D + d]])


def test_cache_entries_rotate_the_stored_key():
    # W_k = I: the rotated key is the RoPE specification of x itself; q and v are 0
    pairs, H = (2, 1, 1), 2
    D = 2 * sum(pairs)
    C = H * D
    gh, gw, t0 = 2, 3, 5
    x = np.random.default_rng(4).standard_normal((2 * gh * gw, C))
    xb = _bits(x)
    w = np.vstack([np.zeros((C, C)), np.eye(C), np.zeros((C, C))])
    q, kr, v = qkv.cache_entries(xb, _bits(w), t0, gh, gw, pairs, 10000.0)
    assert not q.any() and not v.any()
    assert np.array_equal(kr, rope3d.rope_spec_bits(xb.reshape(-1, H, D), t0, gh, gw, pairs, 10000.0))
    # W_k = w3 I with w3 = bf16(1/3) = 0.333984375: each key x * w3 is exact in float64 but
    # not a bf16 value; the cache holds its bf16 rounding, and the rotated key is the
    # specification of that stored key (not a rotation of the unrounded product)
    w3 = 0.333984375
    q, kr, v = qkv.cache_entries(xb, _bits(w * w3), t0, gh, gw, pairs, 10000.0)
    stored = _bits(bf16.bits_to_f64(xb) * w3).reshape(-1, H, D)
    assert not np.array_equal(stored, xb.reshape(-1, H, D))
    assert np.array_equal(kr, rope3d.rope_spec_bits(stored, t0, gh, gw, pairs, 10000.0))


def test_rounding_is_once_from_float64():
    # inputs 1, 2^-8, 2^-30 are exact bf16 values; weight rows sum them
    H, D = 1, 8
    C = H * D
    x = np.zeros((1, C))
    x[0, :3] = [1.0, 2.0 ** -8, 2.0 ** -30]
    w = np.zeros((3 * C, C))
    w[0, :3] = [1, 1, 1]          # q0 = 1 + 2^-8 + 2^-30: just above the tie 1 + 2^-8
    w[1, :2] = [1, 1]             # q1 = 1 + 2^-8: a tie, to even
    w[2, 0], w[2, 1] = 1, 3       # q2 = 1 + 3*2^-8: a tie, to even
    q, _, _ = qkv.project_bits(_bits(x), _bits(w), H, D)
    # rounding the float64 sum once gives 1 + 2^-7; a float32 detour (1 + 2^-8, then the
    # tie to even) would give 1.0
    assert q[0, 0, 0] == 0x3F81
    assert q[0, 0, 1] == 0x3F80
    assert q[0, 0, 2] == 0x3F82


@pytest.mark.parametrize("seed", [5, 6])
def test_float32_accumulation_is_within_one_bf16_step(seed):
    """The tolerance the device parity test uses: a float32 running sum over the 1,536
    input features, rounded to bf16, equals the float64-then-bf16 value except where
    the two straddle a rounding boundary, and then it is within one bf16 step plus the
    worst-case float32 summation error E = (C - 1) 2^-24 sum |x_c w_c| (which matters
    for outputs near zero).  Two weight rows are built to cancel almost exactly."""
    rng = np.random.default_rng(seed)
    C, L, F = 1536, 16, 64
    xb = _bits(rng.standard_normal((L, C)))
    w0 = rng.standard_normal((F, C)) / np.sqrt(C)
    x0 = bf16.bits_to_f64(xb)
    for r in (0, 1):  # make x[r] . w[r] tiny: remove its projection on x[r]
        w0[r] -= (w0[r] @ x0[r]) / (x0[r] @ x0[r]) * x0[r]
    wb = _bits(w0)
    x, w = bf16.bits_to_f64(xb), bf16.bits_to_f64(wb)
    exact = x @ w.T
    acc = np.zeros((L, F), dtype=np.float32)
    for c in range(C):  # float32 products of bf16 values are exact; one rounding per add
        acc = (acc + (x[:, c:c + 1] * w[:, c][None, :]).astype(np.float32)).astype(np.float32)
    dev = bf16.f64_to_bits(acc.astype(np.float64))
    ref = bf16.f64_to_bits(exact)
    same = dev == ref
    assert same.mean() > 0.98
    diff = np.abs(bf16.bits_to_f64(dev) - bf16.bits_to_f64(ref))
    E = (C - 1) * 2.0 ** -24 * (np.abs(x) @ np.abs(w).T)
    assert np.all(diff <= np.abs(bf16.bits_to_f64(ref)) * 2.0 ** -7 * 1.01 + 1.02 * E)
    # away from zero the difference is at most one bf16 step
    big = np.abs(exact) > 64 * E
    assert np.all(diff[big] <= np.abs(bf16.round_f64(exact[big])) * 2.0 ** -7 * 1.0001)
