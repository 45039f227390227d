"""Seeded sweep of small random configurations of rf_rope3d_apply, rf_kvcache_roll and the
grouped roll rf_kvcache_roll_layers, bit-exact against the oracle's bf16 RoPE
specification (oracle.rope3d.rope_spec_bits) and its ring model (oracle.ring.RingModel).

Each case draws a geometry (8 to 200 tokens per frame, 1/2/3/5 heads, a random split of
the 64 rotation pairs over the three axes with empty axes allowed, two RoPE bases) and:
* RoPE of a ragged token range starting at a random frame, read from and written to
  strided views (rows of a wider buffer);
* a ring of 2..7 slots taken through 8 random rolls (start anywhere in the window or just
  past it, 1..W frames: rewrites in place, appends, evictions, wraps), the whole ring
  (K rotated head-major, V in 8-token blocks) and the window compared after every roll;
* three rings of one context rolled together by one grouped launch per step (the same
  schedule, different data per layer, layer inputs in one [layers, tokens, H, D] tensor),
  every ring compared after every step.
"""
import numpy as np
import pytest
import torch

import rolling_window_attention_amd as rf
from rolling_window_attention_amd import synth
from oracle import rope3d as orope
from oracle.ring import RingModel

from gpu_util import down, ring_slot_v, up

pytestmark = pytest.mark.gpu

FRAME_TOKENS = (8, 16, 24, 40, 48, 56, 64, 72, 96, 104, 136, 200)


def _geometry(rng):
    n = int(rng.choice(FRAME_TOKENS))
    divisors = [d for d in range(1, n + 1) if n % d == 0 and d <= 16]
    gh = int(rng.choice(divisors))
    cuts = np.sort(rng.integers(0, 65, size=2))
    pairs = (int(cuts[0]), int(cuts[1] - cuts[0]), int(64 - cuts[1]))
    return synth.Geometry(grid_h=gh, grid_w=n // gh, n_heads=int(rng.choice([1, 2, 3, 5])), pairs=pairs,
                          base=float(rng.choice([10000.0, 500.0])), window=int(rng.integers(2, 8)))


def _spec(g, bits, t0):
    return orope.rope_spec_bits(bits, t0, g.grid_h, g.grid_w, g.pairs, g.base)


def _expected_ring(g, model):
    N, H, D, W = g.tokens_per_frame, g.n_heads, g.head_dim, g.window
    K = np.zeros((W, H, N, D), np.uint16)
    V = np.zeros((W, H, N // 8, D, 8), np.uint16)
    for s in range(W):
        if model.slot_data[s] is not None:
            kb, vb, t = model.slot_data[s]
            K[s] = _spec(g, kb, t).transpose(1, 0, 2)
            V[s] = ring_slot_v(vb)
    return K, V


def _schedule(rng, W, steps=8):
    """(t0, n) of each roll: the first at a random frame, the others inside the window or
    just past its end (as the library requires)."""
    out, first, count = [], 0, 0
    for _ in range(steps):
        n = int(rng.integers(1, W + 1))
        t0 = int(rng.integers(0, 40)) if count == 0 else int(rng.integers(first, first + count + 1))
        out.append((t0, n))
        first, count = rf.plan_roll(W, first, count, t0, n)
    return out


def _frames_of(k, v, N, t0, n):
    return [(k[i * N:(i + 1) * N], v[i * N:(i + 1) * N], t0 + i) for i in range(n)]


@pytest.mark.parametrize("seed", range(24))
def test_random_rope_and_roll(seed):
    rng = np.random.default_rng(7000 + seed)
    g = _geometry(rng)
    N, H, D, W = g.tokens_per_frame, g.n_heads, g.head_dim, g.window
    print(f"seed {seed}: grid {g.grid_h}x{g.grid_w} heads {H} pairs {g.pairs} base {g.base} W {W}", flush=True)
    ctx = rf.Context(g.grid_h, g.grid_w, H, D, g.pairs, g.base, max_frame=128)

    # RoPE of a ragged token range through strided views
    t0 = int(rng.integers(0, 60))
    n_tok = int(rng.integers(1, 4 * N + 1))
    x = synth.frames(g, seed, 0, t0, (n_tok + N - 1) // N, synth.Q)[:n_tok]
    pad = int(rng.integers(0, 3)) * 8
    src = torch.zeros((n_tok, H * D + pad), dtype=torch.bfloat16, device="cuda")
    src[:, :H * D] = up(x).view(n_tok, H * D)
    dst = torch.zeros((n_tok, H * D + 16), dtype=torch.bfloat16, device="cuda")
    ctx.rope3d_apply(src[:, :H * D], t0, y=dst[:, :H * D])
    torch.cuda.synchronize()
    assert np.array_equal(down(dst[:, :H * D].contiguous()).reshape(n_tok, H, D), _spec(g, x, t0)), "rope3d"
    assert not dst[:, H * D:].any(), "rope3d wrote past its rows"

    # one ring through a random roll schedule
    cache = rf.KVCache(ctx, W)
    model = RingModel(W)
    for r, (t0, n) in enumerate(_schedule(rng, W)):
        k = synth.frames(g, seed, 10 + r, t0, n, synth.K)
        v = synth.frames(g, seed, 10 + r, t0, n, synth.V)
        cache.roll(up(k), up(v), t0)
        model.roll(t0, n, _frames_of(k, v, N, t0, n))
        torch.cuda.synchronize()
        assert (cache.first, cache.count) == (model.first, model.count), f"window after roll {r}"
        K, V = _expected_ring(g, model)
        assert np.array_equal(down(cache.k), K), f"K ring after roll {r} ({t0}, {n})"
        assert np.array_equal(down(cache.v), V), f"V ring after roll {r} ({t0}, {n})"


@pytest.mark.parametrize("seed", range(12))
def test_random_grouped_roll(seed):
    rng = np.random.default_rng(8000 + seed)
    g = _geometry(rng)
    N, H, D, W = g.tokens_per_frame, g.n_heads, g.head_dim, g.window
    L = 3
    print(f"seed {seed}: grid {g.grid_h}x{g.grid_w} heads {H} pairs {g.pairs} W {W} layers {L}", flush=True)
    ctx = rf.Context(g.grid_h, g.grid_w, H, D, g.pairs, g.base, max_frame=128)
    caches = [rf.KVCache(ctx, W) for _ in range(L)]
    rings = rf.DeviceRings(caches)
    models = [RingModel(W) for _ in range(L)]
    for r, (t0, n) in enumerate(_schedule(rng, W, steps=6)):
        ks = [synth.frames(g, seed * 16 + l, 10 + r, t0, n, synth.K) for l in range(L)]
        vs = [synth.frames(g, seed * 16 + l, 10 + r, t0, n, synth.V) for l in range(L)]
        rings.roll(up(np.stack(ks)), up(np.stack(vs)), t0)
        torch.cuda.synchronize()
        for l in range(L):
            models[l].roll(t0, n, _frames_of(ks[l], vs[l], N, t0, n))
            c = caches[l]
            assert (c.first, c.count) == (models[l].first, models[l].count), f"layer {l} window, roll {r}"
            K, V = _expected_ring(g, models[l])
            assert np.array_equal(down(c.k), K), f"layer {l} K ring after roll {r}"
            assert np.array_equal(down(c.v), V), f"layer {l} V ring after roll {r}"
