"""Seeded sweep of small random configurations of rf_window_attention against the float64
oracle, every output row checked.

Each case draws a geometry (tokens per frame from 8 to 200: frames shorter than a key
tile, frames whose key tiles straddle frame boundaries; 1, 2, 3 or 5 heads; a random
split of the 64 rotation pairs over time, height and width, zero pairs on an axis
included; two RoPE bases), a ring of 2..7 slots, a history of rolls (random starts inside
the window and random lengths: rewrites in place, appends, evictions, wraps of the ring),
then ONE launch of 1..3 segments, each with its own context range inside the window, its
own query frame and first query token (blocks cut anywhere in a frame) and length, and a
softmax scale (the default 1/sqrt(128) or an explicit one).  The ring's frames are tracked
on the host as the oracle's context (the newest write of each frame).

Inputs are synthetic N(0, 1) bf16 tensors (rolling_window_attention_amd.synth); the
tolerances are the ones of every attention parity test (gpu_util.assert_close).
"""
import numpy as np
import pytest
import torch

import rolling_window_attention_amd as rf
from rolling_window_attention_amd import synth
from oracle import attention as oatt

from gpu_util import assert_close, down, f64, up

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


def _roll_history(rng, g, cache, seed):
    """Random rolls; returns {frame: (k bits, v bits)} as the ring holds them."""
    held = {}
    t_start = int(rng.integers(0, 40))
    for r in range(int(rng.integers(1, 6))):
        n = int(rng.integers(1, g.window + 1))
        if cache.count == 0:
            t0 = t_start
        else:
            t0 = int(rng.integers(cache.first, cache.first + cache.count + 1))
        k = synth.frames(g, seed, r, t0, n, synth.K)
        v = synth.frames(g, seed, r, t0, n, synth.V)
        cache.roll(up(k), up(v), t0)
        N = g.tokens_per_frame
        for i in range(n):
            held[t0 + i] = (k[i * N:(i + 1) * N], v[i * N:(i + 1) * N])
    return {t: held[t] for t in cache.window()}


@pytest.mark.parametrize("seed", range(48))
def test_random_configuration(seed):
    rng = np.random.default_rng(9000 + seed)
    g = _geometry(rng)
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    ctx = rf.Context(g.grid_h, g.grid_w, H, D, g.pairs, g.base, max_frame=256)
    cache = rf.KVCache(ctx, g.window)
    held = _roll_history(rng, g, cache, seed)
    lo, hi = cache.first, cache.first + cache.count
    scale = float(rng.choice([0.0, 0.03, 0.15]))
    segs, refs = [], []
    for i in range(int(rng.integers(1, 4))):
        c0 = int(rng.integers(lo, hi))
        cf = int(rng.integers(1, hi - c0 + 1))
        q_t0 = int(rng.integers(0, 60))
        tok0 = int(rng.integers(0, N))
        n_rows = int(rng.integers(1, 3 * N + 1))
        frames_q = (tok0 + n_rows + N - 1) // N
        q = synth.frames(g, seed, 100 + i, q_t0, frames_q, synth.Q)[tok0:tok0 + n_rows]
        o = torch.empty((n_rows, H, D), dtype=torch.bfloat16, device="cuda")
        segs.append(rf.Segment(up(q), q_t0, o, c0, cf, q_tok0=tok0))
        refs.append((q, q_t0, c0, cf, tok0, o))
    desc = (f"seed {seed}: grid {g.grid_h}x{g.grid_w} heads {H} pairs {g.pairs} base {g.base} "
            f"W {g.window} window [{lo},{hi}) scale {scale} segments "
            + ", ".join(f"q {r[1]}+{r[4]} x{len(r[0])} over [{r[2]},{r[2] + r[3]})" for r in refs))
    print(desc, flush=True)
    rf.window_attention(ctx, cache, segs, scale=scale)
    torch.cuda.synchronize()
    for i, (q, q_t0, c0, cf, tok0, o) in enumerate(refs):
        k = np.concatenate([held[t][0] for t in range(c0, c0 + cf)])
        v = np.concatenate([held[t][1] for t in range(c0, c0 + cf)])
        want = oatt.window_attention(f64(q), q_t0, f64(k), f64(v), c0, g.grid_h, g.grid_w, g.pairs, g.base,
                                     scale=scale if scale else None, q_tok0=tok0, workers=1)
        assert_close(f64(down(o)), want, f"seed {seed} segment {i}")


# Segment lengths around the 32-row boundaries of the waves in a 256-row query tile:
# the last tile of a segment runs only the waves that hold some of its rows, the
# others only stage keys and values.  Checked alone (every tile of the launch cut into
# key ranges and merged) and next to a long segment of 128 tiles per head placed last,
# so that the short segments' tiles fall in the launch's whole-tile round.
WAVE_EDGE_ROWS = (1, 31, 32, 33, 224, 225, 255, 256, 257, 288)


@pytest.mark.parametrize("with_long", [False, True])
def test_segment_lengths_at_wave_boundaries(with_long):
    g = synth.Geometry(grid_h=8, grid_w=12, n_heads=2, window=6)
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    ctx = rf.Context(g.grid_h, g.grid_w, H, D, g.pairs, g.base, max_frame=512)
    cache = rf.KVCache(ctx, g.window)
    k = synth.frames(g, 77, 0, 0, g.window, synth.K)
    v = synth.frames(g, 77, 0, 0, g.window, synth.V)
    cache.roll(up(k), up(v), 0)

    def segment(i, n_rows):
        tok0 = (7 * i) % N
        q = synth.frames(g, 77, 100 + i, 3, (tok0 + n_rows + N - 1) // N, synth.Q)[tok0:tok0 + n_rows]
        o = torch.empty((n_rows, H, D), dtype=torch.bfloat16, device="cuda")
        return rf.Segment(up(q), 3, o, 0, g.window, q_tok0=tok0), (q, tok0, o)

    short = [segment(i, n) for i, n in enumerate(WAVE_EDGE_ROWS)]
    checks = [r for _, r in short]
    groups = [short[:7], short[7:]]
    for gi, grp in enumerate(groups):
        segs = [sg for sg, _ in grp]
        if with_long:  # 256 query tiles in all: the launch's whole-tile round takes the short ones first
            sg, ref = segment(50 + gi, 128 * 256)
            segs.append(sg)
            q, tok0, o = ref
            checks.append((q[:64], tok0, o[:64]))
            checks.append((q[-64:], (tok0 + len(q) - 64) % N, o[-64:], 3 + (tok0 + len(q) - 64) // N))
        print(f"with_long={with_long}: segments of {[len(r[0]) for _, r in grp]} rows", flush=True)
        rf.window_attention(ctx, cache, segs)
    torch.cuda.synchronize()
    for c in checks:
        q, tok0, o = c[:3]
        q_t0 = c[3] if len(c) > 3 else 3
        want = oatt.window_attention(f64(q), q_t0, f64(k), f64(v), 0, g.grid_h, g.grid_w, g.pairs, g.base,
                                     q_tok0=tok0, workers=1)
        assert_close(f64(down(o.contiguous())), want, f"{len(q)} rows from token {tok0} (with_long={with_long})")
