"""Replaying one captured window step as the following steps (rf_set_frame_shift /
rf_add_frame_shift), against the same steps run eagerly on a second context, bit for
bit after every replay: the ring's keys and values and both segments' outputs.

A step s rolls frames s-1 .. s+n-2 (the clean re-encode of s-1 and the new frames) and
runs one batched launch: the denoise segment (query frames s..) and the cache-update
segment (query frame s-1), both over the window's last W frames.  The graph holds the
launches of step s0 and a shift increment; replay i is step s0 + i.  Inputs are the
same tensors every step (their pointers are baked into the graph).
"""
import gc

import numpy as np
import pytest
import torch

import rolling_window_attention_amd as rf
from rolling_window_attention_amd import synth

from gpu_util import down, up

pytestmark = pytest.mark.gpu


def _run(g, n_new, replays, cfg):
    N, H, D, W = g.tokens_per_frame, g.n_heads, g.head_dim, g.window
    nq = n_new - 1  # denoise query frames
    contexts = [rf.Context(g.grid_h, g.grid_w, H, D, g.pairs, g.base, 4096) for _ in range(2)]
    caches = [rf.KVCache(c, W) for c in contexts]
    k0 = synth.frames(g, cfg, 0, 0, W, synth.K + synth.CLEAN)
    v0 = synth.frames(g, cfg, 0, 0, W, synth.V + synth.CLEAN)
    for c in caches:
        c.roll(up(k0), up(v0), 0)
    k = up(synth.frames(g, cfg, 1, 0, n_new, synth.K))
    v = up(synth.frames(g, cfg, 1, 0, n_new, synth.V))
    qa = up(synth.frames(g, cfg, 1, 0, nq, synth.Q))
    qb = up(synth.frame(g, cfg, 1, 0, synth.Q + synth.CLEAN))
    outs = [(torch.empty((nq * N, H, D), dtype=torch.bfloat16, device="cuda"),
             torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda")) for _ in range(2)]
    s0 = W - nq + 1  # first step whose roll appends past the prefilled frames 0..W-1

    def step(i, s):
        ctx, cache, (oa, ob) = contexts[i], caches[i], outs[i]
        cache.roll(k, v, s - 1)
        c0 = s + nq - W
        rf.window_attention(ctx, cache, [rf.Segment(qa, s, oa, c0, W), rf.Segment(qb, s - 1, ob, c0, W)])

    shift = torch.zeros(1, dtype=torch.int64, device="cuda")
    contexts[1].set_frame_shift(shift, replays)
    torch.cuda.synchronize()
    # contexts of earlier tests that sit in reference cycles (exception tracebacks) are
    # freed now rather than by a collection inside the capture
    gc.collect()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(1, s0)
            contexts[1].add_frame_shift(shift, 1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for i in range(replays):
        print(f"replay {i}: step {s0 + i} (N={N}, {n_new} new frames)", flush=True)
        step(0, s0 + i)
        graph.replay()
        torch.cuda.synchronize()
        assert int(shift.item()) == i + 1
        assert np.array_equal(down(caches[1].k), down(caches[0].k)), f"K ring differs at replay {i}"
        assert np.array_equal(down(caches[1].v), down(caches[0].v)), f"V ring differs at replay {i}"
        assert np.array_equal(down(outs[1][0]), down(outs[0][0])), f"denoise output differs at replay {i}"
        assert np.array_equal(down(outs[1][1]), down(outs[0][1])), f"cache-update output differs at replay {i}"
    contexts[1].set_frame_shift(None, 0)


def test_graph_replay_tiny_through_the_ring_wrap():
    _run(synth.TINY, n_new=4, replays=6, cfg=41)


def test_graph_replay_full_size():
    _run(synth.FULL, n_new=16, replays=2, cfg=42)


def test_frame_shift_validation():
    g = synth.TINY
    ctx = rf.Context(g.grid_h, g.grid_w, g.n_heads, g.head_dim, g.pairs, g.base, max_frame=20)
    cache = rf.KVCache(ctx, g.window)
    shift = torch.zeros(1, dtype=torch.int64, device="cuda")
    with pytest.raises(rf.RfError):
        ctx.set_frame_shift(shift, 20)        # clamp beyond the tables
    ctx.set_frame_shift(shift, 10)
    N = g.tokens_per_frame
    kv = torch.zeros((4 * N, g.n_heads, g.head_dim), dtype=torch.bfloat16, device="cuda")
    cache.roll(kv, kv, 6)                     # frames 6..9, + 10 <= 20
    with pytest.raises(rf.RfError) as e:
        cache.roll(kv, kv, 7)                 # frames 7..10 + 10 = 20: beyond the tables
    assert e.value.status == 4
    ctx.set_frame_shift(None, 0)
    cache.roll(kv, kv, 7)                     # without the shift: fine


def test_context_collected_inside_a_capture_is_freed_after_it():
    """A context that is garbage when the collector runs inside a graph capture is not
    freed there (freeing device memory would invalidate the capture) but at the next
    context creation outside it."""
    g = synth.TINY
    gc.collect()  # contexts left in cycles by earlier tests are closed now, outside a capture
    ctx = rf.Context(g.grid_h, g.grid_w, g.n_heads, g.head_dim, g.pairs, g.base, 64)
    assert not rf._pending_destroy
    cycle = [ctx]
    cycle.append(cycle)  # only the cyclic collector can free it now
    del ctx, cycle
    x = torch.zeros(16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    gc.disable()
    try:
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                x.add_(1)
                gc.collect()  # closes the context while the capture is under way
                pending = len(rf._pending_destroy)
                x.add_(1)
    finally:
        gc.enable()
    torch.cuda.current_stream().wait_stream(side)
    assert pending == 1
    graph.replay()
    torch.cuda.synchronize()
    assert float(x[0]) == 2.0
    rf.Context(g.grid_h, g.grid_w, g.n_heads, g.head_dim, g.pairs, g.base, 64).close()
    assert not rf._pending_destroy
