"""rf_window_attention_noalloc (the attention call that takes its split-tile scratch from
the library's static per-device array) against rf_window_attention (the context's
workspace): the same kernels and split, so the outputs must be equal bit for bit.

Two calls in a row through the C ABI, the second smaller: the batched two-phase step at
full size (whole tiles plus a key-split last round), then the lone cache-update pass
(every tile key-split, more split work-groups than the first call's), then a tiny launch
on another context (the array is shared across contexts of one device).
"""
import numpy as np
import pytest
import torch

import rolling_window_attention_amd as rf
from rolling_window_attention_amd import synth

from gpu_util import up

pytestmark = pytest.mark.gpu


def _ctx(g):
    return rf.Context(g.grid_h, g.grid_w, g.n_heads, g.head_dim, g.pairs, g.base, 4096)


def _out(g, n_tokens):
    return torch.full((n_tokens, g.n_heads, g.head_dim), 3.0, dtype=torch.bfloat16, device="cuda")


def _same(a, b, what):
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), what


def _fill(g, cfg, cache, n_frames, t0=0):
    k = synth.frames(g, cfg, 0, t0, n_frames, synth.K)
    v = synth.frames(g, cfg, 0, t0, n_frames, synth.V)
    cache.roll(up(k), up(v), t0)


def test_noalloc_matches_the_workspace_call_on_two_calls_in_a_row():
    g, cfg = synth.FULL, 71
    N = g.tokens_per_frame
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, g.window)
    _fill(g, cfg, cache, g.window)
    qa = up(synth.frames(g, cfg, 1, 6, 15, synth.Q))
    qb = up(synth.frame(g, cfg, 1, 5, synth.Q + synth.CLEAN))

    # call 1: the batched step (23,400 + 1,560 queries over 21 frames)
    print("call 1: batched step, full size", flush=True)
    ref_a, ref_b = _out(g, 15 * N), _out(g, N)
    rf.window_attention(ctx, cache, [rf.Segment(qa, 6, ref_a, 0, 21), rf.Segment(qb, 5, ref_b, 0, 21)])
    got_a, got_b = _out(g, 15 * N), _out(g, N)
    rf.window_attention_noalloc(ctx, cache, [rf.Segment(qa, 6, got_a, 0, 21), rf.Segment(qb, 5, got_b, 0, 21)])
    torch.cuda.synchronize()
    _same(got_a, ref_a, "batched step, denoise segment")
    _same(got_b, ref_b, "batched step, cache-update segment")
    assert bool(torch.isfinite(got_a.float()).all())

    # call 2, smaller: the lone cache-update pass over 16 frames (all tiles key-split)
    print("call 2: lone cache-update pass", flush=True)
    ref, got = _out(g, N), _out(g, N)
    rf.window_attention(ctx, cache, [rf.Segment(qb, 5, ref, 5, 16)])
    rf.window_attention_noalloc(ctx, cache, [rf.Segment(qb, 5, got, 5, 16)])
    torch.cuda.synchronize()
    _same(got, ref, "cache-update pass")

    # call 3, smaller still, on another context of the same device
    print("call 3: tiny geometry", flush=True)
    t = synth.TINY
    tctx = _ctx(t)
    tcache = rf.KVCache(tctx, t.window)
    _fill(t, cfg, tcache, t.window)
    q = up(synth.frames(t, cfg, 1, 2, 3, synth.Q))
    ref, got = _out(t, 3 * t.tokens_per_frame), _out(t, 3 * t.tokens_per_frame)
    rf.window_attention(tctx, tcache, [rf.Segment(q, 2, ref, 0, 5)])
    rf.window_attention_noalloc(tctx, tcache, [rf.Segment(q, 2, got, 0, 5)])
    torch.cuda.synchronize()
    _same(got, ref, "tiny launch")


def test_noalloc_validates_like_the_workspace_call():
    g = synth.TINY
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, g.window)
    q = up(synth.frames(g, 9, 0, 0, 1, synth.Q))
    o = _out(g, g.tokens_per_frame)
    with pytest.raises(rf.RfError) as e:  # empty cache
        rf.window_attention_noalloc(ctx, cache, [rf.Segment(q, 0, o, 0, 1)])
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())
