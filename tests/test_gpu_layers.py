"""Several layers' rings and device-resident ring descriptors, on the GPU:

* rf_kvcache_roll_layers (one launch rolls the same frames into L rings) bit-exact
  against the oracle's ring model and bf16 RoPE specification for every layer, L = 1, 4,
  30, on the tiny grid through the ring's wrap (whole rings after every roll) and at
  the workload geometry (cache-update roll with eviction); the device descriptors'
  windows advance exactly as the host's;
* rf_window_attention_dev (segments over the window the device descriptor holds) equal
  to rf_window_attention over the same frames, bit for bit where the key split is the
  same, and against the oracle;
* the 30-step window fill (context 15 -> 21 frames, then one eviction per step) captured
  ONCE as a graph of one step -- grouped roll of the current frames, attention over the
  device window, roll of the clean frame, frame-shift increment -- and replayed 30 times
  from an empty ring, bit-identical to the same steps run eagerly with host ranges.
"""
import gc

import numpy as np
import pytest
import torch

import rolling_window_attention_amd as rf
from rolling_window_attention_amd import synth
from oracle import rope3d as orope
from oracle.ring import RingModel

from gpu_util import ring_slot_v, RotatedKeys, assert_close, down, f64, oracle_rows, ring_frame_k, ring_frame_v, sample_rows, up

pytestmark = pytest.mark.gpu


def _ctx(g, max_frame=4096):
    return rf.Context(g.grid_h, g.grid_w, g.n_heads, g.head_dim, g.pairs, g.base, max_frame)


def _spec(g, bits, t0):
    return orope.rope_spec_bits(bits, t0, g.grid_h, g.grid_w, g.pairs, g.base)


def _layer_frames(g, cfg, layer, step, t0, n, tensor_id):
    return synth.frames(g, 1000 * cfg + layer, step, t0, n, tensor_id)


def _dev_windows(rings):
    d = rings.buf.cpu().numpy()  # [L, 4] int64: k, v, first, (count | capacity << 32)
    return [(int(r[2]), int(r[3] & 0xFFFFFFFF)) for r in d]


def _expected_ring(g, model, W):
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    K = np.zeros((W, H, N, D), np.uint16)
    V = np.zeros((W, H, N // 8, D, 8), np.uint16)
    for s in range(W):
        if model.slot_data[s] is not None:
            kb, vb, t = model.slot_data[s]
            K[s] = _spec(g, kb, t).transpose(1, 0, 2)
            V[s] = ring_slot_v(vb)
    return K, V


@pytest.mark.parametrize("L", [1, 4, 30])
def test_grouped_roll_tiny_wrap_every_layer_bit_exact(L):
    g = synth.TINY
    W, N = g.window, g.tokens_per_frame
    ctx = _ctx(g)
    caches = [rf.KVCache(ctx, W) for _ in range(L)]
    rings = rf.DeviceRings(caches)
    models = [RingModel(W) for _ in range(L)]
    rng = np.random.default_rng(L)
    t0 = 7
    for step in range(9):
        m = models[0]
        n = int(rng.integers(1, W + 1))
        if m.count:
            t0 = int(rng.integers(m.first, m.first + m.count + 1))
        print(f"L={L} roll {step}: t0={t0} n={n}", flush=True)
        k = np.stack([_layer_frames(g, 51, l, step, t0, n, synth.K) for l in range(L)])
        v = np.stack([_layer_frames(g, 51, l, step, t0, n, synth.V) for l in range(L)])
        rings.roll(up(k), up(v), t0)
        for l in range(L):
            models[l].roll(t0, n, [(k[l, i * N:(i + 1) * N], v[l, i * N:(i + 1) * N], t0 + i) for i in range(n)])
            assert (caches[l].first, caches[l].count) == (models[l].first, models[l].count)
        torch.cuda.synchronize()
        assert _dev_windows(rings) == [(m.first, m.count) for m in models]
        for l in range(L):
            K, V = _expected_ring(g, models[l], W)
            assert np.array_equal(down(caches[l].k), K), f"layer {l}: K ring differs after roll {step}"
            assert np.array_equal(down(caches[l].v), V), f"layer {l}: V ring differs after roll {step}"


@pytest.mark.parametrize("L", [4, 30])
def test_grouped_roll_full_size_cache_update(L):
    """Workload geometry: the rings hold frames 0..20 (descriptors uploaded with that
    window, buffers zero), then ONE launch rolls frame 21 into all L rings: it evicts
    frame 0, so slot 0 of every layer receives that layer's frame 21 bit-exactly and the
    other 20 slots stay untouched."""
    g = synth.FULL
    W, N, H, D = g.window, g.tokens_per_frame, g.n_heads, g.head_dim
    ctx = _ctx(g)
    caches = [rf.KVCache(ctx, W) for _ in range(L)]
    for c in caches:
        c.desc.first, c.desc.count = 0, W
    rings = rf.DeviceRings(caches)
    k = np.stack([_layer_frames(g, 52, l, 1, 21, 1, synth.K + synth.CLEAN) for l in range(L)])
    v = np.stack([_layer_frames(g, 52, l, 1, 21, 1, synth.V + synth.CLEAN) for l in range(L)])
    print(f"grouped roll of frame 21 into {L} rings", flush=True)
    rings.roll(up(k), up(v), 21)
    torch.cuda.synchronize()
    assert _dev_windows(rings) == [(1, W)] * L
    for l, c in enumerate(caches):
        assert (c.first, c.count) == (1, W)
        assert np.array_equal(ring_frame_k(down(c.k[0:1]), 0), _spec(g, k[l], 21)), f"layer {l} K"
        assert np.array_equal(ring_frame_v(down(c.v[0:1]), 0), v[l]), f"layer {l} V"
        assert not bool(c.k[1:].view(torch.int16).any()) and not bool(c.v[1:].view(torch.int16).any())


def test_grouped_roll_of_the_most_layers():
    """The most layers one grouped roll accepts, 65,535 (the grid's y extent), on the tiny
    grid with 2-slot rings (39 GB in all) and the same frames for every layer (layer
    stride 0): two frames, then a third that evicts the first.  Sampled layers' rings
    bit-exact, every layer's device window advanced, 65,536 layers refused."""
    g = synth.TINY
    N = g.tokens_per_frame
    L, W = 65535, 2
    ctx = _ctx(g)
    caches = [rf.KVCache(ctx, W) for _ in range(L)]
    rings = rf.DeviceRings(caches)
    model = RingModel(W)
    for step, (t0, n) in enumerate([(0, 2), (2, 1)]):
        k = synth.frames(g, 52, step, t0, n, synth.K)
        v = synth.frames(g, 52, step, t0, n, synth.V)
        kd, vd = up(k), up(v)
        print(f"{L} layers: roll frames {t0}..{t0 + n - 1}", flush=True)
        rings.roll(kd.unsqueeze(0).expand(L, *kd.shape), vd.unsqueeze(0).expand(L, *vd.shape), t0)
        model.roll(t0, n, [(k[i * N:(i + 1) * N], v[i * N:(i + 1) * N], t0 + i) for i in range(n)])
    torch.cuda.synchronize()
    assert all((c.first, c.count) == (1, 2) for c in caches)
    assert _dev_windows(rings) == [(1, 2)] * L
    K, V = _expected_ring(g, model, W)
    for l in (0, 1, 255, 256, 32767, L - 2, L - 1):
        assert np.array_equal(down(caches[l].k), K), l
        assert np.array_equal(down(caches[l].v), V), l
    with pytest.raises(rf.RfError):
        rf.DeviceRings(caches + [rf.KVCache(ctx, W)])
    del rings, caches
    gc.collect()
    torch.cuda.empty_cache()


def test_grouped_roll_matches_separate_rolls_and_validates():
    """One grouped launch leaves the same bits as L separate rf_kvcache_roll calls (shared
    input with layer stride 0 included); illegal rolls are refused for the group before
    any launch and leave every descriptor as it was."""
    g = synth.TINY
    W, N = g.window, g.tokens_per_frame
    ctx = _ctx(g)
    L = 3
    a = [rf.KVCache(ctx, W) for _ in range(L)]
    b = [rf.KVCache(ctx, W) for _ in range(L)]
    rings = rf.DeviceRings(a)
    k = up(synth.frames(g, 53, 0, 4, 3, synth.K))
    v = up(synth.frames(g, 53, 0, 4, 3, synth.V))
    rings.roll(k.unsqueeze(0).expand(L, *k.shape), v.unsqueeze(0).expand(L, *v.shape), 4)
    for c in b:
        c.roll(k, v, 4)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.k.view(torch.int16), y.k.view(torch.int16))
        assert torch.equal(x.v.view(torch.int16), y.v.view(torch.int16))
        assert x.window() == y.window() == [4, 5, 6]
    kk = k.unsqueeze(0).expand(L, *k.shape)
    for t0 in (8, 3):  # a gap, and a start before the window
        with pytest.raises(rf.RfError) as e:
            rings.roll(kk, kk, t0)
        assert e.value.status == 4
    with pytest.raises(rf.RfError) as e:  # two layers on one ring
        bad = rf.DeviceRings([a[0], a[0]])
        bad.roll(kk[:2], kk[:2], 5)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert [c.window() for c in a] == [[4, 5, 6]] * L
    assert _dev_windows(rings) == [(4, 3)] * L


def test_window_attention_dev_against_host_ranges_and_oracle():
    """Attention over the device window is bit-identical to attention over the same frames
    given as a host range (the launch is cut the same way), on the tiny grid (all tiles
    key-split) and at the workload geometry (the batched step), and matches the oracle."""
    g = synth.TINY
    N = g.tokens_per_frame
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, g.window)
    rings = rf.DeviceRings([cache])
    k = synth.frames(g, 54, 0, 0, 4, synth.K)
    v = synth.frames(g, 54, 0, 0, 4, synth.V)
    rings.roll(up(k).unsqueeze(0), up(v).unsqueeze(0), 0)
    q = synth.frames(g, 54, 0, 1, 3, synth.Q)
    o_dev = torch.empty((3 * N, g.n_heads, g.head_dim), dtype=torch.bfloat16, device="cuda")
    o_host = torch.empty_like(o_dev)
    rf.window_attention_dev(ctx, rings, 0, [rf.Segment(up(q), 1, o_dev, 0, 0)])
    rf.window_attention(ctx, cache, [rf.Segment(up(q), 1, o_host, 0, 4)])
    torch.cuda.synchronize()
    rk = RotatedKeys(g)
    khs = [rk.get(t, 0, k[t * N:(t + 1) * N]) for t in range(4)]
    want = oracle_rows(g, q, 1, khs, [v[t * N:(t + 1) * N] for t in range(4)], np.arange(3 * N))
    assert_close(f64(down(o_dev)), want, "device window, tiny")
    assert torch.equal(o_dev.view(torch.int16), o_host.view(torch.int16))
    with pytest.raises(rf.RfError) as e:  # a segment with a context range
        rf.window_attention_dev(ctx, rings, 0, [rf.Segment(up(q), 1, o_dev, 0, 4)])
    assert e.value.status == 3

    G = synth.FULL
    N = G.tokens_per_frame
    ctx = _ctx(G)
    cache = rf.KVCache(ctx, G.window)
    rings = rf.DeviceRings([cache])
    k = up(synth.frames(G, 55, 0, 3, 21, synth.K)).unsqueeze(0)
    v = up(synth.frames(G, 55, 0, 3, 21, synth.V)).unsqueeze(0)
    rings.roll(k, v, 3)
    qa = up(synth.frames(G, 55, 0, 9, 15, synth.Q))
    qb = up(synth.frame(G, 55, 0, 8, synth.Q + synth.CLEAN))
    outs = [(torch.empty((15 * N, G.n_heads, G.head_dim), dtype=torch.bfloat16, device="cuda"),
             torch.empty((N, G.n_heads, G.head_dim), dtype=torch.bfloat16, device="cuda")) for _ in range(2)]
    print("full-size batched step over the device window", flush=True)
    rf.window_attention_dev(ctx, rings, 0, [rf.Segment(qa, 9, outs[0][0], 0, 0), rf.Segment(qb, 8, outs[0][1], 0, 0)])
    rf.window_attention(ctx, cache, [rf.Segment(qa, 9, outs[1][0], 3, 21), rf.Segment(qb, 8, outs[1][1], 3, 21)])
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))


def _fill_inputs(g, cfg, pool):
    """`pool` distinct step inputs: (k, v) of the 15 current frames, (k, v) of the clean
    frame, q of the 15 current frames (bf16 bits)."""
    out = []
    for i in range(pool):
        out.append((synth.frames(g, cfg, i, 0, 15, synth.K), synth.frames(g, cfg, i, 0, 15, synth.V),
                    synth.frame(g, cfg, i, 0, synth.K + synth.CLEAN), synth.frame(g, cfg, i, 0, synth.V + synth.CLEAN),
                    synth.frames(g, cfg, i, 0, 15, synth.Q)))
    return out


def _fill_replay(g, cfg, steps, pool, check_rows=None):
    """The window fill: step s rolls current frames s..s+14 (noisy), attends with query
    frames s..s+14 over the whole window (min(s,6)+15 frames), then rolls the clean frame
    s.  Eagerly with host ranges on one context; captured once (step 0, device window,
    frame shift) and replayed `steps` times on another.  Step s uses input set s % pool."""
    N, H, D, W = g.tokens_per_frame, g.n_heads, g.head_dim, 21
    host = _fill_inputs(g, cfg, pool)
    data = [tuple(up(x) for x in d) for d in host]
    ctx_e, ctx_g = _ctx(g), _ctx(g)
    ce, cg = rf.KVCache(ctx_e, W), rf.KVCache(ctx_g, W)
    rings = rf.DeviceRings([cg])
    o_e = torch.empty((15 * N, H, D), dtype=torch.bfloat16, device="cuda")
    o_g = torch.empty_like(o_e)
    stage = [torch.empty_like(x) for x in data[0]]  # the graph's fixed input buffers
    shift = torch.zeros(1, dtype=torch.int64, device="cuda")
    ctx_g.set_frame_shift(shift, steps)
    torch.cuda.synchronize()
    gc.collect()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            rings.roll(stage[0].unsqueeze(0), stage[1].unsqueeze(0), 0)
            rf.window_attention_dev(ctx_g, rings, 0, [rf.Segment(stage[4], 0, o_g, 0, 0)])
            rings.roll(stage[2].unsqueeze(0), stage[3].unsqueeze(0), 0)
            ctx_g.add_frame_shift(shift, 1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # the capture enqueued nothing: reset the device window and the shift, then replay
    rings.reset()
    shift.zero_()
    torch.cuda.synchronize()
    for s in range(steps):
        c0 = max(0, s - 6)
        print(f"step {s}: context {s + 15 - c0} frames", flush=True)
        kn, vn, kc, vc, q = data[s % pool]
        ce.roll(kn, vn, s)
        rf.window_attention(ctx_e, ce, [rf.Segment(q, s, o_e, c0, s + 15 - c0)])
        ce.roll(kc, vc, s)
        for dst, src in zip(stage, data[s % pool]):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        assert int(shift.item()) == s + 1
        assert _dev_windows(rings) == [(ce.first, ce.count)]
        assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16)), f"output differs at step {s}"
        assert torch.equal(cg.k.view(torch.int16), ce.k.view(torch.int16)), f"K ring differs at step {s}"
        assert torch.equal(cg.v.view(torch.int16), ce.v.view(torch.int16)), f"V ring differs at step {s}"
        if check_rows is not None and s in check_rows:
            _check_fill_step(g, host, s, o_g)
    ctx_g.set_frame_shift(None, 0)


def _check_fill_step(g, inputs, s, o):
    """Sampled rows of step s's output against the oracle (frames t < s are the clean
    versions written at step t, the others the current ones of step s)."""
    N = g.tokens_per_frame
    pool = len(inputs)
    c0 = max(0, s - 6)
    khs, vs = [], []
    rk = RotatedKeys(g)
    for t in range(c0, s + 15):
        if t < s:
            kb, vb = inputs[t % pool][2], inputs[t % pool][3]
        else:
            kb = inputs[s % pool][0][(t - s) * N:(t - s + 1) * N]
            vb = inputs[s % pool][1][(t - s) * N:(t - s + 1) * N]
        khs.append(rk.get(t, (s, t), kb))
        vs.append(vb)
    rows = sample_rows(15 * N, N, extra=24, seed=s)
    want = oracle_rows(g, inputs[s % pool][4], s, khs, vs, rows)
    assert_close(f64(down(o))[rows], want, f"fill step {s}")


def test_window_fill_replayed_from_one_graph_tiny():
    _fill_replay(synth.Geometry(grid_h=6, grid_w=8), 56, steps=30, pool=5, check_rows=(0, 3, 6, 29))


def test_window_fill_replayed_from_one_graph_full_size():
    _fill_replay(synth.FULL, 57, steps=30, pool=2, check_rows=(2, 29))
