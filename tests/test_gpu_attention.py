"""GPU parity of rf_window_attention against the float64 oracle.

Tolerances (max-abs 2e-2, mean-abs 2e-3 on bf16 inputs) plus rel-L2 <= 1e-2, because at
32,760 keys the output's own spread is ~0.01 and dropping a whole context frame would still
pass the absolute bounds.  Closed-form checks on top: q = 0 returns the mean of the attended
values (frame tags prove which frames were read) and k = 16q makes every query pick its own
token's value.
"""
import gc

import numpy as np
import pytest
import torch

import rolling_window_attention_amd as rf
from rolling_window_attention_amd import synth
from oracle import attention as oatt
from oracle import rope3d as orope

from gpu_util import (RotatedKeys, assert_close, down, f64, oracle_rows, sample_rows, up)

pytestmark = pytest.mark.gpu


def _ctx(g, max_frame=4096):
    return rf.Context(g.grid_h, g.grid_w, g.n_heads, g.head_dim, g.pairs, g.base, max_frame)


def _out(g, n_frames):
    return torch.empty((n_frames * g.tokens_per_frame, g.n_heads, g.head_dim), dtype=torch.bfloat16,
                       device="cuda")


def test_tiny_full_parity():
    """6x8 grid, 2 cached + 3 current frames (240 keys), 3 query frames (144 rows)."""
    g, cfg = synth.TINY, synth.WORKLOAD_IDS["tiny"]
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, g.window)
    kc = synth.frames(g, cfg, 0, 0, 2, synth.K + synth.CLEAN)
    vc = synth.frames(g, cfg, 0, 0, 2, synth.V + synth.CLEAN)
    cache.roll(up(kc), up(vc), 0)
    k = synth.frames(g, cfg, 1, 2, 3, synth.K)
    v = synth.frames(g, cfg, 1, 2, 3, synth.V)
    q = synth.frames(g, cfg, 1, 2, 3, synth.Q)
    cache.roll(up(k), up(v), 2)
    o = _out(g, 3)
    rf.window_attention(ctx, cache, [rf.Segment(up(q), 2, o, 0, 5)])
    torch.cuda.synchronize()
    want = oatt.window_attention(f64(q), 2, f64(np.concatenate([kc, k])),
                                 f64(np.concatenate([vc, v])), 0, g.grid_h, g.grid_w, g.pairs,
                                 g.base)
    assert_close(f64(down(o)), want, "tiny")


def test_time_shift_by_1000_frames():
    """The same frames placed 1,000 frames later (keys rolled at t + 1000, queries at
    q_t0 + 1000): the output changes by rounding only, since the rotation acts on the
    difference of positions; both launches also against the oracle at their own
    positions."""
    g, cfg = synth.TINY, synth.WORKLOAD_IDS["tiny"]
    ctx = _ctx(g)
    outs = []
    k = synth.frames(g, cfg, 0, 0, 5, synth.K)
    v = synth.frames(g, cfg, 0, 0, 5, synth.V)
    q = synth.frames(g, cfg, 0, 2, 3, synth.Q)
    for t in (0, 1000):
        cache = rf.KVCache(ctx, g.window)
        cache.roll(up(k), up(v), t)
        o = _out(g, 3)
        rf.window_attention(ctx, cache, [rf.Segment(up(q), 2 + t, o, t, 5)])
        torch.cuda.synchronize()
        want = oatt.window_attention(f64(q), 2 + t, f64(k), f64(v), t, g.grid_h, g.grid_w, g.pairs, g.base)
        assert_close(f64(down(o)), want, f"frames from {t}")
        outs.append(f64(down(o)))
    assert_close(outs[1], outs[0], "shifted by 1000 frames against unshifted")


def test_tiny_wrap_run_and_two_segments():
    """Twelve steps on a 5-slot ring: each step rolls the clean frame s-1 and the current
    frames s..s+2, then ONE launch runs the denoise segment (3 frames) and the cache-update
    segment (frame s-1) over the window; every output row is checked."""
    g, cfg = synth.TINY, 11
    W, N = g.window, g.tokens_per_frame
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, W)
    frames_k, frames_v = {}, {}
    for s in range(12):
        t0 = max(s - 1, 0)
        ts = list(range(t0, s + 3))
        for t in ts:
            tag = synth.CLEAN if t < s else 0
            frames_k[t] = synth.frame(g, cfg, s, t, synth.K + tag)
            frames_v[t] = synth.frame(g, cfg, s, t, synth.V + tag)
        cache.roll(up(np.concatenate([frames_k[t] for t in ts])),
                   up(np.concatenate([frames_v[t] for t in ts])), t0)
        lo, hi = cache.first, cache.first + cache.count  # window [lo, hi)
        qa = synth.frames(g, cfg, s, s, 3, synth.Q)
        oa = _out(g, 3)
        segs = [rf.Segment(up(qa), s, oa, lo, hi - lo)]
        if s >= 1:
            qb = synth.frame(g, cfg, s, s - 1, synth.Q + synth.CLEAN)
            ob = _out(g, 1)
            segs.append(rf.Segment(up(qb), s - 1, ob, lo, hi - lo))
        print(f"step {s}: window [{lo},{hi}) segments={len(segs)}", flush=True)
        rf.window_attention(ctx, cache, segs)
        torch.cuda.synchronize()
        kk = f64(np.concatenate([frames_k[t] for t in range(lo, hi)]))
        vv = f64(np.concatenate([frames_v[t] for t in range(lo, hi)]))
        want = oatt.window_attention(f64(qa), s, kk, vv, lo, g.grid_h, g.grid_w, g.pairs, g.base)
        assert_close(f64(down(oa)), want, f"step {s} A")
        if s >= 1:
            want = oatt.window_attention(f64(qb), s - 1, kk, vv, lo, g.grid_h, g.grid_w, g.pairs,
                                         g.base)
            assert_close(f64(down(ob)), want, f"step {s} B")


@pytest.mark.parametrize("geom", [synth.TINY, synth.FULL])
def test_zero_query_reads_exactly_the_context_frames(geom):
    """q = 0: every weight is 1, so o = mean of v over the context.  v of frame t is the
    constant t/32 (exact in bf16), so the output names the attended frames."""
    g = geom
    W, N, H, D = g.window, g.tokens_per_frame, g.n_heads, g.head_dim
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, W)
    t_end = W + 3  # roll frames 0..W+2 one by one, so the ring has wrapped
    for t in range(t_end):
        k = synth.frame(g, 5, 0, t, synth.K)
        v = np.full((N, H, D), t / 32.0)
        cache.roll(up(k), up(synth.f32_to_bf16_bits(v.astype(np.float32))), t)
    lo, hi = t_end - W, t_end
    assert cache.window() == list(range(lo, hi))
    q = torch.zeros((N, H, D), dtype=torch.bfloat16, device="cuda")
    for ctx_t0, nf in ((lo, W), (hi - 3, 3), (lo + 1, 1), (lo + 1, W - 2)):
        o = _out(g, 1)
        rf.window_attention(ctx, cache, [rf.Segment(q, 4, o, ctx_t0, nf)])
        torch.cuda.synchronize()
        want = np.mean(np.arange(ctx_t0, ctx_t0 + nf)) / 32.0
        got = f64(down(o))
        print(f"ctx {ctx_t0}+{nf}: want {want:.6f} got [{got.min():.6f}, {got.max():.6f}]", flush=True)
        assert np.all(np.abs(got - want) <= abs(want) * 2.0 ** -7), (ctx_t0, nf)


@pytest.mark.parametrize("geom,nf", [(synth.TINY, 4), (synth.FULL, 4)])
def test_self_match(geom, nf):
    """Context = the query frames and k = 16 q token by token, with every q row scaled to
    norm sqrt(D).  RoPE cancels at equal positions, so a query's own key scores
    16*sqrt(D) ~ 181 while the others score ~N(0, 16^2): each query must return its own
    token's v row."""
    g = geom
    W, N, H, D = g.window, g.tokens_per_frame, g.n_heads, g.head_dim
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, W)
    t0 = 30
    x = np.random.default_rng(77).standard_normal((nf * N, H, D))
    x *= np.sqrt(D) / np.linalg.norm(x, axis=2, keepdims=True)
    q = synth.f32_to_bf16_bits(x.astype(np.float32))
    k = synth.f32_to_bf16_bits((f64(q) * 16.0).astype(np.float32))  # exact: power of two
    v = synth.frames(g, 6, 0, t0, nf, synth.V)
    cache.roll(up(k), up(v), t0)
    o = _out(g, nf)
    rf.window_attention(ctx, cache, [rf.Segment(up(q), t0, o, t0, nf)])
    torch.cuda.synchronize()
    got = f64(down(o))
    want = f64(v)
    err = np.abs(got - want).max()
    print(f"self-match max_abs={err:.3e}", flush=True)
    assert err <= 2.0 ** -7 * np.abs(want).max()


def _fill_steady(g, cfg, s, cache):
    """Bring `cache` to the state after step s: clean frames max(0,s-6)..s-1 (as written at
    steps t+1), current frames s..s+14 drawn at step s.  Returns {t: (k_bits, v_bits, tag)}."""
    N = g.tokens_per_frame
    lo = max(0, s - 6)
    data = {}
    for t in range(lo, s):
        data[t] = (synth.frame(g, cfg, t + 1, t, synth.K + synth.CLEAN),
                   synth.frame(g, cfg, t + 1, t, synth.V + synth.CLEAN), ("clean", t + 1))
    for t in range(s, s + 15):
        data[t] = (synth.frame(g, cfg, s, t, synth.K), synth.frame(g, cfg, s, t, synth.V),
                   ("noisy", s))
    ts = sorted(data)
    # two rolls: clean frames, then the current ones (each <= 21 frames)
    if lo < s:
        cache.roll(up(np.concatenate([data[t][0] for t in range(lo, s)])),
                   up(np.concatenate([data[t][1] for t in range(lo, s)])), lo)
    cache.roll(up(np.concatenate([data[t][0] for t in range(s, s + 15)])),
               up(np.concatenate([data[t][1] for t in range(s, s + 15)])), s)
    assert cache.window() == ts
    return data


def _check_rows(g, rk, data, q_bits, q_t0, o, ctx_lo, ctx_hi, rows, what, q_tok0=0):
    khs = [rk.get(t, data[t][2], data[t][0]) for t in range(ctx_lo, ctx_hi)]
    vs = [data[t][1] for t in range(ctx_lo, ctx_hi)]
    want = oracle_rows(g, q_bits, q_t0, khs, vs, rows, q_tok0=q_tok0)
    got = f64(down(o))[rows]
    assert_close(got, want, what)


def test_cache_update_pass_full_size():
    """1 clean query frame (1,560 rows) over 21 frames (32,760 keys), after a roll that
    evicts the oldest frame; sampled rows incl. frame and tile edges."""
    g, cfg = synth.FULL, synth.WORKLOAD_IDS["cache_update"]
    W, N = g.window, g.tokens_per_frame
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, W)
    data = {}
    for t in range(W):
        data[t] = (synth.frame(g, cfg, 0, t, synth.K), synth.frame(g, cfg, 0, t, synth.V), 0)
    cache.roll(up(np.concatenate([data[t][0] for t in range(W)])),
               up(np.concatenate([data[t][1] for t in range(W)])), 0)
    data[21] = (synth.frame(g, cfg, 1, 21, synth.K + synth.CLEAN),
                synth.frame(g, cfg, 1, 21, synth.V + synth.CLEAN), 1)
    cache.roll(up(data[21][0]), up(data[21][1]), 21)
    assert cache.window() == list(range(1, 22))
    q = synth.frame(g, cfg, 1, 21, synth.Q + synth.CLEAN)
    o = _out(g, 1)
    rf.window_attention(ctx, cache, [rf.Segment(up(q), 21, o, 1, 21)])
    torch.cuda.synchronize()
    rows = sample_rows(N, N, extra=96, seed=1)
    _check_rows(g, RotatedKeys(g), data, q, 21, o, 1, 22, rows, "cache-update")


def test_denoise_pass_full_size_and_determinism():
    """15 query frames (23,400 rows) over 21 frames (32,760 keys) = 6 cached + 15 current."""
    g, cfg = synth.FULL, synth.WORKLOAD_IDS["denoise"]
    N = g.tokens_per_frame
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, g.window)
    data = _fill_steady(g, cfg, 6, cache)
    q = synth.frames(g, cfg, 6, 6, 15, synth.Q)
    qd = up(q)
    o = _out(g, 15)
    rf.window_attention(ctx, cache, [rf.Segment(qd, 6, o, 0, 21)])
    o2 = _out(g, 15)
    rf.window_attention(ctx, cache, [rf.Segment(qd, 6, o2, 0, 21)])
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "not deterministic"
    rows = sample_rows(15 * N, N, extra=160, seed=2)
    _check_rows(g, RotatedKeys(g), data, q, 6, o, 0, 21, rows, "denoise")


def test_batched_two_phase_step_full_size():
    """Steady state step s = 9: ONE launch with the denoise segment (frames 9..23) and the
    cache-update segment (frame 8), both over the window 3..23."""
    g, cfg = synth.FULL, synth.WORKLOAD_IDS["batched"]
    N = g.tokens_per_frame
    s = 9
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, g.window)
    # bring the ring to the state before step s, then roll frame s-1 (clean) + s..s+14
    _fill_steady(g, cfg, s - 1, cache)
    data = {}
    for t in range(s - 6, s):
        data[t] = (synth.frame(g, cfg, t + 1, t, synth.K + synth.CLEAN),
                   synth.frame(g, cfg, t + 1, t, synth.V + synth.CLEAN), ("clean", t + 1))
    for t in range(s, s + 15):
        data[t] = (synth.frame(g, cfg, s, t, synth.K), synth.frame(g, cfg, s, t, synth.V),
                   ("noisy", s))
    cache.roll(up(np.concatenate([data[t][0] for t in range(s - 1, s + 15)])),
               up(np.concatenate([data[t][1] for t in range(s - 1, s + 15)])), s - 1)
    assert cache.window() == list(range(s - 6, s + 15))
    qa = synth.frames(g, cfg, s, s, 15, synth.Q)
    qb = synth.frame(g, cfg, s, s - 1, synth.Q + synth.CLEAN)
    oa, ob = _out(g, 15), _out(g, 1)
    rf.window_attention(ctx, cache, [rf.Segment(up(qa), s, oa, s - 6, 21),
                                     rf.Segment(up(qb), s - 1, ob, s - 6, 21)])
    torch.cuda.synchronize()
    rk = RotatedKeys(g)
    _check_rows(g, rk, data, qa, s, oa, s - 6, s + 15, sample_rows(15 * N, N, extra=96, seed=3),
                "batched A")
    _check_rows(g, rk, data, qb, s - 1, ob, s - 6, s + 15, sample_rows(N, N, extra=64, seed=4),
                "batched B")


def test_largest_ring_with_the_window_across_its_end():
    """The largest ring the library accepts at the full geometry (448 slots: 2.15 GB per K or
    V ring, just under the attention kernel's 32-bit offset limit), with the window's 21
    frames 440..460 in slots 440..447 and 0..12: key and value tiles come from the ring's
    last bytes and across its wrap.  One batched launch (denoise frames 446..460 and the
    cache-update frame 445, both over 440..460); sampled rows of both against the oracle."""
    g, cfg = synth.FULL, synth.WORKLOAD_IDS["batched"]
    N = g.tokens_per_frame
    slot_bytes = N * g.n_heads * g.head_dim * 2
    capacity = (0x7FFFFFF0 - 1) // slot_bytes
    assert capacity == 448
    assert rf.kvcache_bytes(capacity) == capacity * slot_bytes
    with pytest.raises(rf.RfError):
        rf.kvcache_bytes(capacity + 1)
    t_lo, s = 440, 446
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, capacity)
    data = {t: (synth.frame(g, cfg, s, t, synth.K), synth.frame(g, cfg, s, t, synth.V), ("noisy", s))
            for t in range(t_lo, t_lo + g.window)}
    cache.roll(up(np.concatenate([data[t][0] for t in sorted(data)])),
               up(np.concatenate([data[t][1] for t in sorted(data)])), t_lo)
    assert cache.window() == list(range(t_lo, t_lo + g.window))
    qa = synth.frames(g, cfg, s, s, 15, synth.Q)
    qb = synth.frame(g, cfg, s, s - 1, synth.Q + synth.CLEAN)
    oa, ob = _out(g, 15), _out(g, 1)
    rf.window_attention(ctx, cache, [rf.Segment(up(qa), s, oa, t_lo, g.window),
                                     rf.Segment(up(qb), s - 1, ob, t_lo, g.window)])
    torch.cuda.synchronize()
    rk = RotatedKeys(g)
    hi = t_lo + g.window
    _check_rows(g, rk, data, qa, s, oa, t_lo, hi, sample_rows(15 * N, N, extra=64, seed=11),
                "largest ring A")
    _check_rows(g, rk, data, qb, s - 1, ob, t_lo, hi, sample_rows(N, N, extra=48, seed=12),
                "largest ring B")
    del cache
    gc.collect()
    torch.cuda.empty_cache()


def test_largest_segment_the_library_accepts():
    """One segment of the most query tokens the library accepts, 2^24 - 1 (the device's
    token -> frame, row, column division is exact below 2^24): 10,755 frames of queries,
    51.5 GB of Q and as much O, 786,432 query tiles in 3,072 whole rounds, over a 21-frame
    window.  A segment of 2^24 tokens is refused before any launch.  Sampled rows of the
    first and last tiles, frame edges far into the segment and random rows against the
    oracle, each query rotated at its own position."""
    g = synth.FULL
    N, H, D, W = g.tokens_per_frame, g.n_heads, g.head_dim, g.window
    n, q_t0, cfg = (1 << 24) - 1, 5, 61
    ctx = _ctx(g, max_frame=16384)
    cache = rf.KVCache(ctx, W)
    k = synth.frames(g, cfg, 0, 0, W, synth.K)
    v = synth.frames(g, cfg, 0, 0, W, synth.V)
    cache.roll(up(k), up(v), 0)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cfg)
    q_all = torch.randn((n + 1, H, D), generator=gen, device="cuda", dtype=torch.bfloat16)
    o_all = torch.full((n + 1, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rf.RfError, match="too many query tokens"):
        rf.window_attention(ctx, cache, [rf.Segment(q_all, q_t0, o_all, 0, W)])
    q, o = q_all[:n], o_all[:n]
    print(f"one segment of {n} query tokens over {W * N} keys", flush=True)
    rf.window_attention(ctx, cache, [rf.Segment(q, q_t0, o, 0, W)])
    torch.cuda.synchronize()
    rng = np.random.default_rng(cfg)
    last = (n - 1) // 256 * 256
    rows = {0, 1, 31, 32, 255, 256, last - 1, last, last + 31, last + 32, n - 2, n - 1}
    for f in rng.integers(1, n // N, 16):
        rows.update({int(f) * N - 1, int(f) * N})
    rows.update(int(r) for r in rng.integers(0, n, 48))
    rows = np.array(sorted(rows))
    idx = torch.from_numpy(rows).cuda()
    qb = q.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
    got = f64(o.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16))
    kh = orope.rope_exact(f64(k), 0, g.grid_h, g.grid_w, g.pairs, g.base)
    vf = f64(v)
    want = np.empty((len(rows), H, D))
    for j, i in enumerate(rows):
        qh = orope.rope_exact(f64(qb[j:j + 1]), q_t0 + int(i) // N, g.grid_h, g.grid_w, g.pairs,
                                    g.base, tok0=int(i) % N)[0]
        for h in range(H):
            want[j, h] = oatt.attend_head(qh[None, h], kh[:, h], vf[:, h], 1.0 / np.sqrt(D))[0]
    assert_close(got, want, "largest segment")
    del q_all, o_all, q, o, cache
    torch.cuda.empty_cache()


def test_two_contexts_on_two_streams_at_once():
    """Two contexts, each with its own ring and workspace, run batched launches (whole and
    key-split tiles) on two streams at the same time, three each, interleaved; every output
    equals, bit for bit, what the same launch gives alone: the contexts share no state."""
    g, cfg = synth.FULL, synth.WORKLOAD_IDS["batched"]
    N, W = g.tokens_per_frame, g.window
    s = 9
    kall = up(synth.frames(g, cfg, s, s - 6, W, synth.K))
    vall = up(synth.frames(g, cfg, s, s - 6, W, synth.V))
    ctxs = [_ctx(g), _ctx(g)]
    caches = []
    for c in ctxs:
        cache = rf.KVCache(c, W)
        cache.roll(kall, vall, s - 6)
        caches.append(cache)
    qs = [(up(synth.frames(g, cfg + 100 * i, s, s, 15, synth.Q)),
           up(synth.frame(g, cfg + 100 * i, s, s - 1, synth.Q + synth.CLEAN))) for i in range(2)]

    def launch(i, oa, ob):
        rf.window_attention(ctxs[i], caches[i], [rf.Segment(qs[i][0], s, oa, s - 6, W),
                                                 rf.Segment(qs[i][1], s - 1, ob, s - 6, W)])

    alone = []
    for i in range(2):
        oa, ob = _out(g, 15), _out(g, 1)
        launch(i, oa, ob)
        torch.cuda.synchronize()
        alone.append((oa, ob))
    outs = [[(_out(g, 15), _out(g, 1)) for _ in range(3)] for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    main = torch.cuda.current_stream()
    for st in streams:
        st.wait_stream(main)
    print("two contexts, two streams: 3 + 3 batched launches", flush=True)
    for r in range(3):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                launch(i, *outs[i][r])
    torch.cuda.synchronize()
    for i in range(2):
        for r in range(3):
            for got, want in zip(outs[i][r], alone[i]):
                assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (i, r)
    assert not torch.equal(alone[0][0], alone[1][0])  # the two query sets differ


def test_batched_step_full_size_every_row_and_canaries():
    """One full check of the batched step (s = 7): every one of the 23,400 + 1,560 output
    rows x 12 heads against the oracle, with canaries -- rows before and after each output
    and 16 padding columns per row, filled with a sentinel -- that must survive."""
    from threadpoolctl import threadpool_limits
    g, cfg = synth.FULL, 57
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    s = 7
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, g.window)
    _fill_steady(g, cfg, s - 1, cache)
    data = {}
    for t in range(s - 6, s):
        data[t] = (synth.frame(g, cfg, t + 1, t, synth.K + synth.CLEAN),
                   synth.frame(g, cfg, t + 1, t, synth.V + synth.CLEAN))
    for t in range(s, s + 15):
        data[t] = (synth.frame(g, cfg, s, t, synth.K), synth.frame(g, cfg, s, t, synth.V))
    cache.roll(up(np.concatenate([data[t][0] for t in range(s - 1, s + 15)])),
               up(np.concatenate([data[t][1] for t in range(s - 1, s + 15)])), s - 1)
    qa = synth.frames(g, cfg, s, s, 15, synth.Q)
    qb = synth.frame(g, cfg, s, s - 1, synth.Q + synth.CLEAN)
    pad, row = 3, H * D
    sentinel = -12345  # bf16 bits 0xCFC7, a value no output row holds

    def canaried(n):
        full = torch.full((n + 2 * pad, row + 16), sentinel, dtype=torch.int16, device="cuda")
        return full, full.view(torch.bfloat16)[pad:pad + n, :row].view(n, H, D)

    fa, oa = canaried(15 * N)
    fb, ob = canaried(N)
    rf.window_attention(ctx, cache, [rf.Segment(up(qa), s, oa, s - 6, 21),
                                     rf.Segment(up(qb), s - 1, ob, s - 6, 21)])
    torch.cuda.synchronize()
    for full, n, what in ((fa, 15 * N, "A"), (fb, N, "B")):
        f = full.cpu().numpy()
        assert (f[:pad] == sentinel).all() and (f[pad + n:] == sentinel).all(), f"rows around {what} written"
        assert (f[:, row:] == sentinel).all(), f"padding columns of {what} written"
    k = f64(np.concatenate([data[t][0] for t in range(s - 6, s + 15)]))
    v = f64(np.concatenate([data[t][1] for t in range(s - 6, s + 15)]))
    print("oracle over all rows of both segments", flush=True)
    with threadpool_limits(limits=1, user_api="blas"):
        want_a = oatt.window_attention(f64(qa), s, k, v, s - 6, g.grid_h, g.grid_w, g.pairs, g.base)
        want_b = oatt.window_attention(f64(qb), s - 1, k, v, s - 6, g.grid_h, g.grid_w, g.pairs, g.base)
    assert_close(f64(down(oa)), want_a, "batched A, every row")
    assert_close(f64(down(ob)), want_b, "batched B, every row")


def test_dynamic_window_fill_30_steps():
    """30 steps in one process: context grows 15..21 frames as the ring fills, then one
    frame is evicted per step; no reallocation between steps.  Sampled rows every step."""
    g, cfg = synth.FULL, synth.WORKLOAD_IDS["dynamic"]
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, g.window)
    kbuf = torch.empty((16 * N, H, D), dtype=torch.bfloat16, device="cuda")
    vbuf = torch.empty_like(kbuf)
    qbuf = torch.empty((15 * N, H, D), dtype=torch.bfloat16, device="cuda")
    o = _out(g, 15)
    rk = RotatedKeys(g)
    data = {}
    gc.collect()  # earlier tests' contexts are freed now, not by a collection inside the loop
    gc.disable()
    try:
        _dynamic_steps(g, cfg, N, ctx, cache, kbuf, vbuf, qbuf, o, rk, data)
    finally:
        gc.enable()


def _dynamic_steps(g, cfg, N, ctx, cache, kbuf, vbuf, qbuf, o, rk, data):
    mem0 = None
    for s in range(30):
        t0 = max(s - 1, 0)
        for t in range(t0, s + 15):
            tag = ("clean", s) if t < s else ("noisy", s)
            tid = synth.CLEAN if t < s else 0
            data[t] = (synth.frame(g, cfg, s, t, synth.K + tid), synth.frame(g, cfg, s, t, synth.V + tid), tag)
        n = s + 15 - t0
        kbuf[:n * N] = up(np.concatenate([data[t][0] for t in range(t0, s + 15)]))
        vbuf[:n * N] = up(np.concatenate([data[t][1] for t in range(t0, s + 15)]))
        cache.roll(kbuf[:n * N], vbuf[:n * N], t0)
        lo = s - min(s, 6)
        assert cache.window() == list(range(lo, s + 15)), (s, cache.window())
        q = synth.frames(g, cfg, s, s, 15, synth.Q)
        qbuf.copy_(up(q))
        rf.window_attention(ctx, cache, [rf.Segment(qbuf, s, o, lo, s + 15 - lo)])
        torch.cuda.synchronize()
        if mem0 is None:
            mem0 = torch.cuda.memory_allocated()
        assert torch.cuda.memory_allocated() == mem0
        # device-wide free memory (hipMemGetInfo) also sees allocations outside torch's
        # allocator: none while the context grows from 15 to 21 frames (from step 2 on,
        # when torch's cache holds every temporary size the loop uses)
        if s == 2:
            free2 = torch.cuda.mem_get_info()[0]
        elif s > 2:
            assert torch.cuda.mem_get_info()[0] == free2, f"device memory changed at step {s}"
        rows = sample_rows(15 * N, N, extra=8, seed=100 + s) if s in (0, 6, 7, 29) else \
            np.array([0, 777, 15 * N - 1])
        rk.prune(lo)
        print(f"step {s}: ctx {s + 15 - lo} frames, {len(rows)} rows", flush=True)
        _check_rows(g, rk, data, q, s, o, lo, s + 15, rows, f"dynamic step {s}")


def test_token_offset_segments_tiny():
    """Query blocks cut at any token, in one launch: 70 rows from token 29 of frame 2 (into
    frame 4) and 35 rows from token 5 of frame 1, over frames 0..4; every row checked."""
    g, cfg = synth.TINY, 61
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, g.window)
    k = synth.frames(g, cfg, 0, 0, 5, synth.K)
    v = synth.frames(g, cfg, 0, 0, 5, synth.V)
    q = synth.frames(g, cfg, 0, 0, 5, synth.Q)
    cache.roll(up(k), up(v), 0)
    qa, qb = q[2 * N + 29:2 * N + 99], q[N + 5:N + 40]
    oa = torch.empty((70, H, D), dtype=torch.bfloat16, device="cuda")
    ob = torch.empty((35, H, D), dtype=torch.bfloat16, device="cuda")
    rf.window_attention(ctx, cache, [rf.Segment(up(qa), 2, oa, 0, 5, q_tok0=29),
                                     rf.Segment(up(qb), 1, ob, 0, 5, q_tok0=5)])
    torch.cuda.synchronize()
    args = (f64(k), f64(v), 0, g.grid_h, g.grid_w, g.pairs, g.base)
    assert_close(f64(down(oa)), oatt.window_attention(f64(qa), 2, *args, q_tok0=29), "from token 29")
    assert_close(f64(down(ob)), oatt.window_attention(f64(qb), 1, *args, q_tok0=5), "from token 5")


@pytest.mark.parametrize("half", [0, 1])
def test_one_gpu_share_of_the_hybrid_split_full_size(half):
    """One device's share of the heads x sequence split: 3 heads, and one half of the
    step's queries -- denoise tokens 11,700 h .. 11,700 h + 11,699 of frames s..s+14 (the
    second half starts at token 780 of frame s+7) and cache-update tokens 780 h .. 780 h
    + 779 of frame s-1 -- in one launch over the 21-frame window; sampled rows."""
    g, cfg = synth.SHARD, synth.WORKLOAD_IDS["shard"]
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    s = 9
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, g.window)
    _fill_steady(g, cfg, s - 1, cache)
    data = {}
    for t in range(s - 6, s):
        data[t] = (synth.frame(g, cfg, t + 1, t, synth.K + synth.CLEAN),
                   synth.frame(g, cfg, t + 1, t, synth.V + synth.CLEAN), ("clean", t + 1))
    for t in range(s, s + 15):
        data[t] = (synth.frame(g, cfg, s, t, synth.K), synth.frame(g, cfg, s, t, synth.V),
                   ("noisy", s))
    cache.roll(up(np.concatenate([data[t][0] for t in range(s - 1, s + 15)])),
               up(np.concatenate([data[t][1] for t in range(s - 1, s + 15)])), s - 1)
    na, nb = 15 * N // 2, N // 2
    qa = synth.frames(g, cfg, s, s, 15, synth.Q)[half * na:(half + 1) * na]
    qb = synth.frame(g, cfg, s, s - 1, synth.Q + synth.CLEAN)[half * nb:(half + 1) * nb]
    a_t0, a_tok0 = s + (half * na) // N, (half * na) % N
    b_tok0 = half * nb
    oa = torch.empty((na, H, D), dtype=torch.bfloat16, device="cuda")
    ob = torch.empty((nb, H, D), dtype=torch.bfloat16, device="cuda")
    print(f"share {half}: denoise from frame {a_t0} token {a_tok0}, update from token {b_tok0}",
          flush=True)
    rf.window_attention(ctx, cache, [rf.Segment(up(qa), a_t0, oa, s - 6, 21, q_tok0=a_tok0),
                                     rf.Segment(up(qb), s - 1, ob, s - 6, 21, q_tok0=b_tok0)])
    torch.cuda.synchronize()
    rk = RotatedKeys(g)
    rows_a = np.union1d(sample_rows(na, N, extra=64, seed=20 + half),
                        [N - a_tok0 - 1, N - a_tok0])  # both sides of the first frame edge
    _check_rows(g, rk, data, qa, a_t0, oa, s - 6, s + 15, rows_a, f"share {half} denoise",
                q_tok0=a_tok0)
    _check_rows(g, rk, data, qb, s - 1, ob, s - 6, s + 15, sample_rows(nb, N, extra=32, seed=30),
                f"share {half} cache update", q_tok0=b_tok0)


def test_attention_errors():
    g = synth.TINY
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, g.window)
    q = up(synth.frames(g, 9, 0, 0, 1, synth.Q))
    o = _out(g, 1)
    with pytest.raises(rf.RfError) as e:  # empty cache
        rf.window_attention(ctx, cache, [rf.Segment(q, 0, o, 0, 1)])
    assert e.value.status == 4
    k = up(synth.frames(g, 9, 0, 0, 3, synth.K))
    cache.roll(k, k, 0)
    for ctx_t0, nf in ((0, 4), (-1, 2), (3, 1)):
        with pytest.raises(rf.RfError) as e:
            rf.window_attention(ctx, cache, [rf.Segment(q, 0, o, ctx_t0, nf)])
        assert e.value.status == 4
    with pytest.raises(rf.RfError) as e:
        rf.window_attention(ctx, cache, [rf.Segment(q, 0, o, 0, 3)], scale=-1.0)
    assert e.value.status == 3
    with pytest.raises(ValueError):
        rf.window_attention(ctx, cache, [])
    N = g.tokens_per_frame
    for tok0 in (-1, N):  # the first token must lie inside frame q_t0
        with pytest.raises(rf.RfError) as e:
            rf.window_attention(ctx, cache, [rf.Segment(q[:5], 0, o[:5], 0, 3, q_tok0=tok0)])
        assert e.value.status == 3
    with pytest.raises(ValueError):  # q and o of different lengths
        rf.window_attention(ctx, cache, [rf.Segment(q[:5], 0, o[:6], 0, 3)])
    with pytest.raises(rf.RfError) as e:  # an empty query segment: torch hands over a null
        rf.window_attention(ctx, cache, [rf.Segment(q[:0], 0, o[:0], 0, 3)])  # pointer for it
    assert e.value.status in (1, 3)  # RF_ERR_NULL, or RF_ERR_SHAPE for a non-null pointer
    with pytest.raises(ValueError):  # more segments than one launch takes
        rf.window_attention(ctx, cache, [rf.Segment(q[i:i + 1], 0, o[i:i + 1], 0, 3, q_tok0=i)
                                         for i in range(rf.MAX_SEGMENTS + 1)])
    small = _ctx(g, max_frame=20)
    cs = rf.KVCache(small, g.window)
    cs.roll(k, k, 0)
    rf.window_attention(small, cs, [rf.Segment(q[:2], 19, o[:2], 0, 3, q_tok0=N - 2)])  # frame 19 only
    with pytest.raises(rf.RfError) as e:  # token N-1 of frame 19, then frame 20: beyond the tables
        rf.window_attention(small, cs, [rf.Segment(q[:2], 19, o[:2], 0, 3, q_tok0=N - 1)])
    assert e.value.status == 4
    torch.cuda.synchronize()


def test_oversized_ring_is_refused_before_any_launch():
    """A ring whose byte size reaches the attention kernel's 32-bit range (449 slots at
    the workload geometry) is refused with RF_ERR_SHAPE by every call that takes a ring,
    before anything is enqueued: the descriptor points at a small dummy buffer that no
    kernel may touch, and the output canary stays intact."""
    import ctypes
    g = synth.FULL
    ctx = _ctx(g)
    N = g.tokens_per_frame
    dummy = torch.zeros(4096, dtype=torch.bfloat16, device="cuda")
    for capacity, count in ((449, 21), (897, 21)):
        desc = rf.KVCacheDesc(dummy.data_ptr(), dummy.data_ptr(), capacity, count, 0)
        q = torch.zeros((N, g.n_heads, g.head_dim), dtype=torch.bfloat16, device="cuda")
        o = torch.full((N, g.n_heads, g.head_dim), 7.0, dtype=torch.bfloat16, device="cuda")
        seg = rf.SegmentDesc(q.data_ptr(), g.n_heads * g.head_dim, o.data_ptr(), g.n_heads * g.head_dim,
                             20, 0, N, 0, 21, 0)
        st = rf.lib().rf_window_attention(ctx.handle, ctypes.byref(desc), ctypes.byref(seg), 1, 0.0,
                                          rf._stream(None))
        assert st == 3, rf.lib().rf_last_error()
        st = rf.lib().rf_kvcache_roll(ctx.handle, ctypes.byref(desc), q.data_ptr(), g.n_heads * g.head_dim,
                                      q.data_ptr(), g.n_heads * g.head_dim, 20, 1, rf._stream(None))
        assert st == 3, rf.lib().rf_last_error()
        assert (desc.first, desc.count) == (0, count)
        torch.cuda.synchronize()
        assert bool((o == 7.0).all())
    with pytest.raises(rf.RfError) as e:  # the binding refuses before allocating
        rf.KVCache(ctx, 449)
    assert e.value.status == 3


def test_keys_rotated_on_load_variant_full_size():
    """rf_window_attention_rawk (the measurement variant that keeps un-rotated keys in
    the ring and rotates each key tile as it stages it) against the oracle on sampled
    rows of the batched step, and within a bf16 step of the shipped kernel (its float32
    key rotation may round differently from the ring's float64 one)."""
    g, cfg = synth.FULL, 61
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    s = 9
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, g.window)
    data = _fill_steady(g, cfg, s, cache)
    assert cache.window() == list(range(s - 6, s + 15))
    raw = rf.KVCache(ctx, g.window)  # same values, raw keys written head-major by torch
    raw.desc.first, raw.desc.count = cache.first, cache.count
    raw.v.copy_(cache.v)
    for t in range(s - 6, s + 15):
        raw.k[t % g.window] = up(data[t][0]).view(N, H, D).permute(1, 0, 2)
    qa = synth.frames(g, cfg, s, s, 15, synth.Q)
    qb = synth.frame(g, cfg, s, s - 1, synth.Q + synth.CLEAN)
    oa, ob, ra, rb = _out(g, 15), _out(g, 1), _out(g, 15), _out(g, 1)
    rf.window_attention_rawk(ctx, raw, [rf.Segment(up(qa), s, ra, s - 6, 21), rf.Segment(up(qb), s - 1, rb, s - 6, 21)])
    rf.window_attention(ctx, cache, [rf.Segment(up(qa), s, oa, s - 6, 21), rf.Segment(up(qb), s - 1, ob, s - 6, 21)])
    torch.cuda.synchronize()
    rk = RotatedKeys(g)
    _check_rows(g, rk, data, qa, s, ra, s - 6, s + 15, sample_rows(15 * N, N, extra=64, seed=11), "rawk A")
    _check_rows(g, rk, data, qb, s - 1, rb, s - 6, s + 15, sample_rows(N, N, extra=32, seed=12), "rawk B")
    for got, ref in ((ra, oa), (rb, ob)):
        d = (got.float() - ref.float()).abs()
        assert float(d.max()) <= 2.0 ** -7, float(d.max())
    small = _ctx(synth.TINY)
    tc = rf.KVCache(small, synth.TINY.window)
    k = up(synth.frames(synth.TINY, cfg, 0, 0, 2, synth.K))
    tc.roll(k, k, 0)
    with pytest.raises(rf.RfError) as e:  # frames shorter than a key tile
        rf.window_attention_rawk(small, tc, [rf.Segment(k[:4], 0, k[4:8].clone(), 0, 2)])
    assert e.value.status == 3
