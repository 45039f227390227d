"""GPU parity of rf_rope3d_apply and rf_kvcache_roll: bit-exact against the oracle's
bf16 RoPE specification and ring model (tiny and full 30x52x12x128 geometry)."""
import numpy as np
import pytest
import torch

import rolling_window_attention_amd as rf
from rolling_window_attention_amd import synth
from oracle import rope3d as orope
from oracle.ring import RingModel

from gpu_util import ring_slot_v, down, ring_frame_k, ring_frame_v, up

pytestmark = pytest.mark.gpu


def _ctx(g, max_frame=4096):
    return rf.Context(g.grid_h, g.grid_w, g.n_heads, g.head_dim, g.pairs, g.base, max_frame)


def _spec(g, bits, t0):
    return orope.rope_spec_bits(bits, t0, g.grid_h, g.grid_w, g.pairs, g.base)


@pytest.mark.parametrize("geom,t0,n_frames", [(synth.TINY, 3, 7), (synth.TINY, 0, 1),
                                              (synth.FULL, 6, 15)])
def test_rope3d_bit_exact(geom, t0, n_frames):
    print(f"rope3d geom={geom.grid_h}x{geom.grid_w} t0={t0} frames={n_frames}", flush=True)
    ctx = _ctx(geom)
    x = synth.frames(geom, 11, 0, t0, n_frames, synth.Q)
    y = ctx.rope3d_apply(up(x), t0)
    torch.cuda.synchronize()
    assert np.array_equal(down(y), _spec(geom, x, t0))


def test_rope3d_partial_frame_strided_and_in_place():
    g = synth.TINY
    ctx = _ctx(g)
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    n = 2 * N + 13  # a ragged number of tokens
    x = synth.frames(g, 12, 0, 40, 3, synth.Q)[:n]
    want = _spec(g, x, 40)
    # x lives inside a fused [tokens, 3*H*D] projection output (row stride 3*H*D)
    fused = torch.zeros((n, 3, H, D), dtype=torch.bfloat16, device="cuda")
    fused[:, 1] = up(x)
    xs = fused[:, 1]
    out = torch.zeros((n, H, D), dtype=torch.bfloat16, device="cuda")
    ctx.rope3d_apply(xs, 40, y=out)
    ctx.rope3d_apply(xs, 40, y=xs)  # in place, same stride
    torch.cuda.synchronize()
    assert np.array_equal(down(out), want)
    assert np.array_equal(down(fused[:, 1]), want)
    assert not fused[:, 0].any() and not fused[:, 2].any()  # neighbours untouched


def test_one_context_from_four_threads_and_streams():
    """One context shared by four host threads, each on a stream of its own (default
    priority), applying the RoPE and rolling its own ring at once, and one thread's call
    failing validation meanwhile: every output is bit-exact and each thread's error
    detail is its own."""
    import threading
    g = synth.TINY
    ctx = _ctx(g)
    N = g.tokens_per_frame
    xs = [synth.frames(g, 20 + i, 0, 3 * i, 4, synth.Q) for i in range(4)]
    kv = [(synth.frames(g, 30 + i, 0, i, 3, synth.K), synth.frames(g, 30 + i, 0, i, 3, synth.V)) for i in range(4)]
    dev_x = [up(x) for x in xs]
    dev_kv = [(up(k), up(v)) for k, v in kv]
    caches = [rf.KVCache(ctx, g.window) for _ in range(4)]
    ys = [[None] * 5 for _ in range(4)]
    errs = [None] * 4
    torch.cuda.synchronize()
    barrier = threading.Barrier(4)

    def work(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                barrier.wait()
                for r in range(5):
                    ys[i][r] = ctx.rope3d_apply(dev_x[i], 3 * i)
                caches[i].roll(dev_kv[i][0], dev_kv[i][1], i)
                if i == 2:  # a call that fails validation on this thread only
                    with pytest.raises(rf.RfError, match="roll start"):
                        caches[i].roll(dev_kv[i][0], dev_kv[i][1], 100)
                    errs[i] = rf.lib().rf_last_error().decode()
                else:
                    errs[i] = rf.lib().rf_last_error().decode()
                st.synchronize()
        except BaseException as e:  # reported by the main thread
            errs[i] = e

    threads = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    torch.cuda.synchronize()
    for i in range(4):
        assert not isinstance(errs[i], BaseException), errs[i]
        want = _spec(g, xs[i], 3 * i)
        for r in range(5):
            assert np.array_equal(down(ys[i][r]), want), (i, r)
        Kb, Vb = down(caches[i].k), down(caches[i].v)
        for f in range(3):
            slot = (i + f) % g.window
            assert np.array_equal(ring_frame_k(Kb, slot), _spec(g, kv[i][0][f * N:(f + 1) * N], i + f))
            assert np.array_equal(ring_frame_v(Vb, slot), kv[i][1][f * N:(f + 1) * N])
    assert "roll start 100" in errs[2]
    assert all(errs[i] == "" for i in (0, 1, 3)), errs


def test_rope3d_errors():
    g = synth.TINY
    ctx = _ctx(g, max_frame=10)
    x = up(synth.frames(g, 13, 0, 0, 2, synth.Q))
    with pytest.raises(rf.RfError) as e:
        ctx.rope3d_apply(x, 9)  # second frame would be 10 >= max_frame
    assert e.value.status == 4
    with pytest.raises(rf.RfError) as e:
        ctx.rope3d_apply(x, -1)
    assert e.value.status == 4
    # misaligned pointer
    flat = torch.zeros(2 * g.tokens_per_frame * g.n_heads * g.head_dim + 8, dtype=torch.bfloat16,
                       device="cuda")
    mis = flat[1:1 + x.numel()].view(x.shape)
    with pytest.raises(rf.RfError) as e:
        ctx.rope3d_apply(mis, 0)
    assert e.value.status == 2
    # zero tokens is a no-op
    ctx.rope3d_apply(x[:0], 0)


def _expected_ring(g, model, W):
    """Expected ring bits from the oracle ring model (slot_data = (k_bits, v_bits, t))."""
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    K = np.zeros((W, H, N, D), np.uint16)
    V = np.zeros((W, H, N // 8, D, 8), np.uint16)
    for s in range(W):
        if model.slot_data[s] is None:
            continue
        kb, vb, t = model.slot_data[s]
        K[s] = _spec(g, kb, t).transpose(1, 0, 2)
        V[s] = ring_slot_v(vb)
    return K, V


def test_roll_tiny_wrap_bit_exact():
    """Twelve steps of the window schedule on a 5-slot ring (wraps twice), the whole
    ring compared after every roll."""
    g = synth.TINY
    W = g.window
    N = g.tokens_per_frame
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, W)
    model = RingModel(W)
    for s in range(12):
        t0 = max(s - 1, 0)
        n = (s + 3) - t0  # frames t0 .. s+2 (3 current frames plus the clean one)
        n = min(n, W)
        print(f"roll step {s}: t0={t0} n={n}", flush=True)
        k = np.concatenate([synth.frame(g, 1, s, t, synth.K + (synth.CLEAN if t < s else 0))
                            for t in range(t0, t0 + n)])
        v = np.concatenate([synth.frame(g, 1, s, t, synth.V + (synth.CLEAN if t < s else 0))
                            for t in range(t0, t0 + n)])
        cache.roll(up(k), up(v), t0)
        model.roll(t0, n, [(k[i * N:(i + 1) * N], v[i * N:(i + 1) * N], t0 + i) for i in range(n)])
        assert (cache.first, cache.count) == (model.first, model.count)
        torch.cuda.synchronize()
        K, V = _expected_ring(g, model, W)
        assert np.array_equal(down(cache.k), K), f"K ring differs after step {s}"
        assert np.array_equal(down(cache.v), V), f"V ring differs after step {s}"


def test_roll_full_cache_update_bit_exact():
    """Full geometry: fill 21 frames, then roll frame 21 in (evicts frame 0); the new
    slot is bit-exact and the other 20 slots are untouched."""
    g = synth.FULL
    W, N = g.window, g.tokens_per_frame
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, W)
    k0 = synth.frames(g, 2, 0, 0, W, synth.K + synth.CLEAN)
    v0 = synth.frames(g, 2, 0, 0, W, synth.V + synth.CLEAN)
    print("prefill 21 frames", flush=True)
    cache.roll(up(k0), up(v0), 0)
    torch.cuda.synchronize()
    Kb, Vb = down(cache.k), down(cache.v)
    for t in (0, 7, 20):
        assert np.array_equal(ring_frame_k(Kb, t), _spec(g, k0[t * N:(t + 1) * N], t))
        assert np.array_equal(ring_frame_v(Vb, t), v0[t * N:(t + 1) * N])
    k1 = synth.frame(g, 2, 1, 21, synth.K + synth.CLEAN)
    v1 = synth.frame(g, 2, 1, 21, synth.V + synth.CLEAN)
    print("roll frame 21", flush=True)
    cache.roll(up(k1), up(v1), 21)
    assert (cache.first, cache.count) == (1, 21)
    torch.cuda.synchronize()
    K2, V2 = down(cache.k), down(cache.v)
    assert np.array_equal(ring_frame_k(K2, 0), _spec(g, k1, 21))
    assert np.array_equal(ring_frame_v(V2, 0), v1)
    assert np.array_equal(K2[1:], Kb[1:]) and np.array_equal(V2[1:], Vb[1:])


def test_roll_largest_ring_bit_exact():
    """Full geometry, the largest ring the library accepts (448 slots): 16 frames 440..455
    rolled into an empty ring land in slots 440..447 and 0..7, bit-exact against the RoPE
    specification (keys) and the blocked values; a slot between them stays untouched."""
    g = synth.FULL
    N = g.tokens_per_frame
    capacity, t0, n = 448, 440, 16
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, capacity)
    k = synth.frames(g, 3, 0, t0, n, synth.K)
    v = synth.frames(g, 3, 0, t0, n, synth.V)
    print("roll 16 frames into slots 440..447, 0..7 of a 448-slot ring", flush=True)
    cache.roll(up(k), up(v), t0)
    assert (cache.first, cache.count) == (t0, n)
    torch.cuda.synchronize()
    for f in (0, 7, 8, 15):  # slots 440, 447 (the ring's last bytes), 0, 7
        slot = (t0 + f) % capacity
        kb = down(cache.k[slot:slot + 1])
        vb = down(cache.v[slot:slot + 1])
        assert np.array_equal(ring_frame_k(kb, 0), _spec(g, k[f * N:(f + 1) * N], t0 + f)), slot
        assert np.array_equal(ring_frame_v(vb, 0), v[f * N:(f + 1) * N]), slot
    assert not cache.k[100].any() and not cache.v[100].any()
    del cache
    torch.cuda.empty_cache()


def test_roll_of_a_whole_largest_ring():
    """The largest roll: 448 frames (the whole largest accepted ring, 4.3 GB of K and V) in
    one call into an empty ring, starting at frame 900 (slot 4, so it wraps); sampled
    frames bit-exact, among them those in the ring's last and first slots."""
    g = synth.FULL
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    capacity, t0 = 448, 900
    ctx = _ctx(g, max_frame=2048)
    cache = rf.KVCache(ctx, capacity)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    k = torch.randn((capacity * N, H, D), generator=gen, device="cuda", dtype=torch.bfloat16)
    v = torch.randn((capacity * N, H, D), generator=gen, device="cuda", dtype=torch.bfloat16)
    print("roll 448 frames into a 448-slot ring", flush=True)
    cache.roll(k, v, t0)
    assert (cache.first, cache.count) == (t0, capacity)
    torch.cuda.synchronize()
    for f in (0, capacity - 1 - t0 % capacity, capacity - t0 % capacity, 200, capacity - 1):
        slot = (t0 + f) % capacity
        kf, vf = down(k[f * N:(f + 1) * N]), down(v[f * N:(f + 1) * N])
        assert np.array_equal(ring_frame_k(down(cache.k[slot:slot + 1]), 0), _spec(g, kf, t0 + f)), slot
        assert np.array_equal(ring_frame_v(down(cache.v[slot:slot + 1]), 0), vf), slot
    del cache, k, v
    torch.cuda.empty_cache()


def test_rope3d_longest_block_in_place():
    """rf_rope3d_apply on the most tokens the device index math allows (2^24 - 1: 51.5 GB,
    10,755 frames), in place; sampled tokens -- the first and last, frame edges far into
    the block, random ones -- bit-exact against the specification at their own
    positions."""
    g = synth.FULL
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    n, t0 = (1 << 24) - 1, 3
    ctx = _ctx(g, max_frame=16384)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8)
    x = torch.randn((n, H, D), generator=gen, device="cuda", dtype=torch.bfloat16)
    rng = np.random.default_rng(8)
    rows = {0, 1, N - 1, N, n - 2, n - 1}
    for f in rng.integers(1, n // N, 12):
        rows.update({int(f) * N - 1, int(f) * N})
    rows.update(int(r) for r in rng.integers(0, n, 32))
    rows = np.array(sorted(rows))
    idx = torch.from_numpy(rows).cuda()
    before = x.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
    print(f"rope3d in place on {n} tokens", flush=True)
    ctx.rope3d_apply(x, t0, y=x)
    torch.cuda.synchronize()
    after = x.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
    for j, i in enumerate(rows):
        frame = np.zeros((N, H, D), np.uint16)  # the sampled token at its place in its frame
        frame[i % N] = before[j]
        want = _spec(g, frame, t0 + int(i) // N)[i % N]
        assert np.array_equal(after[j], want), int(i)
    del x
    torch.cuda.empty_cache()


def test_roll_strided_inputs_and_errors():
    g = synth.TINY
    W, N, H, D = g.window, g.tokens_per_frame, g.n_heads, g.head_dim
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, W)
    k = synth.frames(g, 3, 0, 10, 2, synth.K)
    v = synth.frames(g, 3, 0, 10, 2, synth.V)
    qkv = torch.zeros((2 * N, 3, H, D), dtype=torch.bfloat16, device="cuda")
    qkv[:, 1] = up(k)
    qkv[:, 2] = up(v)
    cache.roll(qkv[:, 1], qkv[:, 2], 10)  # empty ring starts at frame 10
    assert cache.window() == [10, 11]
    torch.cuda.synchronize()
    Kb, Vb = down(cache.k), down(cache.v)
    assert np.array_equal(ring_frame_k(Kb, 10 % W), _spec(g, k[:N], 10))
    assert np.array_equal(ring_frame_v(Vb, 11 % W), v[N:])
    # a gap (t0 past first+count) and too many frames are rejected; descriptor unchanged
    for t0, frames in ((13, 1), (9, 1), (10, W + 1)):
        kk = up(synth.frames(g, 3, 0, 0, frames, synth.K))
        with pytest.raises(rf.RfError):
            cache.roll(kk, kk, t0)
        assert cache.window() == [10, 11]


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 19_169_280 // 2])
def test_device_copy_bit_exact(nbytes):
    """The bandwidth probe copies exactly (sizes below, at and above whole work-groups)."""
    src = torch.randint(-32768, 32767, (nbytes // 2,), dtype=torch.int16, device="cuda")
    dst = torch.zeros_like(src)
    rf.device_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
