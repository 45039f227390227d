"""GPU parity of rf_qkv_project (the QKV projection fused with the cache write) against
oracle.qkv / oracle.rope3d.

* Identity weight blocks (W = [-I; I; 2I]) make q = -x, k = x and v = 2x exact in
  float32, so the ring must hold bit for bit what a roll of (x, 2x) writes and q must
  be -x: this pins every index of the epilogue (token, head, dimension, slot, frame
  position of the rotation) independently of any rounding.
* Random weights: q, v and the rotated keys equal the oracle's bf16 values except
  where the device's float32 sum and the float64 sum round to different neighbours;
  there they differ by at most one bf16 step plus the worst-case float32 summation
  error E = (C - 1) 2^-24 sum_c |x_c w_c| (oracle test
  test_float32_accumulation_is_within_one_bf16_step checks this bound on a model).
* Full size (16 frames, 24,960 tokens: the last token tile is half full) on sampled
  tokens, into a ring whose slots wrap; an odd head count (feature tiles of 256 + 128);
  argument errors.
"""
import numpy as np
import pytest
import torch

import rolling_window_attention_amd as rf
from rolling_window_attention_amd import synth
from oracle import bf16 as obf
from oracle import qkv as oqkv
from oracle import rope3d as orope

from gpu_util import down, f64, ring_frame_k, ring_frame_v, up

pytestmark = pytest.mark.gpu


def _ctx(g):
    return rf.Context(g.grid_h, g.grid_w, g.n_heads, g.head_dim, g.pairs, g.base, 4096)


def _bits(a):
    return obf.f64_to_bits(np.asarray(a, dtype=np.float64))


def _identity_weight(g):
    c = g.n_heads * g.head_dim
    eye = np.eye(c)
    return _bits(np.vstack([-eye, eye, 2 * eye]))


def _acc_bound(x_bits, w_bits, H, D):
    """Worst-case float32 summation error of each output: (C - 1) 2^-24 sum |x_c w_c|,
    split into q, k, v [rows, H, D]."""
    C = H * D
    e = (C - 1) * 2.0 ** -24 * (np.abs(f64(x_bits)) @ np.abs(f64(w_bits)).T)
    return tuple(e[:, i * C:(i + 1) * C].reshape(-1, H, D) for i in range(3))


def _near(got, want, what, err, min_exact=0.99):
    """bf16 bits: equal almost everywhere, elsewhere within one bf16 step of want plus the
    float32 summation bound err."""
    eq = got == want
    gf, wf = f64(got), f64(want)
    step = np.abs(wf) * 2.0 ** -7 * 1.01 + 1.02 * err
    bad = ~eq & (np.abs(gf - wf) > step)
    print(f"{what}: exact {eq.mean():.5f}, beyond one step {bad.sum()}", flush=True)
    assert eq.mean() >= min_exact, what
    assert not bad.any(), what


def _near_rotated(got, want, k_ref, what, err, min_exact=0.99):
    """Rotated keys: a pair differs when either stored key element rounded differently
    (by at most one step plus err each, as for q and v); the rotation adds the two
    elements' errors, and the result is rounded once more."""
    eq = got == want
    gf, wf = f64(got), f64(want)
    kf = f64(k_ref)
    e = np.abs(kf) * 2.0 ** -7 * 1.01 + 1.02 * err
    pair = np.repeat(e[..., 0::2] + e[..., 1::2], 2, axis=-1)
    bad = ~eq & (np.abs(gf - wf) > pair + np.abs(wf) * 2.0 ** -7 * 1.01)
    print(f"{what}: exact {eq.mean():.5f}, beyond tolerance {bad.sum()}", flush=True)
    assert eq.mean() >= min_exact, what
    assert not bad.any(), what


def _project(g, cache, x_bits, w_bits, t0):
    M = x_bits.shape[0]
    q = torch.empty((M, g.n_heads, g.head_dim), dtype=torch.bfloat16, device="cuda")
    cache.project(up(x_bits), up(w_bits), q, t0)
    torch.cuda.synchronize()
    return down(q)


@pytest.mark.parametrize("geom,calls", [
    (synth.TINY, [(3, 3), (5, 3)]),
    (synth.Geometry(grid_h=4, grid_w=6, n_heads=3, window=4), [(3, 3), (5, 3)]),
    # 16x16 grid, 10 frames per call: 10 token tiles of 256, i.e. one full group of 8
    # token tiles in the kernel's tile order and a partial group of 2 (every tile checked)
    (synth.Geometry(grid_h=16, grid_w=16, n_heads=3, window=12), [(0, 10), (8, 10)]),
    # 5 and 6 heads (reductions of 10 and 12 steps of 64) on 384-token frames: some
    # 256-token tiles lie inside one frame, others straddle two; 7.5 token tiles (the
    # last half full) and, with 5 heads, a last feature tile of 128 features
    (synth.Geometry(grid_h=16, grid_w=24, n_heads=5, window=8), [(0, 5), (4, 5)]),
    (synth.Geometry(grid_h=16, grid_w=24, n_heads=6, window=8), [(0, 5), (4, 5)])])
def test_identity_blocks_match_the_roll_bit_exact(geom, calls):
    """Project frames, then more that overwrite some and wrap the ring (evicting); ring and
    q must equal what rolling (x, 2x) writes and -x."""
    g = geom
    N, H, D, W = g.tokens_per_frame, g.n_heads, g.head_dim, g.window
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, W)
    ref = rf.KVCache(ctx, W)
    w = _identity_weight(g)
    for step, (t0, n) in enumerate(calls):
        print(f"identity blocks H={H}: frames {t0}..{t0 + n - 1}", flush=True)
        x = synth.layer_input(g, 11, step, t0, n)
        q = _project(g, cache, x, w, t0)
        xv = x.reshape(-1, H, D)
        ref.roll(up(xv), up(_bits(2 * f64(xv))), t0)
        torch.cuda.synchronize()
        assert (cache.first, cache.count) == (ref.first, ref.count)
        assert np.array_equal(q, _bits(-f64(xv))), "q != -x"
        assert np.array_equal(down(cache.k), down(ref.k)), "K ring differs from the roll's"
        assert np.array_equal(down(cache.v), down(ref.v)), "V ring differs from the roll's"


def _equal_but_zero_sign(a, b):
    """bf16 tensors equal bit for bit, except that -0 (bits 0x8000) counts as +0."""
    def canon(t):
        bits = t.view(torch.int16)
        return torch.where(bits == -32768, torch.zeros_like(bits), bits)
    return torch.equal(canon(a), canon(b))


def test_identity_blocks_into_the_largest_ring_bit_exact():
    """Full geometry, the largest ring the library accepts (448 slots, 2.15 GB per K or V
    ring): 16 frames 440..455 projected into slots 440..447 and 0..7 of an empty ring.
    With identity weight blocks both rings must equal, bit for bit, those a roll of
    (x, 2x) writes, and q must be -x (compared on the device).  The 38 M inputs hold a
    few exact zeros; there the device's sum of one signed-zero product and exact +0
    products is +0 (IEEE round to nearest), where -x or 2x keep the zero's sign, so +0
    and -0 count as equal."""
    g = synth.FULL
    H, D = g.n_heads, g.head_dim
    capacity, t0, n = 448, 440, 16
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, capacity)
    ref = rf.KVCache(ctx, capacity)
    x = synth.layer_input(g, 14, 0, t0, n)
    xd = up(x)
    q = torch.empty((x.shape[0], H, D), dtype=torch.bfloat16, device="cuda")
    print("identity blocks, 448-slot ring: frames 440..455", flush=True)
    cache.project(xd, up(_identity_weight(g)), q, t0)
    xv = xd.view(-1, H, D)
    ref.roll(xv, (2 * xv.float()).to(torch.bfloat16), t0)
    torch.cuda.synchronize()
    assert (cache.first, cache.count) == (ref.first, ref.count) == (t0, n)
    assert _equal_but_zero_sign(q, -xv), "q != -x"
    assert _equal_but_zero_sign(cache.k, ref.k), "K ring differs from the roll's"
    assert _equal_but_zero_sign(cache.v, ref.v), "V ring differs from the roll's"
    del cache, ref
    torch.cuda.empty_cache()


def test_identity_projection_of_a_whole_largest_ring():
    """The largest projection call: 448 frames (698,880 tokens, 2,730 token tiles) filling
    an empty 448-slot ring from frame 900 (slot 4, so it wraps), identity weight blocks;
    both rings and q against a roll of (x, 2x) and -x, on the device, +0 and -0 equal."""
    g = synth.FULL
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    capacity, t0 = 448, 900
    ctx = rf.Context(g.grid_h, g.grid_w, H, D, g.pairs, g.base, 2048)
    cache = rf.KVCache(ctx, capacity)
    ref = rf.KVCache(ctx, capacity)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(15)
    xd = torch.randn((capacity * N, H * D), generator=gen, device="cuda", dtype=torch.bfloat16)
    q = torch.empty((capacity * N, H, D), dtype=torch.bfloat16, device="cuda")
    print("identity blocks, 448 frames into a 448-slot ring", flush=True)
    cache.project(xd, up(_identity_weight(g)), q, t0)
    xv = xd.view(-1, H, D)
    ref.roll(xv, (2 * xv.float()).to(torch.bfloat16), t0)
    torch.cuda.synchronize()
    assert (cache.first, cache.count) == (ref.first, ref.count) == (t0, capacity)
    assert _equal_but_zero_sign(q, -xv), "q != -x"
    assert _equal_but_zero_sign(cache.k, ref.k), "K ring differs from the roll's"
    assert _equal_but_zero_sign(cache.v, ref.v), "V ring differs from the roll's"
    del cache, ref, xd, q
    torch.cuda.empty_cache()


@pytest.mark.parametrize("geom", [synth.TINY, synth.Geometry(grid_h=4, grid_w=6, n_heads=3, window=4)])
def test_random_weights_tiny(geom):
    g = geom
    N, H, D, W = g.tokens_per_frame, g.n_heads, g.head_dim, g.window
    t0, n = 2, 3
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, W)
    x = synth.layer_input(g, 12, 0, t0, n)
    w = synth.qkv_weight(g, 12)
    print(f"random weights H={H}: {n} frames from {t0}", flush=True)
    q = _project(g, cache, x, w, t0)
    qr, kr, vr = oqkv.project_bits(x, w, H, D)
    eq_, ek, ev = _acc_bound(x, w, H, D)
    krot = orope.rope_spec_bits(kr, t0, g.grid_h, g.grid_w, g.pairs, g.base)
    _near(q, qr, "q", eq_)
    Kb, Vb = down(cache.k), down(cache.v)
    for f in range(n):
        slot = (t0 + f) % W
        sl = slice(f * N, (f + 1) * N)
        _near_rotated(ring_frame_k(Kb, slot), krot[sl], kr[sl], f"K frame {t0 + f}", ek[sl])
        _near(ring_frame_v(Vb, slot), vr[sl], f"V frame {t0 + f}", ev[sl])


def test_full_size_sampled_tokens():
    """16 frames (24,960 tokens, the last token tile half full) appended to a ring that
    holds frames 0..20 (evicts 5..; slots wrap); sampled tokens of every frame against
    the oracle, untouched slots unchanged."""
    g = synth.FULL
    N, H, D, W = g.tokens_per_frame, g.n_heads, g.head_dim, g.window
    ctx = _ctx(g)
    cache = rf.KVCache(ctx, W)
    k0 = synth.frames(g, 13, 0, 0, W, synth.K)
    v0 = synth.frames(g, 13, 0, 0, W, synth.V)
    cache.roll(up(k0), up(v0), 0)
    torch.cuda.synchronize()
    before_k, before_v = down(cache.k), down(cache.v)
    t0, n = 12, 16  # frames 12..27: 12..20 overwritten in place, 21..27 evict 0..6
    x = synth.layer_input(g, 13, 1, t0, n)
    w = synth.qkv_weight(g, 13)
    print("full size: 16 frames", flush=True)
    q = _project(g, cache, x, w, t0)
    assert (cache.first, cache.count) == (7, 21)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([
        rng.integers(0, n * N, 400),
        [0, 255, 256, 1559, 1560, n * N - 129, n * N - 128, n * N - 1],  # tile / frame edges
    ]))
    qr, kr, vr = oqkv.project_bits(x[rows], w, H, D)
    eq_, ek, ev = _acc_bound(x[rows], w, H, D)
    _near(q[rows], qr, "q sampled", eq_)
    Kb, Vb = down(cache.k), down(cache.v)
    f_of = rows // N
    n_of = rows % N
    slots = (t0 + f_of) % W
    got_k = Kb[slots, :, n_of, :]           # [rows, H, D]
    got_v = Vb[slots, :, n_of // 8, :, n_of % 8]  # [rows, H, D] (8-token blocks)
    krot = _rotate_rows(g, kr, t0, rows)
    _near_rotated(got_k, krot, kr, "K sampled", ek)
    _near(got_v, vr, "V sampled", ev)
    # slots of frames 7..11 (7 % 21 .. 11 % 21) were not written
    for t in range(7, 12):
        s = t % W
        assert np.array_equal(Kb[s], before_k[s]) and np.array_equal(Vb[s], before_v[s]), t


def _rotate_rows(g, k_bits, t0, rows):
    """rope_spec_bits of the sampled tokens (rows of frames t0..) at their own positions:
    each frame is rotated whole, zeros where no token was sampled."""
    N = g.tokens_per_frame
    out = np.empty_like(k_bits)
    f_of, n_of = rows // N, rows % N
    for f in np.unique(f_of):
        sel = f_of == f
        blk = np.zeros((N,) + k_bits.shape[1:], np.uint16)
        blk[n_of[sel]] = k_bits[sel]
        out[sel] = orope.rope_spec_bits(blk, t0 + int(f), g.grid_h, g.grid_w, g.pairs, g.base)[n_of[sel]]
    return out


def test_projection_errors():
    g = synth.TINY
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    C = H * D
    ctx = rf.Context(g.grid_h, g.grid_w, H, D, g.pairs, g.base, max_frame=10)
    cache = rf.KVCache(ctx, g.window)
    x = torch.zeros((2 * N, C), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((3 * C, C), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((2 * N, H, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        cache.project(x, w[:C], q, 0)          # weight with C rows instead of 3C
    with pytest.raises(ValueError):
        cache.project(x[:N + 8], w, q[:N + 8], 0)  # not whole frames
    with pytest.raises(rf.RfError) as e:
        cache.project(x, w, q, 9)              # frames 9..10: beyond max_frame 10
    assert e.value.status == 4
    cache.project(x, w, q, 0)
    with pytest.raises(rf.RfError) as e:
        cache.project(x, w, q, 5)              # leaves a gap after frames 0..1
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert (cache.first, cache.count) == (0, 2)


def test_strided_operands_match_dense_bit_exact():
    """x, w and q with row strides larger than C (views into wider buffers) give the
    same q and ring contents, bit for bit, as dense tensors; 4 frames into an empty
    4-frame ring (n_frames = capacity)."""
    g = synth.Geometry(grid_h=4, grid_w=6, n_heads=3, window=4)
    N, H, D, W = g.tokens_per_frame, g.n_heads, g.head_dim, g.window
    C = H * D
    x = synth.layer_input(g, 15, 0, 0, 4)
    w = synth.qkv_weight(g, 15)
    ctx = _ctx(g)
    dense, strided = rf.KVCache(ctx, W), rf.KVCache(ctx, W)
    q_dense = torch.empty((4 * N, H, D), dtype=torch.bfloat16, device="cuda")
    dense.project(up(x), up(w), q_dense, 0)
    xw = torch.zeros((4 * N, C + 72), dtype=torch.bfloat16, device="cuda")
    xw[:, :C] = up(x)
    ww = torch.zeros((3 * C, C + 40), dtype=torch.bfloat16, device="cuda")
    ww[:, :C] = up(w)
    qw = torch.zeros((4 * N, C + 24), dtype=torch.bfloat16, device="cuda")
    strided.project(xw[:, :C], ww[:, :C], qw[:, :C], 0)
    torch.cuda.synchronize()
    assert (strided.first, strided.count) == (dense.first, dense.count) == (0, 4)
    assert np.array_equal(down(qw[:, :C]), down(q_dense).reshape(4 * N, C))
    assert not down(qw[:, C:]).any(), "the padding of q was written"
    assert np.array_equal(down(strided.k), down(dense.k))
    assert np.array_equal(down(strided.v), down(dense.v))
