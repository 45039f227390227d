"""Planted mistakes in the oracle (CPU only).

Each mutant below is one plausible slip in one oracle function -- a wrong sign,
index, axis order or exponent, a dropped or extra step, a transposed layout, a
wrong rounding -- patched in with ``monkeypatch`` for the duration of one test.
The oracle's own pins (the ``test_oracle_*`` modules, run here as plain
functions) must then fail: at least one of them raises.  Before that, the same
pins are run unpatched and must all pass, so a pin that fails for reasons of its
own cannot make a mutant look caught.  The mistakes are planted in the oracle
only, on the CPU; nothing here touches the device library.
"""
import types

import numpy as np
import pytest

from oracle import attention, bf16, precision, qkv, ring, rope3d

import test_oracle_attention as pins_attention
import test_oracle_bf16 as pins_bf16
import test_oracle_precision as pins_precision
import test_oracle_qkv as pins_qkv
import test_oracle_ring as pins_ring
import test_oracle_rope as pins_rope

# the 14-second pin of the precision model runs last, and only where it is needed
_SLOW = {"test_bf16_operands_alone_exceed_the_tolerance_at_scale_one_quarter"}


def _pin_calls(module):
    """(name, function, kwargs) of every pin in a test module, parametrized ones expanded,
    in source order."""
    calls = []
    fns = [getattr(module, n) for n in dir(module) if n.startswith("test_")]
    fns.sort(key=lambda f: f.__code__.co_firstlineno)
    for fn in fns:
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            calls.append((fn.__name__, fn, {}))
            continue
        argnames, values = marks[0].args[0], marks[0].args[1]
        names = [a.strip() for a in argnames.split(",")] if isinstance(argnames, str) else list(argnames)
        for v in values:
            vals = tuple(v) if len(names) > 1 else (v,)
            calls.append((f"{fn.__name__}{list(vals)}", fn, dict(zip(names, vals))))
    slow = [c for c in calls if c[1].__name__ in _SLOW]
    return [c for c in calls if c[1].__name__ not in _SLOW] + slow


def _first_failing_pin(modules):
    """Run the pins of `modules` in order; the name of the first that raises, else None."""
    for module in modules:
        for name, fn, kwargs in _pin_calls(module):
            try:
                with np.errstate(all="ignore"):
                    fn(**kwargs)
            except Exception:  # an assertion, or an error the mistake provokes
                return f"{module.__name__}::{name}"
    return None


# ---- mutants ------------------------------------------------------------------------
# Each takes pytest's monkeypatch and plants one mistake.  The docstring says what a
# slip in the oracle would look like.

def _rope_rotate(x, C, S, half_split=False):
    x0, x1 = (x[..., :x.shape[-1] // 2], x[..., x.shape[-1] // 2:]) if half_split else (x[..., 0::2], x[..., 1::2])
    y0, y1 = x0 * C - x1 * S, x0 * S + x1 * C
    y = np.empty_like(x)
    if half_split:
        y[..., :x.shape[-1] // 2], y[..., x.shape[-1] // 2:] = y0, y1
    else:
        y[..., 0::2], y[..., 1::2] = y0, y1
    return y


def rope_row_and_column_swapped(mp):
    """Row and column of a token exchanged (column-major inside a frame)."""
    real = rope3d.token_positions

    def f(t0, n_tokens, grid_h, grid_w, tok0=0):
        t, r, c = real(t0, n_tokens, grid_h, grid_w, tok0)
        i = (tok0 + np.arange(n_tokens)) % (grid_h * grid_w)
        return t, i % grid_h, i // grid_h
    mp.setattr(rope3d, "token_positions", f)


def rope_frame_index_relative_to_block(mp):
    """Time position counted from the block's first frame instead of the absolute index."""
    real = rope3d.token_positions

    def f(t0, n_tokens, grid_h, grid_w, tok0=0):
        t, r, c = real(t0, n_tokens, grid_h, grid_w, tok0)
        return t - t0, r, c
    mp.setattr(rope3d, "token_positions", f)


def rope_token_offset_ignored(mp):
    """A block cut inside a frame treated as if it started at the frame's first token."""
    real = rope3d.token_positions
    mp.setattr(rope3d, "token_positions", lambda t0, n, gh, gw, tok0=0: real(t0, n, gh, gw, 0))


def rope_exponent_two_j(mp):
    """Frequencies base^(-2j/P) (the 2j/d habit of 1-D RoPE carried into each axis)."""
    mp.setattr(rope3d, "axis_frequencies", lambda P, base: [base ** (-(2.0 * j / P)) for j in range(P)])


def rope_one_frequency_ladder(mp):
    """One ladder base^(-j/64) for every axis instead of base^(-j/P) per axis."""
    mp.setattr(rope3d, "axis_frequencies", lambda P, base: [base ** (-(j / 64.0)) for j in range(P)])


def rope_clockwise(mp):
    """Rotation by -angle (the sine's sign flipped)."""
    real = rope3d.angle_table

    def f(positions, n_pairs, base, f32=False):
        C, S = real(positions, n_pairs, base, f32)
        return C, -S
    mp.setattr(rope3d, "angle_table", f)


def rope_axes_t_w_h(mp):
    """Pair blocks in the order time, width, height."""
    def f(t0, n_tokens, grid_h, grid_w, pairs, base, f32=False, tok0=0):
        t, r, c = rope3d.token_positions(t0, n_tokens, grid_h, grid_w, tok0)
        Ct, St = rope3d.angle_table(t, pairs[0], base, f32)
        Cw, Sw = rope3d.angle_table(c, pairs[1], base, f32)
        Ch, Sh = rope3d.angle_table(r, pairs[2], base, f32)
        return np.concatenate([Ct, Cw, Ch], axis=1), np.concatenate([St, Sw, Sh], axis=1)
    mp.setattr(rope3d, "pair_cos_sin", f)


def rope_half_split_pairs(mp):
    """Pairs (p, p + D/2) (the rotate-half layout) instead of interleaved (2p, 2p+1)."""
    def exact(x, t0, grid_h, grid_w, pairs, base, tok0=0):
        x = np.asarray(x, dtype=np.float64)
        C, S = rope3d.pair_cos_sin(t0, x.shape[0], grid_h, grid_w, pairs, base, tok0=tok0)
        return _rope_rotate(x, C[:, None, :], S[:, None, :], half_split=True)

    def spec(x_bits, t0, grid_h, grid_w, pairs, base):
        x = bf16.bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
        C, S = rope3d.pair_cos_sin(t0, x.shape[0], grid_h, grid_w, pairs, base, f32=True)
        return bf16.f64_to_bits(_rope_rotate(x, C[:, None, :], S[:, None, :], half_split=True))
    mp.setattr(rope3d, "rope_exact", exact)
    mp.setattr(rope3d, "rope_spec_bits", spec)


def rope_spec_with_float64_tables(mp):
    """The bit-exact specification computed with float64 cos/sin (the float32 rounding of
    the device tables left out)."""
    real = rope3d.angle_table
    mp.setattr(rope3d, "angle_table", lambda positions, n_pairs, base, f32=False: real(positions, n_pairs, base, False))


def attention_scale_dropped(mp):
    """Scores not multiplied by the scale."""
    mp.setattr(attention, "attend_head", lambda qh, kh, vh, scale: attention.softmax_rows(qh @ kh.T) @ vh)


def attention_softmax_over_queries(mp):
    """Softmax normalised over the query axis instead of the key axis."""
    def f(s):
        p = np.exp(s - s.max(axis=0, keepdims=True))
        return p / p.sum(axis=0, keepdims=True)
    mp.setattr(attention, "softmax_rows", f)


def attention_weights_not_normalised(mp):
    """exp(s - m) used as weights without dividing by their sum."""
    mp.setattr(attention, "softmax_rows", lambda s: np.exp(s - s.max(axis=1, keepdims=True)))


def attention_keys_not_rotated(mp):
    """RoPE applied to the queries only."""
    calls = {"n": 0}

    def f(x, *args, **kwargs):
        calls["n"] += 1  # window_attention rotates the queries first, then the keys
        return rope3d.rope_exact(x, *args, **kwargs) if calls["n"] % 2 == 1 else np.asarray(x, np.float64)
    mp.setattr(attention, "rope3d", types.SimpleNamespace(rope_exact=f))


def attention_query_token_offset_ignored(mp):
    """Queries of a block cut inside a frame rotated as if it started at the frame's start."""
    def f(x, *args, tok0=0, **kwargs):
        return rope3d.rope_exact(x, *args, **kwargs)
    mp.setattr(attention, "rope3d", types.SimpleNamespace(rope_exact=f))


def ring_slot_off_by_one(mp):
    """Frame t stored in slot (t + 1) mod W."""
    mp.setattr(ring.RingModel, "slot", lambda self, t: (t + 1) % self.capacity)


def ring_evicts_newest(mp):
    """A full ring drops its newest frame instead of its oldest."""
    def roll(self, t0, n, data=None):
        self.check_roll(t0, n)
        if self.count == 0:
            self.first = t0
        evicted = []
        for i in range(n):
            t = t0 + i
            if t >= self.first + self.count:
                if self.count == self.capacity:
                    evicted.append(self.first + self.count - 1)
                    self.first += 1
                else:
                    self.count += 1
            s = self.slot(t)
            self.slot_frame[s], self.slot_data[s] = t, None if data is None else data[i]
        return evicted
    mp.setattr(ring.RingModel, "roll", roll)


def ring_overwrite_counted_as_append(mp):
    """A frame already in the window counted again (the window grows or evicts on it)."""
    def roll(self, t0, n, data=None):
        self.check_roll(t0, n)
        if self.count == 0:
            self.first = t0
        evicted = []
        for i in range(n):
            t = t0 + i
            if self.count == self.capacity:
                evicted.append(self.first)
                self.first += 1
            else:
                self.count += 1
            s = self.slot(t)
            self.slot_frame[s], self.slot_data[s] = t, None if data is None else data[i]
        return evicted
    mp.setattr(ring.RingModel, "roll", roll)


def qkv_k_and_v_swapped(mp):
    """The weight's k and v row blocks read in the wrong order."""
    real = qkv._split

    def f(y, n_heads, head_dim):
        q, k, v = real(y, n_heads, head_dim)
        return q, v, k
    mp.setattr(qkv, "_split", f)


def qkv_features_dimension_major(mp):
    """Feature d * H + h taken as dimension d of head h (dimension-major instead of
    head-major)."""
    def f(y, n_heads, head_dim):
        c = n_heads * head_dim
        shape = (y.shape[0], head_dim, n_heads)
        return tuple(y[:, i * c:(i + 1) * c].reshape(shape).transpose(0, 2, 1) for i in range(3))
    mp.setattr(qkv, "_split", f)


def qkv_key_rotated_before_rounding(mp):
    """The cached key rotated from the float64 projection instead of the stored bf16 key."""
    def f(x_bits, w_bits, t0, grid_h, grid_w, pairs, base):
        n_heads = np.asarray(w_bits).shape[1] // (2 * sum(pairs))
        head_dim = 2 * sum(pairs)
        q, k, v = qkv.project(x_bits, w_bits, n_heads, head_dim)
        kr = rope3d.rope_exact(k, t0, grid_h, grid_w, pairs, base)
        return bf16.f64_to_bits(q), bf16.f64_to_bits(kr), bf16.f64_to_bits(v)
    mp.setattr(qkv, "cache_entries", f)


class _NumpyWith(types.ModuleType):
    """numpy with some functions replaced (for a mutant of a module that calls np.*)."""

    def __init__(self, **replaced):
        super().__init__("numpy_with_replacements")
        self.__dict__.update(replaced)

    def __getattr__(self, name):
        return getattr(np, name)


def bf16_ties_away_from_zero(mp):
    """Halfway cases rounded away from zero instead of to even."""
    mp.setattr(bf16, "np", _NumpyWith(rint=lambda a: np.floor(np.asarray(a) + 0.5)))


def bf16_truncation(mp):
    """Conversion to bf16 by dropping the low bits (truncation toward zero)."""
    def f(x):
        u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32)
        return (u >> np.uint32(16)).astype(np.uint16)
    mp.setattr(bf16, "f64_to_bits", f)


def bf16_double_rounding(mp):
    """float64 -> float32 -> bf16 (two roundings) instead of one direct rounding."""
    real = bf16.f64_to_bits
    mp.setattr(bf16, "f64_to_bits", lambda x: real(np.asarray(x, dtype=np.float64).astype(np.float32)))


def bf16_no_overflow_to_infinity(mp):
    """Values that round past the largest bf16 clamped to it instead of becoming inf."""
    real = bf16.round_f64

    def f(x):
        r = real(x)
        fin = np.isfinite(np.asarray(x, dtype=np.float64))
        return np.where(fin & np.isinf(r), np.copysign(bf16.BF16_MAX, r), r)
    mp.setattr(bf16, "round_f64", f)


def precision_weights_left_unrounded(mp):
    """The bf16 model's softmax weights kept in float64 (one of its roundings dropped)."""
    real = bf16.round_f64
    calls = {"n": 0}

    def f(x):
        x = np.asarray(x, dtype=np.float64)
        if x.ndim == 3:  # the scaled queries, rounded once per call before the head loop
            calls["n"] = 0
            return real(x)
        calls["n"] += 1  # then per head: the weights, then the output
        return x if calls["n"] % 2 == 1 else real(x)
    mp.setattr(precision, "bf16", types.SimpleNamespace(round_f64=f, bits_to_f64=bf16.bits_to_f64))


def precision_query_scale_after_rounding(mp):
    """The query rounded to bf16 before it is multiplied by the scale."""
    real_rotate = precision._rotate_f32_tables

    def f(x, *args, **kwargs):
        return bf16.round_f64(real_rotate(x, *args, **kwargs))
    mp.setattr(precision, "_rotate_f32_tables", f)


MUTANTS = [
    (rope_row_and_column_swapped, [pins_rope]),
    (rope_frame_index_relative_to_block, [pins_rope]),
    (rope_token_offset_ignored, [pins_rope]),
    (rope_exponent_two_j, [pins_rope]),
    (rope_one_frequency_ladder, [pins_rope]),
    (rope_clockwise, [pins_rope]),
    (rope_axes_t_w_h, [pins_rope]),
    (rope_half_split_pairs, [pins_rope]),
    (rope_spec_with_float64_tables, [pins_rope]),
    (attention_scale_dropped, [pins_attention]),
    (attention_softmax_over_queries, [pins_attention]),
    (attention_weights_not_normalised, [pins_attention]),
    (attention_keys_not_rotated, [pins_attention]),
    (attention_query_token_offset_ignored, [pins_attention]),
    (ring_slot_off_by_one, [pins_ring]),
    (ring_evicts_newest, [pins_ring]),
    (ring_overwrite_counted_as_append, [pins_ring]),
    (qkv_k_and_v_swapped, [pins_qkv]),
    (qkv_features_dimension_major, [pins_qkv]),
    (qkv_key_rotated_before_rounding, [pins_qkv]),
    (bf16_ties_away_from_zero, [pins_bf16]),
    (bf16_truncation, [pins_bf16]),
    (bf16_double_rounding, [pins_bf16]),
    (bf16_no_overflow_to_infinity, [pins_bf16]),
    (precision_weights_left_unrounded, [pins_precision]),
    (precision_query_scale_after_rounding, [pins_precision]),
]


def test_every_pin_passes_unpatched():
    """The baseline: with nothing planted, no pin of any module fails."""
    assert _first_failing_pin([pins_rope, pins_attention, pins_ring, pins_qkv, pins_bf16,
                               pins_precision]) is None


@pytest.mark.parametrize("mutant,modules", MUTANTS, ids=[m.__name__ for m, _ in MUTANTS])
def test_planted_mistake_is_caught(mutant, modules, monkeypatch):
    mutant(monkeypatch)
    caught = _first_failing_pin(modules)
    print(f"{mutant.__name__}: caught by {caught}")
    assert caught is not None, f"no pin catches: {mutant.__doc__}"
