"""3D rotary position embedding over (time, row, column) -- oracle, float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: the pages say video RoPE acts on three axes -- time, height and
width -- where an LLM uses one position ("Amazon and Reactor tune Trainium
for real-time video generation", section "Three problems for generic
compilers"; "Optimizing Real-Time Video Generation on Trainium Chips",
section 5 "Three core bottlenecks").  They give no formula; the readings
below are the plainest ones the pages support:

* Token ``i`` of a block that starts at absolute latent frame ``t0`` sits at
  ``(t, r, c) = (t0 + i // N, (i % N) // grid_w, i % grid_w)``, ``N =
  grid_h * grid_w`` (frame-major, row-major inside a frame).  ``t`` is the
  absolute frame index, never re-based as the window rolls.  A block may
  start inside its first frame, at token ``tok0`` of it (a sequence split
  cuts frames; positions are per token): then ``i`` is replaced by
  ``tok0 + i`` above.
* The head dimension is split into ``D/2`` rotation pairs ``(2p, 2p+1)``
  (interleaved).  The first ``P_t`` pairs rotate by the time position, the
  next ``P_h`` by the row, the last ``P_w`` by the column.
* Inside an axis with ``P`` pairs, pair ``j`` has frequency
  ``omega_j = base ** (-j / P)``: each axis is an independent 1-D RoPE of
  dimension ``2P``.
* The rotation is counter-clockwise, i.e. the pair ``x_{2p} + i x_{2p+1}``
  is multiplied by ``exp(i * pos * omega)``; queries and keys alike.

Two functions compute the rotation:

* ``rope_exact``  -- the rotation in float64 with float64 cos/sin; used by the
  attention oracle.
* ``rope_spec_bits`` -- the bit-exact definition of a bf16 RoPE output: the
  cos/sin are first rounded to float32 (the precision of the tables the
  device keeps), the products bf16*fp32 are exact in float64, their
  difference is rounded once to float64, and that value is rounded to the
  nearest bf16 (ties to even) directly.  That makes the output of the RoPE
  and cache-roll kernels unique, so they are compared bit for bit.
"""

import math

import numpy as np

from . import bf16


def token_positions(t0, n_tokens, grid_h, grid_w, tok0=0):
    """(t, r, c) int64 arrays for ``n_tokens`` consecutive tokens from token
    ``tok0`` of frame ``t0``."""
    n = grid_h * grid_w
    if not 0 <= tok0 < n:
        raise ValueError("tok0 must lie inside the first frame")
    i = tok0 + np.arange(n_tokens, dtype=np.int64)
    t = t0 + i // n
    r = (i % n) // grid_w
    c = i % grid_w
    return t, r, c


def axis_frequencies(n_pairs, base):
    """omega_j = base ** (-j / P) for j = 0..P-1, float64 (C ``pow``)."""
    return [base ** (-(float(j) / float(n_pairs))) for j in range(n_pairs)]


def angle_table(positions, n_pairs, base, f32=False):
    """cos/sin of ``pos * omega_j`` for each position (rows) and pair j (cols).

    Computed element by element with the C library's ``cos``/``sin`` through
    Python's ``math`` module, in float64.  ``f32=True`` rounds each value to
    float32 (round to nearest even), the precision of the device tables.
    """
    omegas = axis_frequencies(n_pairs, base)
    pos = [int(p) for p in np.unique(np.asarray(positions, dtype=np.int64))]
    cos = {}
    sin = {}
    for p in pos:
        th = [float(p) * w for w in omegas]
        cos[p] = [math.cos(x) for x in th]
        sin[p] = [math.sin(x) for x in th]
    idx = np.asarray(positions, dtype=np.int64)
    C = np.array([cos[int(p)] for p in idx], dtype=np.float64).reshape(len(idx), n_pairs)
    S = np.array([sin[int(p)] for p in idx], dtype=np.float64).reshape(len(idx), n_pairs)
    if f32:
        C = C.astype(np.float32).astype(np.float64)
        S = S.astype(np.float32).astype(np.float64)
    return C, S


def pair_cos_sin(t0, n_tokens, grid_h, grid_w, pairs, base, f32=False, tok0=0):
    """cos, sin of every rotation pair of every token: two [n_tokens, D/2] arrays."""
    t, r, c = token_positions(t0, n_tokens, grid_h, grid_w, tok0)
    Ct, St = angle_table(t, pairs[0], base, f32)
    Ch, Sh = angle_table(r, pairs[1], base, f32)
    Cw, Sw = angle_table(c, pairs[2], base, f32)
    C = np.concatenate([Ct, Ch, Cw], axis=1)
    S = np.concatenate([St, Sh, Sw], axis=1)
    return C, S


def _check(x, pairs):
    if x.ndim != 3:
        raise ValueError("expected [tokens, heads, head_dim]")
    if x.shape[2] != 2 * sum(pairs):
        raise ValueError("head_dim must equal 2 * sum(pairs)")


def rope_exact(x, t0, grid_h, grid_w, pairs, base, tok0=0):
    """Rotate float64 ``x`` [L, H, D] (token-major, first token = token ``tok0`` of
    frame ``t0``) in float64.

    y_{2p}   = x_{2p} cos - x_{2p+1} sin
    y_{2p+1} = x_{2p} sin + x_{2p+1} cos
    """
    x = np.asarray(x, dtype=np.float64)
    _check(x, pairs)
    C, S = pair_cos_sin(t0, x.shape[0], grid_h, grid_w, pairs, base, f32=False, tok0=tok0)
    C = C[:, None, :]
    S = S[:, None, :]
    x0 = x[:, :, 0::2]
    x1 = x[:, :, 1::2]
    y = np.empty_like(x)
    y[:, :, 0::2] = x0 * C - x1 * S
    y[:, :, 1::2] = x0 * S + x1 * C
    return y


def rope_spec_bits(x_bits, t0, grid_h, grid_w, pairs, base):
    """Bit-exact bf16 RoPE of bf16 ``x_bits`` [L, H, D] (uint16), returning uint16.

    With c32, s32 the float32 roundings of cos and sin:
      y_{2p}   = bf16( fl64( x_{2p} * c32 - x_{2p+1} * s32 ) )
      y_{2p+1} = bf16( fl64( x_{2p} * s32 + x_{2p+1} * c32 ) )
    Each product of a bf16 (8 significant bits) and a float32 (24) has at most
    32 significant bits and is exact in float64, so the only roundings are the
    one float64 sum and the final round-to-nearest-even to bf16.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    _check(x_bits, pairs)
    x = bf16.bits_to_f64(x_bits)
    C, S = pair_cos_sin(t0, x.shape[0], grid_h, grid_w, pairs, base, f32=True)
    C = C[:, None, :]
    S = S[:, None, :]
    x0 = x[:, :, 0::2]
    x1 = x[:, :, 1::2]
    y = np.empty_like(x)
    y[:, :, 0::2] = x0 * C - x1 * S
    y[:, :, 1::2] = x0 * S + x1 * C
    return bf16.f64_to_bits(y)
