"""bf16 precision model of the window attention (oracle package; TEST INFRASTRUCTURE ONLY).

Not the definition of the result: that is ``attention.window_attention``, exact
float64.  This model evaluates the same attention with the roundings that an
implementation keeping bf16 operands for its matrix products makes, and nothing
else (every other step in float64):

* the rotated query, multiplied by c = float32(scale * log2(e)), is rounded to
  bf16 once, so that the scores come out in log2 units; the rotation uses the
  float32 cos/sin of the tables (``rope3d.pair_cos_sin(f32=True)``) with the
  products and the sum in float64, as ``rope3d.rope_spec_bits`` does;
* the rotated key is the bf16 value the cache holds, ``rope3d.rope_spec_bits``;
* the softmax weights 2^(s - m) (m the row maximum) are rounded to bf16 before
  the value product, and the row sum adds those bf16 weights;
* the output is rounded to bf16 (nearest even).

The pages fix no precision ("A kernel-centric path to real-time video
generation on Trainium" and its digests give none); bf16 operands with float32
accumulation is the reading taken here.  What the model is for: its error
against the exact oracle is what these operand roundings alone cost on given
rows, so no bf16 implementation of this reading can be expected to do better.
At large softmax scales that cost grows with the logits and reaches the
absolute tolerance by itself, which is the evidence for where that tolerance
stops being a test of the kernel.  With ``rounding=False`` every rounding is
switched off and the model is the exact oracle again (its pin).
"""

import numpy as np

from . import bf16, rope3d

LOG2E = 1.4426950408889634


def _rotate_f32_tables(x, t0, grid_h, grid_w, pairs, base, tok0=0):
    """float64 rotation of float64 x [L, H, D] with the float32-rounded cos/sin."""
    C, S = rope3d.pair_cos_sin(t0, x.shape[0], grid_h, grid_w, pairs, base, f32=True, tok0=tok0)
    C, S = C[:, None, :], S[:, None, :]
    x0, x1 = x[:, :, 0::2], x[:, :, 1::2]
    y = np.empty_like(x)
    y[:, :, 0::2] = x0 * C - x1 * S
    y[:, :, 1::2] = x0 * S + x1 * C
    return y


def attend_rows(q_bits, q_t0, k_bits, v_bits, ctx_t0, grid_h, grid_w, pairs, base,
                scale=None, rows=None, rounding=True, q_tok0=0):
    """Attention of the selected query rows over the context, with the bf16 roundings.

    q_bits: [Lq, H, D] bf16 bits of raw queries, the first being token q_tok0 of frame
    q_t0; k_bits, v_bits: [Lk, H, D] bf16 bits of the raw keys and the values of the
    context frames ctx_t0, ...; rows: query indices (default all).  Returns float64
    [len(rows), H, D].
    """
    q = bf16.bits_to_f64(q_bits)
    D = q.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    v = bf16.bits_to_f64(v_bits)
    if rounding:
        c = float(np.float32(np.float32(scale) * np.float32(LOG2E)))
        qs = bf16.round_f64(_rotate_f32_tables(q, q_t0, grid_h, grid_w, pairs, base, q_tok0)[rows] * c)
        kh = bf16.bits_to_f64(rope3d.rope_spec_bits(k_bits, ctx_t0, grid_h, grid_w, pairs, base))
    else:
        c = scale * LOG2E
        qs = rope3d.rope_exact(q, q_t0, grid_h, grid_w, pairs, base, tok0=q_tok0)[rows] * c
        kh = rope3d.rope_exact(bf16.bits_to_f64(k_bits), ctx_t0, grid_h, grid_w, pairs, base)
    out = np.empty((len(rows), q.shape[1], D))
    for h in range(q.shape[1]):
        s = qs[:, h, :] @ kh[:, h, :].T            # log2 units
        p = np.exp2(s - s.max(axis=1, keepdims=True))
        if rounding:
            p = bf16.round_f64(p)
        o = (p @ v[:, h, :]) / p.sum(axis=1, keepdims=True)
        out[:, h, :] = bf16.round_f64(o) if rounding else o
    return out
