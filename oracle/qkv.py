"""QKV projection of a self-attention layer feeding the rolling KV cache -- oracle,
float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: the pages describe the layer's self-attention over 12 heads ("A
kernel-centric path to real-time video generation on Trainium", ai4snews
digest, second paragraph; "Optimizing Real-Time Video Generation on Trainium
Chips", section 7 "Hybrid sharding solution") and say that every layer reads
and writes a rolling KV cache and rotates its queries and keys over three axes
("Amazon and Reactor tune Trainium for real-time video generation", section
"Three problems for generic compilers").  They do not print the projection
that produces q, k and v.  The reading taken here is the standard one of
multi-head self-attention:

* the model width is ``C = H * D`` (12 heads of 128: 1,536);
* one weight matrix ``W`` of shape ``[3C, C]`` (the layout of a linear layer:
  output features by input features) holds the q rows, then the k rows, then
  the v rows; inside each block of ``C`` rows, feature ``h * D + d`` is
  dimension ``d`` of head ``h``;
* for the layer input ``x`` of shape ``[L, C]`` (token-major),
  ``y = x W^T``, ``q = y[:, :C]``, ``k = y[:, C:2C]``, ``v = y[:, 2C:]``, each
  viewed as ``[L, H, D]``;
* what the cache receives is what the roll receives: ``k`` and ``v`` stored
  as bf16 (round to nearest even), and the rotated key is the bit-exact bf16
  RoPE of that stored ``k`` (``rope3d.rope_spec_bits``).

Functions:

* ``project`` -- q, k, v in float64 from bf16 inputs: numpy's float64 matrix
  product of the exact input values (the products are exact; the 1,536-term
  sums are rounded in float64 only).
* ``project_bits`` -- the same rounded once to bf16, the reference for a
  device that accumulates in float32 and then rounds: where the float32 sum
  lands on the other side of a bf16 rounding boundary the device value is one
  bf16 step away, so parity is checked as "bit-exact almost everywhere, one
  step elsewhere" (see the tests).
* ``cache_entries`` -- (q, rotated k, v) as bf16 bits: what the fused
  projection writes for queries and into the ring slots.
"""

import numpy as np

from . import bf16, rope3d


def _split(y, n_heads, head_dim):
    c = n_heads * head_dim
    shape = (y.shape[0], n_heads, head_dim)
    return y[:, :c].reshape(shape), y[:, c:2 * c].reshape(shape), y[:, 2 * c:].reshape(shape)


def project(x_bits, w_bits, n_heads, head_dim):
    """q, k, v (float64, [L, H, D] each) of bf16 ``x_bits`` [L, C] and ``w_bits`` [3C, C]."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    c = n_heads * head_dim
    if x_bits.ndim != 2 or x_bits.shape[1] != c:
        raise ValueError("x must be [L, H*D]")
    if w_bits.shape != (3 * c, c):
        raise ValueError("w must be [3*H*D, H*D]")
    y = bf16.bits_to_f64(x_bits) @ bf16.bits_to_f64(w_bits).T
    return _split(y, n_heads, head_dim)


def project_bits(x_bits, w_bits, n_heads, head_dim):
    """q, k, v of ``project`` rounded to bf16 (nearest, ties to even), as uint16 bits."""
    return tuple(bf16.f64_to_bits(a) for a in project(x_bits, w_bits, n_heads, head_dim))


def cache_entries(x_bits, w_bits, t0, grid_h, grid_w, pairs, base):
    """(q bits, rotated k bits, v bits), each [L, H, D], for tokens of frames t0.. .

    The rotated key is RoPE of the stored bf16 key, exactly as the cache roll
    would rotate it."""
    n_heads = np.asarray(w_bits).shape[1] // (2 * sum(pairs))
    head_dim = 2 * sum(pairs)
    q, k, v = project_bits(x_bits, w_bits, n_heads, head_dim)
    return q, rope3d.rope_spec_bits(k, t0, grid_h, grid_w, pairs, base), v
