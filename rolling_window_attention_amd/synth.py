"""Seeded synthetic inputs and workload geometry for tests and the benchmark.

Holds none of the method's arithmetic: it draws N(0,1) float32 samples and
stores them as bf16 (round to nearest even), frame by frame, and describes
the workloads' shapes.  Both the HIP path and the CPU oracle consume exactly
these bf16 bit patterns.

A frame's tensor depends only on (workload id, step, frame index, tensor id),
never on how frames are batched into calls:
``numpy.random.default_rng([cfg, step, t, tensor_id]).standard_normal``.
Tensor ids: 0 = q, 1 = k, 2 = v of the noisy (denoise-pass) frame; 3, 4, 5 the
same of the clean frame that the cache-update pass writes; 6 the layer input x
that the QKV projection maps to q, k, v (its weight comes from ``qkv_weight``).
"""

from dataclasses import dataclass

import numpy as np

Q, K, V = 0, 1, 2
CLEAN = 3


@dataclass(frozen=True)
class Geometry:
    grid_h: int = 30
    grid_w: int = 52
    n_heads: int = 12
    head_dim: int = 128
    pairs: tuple = (22, 21, 21)
    base: float = 10000.0
    window: int = 21

    @property
    def tokens_per_frame(self):
        return self.grid_h * self.grid_w


# Latent grid 30x52 (1,560 tokens per frame), 12 heads of 128, 21-frame ring.
FULL = Geometry()
# The tiny case: 6x8 grid (48 tokens per frame), 5-frame window.
TINY = Geometry(grid_h=6, grid_w=8, window=5)

# One GPU's share of the hybrid heads x sequence split over eight devices: 3 of the 12
# heads (its query half is a token range of the full step's queries).
SHARD = Geometry(n_heads=3)

WORKLOAD_IDS = {"tiny": 1, "cache_update": 2, "denoise": 3, "dynamic": 4, "batched": 5, "shard": 7}


def f32_to_bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def frame(geom, cfg, step, t, tensor_id):
    """One frame's tensor: bf16 bits [N, H, D] drawn from N(0, 1)."""
    rng = np.random.default_rng([int(cfg), int(step), int(t), int(tensor_id)])
    shape = (geom.tokens_per_frame, geom.n_heads, geom.head_dim)
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


# Tensor id of a frame's layer input x (the QKV projection's input), [N, H*D].
LAYER_IN = 6


def layer_input(geom, cfg, step, t0, n):
    """Frames t0..t0+n-1 of the layer input: bf16 bits [n*N, H*D] drawn from N(0, 1)."""
    x = frames(geom, cfg, step, t0, n, LAYER_IN)
    return x.reshape(x.shape[0], geom.n_heads * geom.head_dim)


def qkv_weight(geom, cfg):
    """A projection weight [3C, C] (C = H*D): bf16 bits drawn from N(0, 1/C), so that
    projections of N(0, 1) inputs are again about N(0, 1)."""
    c = geom.n_heads * geom.head_dim
    rng = np.random.default_rng([int(cfg), 1 << 20, 3, c])
    w = rng.standard_normal((3 * c, c), dtype=np.float32) * np.float32(1.0 / np.sqrt(c))
    return f32_to_bf16_bits(w)


def frames(geom, cfg, step, t0, n, tensor_id):
    """Frames t0..t0+n-1 stacked token-major: bf16 bits [n*N, H, D]."""
    return np.concatenate([frame(geom, cfg, step, t, tensor_id) for t in range(t0, t0 + n)],
                          axis=0)
