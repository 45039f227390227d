"""Helpers for the GPU parity tests: moving bf16 bit patterns to and from the device,
building the oracle's expectation for ring contents and attention rows."""
import numpy as np
import torch

from oracle import attention as oatt
from oracle import bf16 as obf
from oracle import rope3d as orope

TOL_MAX_ABS = 2e-2
TOL_MEAN_ABS = 2e-3
TOL_REL_L2 = 1e-2


def dev():
    return torch.device("cuda:0")


def up(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def down(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits):
    return obf.bits_to_f64(bits)


def ring_frame_k(cache_k_bits, slot):
    """Ring K slot [H, N, D] -> token-major [N, H, D]."""
    return cache_k_bits[slot].transpose(1, 0, 2)


def ring_frame_v(cache_v_bits, slot):
    """Ring V slot [H, N/8, D, 8] (8-token blocks) -> token-major [N, H, D]."""
    H, G, D, _ = cache_v_bits[slot].shape
    return cache_v_bits[slot].transpose(1, 3, 0, 2).reshape(G * 8, H, D)


def ring_slot_v(v_bits):
    """Token-major [N, H, D] -> a ring V slot [H, N/8, D, 8]."""
    N, H, D = v_bits.shape
    return v_bits.reshape(N // 8, 8, H, D).transpose(2, 0, 3, 1)


def errors(got, want):
    d = np.abs(got - want)
    rel = np.linalg.norm((got - want).ravel()) / max(np.linalg.norm(want.ravel()), 1e-300)
    return d.max(), d.mean(), rel


def assert_close(got, want, what=""):
    mx, mean, rel = errors(got, want)
    print(f"{what}: max_abs={mx:.3e} mean_abs={mean:.3e} rel_l2={rel:.3e}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert mx <= TOL_MAX_ABS, (what, mx)
    assert mean <= TOL_MEAN_ABS, (what, mean)
    assert rel <= TOL_REL_L2, (what, rel)


class RotatedKeys:
    """The oracle's exact float64 rotation of each context frame's raw keys, cached per
    (frame, content key) so that multi-step tests rotate each frame once."""

    def __init__(self, geom):
        self.g = geom
        self.cache = {}

    def get(self, t, tag, k_bits):
        key = (t, tag)
        if key not in self.cache:
            g = self.g
            self.cache[key] = orope.rope_exact(f64(k_bits), t, g.grid_h, g.grid_w, g.pairs, g.base)
        return self.cache[key]

    def prune(self, min_t):
        """Forget frames older than min_t."""
        for key in [k for k in self.cache if k[0] < min_t]:
            del self.cache[key]


def oracle_rows(geom, q_bits, q_t0, kh_frames, v_frames, rows, scale=None, q_tok0=0):
    """Oracle attention for selected query rows, from pre-rotated context keys.

    kh_frames: list of float64 [N, H, D] rotated keys (oracle rope_exact) of the context
    frames in order; v_frames: list of bf16 bit arrays [N, H, D]; q_bits' first token is
    token q_tok0 of frame q_t0."""
    g = geom
    kh = np.concatenate(kh_frames, axis=0)
    v = np.concatenate([f64(x) for x in v_frames], axis=0)
    qh = orope.rope_exact(f64(q_bits), q_t0, g.grid_h, g.grid_w, g.pairs, g.base, tok0=q_tok0)[rows]
    D = q_bits.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((len(rows), q_bits.shape[1], D))
    for h in range(q_bits.shape[1]):
        out[:, h, :] = oatt.attend_head(qh[:, h, :], kh[:, h, :], v[:, h, :], scale)
    return out


def sample_rows(n_tokens, N, block_m=256, extra=64, seed=0):
    """Rows that cover frame edges, query-tile edges (block_m rows), the 32-row wave edges
    of the first and the last (ragged) tile, and random interior rows."""
    rng = np.random.default_rng(seed)
    s = {0, 1, n_tokens - 1, n_tokens - 2}
    for f0 in range(0, n_tokens, N):
        s.update({f0, f0 + N - 1})
    last_tile = (n_tokens - 1) // block_m * block_m
    s.update({last_tile, last_tile - 1})
    for base in (0, last_tile):
        for w in range(0, block_m, 32):
            s.update({base + w, base + w - 1, base + w + 31})
    s.update(int(x) for x in rng.integers(0, n_tokens, extra))
    return np.array(sorted(x for x in s if 0 <= x < n_tokens))
