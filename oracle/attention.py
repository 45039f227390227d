"""Non-causal softmax attention over the window's context frames (oracle, float64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: the DiT self-attention in which the current block of query tokens
(23,400 = 15 frames of 1,560) attends to 32,760 context tokens (21 frames)
across 12 heads, said to take about 70% of compute time ("A kernel-centric
path to real-time video generation on Trainium", ai4snews digest, second
paragraph; "Optimizing Real-Time Video Generation on Trainium Chips",
section 4 "Rolling Forcing advantages").  The pages do not write the formula
out; the plain reading is multi-head scaled dot-product attention with 3D
RoPE applied to queries and keys, every query seeing every context key:

  q^_i = RoPE(q_i, pos(i)),  k^_j = RoPE(k_j, pos(j))
  s_ij = scale * <q^_i, k^_j>,        scale = 1/sqrt(D) unless given
  o_i  = sum_j exp(s_ij - m_i) v_j / sum_j exp(s_ij - m_i),  m_i = max_j s_ij

per head, everything in float64.  Keys are the tokens of the context frames
``ctx_t0 .. ctx_t0+F-1`` in frame-major, row-major order; the result does not
depend on that order (the softmax is over a set).

Rows are processed in blocks only to bound memory; each output row is
computed by the formula above on its own.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import rope3d


def softmax_rows(s):
    """Row-wise softmax of a float64 matrix, max-subtracted."""
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return p / p.sum(axis=1, keepdims=True)


def attend_head(qh, kh, vh, scale):
    """One head: qh [Lq, D], kh [Lk, D], vh [Lk, D] (already rotated) -> [Lq, D]:
    the softmax weights of each row's scores, times the values."""
    return softmax_rows((qh @ kh.T) * scale) @ vh


def window_attention(q, q_t0, k, v, ctx_t0, grid_h, grid_w, pairs, base,
                     scale=None, rows=None, block=256, workers=None, q_tok0=0):
    """Attention of query tokens over context tokens, float64.

    q      : [Lq, H, D] raw (un-rotated) queries of frames q_t0, q_t0+1, ...,
             the first being token q_tok0 of frame q_t0 (a block cut out of a
             frame sequence at any token; 0 = whole frames)
    k, v   : [Lk, H, D] raw keys / values of the context frames ctx_t0, ...
             (Lk a whole number of frames)
    rows   : optional 1-D array of query-token indices to compute (sampling);
             positions still come from each row's own index.
    Returns [len(rows) or Lq, H, D] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L, H, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    qh_all = rope3d.rope_exact(q, q_t0, grid_h, grid_w, pairs, base, tok0=q_tok0)
    if rows is not None:
        qh_all = qh_all[np.asarray(rows, dtype=np.int64)]
    kh_all = rope3d.rope_exact(k, ctx_t0, grid_h, grid_w, pairs, base)
    nq = qh_all.shape[0]
    out = np.empty((nq, H, D), dtype=np.float64)

    jobs = [(h, r0) for h in range(H) for r0 in range(0, nq, block)]

    def run(job):
        h, r0 = job
        r1 = min(r0 + block, nq)
        out[r0:r1, h, :] = attend_head(qh_all[r0:r1, h, :], kh_all[:, h, :],
                                       v[:, h, :], scale)

    if workers is None:
        workers = max(1, len(os.sched_getaffinity(0)))
    if workers == 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(run, jobs))
    return out
