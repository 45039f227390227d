"""The path end to end on the GPU: layer inputs projected into the ring and the queries
(rf_qkv_project), then one batched attention launch (rf_window_attention) over the
ring, against the oracle's composition of the same steps (oracle.qkv, then
oracle.attention on the projected bf16 q, k, v), within the attention tolerance.

Tiny grid, 5-frame window: frames 0..4 are projected as a prefill; step s = 3 then
projects frames 2..5 (the clean re-encode of frame 2 and the noisy frames 3..5, which
appends frame 5 and evicts frame 0) and attends with the denoise segment (queries of
frames 3..5) and the cache-update segment (queries of frame 2) over frames 1..5.
"""
import numpy as np
import pytest
import torch

import rolling_window_attention_amd as rf
from rolling_window_attention_amd import synth
from oracle import attention as oatt
from oracle import qkv as oqkv

from gpu_util import assert_close, down, f64, up

pytestmark = pytest.mark.gpu


def test_projection_then_attention_matches_the_oracle():
    g = synth.TINY
    N, H, D, W = g.tokens_per_frame, g.n_heads, g.head_dim, g.window
    ctx = rf.Context(g.grid_h, g.grid_w, H, D, g.pairs, g.base, 4096)
    cache = rf.KVCache(ctx, W)
    w = synth.qkv_weight(g, 51)
    x_pre = synth.layer_input(g, 51, 0, 0, W)       # frames 0..4
    x_step = synth.layer_input(g, 51, 1, 2, 4)      # frames 2..5 (step 3)
    q_pre = torch.empty((W * N, H, D), dtype=torch.bfloat16, device="cuda")
    q_step = torch.empty((4 * N, H, D), dtype=torch.bfloat16, device="cuda")
    print("project prefill 0..4, then step 3: frames 2..5", flush=True)
    cache.project(up(x_pre), up(w), q_pre, 0)
    cache.project(up(x_step), up(w), q_step, 2)
    assert (cache.first, cache.count) == (1, 5)
    oa = torch.empty((3 * N, H, D), dtype=torch.bfloat16, device="cuda")
    ob = torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda")
    rf.window_attention(ctx, cache, [rf.Segment(q_step[N:], 3, oa, 1, 5), rf.Segment(q_step[:N], 2, ob, 1, 5)])
    torch.cuda.synchronize()

    # oracle: what the ring holds for frames 1..5 and the step's queries
    _, k_pre, v_pre = oqkv.project_bits(x_pre, w, H, D)
    q_s, k_s, v_s = oqkv.project_bits(x_step, w, H, D)
    k_ctx = np.concatenate([k_pre[N:2 * N], k_s])   # frame 1 from the prefill, 2..5 from the step
    v_ctx = np.concatenate([v_pre[N:2 * N], v_s])
    want_a = oatt.window_attention(f64(q_s[N:]), 3, f64(k_ctx), f64(v_ctx), 1, g.grid_h, g.grid_w, g.pairs, g.base)
    want_b = oatt.window_attention(f64(q_s[:N]), 2, f64(k_ctx), f64(v_ctx), 1, g.grid_h, g.grid_w, g.pairs, g.base)
    assert_close(f64(down(oa)), want_a, "denoise segment")
    assert_close(f64(down(ob)), want_b, "cache-update segment")
