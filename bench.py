"""Benchmark of the rolling-window attention hot path on one MI355X.

A step is one steady-state window step of the batched two-phase schedule: the
16-frame cache roll (clean frame s-1 plus current frames s..s+14: RoPE'd K and
transposed V into the 21-slot ring), then ONE rf_window_attention launch with the
denoise segment (15 frames = 23,400 queries) and the cache-update segment (1 frame =
1,560 queries), both over the 21-frame window (32,760 keys), 12 heads of 128.
Inputs are seeded N(0,1) bf16 tensors already resident in HBM.

Prints ONE JSON line.  `value` is attention TFLOP/s over the whole step (algorithmic
flops 4*Lq*Lk*H*D of both segments / step time); `roofline` is the attention kernel's
own rate from HIP events on the launch stream against the dense bf16 MFMA peak.
"""
import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s + ms/layer at 23,400q x 32,760kv x 12h; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "window_attn_traffic.json")
KERNEL_SOURCES = ["csrc/window_attn.hip", "csrc/device_common.h", "csrc/kernels.h", "build.py"]


def kernel_source_hash(package_dir=None):
    """Hash of what the attention kernel is made from (its sources and the build script,
    which sets its register split) without comments and blank lines, so a comment edit
    does not invalidate counter figures taken on the same code."""
    import re
    package_dir = package_dir or os.path.join(ROOT, "rolling_window_attention_amd")
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        comment = r"#.*" if name.endswith(".py") else r"//.*"
        with open(os.path.join(package_dir, name)) as f:
            for line in f:
                code = re.sub(comment, "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(flops_per_launch):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


class ClockSampler:
    """Samples the GPU's effective shader clock (MHz) with amdsmi from a host thread while
    the timed loop runs: the firmware metrics' current gfx clock of each XCD, averaged
    over the XCDs (the clock query's `clk` field gives the DPM level, 2,400 MHz, which
    the chip does not hold under this load).  Read-only queries; None if amdsmi is
    unavailable."""

    def __init__(self, period_s=0.002):
        import threading
        self.period = period_s
        self.samples = []
        self.ok = False
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            self._read()
            self.ok = True
        except Exception:  # no amdsmi, no permission, no device: no clock figure
            self.ok = False

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        per_xcd = [v for v in (m.get("current_gfxclks") or []) if isinstance(v, (int, float)) and v > 0]
        if per_xcd:
            return float(np.mean(per_xcd))
        v = m.get("current_gfxclk")
        if isinstance(v, (int, float)) and v > 0:
            return float(v)
        raise RuntimeError("no gfx clock in the metrics")

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception:
                return
            time.sleep(self.period)

    def start(self):
        if self.ok:
            import threading
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self, skip_s=0.0):
        """Stop sampling; summarise the samples taken after the first skip_s seconds."""
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        if self.ok:
            try:
                self._smi.amdsmi_shut_down()
            except Exception:
                pass
        vals = [v for v in self.samples[int(skip_s / self.period):] if isinstance(v, (int, float)) and v > 0]
        if not vals:
            return None
        return {"median": float(np.median(vals)), "min": float(min(vals)), "max": float(max(vals)),
                "samples": len(vals)}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--pool", type=int, default=4, help="distinct pre-generated step inputs")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle run time")
    p.add_argument("--no-clock", action="store_true",
                   help="skip the untimed ~1.5 s phase that samples the shader clock")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the untimed denoise-only and RoPE launches (profiling runs, so "
                        "that every attention dispatch traced is a batched step)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a 1 GiB device copy (for counter calibration runs)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(librfattn has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch

    import rolling_window_attention_amd as rf
    from rolling_window_attention_amd import synth

    g = synth.FULL
    N, H, D, W = g.tokens_per_frame, g.n_heads, g.head_dim, g.window
    cfg = synth.WORKLOAD_IDS["batched"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    ctx = rf.Context(g.grid_h, g.grid_w, H, D, g.pairs, g.base, max_frame=8192)
    cache = rf.KVCache(ctx, W)

    # ---- untimed setup: ring at the state after step 6 (frames 0..20), input pool ----
    # Step s (s >= 7) rolls frames s-1 (clean) .. s+14 (current) and attends over s-6..s+14.
    # The step inputs cycle through a pool of pre-generated, HBM-resident tensors.
    s0 = 7
    written = {}  # frame -> (k bits, v bits) last written there, replayed for the oracle
    for t in range(21):
        st, tid = (t + 1, synth.CLEAN) if t < 6 else (6, 0)
        written[t] = (synth.frame(g, cfg, st, t, synth.K + tid), synth.frame(g, cfg, st, t, synth.V + tid))
    cache.roll(up(np.concatenate([written[t][0] for t in range(21)])),
               up(np.concatenate([written[t][1] for t in range(21)])), 0)
    pool, pool_bits = [], []
    for i in range(args.pool):
        s = s0 + i
        ks = [synth.frame(g, cfg, s, s - 1, synth.K + synth.CLEAN)] + \
             [synth.frame(g, cfg, s, t, synth.K) for t in range(s, s + 15)]
        vs = [synth.frame(g, cfg, s, s - 1, synth.V + synth.CLEAN)] + \
             [synth.frame(g, cfg, s, t, synth.V) for t in range(s, s + 15)]
        qa = np.concatenate([synth.frame(g, cfg, s, t, synth.Q) for t in range(s, s + 15)])
        qb = synth.frame(g, cfg, s, s - 1, synth.Q + synth.CLEAN)
        pool.append(dict(k=up(np.concatenate(ks)), v=up(np.concatenate(vs)), qa=up(qa), qb=up(qb)))
        pool_bits.append((ks, vs, qa, qb))
    oa = torch.empty((15 * N, H, D), dtype=torch.bfloat16, device=dev)
    ob = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    lq = 16 * N
    lk = 21 * N
    flops_step = 4.0 * lq * lk * H * D
    flops_denoise = 4.0 * 15 * N * lk * H * D
    roll_bytes = 16 * N * H * D * 2 * 4  # K and V: 2 B read + 2 B write per element

    step_idx = [s0]

    def run_step(ev=None):
        s = step_idx[0]
        p = pool[(s - s0) % args.pool]
        ks, vs, _, _ = pool_bits[(s - s0) % args.pool]
        for j in range(16):
            written[s - 1 + j] = (ks[j], vs[j])
        if ev:
            ev[0].record(stream)
        cache.roll(p["k"], p["v"], s - 1)
        if ev:
            ev[1].record(stream)
        rf.window_attention(ctx, cache, [rf.Segment(p["qa"], s, oa, s - 6, 21),
                                         rf.Segment(p["qb"], s - 1, ob, s - 6, 21)])
        if ev:
            ev[2].record(stream)
        step_idx[0] += 1

    # Shader clock under this load: the firmware metrics refresh too slowly for the
    # short timed loop, so sample during ~1.5 s of the same steps first (untimed) and
    # keep the samples of the last second.  This runs before the warm-up steps:
    # stopping the sampler idles the GPU for tens of ms, after which the clock needs
    # a few launches to come back up, and the warm-up steps absorb that.
    clock = ClockSampler(period_s=0.005)
    sclk = None
    if clock.ok and not args.no_clock:
        clock.start()
        t_end_clock = time.perf_counter() + 1.5
        while time.perf_counter() < t_end_clock:
            for _ in range(20):
                run_step()
            torch.cuda.synchronize()
        sclk = clock.stop(skip_s=0.5)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        run_step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = t_start.elapsed_time(t_end) / args.steps
    roll_each = np.array([e[0].elapsed_time(e[1]) for e in evs])
    attn_each = np.array([e[1].elapsed_time(e[2]) for e in evs])
    roll_ms = float(np.mean(roll_each))
    attn_ms = float(np.mean(attn_each))
    last_s = step_idx[0] - 1

    def pct(x):
        return {f"p{q}": round(float(np.percentile(x, q)), 4) for q in (10, 50, 90)}

    # ---- extras (not part of the timed steps): denoise-only launch, the cache-update
    # pass alone, standalone RoPE, cold/warm single calls, the 30-step dynamic fill ----
    denoise_ms = rope_ms = update_ms = None
    dynamic = projection = replay = share = rawk = grouped = tiny = fill_replay = None
    cold_warm = {}
    rope_bytes = 15 * N * H * D * 2 * 2
    if not args.no_extras:
        p = pool[(last_s - s0) % args.pool]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        od = torch.empty_like(oa)
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            rf.window_attention(ctx, cache, [rf.Segment(p["qa"], last_s, od, last_s - 6, 21)])
        e1.record(stream)
        torch.cuda.synchronize()
        denoise_ms = e0.elapsed_time(e1) / reps
        qr = torch.empty_like(p["qa"])
        e0.record(stream)
        for _ in range(reps):
            ctx.rope3d_apply(p["qa"], last_s, y=qr)
        e1.record(stream)
        torch.cuda.synchronize()
        rope_ms = e0.elapsed_time(e1) / reps
        # the cache-update segment alone (1,560 query rows): too few query tiles to
        # fill the GPU, so the launch is entirely key-split
        ou = torch.empty_like(ob)
        e0.record(stream)
        for _ in range(reps):
            rf.window_attention(ctx, cache, [rf.Segment(p["qb"], last_s - 1, ou, last_s - 6, 21)])
        e1.record(stream)
        torch.cuda.synchronize()
        update_ms = e0.elapsed_time(e1) / reps
        rawk = keys_rotated_on_load(rf, ctx, cache, written, last_s, p, g, stream)
        dynamic = dynamic_fill(rf, ctx, W, N, H, D, pool, pool_bits, stream)
        grouped = grouped_roll(rf, ctx, g, stream)
        tiny = tiny_window(rf, synth, stream)
        projection = qkv_projection(rf, synth, g, ctx, W, stream)
        share = hybrid_share(rf, synth, W, stream)
        replay = graph_replay(rf, synth, g, W, pool)
        fill_replay = fill_graph_replay(rf, g, W, pool)

        # cold (a 1 GiB fill evicts L2 and the 256 MB MALL before each rep) and warm
        # single-call times of the standalone RoPE and of the step's roll; the roll
        # rewrites the last step's own frames, so the ring contents do not change
        flush = torch.empty(1 << 28, dtype=torch.int32, device=dev)
        p_last = pool[(last_s - s0) % args.pool]
        # the 1-frame roll rewrites the last step's newest frame (s+14) in place
        # plain device copies (rf_device_copy) moving the same bytes as the RoPE of Q and
        # the 16- and 1-frame rolls: the bandwidth one launch of that size reaches at best
        c_src = torch.empty(16 * N * H * D * 2, dtype=torch.bfloat16, device=dev)
        c_dst = torch.empty_like(c_src)
        n_q = 15 * N * H * D
        n_1 = N * H * D * 2
        single = {"rope3d_q": lambda: ctx.rope3d_apply(p["qa"], last_s, y=qr),
                  "roll_16": lambda: cache.roll(p_last["k"], p_last["v"], last_s - 1),
                  "roll_1": lambda: cache.roll(p_last["k"][15 * N:], p_last["v"][15 * N:], last_s + 14),
                  "copy_rope3d_q_bytes": lambda: rf.device_copy(c_dst[:n_q], c_src[:n_q]),
                  "copy_roll_16_bytes": lambda: rf.device_copy(c_dst, c_src),
                  "copy_roll_1_bytes": lambda: rf.device_copy(c_dst[:n_1], c_src[:n_1])}
        # Each timed call is enqueued while the GPU is still busy (behind the flush, or
        # behind torch's bounded spin kernel for the warm call), so the events measure the
        # GPU's time and not the host's launch latency on an idle GPU.
        def busy():
            try:
                torch.cuda._sleep(100000)
            except Exception:
                pass

        cold_warm = {}
        for name, fn in single.items():
            cold, warm = [], []
            for _ in range(reps):
                flush.zero_()
                e0.record(stream); fn(); e1.record(stream); torch.cuda.synchronize()
                cold.append(e0.elapsed_time(e1))
                busy()
                e0.record(stream); fn(); e1.record(stream); torch.cuda.synchronize()
                warm.append(e0.elapsed_time(e1))
            cold_warm[name] = (float(np.median(cold)), float(np.median(warm)))
        del flush, c_src, c_dst

    if args.calibrate_copy:
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    attn_tflops = flops_step / (attn_ms * 1e-3) / 1e12
    value = flops_step / (step_ms * 1e-3) / 1e12
    traffic = measured_traffic(flops_step)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "batched two-phase window step: 16-frame cache roll + one attention launch "
                        "(denoise 23,400q + cache-update 1,560q) over 32,760 kv, 12 heads x 128",
            "q_tokens": [15 * N, N], "kv_tokens": lk, "heads": H, "head_dim": D,
            "grid": f"{g.grid_h}x{g.grid_w}", "window_frames": W, "roll_frames": 16,
            "input_pool": args.pool,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "window_attn_kernel",
            "flops_per_launch": flops_step,
            "ms_per_launch": round(attn_ms, 4),
            # peak scales with the shader clock: 2.5 PFLOP/s is quoted at 2,400 MHz
            "sclk_mhz": sclk,
            "frac_at_sclk": (round(attn_tflops / (PEAK_BF16_TFLOPS * sclk["median"] / 2400.0), 4)
                             if sclk else None),
        },
        "ms_attention": round(attn_ms, 4),
        "ms_roll": round(roll_ms, 4),
        "per_launch_ms": {"attention": pct(attn_each), "roll": pct(roll_each)},
        "roll_GBps": round(roll_bytes / (roll_ms * 1e-3) / 1e9, 1),
        "roll_hbm_frac": round(roll_bytes / (roll_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "wall_s_timed": round(wall, 3),
    }
    if denoise_ms is not None:
        out["denoise_only"] = {
            "q_tokens": 15 * N, "kv_tokens": lk, "ms": round(denoise_ms, 4),
            "TFLOP/s": round(flops_denoise / (denoise_ms * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(flops_denoise / (denoise_ms * 1e-3) / 1e12
                                    / PEAK_BF16_TFLOPS, 4)}
        out["rope3d_q"] = {
            "tokens": 15 * N, "ms": round(rope_ms, 4),
            "GB/s": round(rope_bytes / (rope_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(rope_bytes / (rope_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        nbytes = {"rope3d_q": rope_bytes, "roll_16": roll_bytes, "roll_1": roll_bytes // 16,
                  "copy_rope3d_q_bytes": rope_bytes, "copy_roll_16_bytes": roll_bytes,
                  "copy_roll_1_bytes": roll_bytes // 16}
        out["cold_warm"] = {
            name: {"bytes": nbytes[name], "cold_ms": round(c, 4), "warm_ms": round(w, 4),
                   "cold_hbm_frac": round(nbytes[name] / (c * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                   "warm_hbm_frac": round(nbytes[name] / (w * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            for name, (c, w) in cold_warm.items()}
        for name in ("rope3d_q", "roll_16", "roll_1"):  # time of the same bytes copied / kernel time
            cc, cw = cold_warm["copy_" + name + "_bytes"]
            kc, kw = cold_warm[name]
            out["cold_warm"][name]["cold_frac_of_copy"] = round(cc / kc, 4)
            out["cold_warm"][name]["warm_frac_of_copy"] = round(cw / kw, 4)

    if update_ms is not None:
        flops_update = 4.0 * N * lk * H * D
        out["cache_update_only"] = {
            "q_tokens": N, "kv_tokens": lk, "ms": round(update_ms, 4),
            "TFLOP/s": round(flops_update / (update_ms * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(flops_update / (update_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    if dynamic is not None:
        out["dynamic_30_steps"] = dynamic
    if projection is not None:
        out["qkv_projection_16"] = projection
    if share is not None:
        out["hybrid_share_3_heads"] = share
    if replay is not None:
        out["graph_replay_30_steps"] = replay
    if fill_replay is not None:
        out["fill_graph_replay_30_steps"] = fill_replay
    if rawk is not None:
        out["keys_rotated_on_load"] = rawk
    if grouped is not None:
        out["grouped_roll_30_layers"] = grouped

    if not args.no_cpu_baseline:
        ctx_frames = [written[t] for t in range(last_s - 6, last_s + 15)]
        _, _, qa_bits, qb_bits = pool_bits[(last_s - s0) % args.pool]
        out["cpu_baseline"] = cpu_baseline(args, g, last_s, ctx_frames, qa_bits, oa, qb_bits, ob)
        if tiny is not None:
            out["cpu_baseline"]["tiny_window"] = oracle_tiny(g_tiny=synth.TINY, tiny=tiny)
        if dynamic is not None:
            out["cpu_baseline"]["dynamic_steps"] = oracle_dynamic_steps(g, dynamic.pop("_keep"))
    if dynamic is not None:
        dynamic.pop("_keep", None)

    print(json.dumps(out), flush=True)


DYNAMIC_ORACLE_STEPS = (0, 6, 7, 29)


def dynamic_fill(rf, ctx, W, N, H, D, pool, pool_bits, stream):
    """The 30-step dynamic fill from an empty ring: step s rolls frames max(s-1, 0) ..
    s+14 (the clean re-encode of frame s-1 rewrites its slot) and runs the denoise
    segment (query frames s..s+14) over the min(s, 6) + 15 frames s-min(s,6) .. s+14:
    15, 16, .. 21 context frames, then 21 with one eviction per step.  Inputs cycle
    through the step pool (synthetic; parity of this loop is a GPU test).  Timed as one
    stretch of 30 steps after one untimed pass, which also keeps the outputs and context
    frames of steps 0, 6, 7 and 29 for the oracle's timing."""
    import torch

    o = torch.empty((15 * N, H, D), dtype=torch.bfloat16, device=pool[0]["qa"].device)
    keep = {}

    def run(cache, record=False):
        written = {}
        for s in range(30):
            i = s % len(pool)
            p = pool[i]
            ks, vs, qa_bits, _ = pool_bits[i]
            first = 0 if s == 0 else s - 1
            j0 = 1 if s == 0 else 0
            if s == 0:
                cache.roll(p["k"][N:], p["v"][N:], 0)
            else:
                cache.roll(p["k"], p["v"], s - 1)
            for j in range(j0, 16):
                written[first + j - j0] = (ks[j], vs[j])
            c = min(s, 6)
            rf.window_attention(ctx, cache, [rf.Segment(p["qa"], s, o, s - c, c + 15)])
            if record and s in DYNAMIC_ORACLE_STEPS:
                keep[s] = dict(out=o.view(torch.int16).cpu().numpy().view(np.uint16), q=qa_bits,
                               ctx=[written[t] for t in range(s - c, s + 15)], ctx_t0=s - c)

    run(rf.KVCache(ctx, W), record=True)
    cache = rf.KVCache(ctx, W)  # an empty ring again, allocated before the timed stretch
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run(cache)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    flops = sum(4.0 * 15 * N * (min(s, 6) + 15) * N * H * D for s in range(30))
    res = {"steps": 30, "context_frames": [min(s, 6) + 15 for s in range(30)],
           "ms_total": round(ms, 3), "ms_per_step": round(ms / 30, 4),
           "TFLOP": round(flops / 1e12, 2), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
           "_keep": keep}
    return res


def keys_rotated_on_load(rf, ctx, cache, written, s, p, g, stream, reps=10):
    """Ablation of rotating keys once when they enter the ring: rf_window_attention_rawk
    keeps the same window's keys un-rotated and rotates every key tile as it is staged
    (once per query tile that reads it), on the batched step's two segments; next to
    the shipped launch on the rotated ring, same queries, same window."""
    import torch

    N, H, D, W = g.tokens_per_frame, g.n_heads, g.head_dim, g.window
    dev = torch.device("cuda:0")
    raw = rf.KVCache(ctx, W)
    raw.desc.first, raw.desc.count = cache.first, cache.count
    raw.v.copy_(cache.v)
    for t in range(s - 6, s + 15):  # raw keys head-major (torch permute: setup, untimed)
        kb = torch.from_numpy(np.ascontiguousarray(written[t][0]).view(np.int16)).to(dev)
        raw.k[t % W] = kb.view(torch.bfloat16).view(N, H, D).permute(1, 0, 2)
    oa = torch.empty_like(p["qa"])
    ob = torch.empty_like(p["qb"])
    res = {}
    for name, fn, c in (("rotated_once_in_ring_ms", rf.window_attention, cache),
                        ("rotated_per_tile_on_load_ms", rf.window_attention_rawk, raw)):
        segs = [rf.Segment(p["qa"], s, oa, s - 6, 21), rf.Segment(p["qb"], s - 1, ob, s - 6, 21)]
        fn(ctx, c, segs)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn(ctx, c, segs)
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) / reps, 4)
    res["slowdown"] = round(res["rotated_per_tile_on_load_ms"] / res["rotated_once_in_ring_ms"], 4)
    del raw
    return res


def grouped_roll(rf, ctx, g, stream, layers=30, reps=10):
    """The 1-frame roll (cache update: one clean frame into each layer's ring, evicting
    the oldest) for `layers` layers: ONE rf_kvcache_roll_layers launch against `layers`
    separate rf_kvcache_roll launches, cold (a 1 GiB fill evicts L2 and the MALL before
    each rep) and warm.  Algorithmic bytes: 2 B read + 2 B written per K and V element.
    Synthetic inputs; the rings start full (frames 0..20) and every rep rolls frame 21
    again (an overwrite in place after the first)."""
    import torch

    N, H, D, W = g.tokens_per_frame, g.n_heads, g.head_dim, g.window
    dev = torch.device("cuda:0")
    caches = [rf.KVCache(ctx, W) for _ in range(layers)]
    for c in caches:
        c.desc.first, c.desc.count = 0, W
    rings = rf.DeviceRings(caches)
    torch.manual_seed(3)
    k = torch.randn((layers, N, H, D), device=dev).to(torch.bfloat16)
    v = torch.randn((layers, N, H, D), device=dev).to(torch.bfloat16)
    flush = torch.empty(1 << 28, dtype=torch.int32, device=dev)
    nbytes = layers * N * H * D * 2 * 4
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def separate():
        for l, c in enumerate(caches):
            c.roll(k[l], v[l], 21)

    def busy():
        try:
            torch.cuda._sleep(100000)
        except Exception:
            pass

    c_src = torch.empty(nbytes // 4, dtype=torch.int16, device=dev)  # bytes/2 copied = bytes moved
    c_dst = torch.empty_like(c_src)
    res = {"layers": layers, "frames": 1, "bytes": nbytes}
    for name, fn in (("grouped", lambda: rings.roll(k, v, 21)), ("separate", separate),
                     ("copy_same_bytes", lambda: rf.device_copy(c_dst, c_src))):
        fn()
        cold, warm = [], []
        for _ in range(reps):
            flush.zero_()
            e0.record(stream); fn(); e1.record(stream); torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
            busy()
            e0.record(stream); fn(); e1.record(stream); torch.cuda.synchronize()
            warm.append(e0.elapsed_time(e1))
        c_ms, w_ms = float(np.median(cold)), float(np.median(warm))
        res[name] = {"cold_ms": round(c_ms, 4), "warm_ms": round(w_ms, 4),
                     "cold_hbm_frac": round(nbytes / (c_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "warm_hbm_frac": round(nbytes / (w_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    for name in ("grouped", "separate"):
        res[name]["cold_frac_of_copy"] = round(res["copy_same_bytes"]["cold_ms"] / res[name]["cold_ms"], 4)
        res[name]["warm_frac_of_copy"] = round(res["copy_same_bytes"]["warm_ms"] / res[name]["warm_ms"], 4)
    del flush, caches, rings, c_src, c_dst
    return res


def tiny_window(rf, synth, stream):
    """The tiny configuration: 6x8 grid (48 tokens per frame), 12 heads of 128, a 5-slot
    ring; frames 0-1 rolled in first, then frames 2-4 rolled and attended by query frames
    2-4 (144 queries) over frames 0-4 (240 keys).  Returns the GPU output and inputs for
    the oracle's timing and parity."""
    import torch

    g = synth.TINY
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    dev = torch.device("cuda:0")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    cfg = synth.WORKLOAD_IDS["tiny"]
    k = synth.frames(g, cfg, 0, 0, 5, synth.K)
    v = synth.frames(g, cfg, 0, 0, 5, synth.V)
    q = synth.frames(g, cfg, 0, 2, 3, synth.Q)
    ctx = rf.Context(g.grid_h, g.grid_w, H, D, g.pairs, g.base, 64)
    cache = rf.KVCache(ctx, g.window)
    cache.roll(up(k[:2 * N]), up(v[:2 * N]), 0)
    o = torch.empty((3 * N, H, D), dtype=torch.bfloat16, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    cache.roll(up(k[2 * N:]), up(v[2 * N:]), 2)
    rf.window_attention(ctx, cache, [rf.Segment(up(q), 2, o, 0, 5)])
    e1.record(stream)
    torch.cuda.synchronize()
    return dict(k=k, v=v, q=q, out=o.view(torch.int16).cpu().numpy().view(np.uint16),
                gpu_ms=e0.elapsed_time(e1))


def _parity(got_bits, want):
    from oracle import bf16 as obf
    got = obf.bits_to_f64(got_bits)
    d = np.abs(got - want)
    return {"max_abs": float(d.max()), "mean_abs": float(d.mean()),
            "rel_l2": float(np.linalg.norm((got - want).ravel()) / np.linalg.norm(want.ravel()))}


def oracle_tiny(g_tiny, tiny):
    """The oracle on the whole tiny configuration (144 queries x 240 keys x 12 heads)."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as oatt
    from oracle import bf16 as obf
    g = g_tiny
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    t0 = time.perf_counter()
    with threadpool_limits(limits=1, user_api="blas"):
        want = oatt.window_attention(obf.bits_to_f64(tiny["q"]), 2, obf.bits_to_f64(tiny["k"]),
                                     obf.bits_to_f64(tiny["v"]), 0, g.grid_h, g.grid_w, g.pairs, g.base,
                                     workers=1)
    secs = time.perf_counter() - t0
    flops = 4.0 * 3 * N * 5 * N * H * D
    return {"queries": 3 * N, "keys": 5 * N, "seconds": round(secs, 4), "cores": 1,
            "TFLOP/s": round(flops / secs / 1e12, 6), "gpu_ms_roll_and_attention": round(tiny["gpu_ms"], 4),
            "parity": _parity(tiny["out"], want)}


def oracle_dynamic_steps(g, keep):
    """The oracle on whole steps of the 30-step fill (all 23,400 queries x 12 heads over
    15, 21, 21 and 21 context frames at steps 0, 6, 7, 29), with parity against the GPU
    output of the same step."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as oatt
    from oracle import bf16 as obf
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    workers = max(1, len(os.sched_getaffinity(0)))
    res = {}
    for s, kp in sorted(keep.items()):
        k = obf.bits_to_f64(np.concatenate([f[0] for f in kp["ctx"]]))
        v = obf.bits_to_f64(np.concatenate([f[1] for f in kp["ctx"]]))
        t0 = time.perf_counter()
        with threadpool_limits(limits=1, user_api="blas"):
            want = oatt.window_attention(obf.bits_to_f64(kp["q"]), s, k, v, kp["ctx_t0"], g.grid_h, g.grid_w,
                                         g.pairs, g.base, block=64, workers=workers)
        secs = time.perf_counter() - t0
        flops = 4.0 * 15 * N * len(kp["ctx"]) * N * H * D
        res[str(s)] = {"context_frames": len(kp["ctx"]), "seconds": round(secs, 2), "cores": workers,
                       "TFLOP/s": round(flops / secs / 1e12, 6), "parity": _parity(kp["out"], want)}
    return res


def qkv_projection(rf, synth, g, ctx, W, stream, reps=10):
    """rf_qkv_project of the step's 16 frames (24,960 tokens x 1,536 -> 4,608 features):
    q token-major, rotated keys and transposed values into a 21-frame ring.  Synthetic
    layer input and N(0, 1/C) weights.  For context, the time of torch's library GEMM of
    the same shape alone (no epilogue, no cache write) is reported next to it."""
    import torch

    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    C = H * D
    dev = torch.device("cuda:0")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    x = up(synth.layer_input(g, 14, 0, 0, 16))
    w = up(synth.qkv_weight(g, 14))
    q = torch.empty((16 * N, H, D), dtype=torch.bfloat16, device=dev)
    cache = rf.KVCache(ctx, W)
    cache.project(x, w, q, 0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        cache.project(x, w, q, 0)  # rewrites frames 0..15 in place
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    y = x @ w.t()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        y = x @ w.t()
    e1.record(stream)
    torch.cuda.synchronize()
    lib_ms = e0.elapsed_time(e1) / reps
    flops = 2.0 * 16 * N * 3 * C * C
    del y, cache
    return {"tokens": 16 * N, "in_features": C, "out_features": 3 * C, "ms": round(ms, 4),
            "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "library_gemm_only_ms": round(lib_ms, 4)}


def hybrid_share(rf, synth, W, stream, reps=10):
    """One device's share of the heads x sequence split over eight devices: 3 of the 12
    heads and the second half of a batched step's queries -- denoise tokens 11,700..23,399
    (from token 780 of the step's eighth frame) and cache-update tokens 780..1,559 -- in
    one launch over 21 context frames (32,760 keys).  Synthetic 3-head ring and queries."""
    import torch

    g = synth.SHARD
    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    cfg = synth.WORKLOAD_IDS["shard"]
    dev = torch.device("cuda:0")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    ctx = rf.Context(g.grid_h, g.grid_w, H, D, g.pairs, g.base, 4096)
    cache = rf.KVCache(ctx, W)
    s = 9
    cache.roll(up(synth.frames(g, cfg, s, s - 6, W, synth.K)),
               up(synth.frames(g, cfg, s, s - 6, W, synth.V)), s - 6)
    half = N // 2
    qa = up(synth.frames(g, cfg, s, s + 7, 8, synth.Q)[half:])   # 11,700 tokens
    qb = up(synth.frame(g, cfg, s, s - 1, synth.Q + synth.CLEAN)[half:])
    oa, ob = torch.empty_like(qa), torch.empty_like(qb)
    segs = [rf.Segment(qa, s + 7, oa, s - 6, W, q_tok0=half),
            rf.Segment(qb, s - 1, ob, s - 6, W, q_tok0=half)]
    for _ in range(2):
        rf.window_attention(ctx, cache, segs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        rf.window_attention(ctx, cache, segs)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nq = qa.shape[0] + qb.shape[0]
    flops = 4.0 * nq * W * N * H * D
    del cache, ctx
    return {"heads": H, "q_tokens": [qa.shape[0], qb.shape[0]], "kv_tokens": W * N, "ms": round(ms, 4),
            "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
            "frac_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def graph_replay(rf, synth, g, W, pool, steps=30):
    """The batched window step run eagerly for 30 steps, then captured once (with the
    device frame shift and its increment) and replayed for the next 30 steps, on a
    context of its own.  GPU time per step (events around each stretch) and host time
    to enqueue a step (the Python loop without the final synchronisation)."""
    import torch

    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    dev = torch.device("cuda:0")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    ctx = rf.Context(g.grid_h, g.grid_w, H, D, g.pairs, g.base, max_frame=8192)
    cache = rf.KVCache(ctx, W)
    cfg = synth.WORKLOAD_IDS["batched"]
    cache.roll(up(synth.frames(g, cfg, 0, 0, W, synth.K + synth.CLEAN)),
               up(synth.frames(g, cfg, 0, 0, W, synth.V + synth.CLEAN)), 0)
    p = pool[0]
    oa = torch.empty((15 * N, H, D), dtype=torch.bfloat16, device=dev)
    ob = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev)

    def step(s):
        cache.roll(p["k"], p["v"], s - 1)
        rf.window_attention(ctx, cache, [rf.Segment(p["qa"], s, oa, s - 6, 21),
                                         rf.Segment(p["qb"], s - 1, ob, s - 6, 21)])

    s = 7
    for _ in range(3):
        step(s)
        s += 1
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    h0 = time.perf_counter()
    for _ in range(steps):
        step(s)
        s += 1
    host_eager = (time.perf_counter() - h0) / steps
    e1.record(stream)
    torch.cuda.synchronize()
    gpu_eager = e0.elapsed_time(e1) / steps

    shift = torch.zeros(1, dtype=torch.int64, device=dev)
    ctx.set_frame_shift(shift, steps + 1)
    gc.collect()  # free unreachable contexts now, not inside the capture
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(s)
            ctx.add_frame_shift(shift, 1)
    stream.wait_stream(side)
    graph.replay()  # step s, untimed
    torch.cuda.synchronize()
    e0.record(stream)
    h0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    host_graph = (time.perf_counter() - h0) / steps
    e1.record(stream)
    torch.cuda.synchronize()
    gpu_graph = e0.elapsed_time(e1) / steps
    assert int(shift.item()) == steps + 1
    ctx.set_frame_shift(None, 0)
    return {"steps": steps, "gpu_ms_per_step_eager": round(gpu_eager, 4),
            "gpu_ms_per_step_graph": round(gpu_graph, 4),
            "host_us_per_step_eager": round(host_eager * 1e6, 1),
            "host_us_per_step_graph": round(host_graph * 1e6, 1)}


def fill_graph_replay(rf, g, W, pool, steps=30):
    """The 30-step window fill from an empty ring (context 15 -> 21 frames, then one
    eviction per step), each step = roll of the 15 current frames, denoise attention over
    the whole window, roll of the finished clean frame.  Eagerly with host frame ranges,
    then as 30 replays of ONE captured step that reads its window from a device ring
    descriptor and its frame indices from the device frame shift (the ring reset on the
    device first).  GPU time for the 30 steps (events) and host time to enqueue them."""
    import torch

    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    dev = torch.device("cuda:0")
    p = pool[0]
    kn, vn = p["k"][N:], p["v"][N:]          # 15 current frames
    kc, vc = p["k"][:N], p["v"][:N]          # one clean frame
    q = p["qa"]
    o = torch.empty((15 * N, H, D), dtype=torch.bfloat16, device=dev)
    ctx_e = rf.Context(g.grid_h, g.grid_w, H, D, g.pairs, g.base, max_frame=8192)
    ctx_g = rf.Context(g.grid_h, g.grid_w, H, D, g.pairs, g.base, max_frame=8192)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def eager(cache):
        for s in range(steps):
            cache.roll(kn, vn, s)
            c0 = max(0, s - 6)
            rf.window_attention(ctx_e, cache, [rf.Segment(q, s, o, c0, s + 15 - c0)])
            cache.roll(kc, vc, s)

    eager(rf.KVCache(ctx_e, W))  # untimed pass
    ce = rf.KVCache(ctx_e, W)
    torch.cuda.synchronize()
    e0.record(stream)
    h0 = time.perf_counter()
    eager(ce)
    host_eager = (time.perf_counter() - h0) / steps
    e1.record(stream)
    torch.cuda.synchronize()
    gpu_eager = e0.elapsed_time(e1) / steps

    cg = rf.KVCache(ctx_g, W)
    rings = rf.DeviceRings([cg])
    shift = torch.zeros(1, dtype=torch.int64, device=dev)
    ctx_g.set_frame_shift(shift, steps)
    gc.collect()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            rings.roll(kn.unsqueeze(0), vn.unsqueeze(0), 0)
            rf.window_attention_dev(ctx_g, rings, 0, [rf.Segment(q, 0, o, 0, 0)])
            rings.roll(kc.unsqueeze(0), vc.unsqueeze(0), 0)
            ctx_g.add_frame_shift(shift, 1)
    stream.wait_stream(side)
    res = {"steps": steps}
    for rep in range(2):  # the first pass untimed
        rings.reset()
        shift.zero_()
        torch.cuda.synchronize()
        e0.record(stream)
        h0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        host_graph = (time.perf_counter() - h0) / steps
        e1.record(stream)
        torch.cuda.synchronize()
        gpu_graph = e0.elapsed_time(e1) / steps
    assert int(shift.item()) == steps
    same = bool(torch.equal(cg.k.view(torch.int16), ce.k.view(torch.int16)) and
                torch.equal(cg.v.view(torch.int16), ce.v.view(torch.int16)))
    ctx_g.set_frame_shift(None, 0)
    res.update({"gpu_ms_per_step_eager": round(gpu_eager, 4), "gpu_ms_per_step_graph": round(gpu_graph, 4),
                "host_us_per_step_eager": round(host_eager * 1e6, 1),
                "host_us_per_step_graph": round(host_graph * 1e6, 1),
                "rings_equal_after_30_steps": same})
    del rings, cg, ce
    return res


def cpu_baseline(args, g, s, ctx_frames, qa_bits, oa, qb_bits, ob):
    """The fp64 oracle timed on the host cores on a bounded sample of the same workload:
    R query rows of the denoise segment (all 12 heads) over the full 32,760-key window,
    including the oracle's rotation of the context keys.  Scaled to TFLOP/s by the sampled
    rows' algorithmic flops.  The sampled rows also give a parity spot check of the last
    timed step.  The step's cache-update segment (1,560 rows, the cache-update pass on its
    own) is timed in full beside it, with its own parity check."""
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import attention as oatt
    from oracle import bf16 as obf

    N, H, D = g.tokens_per_frame, g.n_heads, g.head_dim
    lk = 21 * N
    k = obf.bits_to_f64(np.concatenate([f[0] for f in ctx_frames]))
    v = obf.bits_to_f64(np.concatenate([f[1] for f in ctx_frames]))
    q = obf.bits_to_f64(qa_bits)
    workers = max(1, len(os.sched_getaffinity(0)))

    def run(rows):
        t0 = time.perf_counter()
        with threadpool_limits(limits=1, user_api="blas"):
            o = oatt.window_attention(q, s, k, v, s - 6, g.grid_h, g.grid_w, g.pairs, g.base,
                                      rows=rows, block=64, workers=workers)
        return o, time.perf_counter() - t0

    # two probes separate the fixed cost (rotating the context keys) from the
    # per-row cost; then size the sample for about `cpu_seconds` of oracle time
    rng = np.random.default_rng(0)
    _, t_a = run(np.sort(rng.choice(15 * N, 64, replace=False)))
    _, t_b = run(np.sort(rng.choice(15 * N, 576, replace=False)))
    per_row = max((t_b - t_a) / 512.0, 1e-6)
    fixed = max(t_a - 64 * per_row, 0.0)
    n_rows = int(np.clip((args.cpu_seconds - fixed) / per_row, 64, 15 * N))
    rows = np.sort(rng.choice(15 * N, n_rows, replace=False))
    o, secs = run(rows)
    flops = 4.0 * n_rows * lk * H * D
    got = obf.bits_to_f64(oa.view(torch.int16).cpu().numpy().view(np.uint16))[rows]
    err = np.abs(got - o)
    rel = float(np.linalg.norm((got - o).ravel()) / np.linalg.norm(o.ravel()))

    # the cache-update segment in full: queries of frame s-1 over the same window
    qb = obf.bits_to_f64(qb_bits)
    t0 = time.perf_counter()
    with threadpool_limits(limits=1, user_api="blas"):
        o_b = oatt.window_attention(qb, s - 1, k, v, s - 6, g.grid_h, g.grid_w, g.pairs, g.base,
                                    block=64, workers=workers)
    secs_b = time.perf_counter() - t0
    got_b = obf.bits_to_f64(ob.view(torch.int16).cpu().numpy().view(np.uint16))
    rel_b = float(np.linalg.norm((got_b - o_b).ravel()) / np.linalg.norm(o_b.ravel()))
    flops_b = 4.0 * N * lk * H * D
    return {
        "value": round(flops / secs / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{n_rows} of 23,400 denoise query rows x 12 heads over 32,760 keys of the last "
                  f"timed step (incl. rotating the 21 context frames), fp64 numpy",
        "seconds": round(secs, 2),
        "cpu_model": host_cpu_model(),
        "parity_rows": {"max_abs": float(err.max()), "mean_abs": float(err.mean()), "rel_l2": rel},
        "cache_update_pass": {"rows": N, "seconds": round(secs_b, 2),
                              "TFLOP/s": round(flops_b / secs_b / 1e12, 6),
                              "parity": {"max_abs": float(np.abs(got_b - o_b).max()),
                                         "mean_abs": float(np.abs(got_b - o_b).mean()),
                                         "rel_l2": rel_b}},
    }


def host_cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
