#!/usr/bin/env python3
"""Benchmark of one latent-KV (VideoMLA) chunk step on one MI355X.

Workload: one Wan2.1-1.3B-shaped layer (hidden 1536, 12 heads x 128, latent
192 + positional 32), a 3-frame chunk (3 x 30 x 52 = 4680 query tokens)
written into and attending over a full 21-frame ring window (32760 cached
tokens), bf16 storage with fp32 accumulation, batch 1, seeded synthetic
inputs (x ~ N(0,1), weights ~ N(0, 1/fan_in), queries ~ N(0,1)).

One step = cache write of the chunk's 3 frames (down-projection into the
ring) + query absorb/rotate + latent flash attention + W_uv up-projection,
all inputs resident in HBM. Prints one JSON line (see the keys below).

  python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA chunk-attention TFLOP/s + cache-write GB/s, Wan-1.3B shape, 1 MI355X"
PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 matrix peak (AMD spec)
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
COUNTERS_FILE = os.path.join(ROOT, "profiles", "flash_mla_wan_traffic.json")
CEILING_LIB = os.path.join(ROOT, "latent_kv_attention_amd", "libmla355_ceiling.so")
# sources of the attention entry point's kernels and of its work split; the
# committed traffic record is used only while these are unchanged
FLASH_SOURCES = ["latent_kv_attention_amd/csrc/flash_mla.hip", "latent_kv_attention_amd/csrc/mla_common.hpp",
                 "latent_kv_attention_amd/csrc/rope_device.hpp", "latent_kv_attention_amd/csrc/mla_internal.hpp",
                 "latent_kv_attention_amd/csrc/mla_abi.hip", "latent_kv_attention_amd/build.py"]
# The roofline unit: one mla_flash_attend call. HIP events on the launch
# stream bracket the call, which launches these kernels (the main kernel is
# about 95% of the time; the merge combines row blocks split between
# work-groups; the window's kR rotation and the exact fallback are small).
FLASH_KERNELS = ["flash_mla_kernel", "flash_combine_kernel", "rope_window_kernel", "flash_exact_kernel"]


def flash_source_hash() -> str:
    h = hashlib.sha256()
    for f in FLASH_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def mfma_ceiling(iters: int = 20000, reps: int = 5):
    """Dense bf16 matrix-core rate of a pure product loop (no memory or LDS
    traffic) in the attention kernel's occupancy: one 512-thread work-group
    per compute unit, 8 independent accumulators per wave. HIP events on the
    launch stream around single launches, median of `reps`. None when the
    probe library has not been built."""
    import ctypes
    import numpy as np
    import torch
    if not os.path.exists(CEILING_LIB):
        return None
    lib = ctypes.CDLL(CEILING_LIB)
    lib.mla_ceiling_flops.restype = ctypes.c_double
    lib.mla_ceiling_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.mla_ceiling_run.restype = ctypes.c_int32
    lib.mla_ceiling_run.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def run(n):
        rc = lib.mla_ceiling_run(blocks, n, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"mla_ceiling_run failed: {rc}")

    run(1000)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run(iters)
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ms = float(np.median(ts))
    tflops = lib.mla_ceiling_flops(blocks, iters) / (ms * 1e-3) / 1e12
    return {"what": f"pure v_mfma_f32_16x16x32_bf16 loop, {blocks} work-groups x 8 waves (2 per SIMD)",
            "ms": round(ms, 4), "TFLOPs": round(tflops, 1), "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4)}


def step_flops(cfg):
    """Algorithmic FLOPs of one step, absorbed form (what the kernels compute)."""
    nq, nk, H = cfg.n_q, cfg.n_k, cfg.n_heads
    cache_write = 2.0 * nq * cfg.hidden * (cfg.d_c + cfg.d_rope)
    absorb = 2.0 * nq * H * cfg.d_head * cfg.d_c
    flash = 2.0 * nq * H * nk * (cfg.d_c + cfg.d_rope + cfg.d_c)
    up = 2.0 * nq * H * cfg.d_c * cfg.d_head
    nonabs = 2.0 * nq * H * nk * (cfg.d_head + cfg.d_rope + cfg.d_head)
    return dict(cache_write=cache_write, absorb=absorb, flash=flash, up_v=up,
                total=cache_write + absorb + flash + up, flash_nonabsorbed_equiv=nonabs)


def cache_write_bytes(cfg):
    """Algorithmic HBM bytes of the chunk's cache write: x read once, the
    stacked down-projection read once, the new cache rows written once."""
    e = 2 if cfg.dtype == "bf16" else 4
    return e * (cfg.n_q * cfg.hidden + (cfg.d_c + cfg.d_rope) * cfg.hidden + cfg.n_q * (cfg.d_c + cfg.d_rope))


def cpu_model() -> str:
    """Model name of the host CPU, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# worker threads the oracle may use: the host CPUs this process may run on,
# at most 16 (the CPU share of one GPU on the machines this runs on)
CPU_THREAD_CAP = 16


def cpu_baseline(cfg, sample_tokens: int, seed: int = 0, gpu_out=None):
    """The fp64 oracle as it stands, on a bounded sample of the same workload:
    latents of the whole 21-frame window, explicit per-head reconstruction of
    every key and value, and attention for the first `sample_tokens` query
    tokens of the chunk (all heads, full window). Credited with the absorbed-
    path FLOPs of that sample (cache write of the chunk + attention of those
    rows), so the rate is in the metric's unit. With gpu_out (the timed
    step's output, same seeded inputs) the oracle rows are also compared with
    it element by element."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from harness import chunk_queries, frame_tokens, layer_weights
    from oracle import mla_oracle as O

    affinity = len(os.sched_getaffinity(0))
    cores = min(affinity, CPU_THREAD_CAP)
    w = layer_weights(cfg, seed)
    frames = list(range(cfg.window_frames))
    xs = [frame_tokens(cfg, f, seed) for f in frames]
    chunk_first = cfg.window_frames - cfg.chunk_frames
    qn, qr = chunk_queries(cfg, chunk_first, seed)
    with threadpool_limits(limits=cores):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        t0 = time.perf_counter()
        c, kr = O.latents(np.concatenate(xs), w["w_dkv"], w["w_kr"])
        k_nope, v = O.reconstruct(c, w["w_uk"], w["w_uv"])
        t, y, x = O.frame_positions(frames, cfg.grid_y, cfg.grid_x)
        k_rope = O.rope3d(kr, t, y, x, cfg.rope_split, cfg.rope_base)
        rows = np.arange(sample_tokens)
        tq, yq, xq = O.frame_positions(chunk_first + np.arange(cfg.chunk_frames), cfg.grid_y, cfg.grid_x)
        q_rope = O.rope3d(qr[rows], tq[rows], yq[rows], xq[rows], cfg.rope_split, cfg.rope_base)
        ref = O.attend(qn[rows], q_rope, k_nope, k_rope, v, O.default_scale(cfg.d_head, cfg.d_rope))
        dt = time.perf_counter() - t0
    fl = step_flops(cfg)
    frac = sample_tokens / cfg.n_q
    credited = fl["cache_write"] + frac * (fl["absorb"] + fl["flash"] + fl["up_v"])
    res = {"value": credited / dt / 1e12, "unit": "TFLOP/s", "cores": int(min(cores, used)), "kind": "oracle",
           "sample": f"fp64 oracle: latents of 21 frames x 1560 tokens, per-head reconstruction of all "
                     f"32760 keys and values, attention of the first {sample_tokens} of 4680 query tokens "
                     f"(all 12 heads, full window); {dt:.2f} s, credited with the chunk cache write plus "
                     f"{sample_tokens}/4680 of the attention-side FLOPs",
           "seconds": round(dt, 3), "cpu_model": cpu_model(), "host_logical_cpus": os.cpu_count(),
           "affinity_cpus": affinity, "thread_cap": CPU_THREAD_CAP}
    if gpu_out is not None:
        got = np.asarray(gpu_out, np.float64)[:sample_tokens]
        d = np.abs(got - ref)
        res["parity_vs_gpu_out"] = {
            "outputs_compared": int(d.size), "max_abs": float(d.max()), "mean_abs": float(d.mean()),
            "rel_rms": float(np.linalg.norm(got - ref) / np.linalg.norm(ref)),
            "gates": {"max_abs": 2e-2, "mean_abs": 2e-3, "rel_rms": 1e-2},
            "pass": bool(d.max() <= 2e-2 and d.mean() <= 2e-3 and np.linalg.norm(got - ref) <= 1e-2 * np.linalg.norm(ref))}
    return res


def setup_step(cfg, kv_splits, dev="cuda"):
    """Seeded inputs and buffers of one chunk step at `cfg`: the window's first
    frames are written, then step() writes the chunk and runs absorb, attention
    and up-projection. Returns a namespace with the buffers and step()."""
    import types

    import numpy as np
    import torch

    import latent_kv_attention_amd as mla
    from harness import chunk_queries, frame_tokens, layer_weights
    from harness.torch_io import to_torch

    T = cfg.tokens_per_frame
    print(f"[bench] generating inputs ({cfg.name}: d_c {cfg.d_c}, d_rope {cfg.d_rope})", file=sys.stderr, flush=True)
    w = {k: to_torch(v, cfg.dtype, dev) for k, v in layer_weights(cfg, 0).items()}
    chunk_first = cfg.window_frames - cfg.chunk_frames
    x_pre = to_torch(np.concatenate([frame_tokens(cfg, f) for f in range(chunk_first)]), cfg.dtype, dev)
    x_chunk = to_torch(np.concatenate([frame_tokens(cfg, chunk_first + i) for i in range(cfg.chunk_frames)]),
                       cfg.dtype, dev)
    qn_h, qr_h = chunk_queries(cfg, chunk_first)
    qn, qr = to_torch(qn_h, cfg.dtype, dev), to_torch(qr_h, cfg.dtype, dev)

    shape = mla.make_shape(cfg, batch=1)
    n_t = 64
    tables = torch.empty(mla.rope3d_table_floats(shape, n_t), dtype=torch.float32, device=dev)
    mla.rope3d_tables(shape, 0, n_t, tables)
    cache = torch.zeros(1, cfg.window_frames, T, cfg.d_c + cfg.d_rope, dtype=torch.bfloat16, device=dev)
    slot_frame = torch.full((1, cfg.window_frames), -1, dtype=torch.int32, device=dev)
    mla.cache_write(shape, x_pre, w["w_dkv"], w["w_kr"], 0, chunk_first, cache, slot_frame)
    del x_pre
    Q = mla.qabs_dim(shape)
    q_abs = torch.empty(cfg.n_q, cfg.n_heads, Q, dtype=torch.bfloat16, device=dev)
    o_lat = torch.empty(cfg.n_q, cfg.n_heads, cfg.d_c, dtype=torch.bfloat16, device=dev)
    out = torch.empty(cfg.n_q, cfg.n_heads, cfg.d_head, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mla.flash_workspace_bytes(shape, cfg.chunk_frames, kv_splits), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev:
            ev[0].record()
        mla.cache_write(shape, x_chunk, w["w_dkv"], w["w_kr"], chunk_first, cfg.chunk_frames, cache, slot_frame)
        if ev:
            ev[1].record()
        mla.absorb_q(shape, qn, qr, chunk_first, cfg.chunk_frames, w["w_uk"], tables, 0, n_t, q_abs)
        if ev:
            ev[2].record()
        mla.flash_attend(shape, q_abs, cfg.chunk_frames, cache, slot_frame, tables, 0, n_t, o_lat, ws, kv_splits)
        if ev:
            ev[3].record()
        mla.up_v(shape, o_lat, cfg.chunk_frames, w["w_uv"], out)
        if ev:
            ev[4].record()

    def write():
        mla.cache_write(shape, x_chunk, w["w_dkv"], w["w_kr"], chunk_first, cfg.chunk_frames, cache, slot_frame)

    def flash():
        mla.flash_attend(shape, q_abs, cfg.chunk_frames, cache, slot_frame, tables, 0, n_t, o_lat, ws, kv_splits)

    return types.SimpleNamespace(shape=shape, w=w, x_chunk=x_chunk, chunk_first=chunk_first, cache=cache,
                                 slot_frame=slot_frame, out=out, step=step, write=write, flash=flash, qn=qn, qr=qr,
                                 tables=tables, n_t=n_t)


def graph_replay_writes(ctx, xs_cold, cw_bytes):
    """GPU-side time of the chunk's cache write: len(xs_cold) writes captured
    in one HIP graph, replayed between events on the launch stream, once over
    the distinct (cold) x buffers and once over one buffer (warm). Each
    replay's cache rows are compared with those of an eager write of the
    same inputs (every buffer holds the same tokens)."""
    import torch

    import latent_kv_attention_amd as mla

    cfg_frames = ctx.cache.shape[1]
    n_frames = ctx.x_chunk.shape[0] // ctx.cache.shape[2]
    slots = [(ctx.chunk_first + i) % cfg_frames for i in range(n_frames)]
    w = ctx.w
    mla.cache_write(ctx.shape, ctx.x_chunk, w["w_dkv"], w["w_kr"], ctx.chunk_first, n_frames, ctx.cache,
                    ctx.slot_frame)
    torch.cuda.synchronize()
    ref = ctx.cache[:, slots].clone()
    out = {"what": f"{len(xs_cold)} cache writes of the chunk replayed from one HIP graph, events around the replay "
                   "(no host launch path between the kernels); per write"}
    for label, bufs in (("cold", xs_cold), ("warm", [ctx.x_chunk] * len(xs_cold))):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for xb in bufs:
                mla.cache_write(ctx.shape, xb, w["w_dkv"], w["w_kr"], ctx.chunk_first, n_frames, ctx.cache,
                                ctx.slot_frame)
        ok = True
        times = []
        for _ in range(3):
            ctx.cache[:, slots] = 0
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) / len(bufs))
            ok = ok and bool(torch.equal(ctx.cache[:, slots], ref))
        del g
        ms = float(min(times[1:]))
        out[label] = {"ms": round(ms, 5), "GBps": round(cw_bytes / (ms * 1e-3) / 1e9, 1),
                      "hbm_frac": round(cw_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4), "matches_eager": ok}
    return out


def settle_clock(ctx, window=20, tol=0.01, min_windows=5, max_windows=40):
    """The GPU raises its clock over the first tens of milliseconds of load
    after idle (set-up is mostly host work): a timed window started from idle
    runs the step 4-25% slower than the sustained rate. Before the warm-up and
    timed steps, run at least `min_windows` windows of `window` steps, until
    two consecutive windows agree within `tol` (at most `max_windows`).
    Returns the first and last window times, reported in the bench line."""
    import torch

    ts = []
    for _ in range(max_windows):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(window):
            ctx.step()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / window)
        if len(ts) >= min_windows and abs(ts[-1] - ts[-2]) <= tol * ts[-1]:
            break
    print(f"[bench] clock settle: {len(ts)} windows of {window} steps, {ts[0]:.4f} -> {ts[-1]:.4f} ms/step",
          file=sys.stderr, flush=True)
    return {"what": f"untimed windows of {window} steps run before the warm-up, at least {min_windows} and until two "
                    f"consecutive windows agree within {tol:.0%} (the clock ramps up under load after idle)",
            "windows": len(ts), "first_window_ms_per_step": round(ts[0], 4), "last_window_ms_per_step": round(ts[-1], 4)}


def time_steps(ctx, steps, warmup):
    """W untimed steps, then K timed ones between events on the launch stream;
    returns (ms per step, mean ms of each of the four calls)."""
    import numpy as np
    import torch

    print(f"[bench] warmup {warmup} steps", file=sys.stderr, flush=True)
    for _ in range(warmup):
        ctx.step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(steps):
        ctx.step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / steps
    names = ["cache_write", "absorb_q", "flash_attend", "up_v"]
    per = {n: float(np.mean([e[k].elapsed_time(e[k + 1]) for e in evs])) for k, n in enumerate(names)}
    print(f"[bench] timed {steps} steps: {ms_step:.4f} ms/step {per}", file=sys.stderr, flush=True)
    assert torch.isfinite(ctx.out.float()).all(), "non-finite output"
    return ms_step, per


# latent widths of the sweep: (d_c, d_rope, RoPE axis split)
SWEEP_WIDTHS = [(128, 32, (8, 12, 12)), (192, 32, (8, 12, 12)), (160, 64, (16, 24, 24)), (192, 64, (16, 24, 24))]


def latent_sweep(base, args):
    """The same chunk step at each latent width the library instantiates (the
    pages' ablations vary the latent size and the content/positional split;
    performance only, weights are synthetic). One JSON line per width; these
    lines are a separate report, not the bench line."""
    import torch

    for dc, dr, split in SWEEP_WIDTHS:
        cfg = base.with_(d_c=dc, d_rope=dr, rope_split=split)
        ctx = setup_step(cfg, args.kv_splits)
        settle_clock(ctx)
        ms_step, per = time_steps(ctx, args.steps, args.warmup)
        fl = step_flops(cfg)
        fl_tf = fl["flash"] / (per["flash_attend"] * 1e-3) / 1e12
        print(json.dumps({
            "report": "latent-width sweep, Wan2.1-1.3B-shaped chunk step (4680 queries x 32760 keys), 1 MI355X",
            "d_c": dc, "d_rope": dr, "rope_split": list(split), "cached_scalars_per_token": dc + dr,
            "window_cache_MB": round(cfg.window_frames * cfg.tokens_per_frame * (dc + dr) * 2 / 1e6, 2),
            "ms_per_step": round(ms_step, 4), "kernel_ms": {k: round(v, 4) for k, v in per.items()},
            "step_TFLOPs": round(fl["total"] / (ms_step * 1e-3) / 1e12, 2), "flash_TFLOPs": round(fl_tf, 2),
            "flash_frac_of_bf16_peak": round(fl_tf / PEAK_BF16_TFLOPS, 4),
            "flash_TFLOPs_nonabsorbed_equiv": round(fl["flash_nonabsorbed_equiv"] / (per["flash_attend"] * 1e-3)
                                                    / 1e12, 2),
            "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic"}), flush=True)
        del ctx
        torch.cuda.empty_cache()


def per_head_report(base, args):
    """The chunk step by the per-head form (cache write, then
    mla_chunk_attend_heads: kR rotation, key/value expansion for every head,
    query scaling and rotation, per-head attention) next to the latent form,
    at each latent width of the sweep. One JSON report line per width; not
    the bench line."""
    import numpy as np
    import torch

    import latent_kv_attention_amd as mla

    # every latent width at the 3-frame chunk, then 1- and 2-frame chunks at the
    # Wan width (the expansion is per call, so its share grows as the chunk shrinks)
    cases = [base.with_(d_c=dc, d_rope=dr, rope_split=split) for dc, dr, split in SWEEP_WIDTHS]
    cases += [base.with_(chunk_frames=nf) for nf in (1, 2)]
    for cfg in cases:
        dc, dr = cfg.d_c, cfg.d_rope
        ctx = setup_step(cfg, args.kv_splits)
        settle_clock(ctx)
        ms_latent, per_latent = time_steps(ctx, args.steps, args.warmup)
        ws = torch.empty(mla.chunk_attend_heads_workspace_bytes(ctx.shape, cfg.chunk_frames), dtype=torch.uint8,
                         device="cuda")
        out_h = torch.empty_like(ctx.out)

        def attend():
            mla.chunk_attend_heads(ctx.shape, ctx.qn, ctx.qr, ctx.chunk_first, cfg.chunk_frames, ctx.w["w_uk"],
                                   ctx.w["w_uv"], ctx.cache, ctx.slot_frame, ctx.tables, 0, ctx.n_t, out_h, ws)

        for _ in range(args.warmup):
            ctx.write()
            attend()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for e in evs:
            e[0].record()
            ctx.write()
            e[1].record()
            attend()
            e[2].record()
        torch.cuda.synchronize()
        ms_w = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        ms_a = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        diff = (out_h.float() - ctx.out.float()).abs()
        nq, nk, H = cfg.n_q, cfg.n_k, cfg.n_heads
        attn_fl = 2.0 * nq * nk * H * (cfg.d_head + cfg.d_rope + cfg.d_head)
        expand_fl = 4.0 * nk * H * cfg.d_head * cfg.d_c
        latent_ms = per_latent["absorb_q"] + per_latent["flash_attend"] + per_latent["up_v"]
        print(json.dumps({
            "report": f"per-head form vs latent form, Wan2.1-1.3B-shaped chunk step ({cfg.n_q} queries x 32760 keys), "
                      "1 MI355X",
            "d_c": dc, "d_rope": dr, "d_head": cfg.d_head, "chunk_frames": cfg.chunk_frames, "n_q": cfg.n_q,
            "per_head_attend_ms": round(ms_a, 4), "latent_attend_ms": round(latent_ms, 4),
            "per_head_step_ms": round(ms_w + ms_a, 4), "latent_step_ms": round(ms_latent, 4),
            "speedup_attend": round(latent_ms / ms_a, 3),
            "per_head_own_TFLOPs": round((attn_fl + expand_fl) / (ms_a * 1e-3) / 1e12, 2),
            "per_head_attention_flops": attn_fl, "per_head_expansion_flops": expand_fl,
            "max_abs_diff_vs_latent_form": round(float(diff.max()), 5),
            "form_mla_chunk_attend_takes": {mla.FORM_LATENT: "latent", mla.FORM_HEADS: "per-head"}[
                mla.chunk_attend_form(ctx.shape, cfg.chunk_frames)],
            "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic"}), flush=True)
        del ctx, ws, out_h
        torch.cuda.empty_cache()


def frame_causal_report(cfg, args):
    """The attention side with and without the frame-causal mask inside the
    chunk, at the Wan shape, in both forms (mla_chunk_attend_latent /
    mla_chunk_attend_latent_frame_causal and mla_chunk_attend_heads /
    mla_chunk_attend_heads_frame_causal). One JSON report line."""
    import numpy as np
    import torch

    import latent_kv_attention_amd as mla

    ctx = setup_step(cfg, 0)
    settle_clock(ctx)
    ctx.write()
    ws = torch.empty(mla.chunk_attend_workspace_bytes(ctx.shape, cfg.chunk_frames), dtype=torch.uint8, device="cuda")
    hws = torch.empty(mla.chunk_attend_heads_workspace_bytes(ctx.shape, cfg.chunk_frames), dtype=torch.uint8,
                      device="cuda")
    calls = {"latent_full": (mla.chunk_attend_latent, ws),
             "latent_causal": (mla.chunk_attend_latent_frame_causal, ws),
             "heads_full": (mla.chunk_attend_heads, hws),
             "heads_causal": (mla.chunk_attend_heads_frame_causal, hws)}
    outs = {k: torch.empty_like(ctx.out) for k in calls}
    ts = {k: [] for k in calls}
    for rnd in range(args.warmup + args.steps):
        for k, (fn, w) in calls.items():
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn(ctx.shape, ctx.qn, ctx.qr, ctx.chunk_first, cfg.chunk_frames, ctx.w["w_uk"], ctx.w["w_uv"], ctx.cache,
               ctx.slot_frame, ctx.tables, 0, ctx.n_t, outs[k], w)
            b.record()
            torch.cuda.synchronize()
            if rnd >= args.warmup:
                ts[k].append(a.elapsed_time(b))
    T = cfg.tokens_per_frame
    last = (cfg.chunk_frames - 1) * T
    # keys each chunk frame may not see: the later chunk frames
    masked_frac = sum(cfg.chunk_frames - 1 - k for k in range(cfg.chunk_frames)) / (cfg.chunk_frames * cfg.window_frames)
    ms = {k: float(np.median(v)) for k, v in ts.items()}
    selected = "heads" if mla.chunk_attend_form(ctx.shape, cfg.chunk_frames) == mla.FORM_HEADS else "latent"
    print(json.dumps({
        "report": "frame-causal vs full attention inside the chunk, both forms, Wan2.1-1.3B-shaped chunk step "
                  "(4680 queries x 32760 keys), 1 MI355X",
        **{f"{k}_attend_ms": round(v, 4) for k, v in ms.items()},
        "masked_key_fraction": round(masked_frac, 4),
        "latent_time_ratio": round(ms["latent_causal"] / ms["latent_full"], 4),
        "heads_time_ratio": round(ms["heads_causal"] / ms["heads_full"], 4),
        "selected_form": selected,
        "rows_identical_in_last_frame": {
            f: bool(torch.equal(outs[f + "_full"][last:], outs[f + "_causal"][last:])) for f in ("latent", "heads")},
        "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic"}), flush=True)


def projections_report(cfg, args):
    """The query path (mla_query_project: query latent, per-head content and
    positional queries) and the output projection (mla_output_project) at the
    Wan shape, and the whole layer built from them (query path, cache write,
    mla_chunk_attend, output projection). One JSON report line."""
    import numpy as np
    import torch

    import latent_kv_attention_amd as mla
    from harness import frame_tokens, layer_weights, query_weights
    from harness.torch_io import to_torch
    from latent_kv_attention_amd.layer import LatentLayer

    dev = "cuda"
    print(f"[bench] projections: generating inputs (d_cq {cfg.q_latent})", file=sys.stderr, flush=True)
    w = {k: to_torch(v, cfg.dtype, dev) for k, v in {**layer_weights(cfg, 0), **query_weights(cfg, 0)}.items()}
    layer = LatentLayer(cfg, w, batch=1, rope_n_t=64)
    chunk_first = cfg.window_frames - cfg.chunk_frames
    x_pre = to_torch(np.concatenate([frame_tokens(cfg, f) for f in range(chunk_first)])[None], cfg.dtype, dev)
    layer.write(x_pre, 0, chunk_first)
    del x_pre
    x = to_torch(np.concatenate([frame_tokens(cfg, chunk_first + i) for i in range(cfg.chunk_frames)])[None],
                 cfg.dtype, dev)
    o = torch.randn(1, cfg.n_q, cfg.n_heads, cfg.d_head, device=dev).to(torch.bfloat16)
    u = torch.empty(1, cfg.n_q, cfg.hidden, dtype=torch.bfloat16, device=dev)
    # the same products through torch's library GEMM (context only)
    x2, o2 = x.view(cfg.n_q, cfg.hidden), o.view(cfg.n_q, cfg.n_heads * cfg.d_head)
    w_q = torch.cat([w["w_uq"].reshape(-1, cfg.q_latent), w["w_qr"].reshape(-1, cfg.q_latent)]).contiguous()
    lin = torch.nn.functional.linear
    # the fused query path (absorbed weights) on a second layer of the same weights and window
    fused = LatentLayer(cfg, w, batch=1, rope_n_t=64)
    fused.cache.copy_(layer.cache)
    fused.slot_frame.copy_(layer.slot_frame)
    fused.absorb_query_weights()
    Q = mla.qabs_dim(layer.shape)
    q_abs = torch.empty(1, cfg.n_q, cfg.n_heads, Q, dtype=torch.bfloat16, device=dev)

    def unfused_query_to_qabs():
        _, qn, qr = layer.project_queries(x, cfg.chunk_frames)
        mla.absorb_q(layer.shape, qn, qr, chunk_first, cfg.chunk_frames, w["w_uk"], layer.tables, 0, 64, q_abs)

    calls = {
        "query_project": lambda: layer.project_queries(x, cfg.chunk_frames),
        "query_to_qabs_unfused": unfused_query_to_qabs,
        "query_project_absorbed": lambda: fused.project_queries_absorbed(x, chunk_first, cfg.chunk_frames),
        "output_project": lambda: layer.project_output(o, cfg.chunk_frames, out=u),
        "layer_step": lambda: layer.step(x, chunk_first, cfg.chunk_frames),
        "layer_step_fused": lambda: fused.step(x, chunk_first, cfg.chunk_frames),
        # frame-causal layer step (the form mla_chunk_attend_form names): one
        # call (query latent and cache write in one product over x) against
        # the four calls one by one
        "layer_step_causal_one_call": lambda: layer.step(x, chunk_first, cfg.chunk_frames, frame_causal=True),
        "layer_step_causal_four_calls": lambda: layer.step_composed(x, chunk_first, cfg.chunk_frames,
                                                                    frame_causal=True),
        "library_query": lambda: lin(lin(x2, w["w_dq"]), w_q),
        "library_output": lambda: lin(o2, w["w_o"]),
    }
    # each sample: `reps` calls back to back between two events on the stream
    reps = 10
    ts = {k: [] for k in calls}
    for rnd in range(args.warmup + args.steps):
        for k, fn in calls.items():
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            if rnd >= args.warmup:
                ts[k].append(a.elapsed_time(b) / reps)
    ms = {k: float(np.median(v)) for k, v in ts.items()}
    M, H = cfg.n_q, cfg.n_heads
    q_fl = 2.0 * M * (cfg.hidden * cfg.q_latent + cfg.q_latent * H * (cfg.d_head + cfg.d_rope))
    o_fl = 2.0 * M * H * cfg.d_head * cfg.hidden
    tf = lambda fl, t: fl / (t * 1e-3) / 1e12
    print(json.dumps({
        "report": "query path and output projection around the chunk step, Wan2.1-1.3B shape (4680 chunk tokens, "
                  "hidden 1536, d_cq %d), 1 MI355X" % cfg.q_latent,
        "query_project_ms": round(ms["query_project"], 4), "query_project_flops": q_fl,
        "query_project_TFLOPs": round(tf(q_fl, ms["query_project"]), 1),
        "output_project_ms": round(ms["output_project"], 4), "output_project_flops": o_fl,
        "output_project_TFLOPs": round(tf(o_fl, ms["output_project"]), 1),
        "projections_frac_of_bf16_peak": round(tf(q_fl + o_fl, ms["query_project"] + ms["output_project"])
                                               / PEAK_BF16_TFLOPS, 4),
        "library_gemm_query_ms": round(ms["library_query"], 4),
        "library_gemm_output_ms": round(ms["library_output"], 4),
        "layer_step_ms": round(ms["layer_step"], 4),
        "query_to_qabs_unfused_ms": round(ms["query_to_qabs_unfused"], 4),
        "query_project_absorbed_ms": round(ms["query_project_absorbed"], 4),
        "query_project_absorbed_TFLOPs": round(tf(2.0 * M * cfg.q_latent * (cfg.hidden + H * Q),
                                                  ms["query_project_absorbed"]), 1),
        "layer_step_fused_ms": round(ms["layer_step_fused"], 4),
        "layer_step_form": {mla.FORM_LATENT: "latent", mla.FORM_HEADS: "per-head"}[
            mla.chunk_attend_form(layer.shape, cfg.chunk_frames)],
        "layer_step_frame_causal_one_call_ms": round(ms["layer_step_causal_one_call"], 4),
        "layer_step_frame_causal_four_calls_ms": round(ms["layer_step_causal_four_calls"], 4),
        "projections_share_of_layer": round((ms["query_project"] + ms["output_project"]) / ms["layer_step"], 4),
        "finite": bool(torch.isfinite(u.float()).all()),
        "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic"}), flush=True)


def configs_report(args):
    """Multi-layer and multi-stream workloads of the Wan shape, one JSON report
    line each (not the bench line): a 30-layer model whose windows fill over 7
    chunks; 8 streams with full windows through 30 layers; an 80-chunk,
    30-layer rollout whose rings evict from the 8th chunk on. Each layer has
    its own weights and ring; per layer and chunk: cache write, query absorb,
    attention, up-projection (mla_cache_write + mla_chunk_attend). Inputs
    come from device-resident pools (64 token frames, 4 query sets); the
    content does not change the work. Timed with HIP events around the whole
    run after one untimed warm-up chunk per layer."""
    import numpy as np
    import torch

    import latent_kv_attention_amd as mla
    from harness import chunk_queries, frame_tokens, get_config, layer_weights
    from harness.torch_io import to_torch
    from latent_kv_attention_amd.layer import LatentLayer

    dev = "cuda"
    base = get_config("wan")
    T = base.tokens_per_frame
    print("[bench] configs: device pools", file=sys.stderr, flush=True)
    # token pool with two wrap-around frames, so any 3 consecutive pool frames are one view
    pool = torch.empty(66, T, base.hidden, dtype=torch.bfloat16, device=dev)
    for i in range(64):
        pool[i] = to_torch(frame_tokens(base, i), "bf16", dev)
    pool[64:] = pool[:2]
    qpool = [tuple(to_torch(a, "bf16", dev) for a in chunk_queries(base, 3 * i)) for i in range(4)]

    def x_of(stream, layer, f0):
        i = (f0 + 7 * layer + 13 * stream) % 64
        return pool[i:i + 3].reshape(1, 3 * T, base.hidden)

    def run(name, B, n_chunks, prefill_frames):
        cfg = get_config(name)
        L = cfg.layers
        layers = []
        for l in range(L):
            wd = {k: to_torch(v, "bf16", dev) for k, v in layer_weights(cfg, 0, l).items()}
            layers.append(LatentLayer(cfg, wd, batch=B, rope_n_t=256))
        xb = torch.empty(B, 3 * T, base.hidden, dtype=torch.bfloat16, device=dev)
        qn = torch.stack([qpool[b % 4][0] for b in range(B)])
        qr = torch.stack([qpool[b % 4][1] for b in range(B)])
        out = torch.empty(B, 3 * T, cfg.n_heads, cfg.d_head, dtype=torch.bfloat16, device=dev)

        def fill(l, f0):
            for b in range(B):
                xb[b] = x_of(b, l, f0)[0]
            return xb

        for l, layer in enumerate(layers):  # prefill (untimed)
            for f0 in range(0, prefill_frames, 3):
                layer.write(fill(l, f0), f0, 3)
        first = prefill_frames
        method = {("latent", False): "attend_latent", ("selected", False): "attend",
                  ("latent", True): "attend_latent_frame_causal",
                  ("selected", True): "attend_frame_causal"}[(args.configs_form, args.configs_causal)]
        attend = lambda layer, *a, **k: getattr(layer, method)(*a, **k)
        for l, layer in enumerate(layers):  # warm-up chunk, rewritten in the timed run
            layer.write(fill(l, first), first, 3)
            attend(layer, qn, qr, first, 3, out=out)
        torch.cuda.synchronize()
        # token inputs of every (chunk, layer) gathered before the clock starts
        xs = {}
        for k in range(n_chunks):
            for l in range(L):
                f0 = first + 3 * k
                key = tuple((f0 + 7 * l + 13 * b) % 64 for b in range(B))
                if key not in xs:
                    xs[key] = torch.stack([x_of(b, l, f0)[0] for b in range(B)]) if B > 1 else x_of(0, l, f0)
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for k in range(n_chunks):
            f0 = first + 3 * k
            for l, layer in enumerate(layers):
                key = tuple((f0 + 7 * l + 13 * b) % 64 for b in range(B))
                layer.write(xs[key], f0, 3)
                attend(layer, qn, qr, f0, 3, out=out)
        e.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(e)
        assert torch.isfinite(out.float()).all()
        # attention FLOPs: window of min(W, frames written) frames at each chunk
        fl = 0.0
        for k in range(n_chunks):
            nk = min(cfg.window_frames, first + 3 * k + 3) * T
            fl += L * B * 2.0 * 3 * T * nk * cfg.n_heads * (2 * cfg.d_c + cfg.d_rope)
        slots = [int(v) for v in layers[0].slot_frame[0].cpu()]
        del layers
        torch.cuda.empty_cache()
        return ms, fl, slots

    runs = [("wan_fill30", 1, 7, 0, "30 layers x 7 chunks, windows filling 3 -> 21 frames"),
            ("wan_batch8", 8, 1, 18, "8 streams x 30 layers, one chunk over full 21-frame windows"),
            ("wan_rollout", 1, 80, 0, "80 chunks x 30 layers (frames 0..239), rings evicting from chunk 8")]
    for name, B, n_chunks, prefill, what in runs:
        if args.configs and name not in args.configs:
            continue
        print(f"[bench] configs: {name}", file=sys.stderr, flush=True)
        ms, fl, slots = run(name, B, n_chunks, prefill)
        print(json.dumps({
            "report": f"Wan2.1-1.3B-shaped workload: {what}, 1 MI355X",
            "config": name, "form": args.configs_form, "mask": "frame-causal" if args.configs_causal else "none",
            "streams": B, "layers": 30, "chunks": n_chunks,
            "total_ms": round(ms, 2),
            "ms_per_layer_chunk": round(ms / (30 * n_chunks), 4),
            "ms_per_chunk_all_layers": round(ms / n_chunks, 3),
            "attention_TFLOP": round(fl / 1e12, 2), "TFLOPs": round(fl / (ms * 1e-3) / 1e12, 1),
            "cache_MB_resident": round(30 * B * 21 * T * 224 * 2 / 1e6, 1),
            "last_slot_frames_layer0": slots,
            "dtype": "bf16", "data": "synthetic"}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--kv-splits", type=int, default=0, help="flash key-range splits (0 = automatic)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4680)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-buffers", type=int, default=40,
                    help="rotating x buffers for the cold-cache cache-write measurement (0 = skip)")
    ap.add_argument("--per-head", action="store_true",
                    help="time the per-head form against the latent form at every width (report lines) and exit")
    ap.add_argument("--frame-causal", action="store_true",
                    help="time the attention side with and without the frame-causal mask (report line) and exit")
    ap.add_argument("--projections", action="store_true",
                    help="time the query path, the output projection and the whole layer (report line) and exit")
    ap.add_argument("--configs", nargs="*", default=None, metavar="NAME",
                    help="time the 30-layer fill (wan_fill30), 8-stream (wan_batch8) and 80-chunk rollout "
                         "(wan_rollout) workloads, or only those named (report lines) and exit")
    ap.add_argument("--configs-form", choices=["latent", "selected"], default="latent",
                    help="attention form of --configs: the latent form (mla_chunk_attend_latent, the benchmark's "
                         "kernel) or the one mla_chunk_attend selects for the shape")
    ap.add_argument("--configs-causal", action="store_true",
                    help="--configs with the frame-causal mask inside each chunk (the attention FLOPs stay "
                         "those of the unmasked step)")
    ap.add_argument("--latent-sweep", action="store_true",
                    help="time the step at every latent width with kernels (one report line each) and exit")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only time the pure matrix-core loop (the attainable bf16 rate) and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (to scale HBM byte counters) and exit")
    args = ap.parse_args()

    if args.mfma_ceiling:
        print(json.dumps({"mfma_attainable": mfma_ceiling()}), flush=True)
        return

    if args.copy_calibration:
        import torch
        n = 1 << 29  # bf16 elements = 1 GiB
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "launches": 3}), flush=True)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library has no multi-GPU path (independent streams shard over GPUs with no exchange).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import latent_kv_attention_amd as mla
    from harness import get_config

    if not os.path.exists(mla.LIB_PATH):
        from latent_kv_attention_amd import build as _build
        _build.build()
    mla.lib()
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    cfg = get_config("wan")
    if args.latent_sweep:
        latent_sweep(cfg, args)
        return
    if args.per_head:
        per_head_report(cfg, args)
        return
    if args.frame_causal:
        frame_causal_report(cfg, args)
        return
    if args.projections:
        projections_report(cfg, args)
        return
    if args.configs is not None:
        configs_report(args)
        return
    ctx = setup_step(cfg, args.kv_splits)
    settle = settle_clock(ctx)
    ms_step, per = time_steps(ctx, args.steps, args.warmup)
    shape, w, x_chunk, chunk_first, cache, slot_frame = (ctx.shape, ctx.w, ctx.x_chunk, ctx.chunk_first, ctx.cache,
                                                        ctx.slot_frame)

    # cold-cache cache write: rotate the input over more distinct buffers than the
    # 256 MB last-level cache holds
    cold = copy_single = copy_bytes = graph_writes = None
    if args.cold_buffers > 0:
        xs_cold = [x_chunk.clone() for _ in range(args.cold_buffers)]
        for i in range(3):
            mla.cache_write(shape, xs_cold[i], w["w_dkv"], w["w_kr"], chunk_first, cfg.chunk_frames, cache,
                            slot_frame)
        torch.cuda.synchronize()
        ce = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.cold_buffers)]
        for i, xb in enumerate(xs_cold):
            ce[i][0].record()
            mla.cache_write(shape, xb, w["w_dkv"], w["w_kr"], chunk_first, cfg.chunk_frames, cache, slot_frame)
            ce[i][1].record()
        torch.cuda.synchronize()
        cold = float(np.mean([a.elapsed_time(b) for a, b in ce[3:]]))
        # for reference a plain device copy of each x buffer (reads and writes
        # its 14.38 MB), timed the same way (single launches between events):
        # the rate a streaming kernel reaches at this transfer size on this GPU
        dst = torch.empty_like(x_chunk)
        ce = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in xs_cold]
        for i, xb in enumerate(xs_cold):
            ce[i][0].record()
            dst.copy_(xb)
            ce[i][1].record()
        torch.cuda.synchronize()
        copy_single = float(np.mean([a.elapsed_time(b) for a, b in ce[3:]]))
        copy_bytes = 2 * x_chunk.numel() * x_chunk.element_size()
        del dst
        # the same writes replayed from a HIP graph, so that the kernels run
        # back to back with no host launch path between them: events around
        # a replay give the GPU-side time per write, with x cold (the 40
        # rotating buffers) and warm (one buffer 40 times)
        graph_writes = graph_replay_writes(ctx, xs_cold, cache_write_bytes(cfg))
        del xs_cold

    # larger writes, where the launch cost is spread over more bytes: a
    # 21-frame prefill of one stream, and a 3-frame chunk of 8 streams
    # (seeded device-side tokens; content does not change the work)
    big_writes = {}
    gen = torch.Generator(device="cuda").manual_seed(0)
    for label, B, nf in (("prefill_21_frames", 1, 21), ("batch8_3_frames", 8, 3)):
        shp = mla.make_shape(cfg, batch=B)
        xb = torch.randn(B, nf * cfg.tokens_per_frame, cfg.hidden, generator=gen, device="cuda").to(torch.bfloat16)
        cb = torch.zeros(B, cfg.window_frames, cfg.tokens_per_frame, cfg.d_c + cfg.d_rope, dtype=torch.bfloat16,
                         device="cuda")
        sb = torch.full((B, cfg.window_frames), -1, dtype=torch.int32, device="cuda")
        ts = []
        for i in range(6):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            mla.cache_write(shp, xb, w["w_dkv"], w["w_kr"], 0, nf, cb, sb)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        rows = B * nf * cfg.tokens_per_frame
        byts = rows * cfg.hidden * 2 + (cfg.d_c + cfg.d_rope) * cfg.hidden * 2 + rows * (cfg.d_c + cfg.d_rope) * 2
        ms = float(np.median(ts[1:]))
        big_writes[label] = {"bytes": byts, "ms": round(ms, 4), "GBps": round(byts / (ms * 1e-3) / 1e9, 1),
                             "hbm_frac": round(byts / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
        del xb, cb, sb

    fl = step_flops(cfg)
    cw_bytes = cache_write_bytes(cfg)
    flash_tflops = fl["flash"] / (per["flash_attend"] * 1e-3) / 1e12
    ceiling = mfma_ceiling()
    traffic = None
    if os.path.exists(COUNTERS_FILE):
        rec = json.load(open(COUNTERS_FILE))
        if rec.get("source_hash") == flash_source_hash():
            traffic = rec.get("hbm_bytes_per_launch")
    result = {
        "metric": METRIC,
        "value": round(fl["total"] / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Wan2.1-1.3B-shaped layer, 3-frame chunk (4680 queries) over a full 21-frame "
                               "window (32760 latent tokens), batch 1",
                   "hidden": cfg.hidden, "n_heads": cfg.n_heads, "d_head": cfg.d_head, "d_c": cfg.d_c,
                   "d_rope": cfg.d_rope, "rope_split": list(cfg.rope_split), "grid": [cfg.grid_y, cfg.grid_x],
                   "chunk_frames": cfg.chunk_frames, "window_frames": cfg.window_frames, "batch": 1,
                   "kv_splits": args.kv_splits},
        "roofline": {"kernel": "mla_flash_attend (" + " + ".join(FLASH_KERNELS) + ")", "bound": "mfma",
                     "achieved": round(flash_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(flash_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "flops_per_launch": fl["flash"],
                     "frac_of_attainable": round(flash_tflops / ceiling["TFLOPs"], 4) if ceiling else None},
        "mfma_attainable": ceiling,
        "cache_write_GBps": round(cw_bytes / (per["cache_write"] * 1e-3) / 1e9, 1),
        "cache_write_cold_GBps": round(cw_bytes / (cold * 1e-3) / 1e9, 1) if cold else None,
        "cache_write_hbm_frac_cold": round(cw_bytes / (cold * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4) if cold else None,
        "kernel_ms": {k: round(v, 4) for k, v in per.items()},
        "cache_write_cold_ms": round(cold, 4) if cold else None,
        "cache_write_graph": graph_writes,
        "cache_write_large": big_writes,
        "copy_reference": {"what": "device copy of a 14.38 MB x buffer (cold, single launches), reads + writes",
                           "bytes": copy_bytes, "ms": round(copy_single, 4),
                           "GBps": round(copy_bytes / (copy_single * 1e-3) / 1e9, 1)} if cold else None,
        "flash_TFLOPs_nonabsorbed_equiv": round(fl["flash_nonabsorbed_equiv"] / (per["flash_attend"] * 1e-3) / 1e12,
                                                2),
        "step_flops": fl["total"],
        "cache_write_bytes": cw_bytes,
        "clock_settle": settle,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline: oracle on {args.cpu_sample_tokens} query tokens", file=sys.stderr,
              flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_sample_tokens, gpu_out=ctx.out.float().cpu().numpy())
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
