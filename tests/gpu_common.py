"""Shared helpers of the GPU parity tests: seeded inputs on the device, the
oracle on the same rounded values, and the error gates."""
from __future__ import annotations

import numpy as np

from harness import chunk_queries, frame_tokens, layer_weights
from harness.torch_io import to_numpy, to_torch
from oracle import mla_oracle as O

# gates: bf16 inputs with fp32 accumulation, and the fp32 configuration
BF16_MAX_ABS, BF16_MEAN_ABS, BF16_REL_RMS = 2e-2, 2e-3, 1e-2
F32_MAX_ABS = 1e-4


def errors(gpu: np.ndarray, ref: np.ndarray) -> dict:
    d = np.abs(gpu - ref)
    return dict(max_abs=float(d.max()) if d.size else 0.0, mean_abs=float(d.mean()) if d.size else 0.0,
                rel_rms=float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30)))


def assert_step_close(gpu, ref, dtype: str, label: str = "", sharp: bool = False):
    """bf16: max-abs <= 2e-2, mean-abs <= 2e-3 and relative RMS <= 1e-2; fp32:
    max-abs <= 1e-4. sharp=True (queries scaled up, outputs several times
    larger than at the nominal distribution, where the absolute bf16 gates are
    stated) keeps the relative-RMS gate and scales the absolute ones by the
    output's RMS relative to 0.1."""
    e = errors(gpu, ref)
    print(f"[parity] {label} {e}", flush=True)
    if dtype == "bf16":
        k = max(1.0, float(np.sqrt(np.mean(ref ** 2))) / 0.1) if sharp else 1.0
        assert (e["max_abs"] <= BF16_MAX_ABS * k and e["mean_abs"] <= BF16_MEAN_ABS * k
                and e["rel_rms"] <= BF16_REL_RMS), e
    else:
        assert e["max_abs"] <= F32_MAX_ABS * (max(1.0, float(np.abs(ref).max())) if sharp else 1.0), e
    assert np.isfinite(gpu).all()


def assert_rounded_close(gpu, ref, dtype: str, rel=None, abs_=1e-5, label=""):
    """Stage outputs stored in `dtype`: bf16 allows the final round to nearest
    (half an ulp, 2^-9 relative) plus fp32 accumulation error."""
    rel = rel if rel is not None else (2.0 ** -8 if dtype == "bf16" else 1e-5)
    d = np.abs(gpu - ref)
    bound = rel * np.abs(ref) + abs_
    bad = d > bound
    print(f"[stage] {label} max_abs={d.max() if d.size else 0:.3e} violations={int(bad.sum())}", flush=True)
    assert not bad.any(), (label, float(d.max()), int(bad.sum()))


class Stream:
    """One stream's seeded frames/queries, on the host (rounded float64)."""

    def __init__(self, cfg, seed=0, stream=0, layer=0, pooled=False):
        self.cfg, self.seed, self.stream, self.layer, self.pooled = cfg, seed, stream, layer, pooled

    def x(self, frame):
        return frame_tokens(self.cfg, frame, self.seed, self.stream, self.layer, pooled=self.pooled)

    def xs(self, first, n):
        return np.concatenate([self.x(first + i) for i in range(n)])

    def q(self, first, q_scale=1.0, n_frames=None):
        return chunk_queries(self.cfg, first, self.seed, self.stream, self.layer, q_scale=q_scale, n_frames=n_frames)


def device_weights(cfg, seed=0, layer=0):
    w = layer_weights(cfg, seed, layer)
    return w, {k: to_torch(v, cfg.dtype) for k, v in w.items()}


def oracle_step_rows(cfg, w, stream_frames_x: dict, window_frames, q_nope, q_r, q_frame_first, rows=None,
                     frame_causal=False):
    """Oracle output for the chosen query rows (all heads, full window; under
    the frame-causal mask when asked)."""
    c_list, kr_list = [], []
    for f in window_frames:
        c, kr = O.latents(stream_frames_x[f], w["w_dkv"], w["w_kr"])
        c_list.append(c)
        kr_list.append(kr)
    c = np.concatenate(c_list) if c_list else np.zeros((0, cfg.d_c))
    kr = np.concatenate(kr_list) if kr_list else np.zeros((0, cfg.d_rope))
    t, y, x = O.frame_positions(list(window_frames), cfg.grid_y, cfg.grid_x)
    k_nope, v = O.reconstruct(c, w["w_uk"], w["w_uv"])
    k_rope = O.rope3d(kr, t, y, x, cfg.rope_split, cfg.rope_base)
    nq = q_nope.shape[0]
    tq, yq, xq = O.frame_positions(q_frame_first + np.arange(nq // cfg.tokens_per_frame), cfg.grid_y, cfg.grid_x)
    if rows is None:
        rows = np.arange(nq)
    q_rope = O.rope3d(q_r[rows], tq[rows], yq[rows], xq[rows], cfg.rope_split, cfg.rope_base)
    visible = O.frame_causal_mask(tq[rows], t) if frame_causal else None
    return O.attend(q_nope[rows], q_rope, k_nope, k_rope, v, O.default_scale(cfg.d_head, cfg.d_rope),
                    visible=visible)


class LatentMemo:
    """Oracle latents (c, kR) of one stream's frames under one layer's weights,
    computed once per frame and reused across chunks."""

    def __init__(self, cfg, w, stream: Stream):
        self.cfg, self.w, self.stream, self.memo = cfg, w, stream, {}

    def get(self, f):
        if f not in self.memo:
            self.memo[f] = O.latents(self.stream.x(f), self.w["w_dkv"], self.w["w_kr"])
        return self.memo[f]


def oracle_rows_memo(cfg, w, memo: LatentMemo, window_frames, q_nope, q_r, q_frame_first, rows, frame_causal=False):
    """oracle_step_rows with the window's latents taken from a LatentMemo."""
    window_frames = list(window_frames)
    c = np.concatenate([memo.get(f)[0] for f in window_frames])
    kr = np.concatenate([memo.get(f)[1] for f in window_frames])
    t, y, x = O.frame_positions(window_frames, cfg.grid_y, cfg.grid_x)
    k_nope, v = O.reconstruct(c, w["w_uk"], w["w_uv"])
    k_rope = O.rope3d(kr, t, y, x, cfg.rope_split, cfg.rope_base)
    nq = q_nope.shape[0]
    tq, yq, xq = O.frame_positions(q_frame_first + np.arange(nq // cfg.tokens_per_frame), cfg.grid_y, cfg.grid_x)
    q_rope = O.rope3d(q_r[rows], tq[rows], yq[rows], xq[rows], cfg.rope_split, cfg.rope_base)
    visible = O.frame_causal_mask(tq[rows], t) if frame_causal else None
    return O.attend(q_nope[rows], q_rope, k_nope, k_rope, v, O.default_scale(cfg.d_head, cfg.d_rope),
                    visible=visible)


def sample_rows(cfg, n, seed):
    """n query rows of a chunk: first/last, frame and 128-key-tile boundaries, random rest."""
    T, nq = cfg.tokens_per_frame, cfg.chunk_frames * cfg.tokens_per_frame
    edge = [r for r in (0, 1, 10, 11, 21, 22, T - 1, T, nq // 2, nq - 22, nq - 1) if r < nq]
    rng = np.random.default_rng(seed)
    rest = rng.choice(nq, max(0, n - len(edge)), replace=False)
    return np.unique(np.concatenate([edge, rest]).astype(np.int64))


__all__ = ["errors", "assert_step_close", "assert_rounded_close", "Stream", "device_weights", "oracle_step_rows",
           "LatentMemo", "oracle_rows_memo", "sample_rows", "to_numpy", "to_torch"]
