"""Seeded synthetic inputs for the latent-KV chunk-attention step.

Every draw uses numpy's PCG64 seeded from SeedSequence([seed, stream, layer,
tag, index]), so any frame, query chunk or weight can be regenerated alone.
Values are drawn in float64 and rounded once to the storage precision; the
CPU oracle and the HIP path then consume the same rounded values.

Distributions: x ~ N(0, 1) per token; weights ~ N(0, 1/fan_in) with fan_in =
hidden for the down-projections and d_c for the up-projections; the query
parts q_nope and q_rope ~ N(0, 1), which is the distribution of x·W_q with
W_q ~ N(0, 1/hidden) (the query projection itself is outside the step).
"""
from __future__ import annotations

import numpy as np

from .configs import MLAConfig

TAG_W_DKV, TAG_W_KR, TAG_W_UK, TAG_W_UV, TAG_X, TAG_QN, TAG_QR, TAG_POOL = range(1, 9)
TAG_W_DQ, TAG_W_UQ, TAG_W_QR, TAG_W_O = range(9, 13)


def _rng(seed: int, stream: int, layer: int, tag: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, layer, tag, index])))


def to_bf16_bits(a) -> np.ndarray:
    """Round to bfloat16 (round to nearest, ties to even, via float32) -> uint16 bits."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(f)
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def from_bf16_bits(b) -> np.ndarray:
    """uint16 bfloat16 bits -> float64 values."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def round_to(a, dtype: str) -> np.ndarray:
    """Round float64 values to the storage precision and return them as float64."""
    if dtype == "bf16":
        return from_bf16_bits(to_bf16_bits(a))
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def layer_weights(cfg: MLAConfig, seed: int = 0, layer: int = 0) -> dict:
    """Per-layer weights, rounded to cfg.dtype, as float64 arrays.

    w_dkv [d_c, hidden], w_kr [d_rope, hidden], w_uk [n_heads, d_head, d_c],
    w_uv [n_heads, d_head, d_c] (row h, i, : of w_uk maps the latent to
    component i of head h's key; likewise w_uv for the value).
    """
    h, dc, dr, nh, dh = cfg.hidden, cfg.d_c, cfg.d_rope, cfg.n_heads, cfg.d_head
    w_dkv = _rng(seed, 0, layer, TAG_W_DKV, 0).standard_normal((dc, h)) / np.sqrt(h)
    w_kr = _rng(seed, 0, layer, TAG_W_KR, 0).standard_normal((dr, h)) / np.sqrt(h)
    w_uk = _rng(seed, 0, layer, TAG_W_UK, 0).standard_normal((nh, dh, dc)) / np.sqrt(dc)
    w_uv = _rng(seed, 0, layer, TAG_W_UV, 0).standard_normal((nh, dh, dc)) / np.sqrt(dc)
    return {k: round_to(v, cfg.dtype) for k, v in
            dict(w_dkv=w_dkv, w_kr=w_kr, w_uk=w_uk, w_uv=w_uv).items()}


def query_weights(cfg: MLAConfig, seed: int = 0, layer: int = 0) -> dict:
    """Query-path and output weights of one layer, rounded to cfg.dtype.

    w_dq [d_cq, hidden], w_uq [n_heads, d_head, d_cq], w_qr [n_heads, d_rope, d_cq],
    w_o [hidden, n_heads * d_head]; d_cq = cfg.q_latent. Scaled by 1/sqrt(fan-in)
    so that queries and outputs keep unit-order entries for unit-order tokens.
    """
    h, dq, dr, nh, dh = cfg.hidden, cfg.q_latent, cfg.d_rope, cfg.n_heads, cfg.d_head
    w_dq = _rng(seed, 0, layer, TAG_W_DQ, 0).standard_normal((dq, h)) / np.sqrt(h)
    w_uq = _rng(seed, 0, layer, TAG_W_UQ, 0).standard_normal((nh, dh, dq)) / np.sqrt(dq)
    w_qr = _rng(seed, 0, layer, TAG_W_QR, 0).standard_normal((nh, dr, dq)) / np.sqrt(dq)
    w_o = _rng(seed, 0, layer, TAG_W_O, 0).standard_normal((h, nh * dh)) / np.sqrt(nh * dh)
    return {k: round_to(v, cfg.dtype) for k, v in dict(w_dq=w_dq, w_uq=w_uq, w_qr=w_qr, w_o=w_o).items()}


POOL_FRAMES = 64


def frame_tokens(cfg: MLAConfig, frame: int, seed: int = 0, stream: int = 0, layer: int = 0,
                 pooled: bool = False) -> np.ndarray:
    """Latent tokens x [tokens_per_frame, hidden] of one frame, rounded to cfg.dtype.

    pooled=True draws from a shared pool of 64 frames indexed by
    (frame + 7*layer + 13*stream) mod 64, for long multi-layer workloads where
    content does not matter for timing.
    """
    shape = (cfg.tokens_per_frame, cfg.hidden)
    if pooled:
        idx = (frame + 7 * layer + 13 * stream) % POOL_FRAMES
        g = _rng(seed, 0, 0, TAG_POOL, idx)
    else:
        g = _rng(seed, stream, layer, TAG_X, frame)
    return round_to(g.standard_normal(shape), cfg.dtype)


def chunk_queries(cfg: MLAConfig, chunk_frame_first: int, seed: int = 0, stream: int = 0,
                  layer: int = 0, q_scale: float = 1.0, n_frames: int | None = None):
    """Query parts of one chunk: q_nope [N_q, n_heads, d_head], q_r [N_q, n_heads, d_rope]
    (q_r unrotated), rounded to cfg.dtype. q_scale multiplies both before rounding
    (q_scale = 4 gives the sharp-softmax variant)."""
    nf = cfg.chunk_frames if n_frames is None else n_frames
    nq = nf * cfg.tokens_per_frame
    qn = _rng(seed, stream, layer, TAG_QN, chunk_frame_first).standard_normal((nq, cfg.n_heads, cfg.d_head))
    qr = _rng(seed, stream, layer, TAG_QR, chunk_frame_first).standard_normal((nq, cfg.n_heads, cfg.d_rope))
    return round_to(qn * q_scale, cfg.dtype), round_to(qr * q_scale, cfg.dtype)
