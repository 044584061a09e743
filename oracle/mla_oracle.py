"""fp64 CPU oracle for the VideoMLA latent-KV streaming chunk-attention step.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module; the product path never does. It shares no
code with the HIP path and imports nothing from it.

Sources (web pages on "VideoMLA: Low-Rank Latent KV Cache for Minute-Scale
Autoregressive Video Diffusion"):
  [Method]    hyper.ai paper summary, "Method" section (same text on its
              Chinese and Korean editions).
  [Abstract]  chatpaper.ai, English abstract.
  [Fig. 1]    ai-papers.net explainer, the architecture paragraph under Fig. 1
              (192-d content latent, 3D-RoPE, 3072 -> 224 scalars per token).

What is computed, per layer and per stream:
  c_j   = W_dkv x_j                     content latent, written to the cache  [Method]
  kR_j  = W_kR  x_j                     one head-shared positional key, stored
                                        unrotated                             [Method]
  k_jh  = W_uk[h] c_j,  v_jh = W_uv[h] c_j   per-head reconstruction          [Method]
  k^rope_j = R(t_j, y_j, x_j) kR_j      3D-RoPE applied at attention time     [Method], [Fig. 1]
  s_ijh = scale (q_ih . k_jh + R(p_i) qR_ih . k^rope_j)   content + positional [Method]
  o_ih  = sum_j softmax_j(s_ijh) v_jh   over every valid key of the sliding
                                        window, the chunk's own frames included [Abstract]
Query path and output (layer_step):
  cQ_i  = W_dq x_i                      query latent of the token             [Method]
  q_ih  = W_uq[h] cQ_i,  qR_ih = W_qr[h] cQ_i   per-head content query and
                                        unrotated positional query            [Method]
  u_i   = W_o [o_i1 ; ... ; o_iH]       output projection of the concatenated
                                        heads (reading: standard multi-head
                                        attention; the pages do not name it)

Readings where the pages are silent (each one is listed with its reason in
the design notes of the repository):
  * RoPE rotates interleaved pairs (2k, 2k+1); each axis a in (t, y, x) owns a
    contiguous block of d_a dims in that order, with angle pos * base^(-2k/d_a).
  * Token order inside a frame is row-major (y major); y, x are 0-based; t is
    the absolute latent-frame index.
  * scale defaults to 1/sqrt(d_head + d_rope).
  * Every query attends every valid window key (no intra-chunk mask); a query
    with no valid key outputs zeros.
  * Frame-causal variant (chunk-wise autoregressive reading, hyper.ai summary,
    Method, and chatpaper.ai abstract): a query of frame f attends only keys of
    frames <= f; earlier chunks are wholly visible and the query's own frame is
    visible. Off unless asked for.
  * The ring buffer keeps frame f in slot f mod W; a slot is valid iff its
    recorded frame index is >= 0.
  * Query path: the pages derive the query latent from the token and the
    per-head positional query from the query latent; the per-head content
    query is read as coming from the same latent through its own per-head
    up-projection. Its width d_cq is not given; no normalisation is applied
    between the projections (none is named).

Functions marked "absorbed" re-associate the same products (the GPU's form);
they are used for stage-by-stage checks and as a self-check, never as the
reference for the full step, which reconstructs keys and values explicitly.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "default_scale", "rope_inv_freq", "rope_axis_cos_sin", "rope_tables", "rope_tables_flat",
    "rotate_pairs", "rope3d", "frame_positions", "latents", "reconstruct", "attend",
    "RingCache", "chunk_step", "absorbed_query", "attend_latent", "up_project", "frame_causal_mask",
    "chunk_step_absorbed", "cache_scalars_per_token", "dense_scalars_per_token",
    "query_project", "output_project", "layer_step",
]


# ---------------------------------------------------------------- counts [Method], [Fig. 1]

def cache_scalars_per_token(d_c: int, d_rope: int) -> int:
    """Scalars one cached token holds per layer: the content latent plus the
    shared positional key [Method]."""
    return d_c + d_rope


def dense_scalars_per_token(n_heads: int, d_head: int) -> int:
    """Scalars a dense per-head K/V cache holds per token per layer [Method]."""
    return 2 * n_heads * d_head


def default_scale(d_head: int, d_rope: int) -> float:
    """Softmax temperature 1/sqrt(width of the two-part score) (a reading: the
    pages give no scale)."""
    return 1.0 / np.sqrt(d_head + d_rope)


# ---------------------------------------------------------------- 3D-RoPE [Method], [Fig. 1]

def rope_inv_freq(d_axis: int, base: float) -> np.ndarray:
    """Per-pair angular frequencies base^(-2k/d_axis), k = 0 .. d_axis/2 - 1."""
    k = np.arange(d_axis // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * k / d_axis)


def rope_axis_cos_sin(pos, d_axis: int, base: float):
    """cos and sin of pos * base^(-2k/d_axis): arrays [len(pos), d_axis/2]."""
    ang = np.asarray(pos, dtype=np.float64)[:, None] * rope_inv_freq(d_axis, base)[None, :]
    return np.cos(ang), np.sin(ang)


def rope_tables(split, base: float, t_first: int, n_t: int, grid_y: int, grid_x: int) -> dict:
    """cos/sin per axis: t over [t_first, t_first + n_t), y over the grid rows,
    x over the grid columns."""
    d_t, d_y, d_x = split
    return {
        "t": rope_axis_cos_sin(np.arange(t_first, t_first + n_t), d_t, base),
        "y": rope_axis_cos_sin(np.arange(grid_y), d_y, base),
        "x": rope_axis_cos_sin(np.arange(grid_x), d_x, base),
    }


def rope_tables_flat(split, base, t_first, n_t, grid_y, grid_x) -> np.ndarray:
    """The tables above concatenated as cos_t, sin_t, cos_y, sin_y, cos_x, sin_x,
    each row-major [positions][pairs]."""
    tb = rope_tables(split, base, t_first, n_t, grid_y, grid_x)
    parts = []
    for a in ("t", "y", "x"):
        c, s = tb[a]
        parts += [c.ravel(), s.ravel()]
    return np.concatenate(parts)


def rotate_pairs(v: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate each interleaved pair (v[2k], v[2k+1]) by the angle whose cos/sin
    are given (broadcast over the leading axes)."""
    v0 = v[..., 0::2]
    v1 = v[..., 1::2]
    out = np.empty(np.broadcast_shapes(v.shape), dtype=np.float64)
    out[..., 0::2] = v0 * cos - v1 * sin
    out[..., 1::2] = v0 * sin + v1 * cos
    return out


def rope3d(v: np.ndarray, t, y, x, split, base: float) -> np.ndarray:
    """3D-RoPE: v has tokens on axis 0 and the rotary dims on the last axis
    (any axes between, e.g. heads, share the token's position). The first d_t
    dims rotate with t, the next d_y with y, the last d_x with x."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[0]
    mid = (1,) * (v.ndim - 2)
    out = np.empty_like(v)
    o = 0
    for pos, d in ((t, split[0]), (y, split[1]), (x, split[2])):
        c, s = rope_axis_cos_sin(np.broadcast_to(np.asarray(pos), (n,)), d, base)
        c = c.reshape((n,) + mid + (d // 2,))
        s = s.reshape((n,) + mid + (d // 2,))
        out[..., o:o + d] = rotate_pairs(v[..., o:o + d], c, s)
        o += d
    return out


def frame_positions(frames, grid_y: int, grid_x: int):
    """(t, y, x) of every token of the given frames, frame-major, row-major
    inside a frame."""
    frames = np.asarray(frames, dtype=np.int64)
    tok = np.arange(grid_y * grid_x)
    t = np.repeat(frames, grid_y * grid_x)
    y = np.tile(tok // grid_x, len(frames))
    x = np.tile(tok % grid_x, len(frames))
    return t, y, x


# ---------------------------------------------------------------- projections [Method]

def latents(x: np.ndarray, w_dkv: np.ndarray, w_kr: np.ndarray):
    """Joint down-projection c = W_dkv x and positional key kR = W_kR x for each
    token row of x [N, hidden]: returns c [N, d_c], kR [N, d_rope]."""
    x = np.asarray(x, dtype=np.float64)
    return x @ np.asarray(w_dkv, np.float64).T, x @ np.asarray(w_kr, np.float64).T


def reconstruct(c: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray):
    """Per-head keys and values from the shared latent: k[j, h] = W_uk[h] c_j,
    v[j, h] = W_uv[h] c_j. c [N, d_c], W [n_h, d_h, d_c] -> [N, n_h, d_h] each."""
    c = np.asarray(c, np.float64)
    k = np.einsum("hdc,nc->nhd", np.asarray(w_uk, np.float64), c, optimize=True)
    v = np.einsum("hdc,nc->nhd", np.asarray(w_uv, np.float64), c, optimize=True)
    return k, v


# ---------------------------------------------------------------- attention [Method], [Abstract]

def frame_causal_mask(q_frames, k_frames) -> np.ndarray:
    """visible[i, j] = key j's frame <= query i's frame (the frame-causal variant)."""
    return np.asarray(q_frames)[:, None] >= np.asarray(k_frames)[None, :]


def _masked_softmax_rows(s: np.ndarray, visible) -> np.ndarray:
    """Row softmax of s [..., Nk] over the keys marked visible (all when None);
    rows with no visible key get all-zero weights."""
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m)
    tot = p.sum(axis=-1, keepdims=True)
    return np.divide(p, tot, out=np.zeros_like(p), where=tot > 0)


def attend(q_nope, q_rope, k_nope, k_rope, v, scale: float, block: int = 64, visible=None) -> np.ndarray:
    """Two-part-score softmax attention with explicit per-head keys and values.

    q_nope [Nq, H, dh], q_rope [Nq, H, dr] (already rotated), k_nope [Nk, H, dh],
    k_rope [Nk, dr] (already rotated, shared by all heads), v [Nk, H, dh].
    Softmax over all Nk keys (or over the keys visible[i] marks for query i),
    max-subtracted, two passes. Returns [Nq, H, dh]; zeros for a query with no
    key.
    """
    q_nope = np.asarray(q_nope, np.float64)
    nq, nh, dh = q_nope.shape
    out = np.zeros((nq, nh, v.shape[-1] if np.ndim(v) == 3 else dh))
    if k_nope.shape[0] == 0:
        return out
    kn = np.ascontiguousarray(np.transpose(k_nope, (1, 2, 0)))  # [H, dh, Nk]
    vv = np.ascontiguousarray(np.transpose(v, (1, 0, 2)))  # [H, Nk, dh]
    krt = np.ascontiguousarray(np.asarray(k_rope, np.float64).T)  # [dr, Nk]
    for i0 in range(0, nq, block):
        i1 = min(nq, i0 + block)
        qn = np.transpose(q_nope[i0:i1], (1, 0, 2))  # [H, b, dh]
        qr = np.transpose(np.asarray(q_rope[i0:i1], np.float64), (1, 0, 2))  # [H, b, dr]
        s = (np.matmul(qn, kn) + np.matmul(qr, krt)) * scale  # [H, b, Nk]
        p = _masked_softmax_rows(s, None if visible is None else visible[None, i0:i1])
        out[i0:i1] = np.transpose(np.matmul(p, vv), (1, 0, 2))
    return out


# ---------------------------------------------------------------- ring-buffer window [Abstract]

class RingCache:
    """Sliding window of W frames: frame f lives in slot f mod W; writing a
    frame evicts whatever the slot held. slot_frame[s] = -1 marks an empty slot."""

    def __init__(self, window_frames: int, tokens_per_frame: int, d_c: int, d_rope: int):
        self.W, self.T = window_frames, tokens_per_frame
        self.slot_frame = np.full(window_frames, -1, dtype=np.int32)
        self.c = np.zeros((window_frames, tokens_per_frame, d_c))
        self.kr = np.zeros((window_frames, tokens_per_frame, d_rope))

    def write(self, frame_first: int, c_rows: np.ndarray, kr_rows: np.ndarray) -> None:
        n = c_rows.shape[0] // self.T
        if n > self.W:
            raise ValueError("more frames than the window holds")
        for i in range(n):
            f = frame_first + i
            s = f % self.W
            self.slot_frame[s] = f
            self.c[s] = c_rows[i * self.T:(i + 1) * self.T]
            self.kr[s] = kr_rows[i * self.T:(i + 1) * self.T]

    def valid_slots(self) -> np.ndarray:
        return np.nonzero(self.slot_frame >= 0)[0]

    def keys(self, grid_y: int, grid_x: int):
        """Latents and positions of every valid slot: c [Nk, d_c], kR [Nk, dr], t, y, x."""
        slots = self.valid_slots()
        c = self.c[slots].reshape(-1, self.c.shape[-1])
        kr = self.kr[slots].reshape(-1, self.kr.shape[-1])
        t, y, x = frame_positions(self.slot_frame[slots], grid_y, grid_x)
        return c, kr, t, y, x


def chunk_step(cfg_dims: dict, w: dict, ring: RingCache, x_chunk, frame_first: int,
               q_nope, q_r, scale: float | None = None, write: bool = True,
               frame_causal: bool = False) -> np.ndarray:
    """One layer's streaming chunk step for one stream, reconstructing per-head
    keys and values explicitly (no absorption).

    cfg_dims: d_head, d_rope, rope_split, rope_base, grid_y, grid_x.
    w: w_dkv, w_kr, w_uk, w_uv. x_chunk [n_frames*T, hidden] are the chunk's
    tokens (frames frame_first ..), q_nope/q_r their queries. Returns
    out [Nq, n_h, d_h]. frame_causal: a query of frame f sees keys of frames <= f.
    """
    gy, gx = cfg_dims["grid_y"], cfg_dims["grid_x"]
    split, base = cfg_dims["rope_split"], cfg_dims["rope_base"]
    if scale is None:
        scale = default_scale(cfg_dims["d_head"], cfg_dims["d_rope"])
    if write:
        c_new, kr_new = latents(x_chunk, w["w_dkv"], w["w_kr"])
        ring.write(frame_first, c_new, kr_new)
    c, kr, t, y, x = ring.keys(gy, gx)
    k_nope, v = reconstruct(c, w["w_uk"], w["w_uv"])
    k_rope = rope3d(kr, t, y, x, split, base)
    nq = np.asarray(q_nope).shape[0]
    tq, yq, xq = frame_positions(frame_first + np.arange(nq // (gy * gx)), gy, gx)
    q_rope = rope3d(q_r, tq, yq, xq, split, base)
    visible = frame_causal_mask(tq, t) if frame_causal else None
    return attend(q_nope, q_rope, k_nope, k_rope, v, scale, visible=visible)


# ---------------------------------------------------------------- query path and output [Method]

def query_project(x, w_dq, w_uq, w_qr):
    """Query latent and per-head queries of tokens x [N, hidden]:
    cQ = x W_dq^T [N, d_cq]; q_nope[i, h] = W_uq[h] cQ_i [N, H, d_h];
    q_r[i, h] = W_qr[h] cQ_i [N, H, d_rope], unrotated (the rotation belongs to
    the attention, where the query's position is known)."""
    x = np.asarray(x, np.float64)
    c_q = x @ np.asarray(w_dq, np.float64).T
    q_nope = np.einsum("nc,hdc->nhd", c_q, np.asarray(w_uq, np.float64), optimize=True)
    q_r = np.einsum("nc,hdc->nhd", c_q, np.asarray(w_qr, np.float64), optimize=True)
    return c_q, q_nope, q_r


def output_project(o, w_o) -> np.ndarray:
    """u_i = W_o [o_i1 ; ... ; o_iH]: o [N, H, d_h], W_o [hidden, H*d_h] -> [N, hidden]."""
    o = np.asarray(o, np.float64)
    return o.reshape(o.shape[0], -1) @ np.asarray(w_o, np.float64).T


def layer_step(cfg_dims: dict, w: dict, ring: RingCache, x_chunk, frame_first: int, scale: float | None = None,
               frame_causal: bool = False):
    """The whole attention layer for one chunk of one stream: the chunk's tokens
    give the queries (query_project) and, through the cache write, keys of the
    window; the heads' outputs are projected back to the token width.
    w additionally holds w_dq, w_uq, w_qr, w_o. Returns (u [Nq, hidden],
    out [Nq, H, d_h], q_nope, q_r)."""
    _, q_nope, q_r = query_project(x_chunk, w["w_dq"], w["w_uq"], w["w_qr"])
    out = chunk_step(cfg_dims, w, ring, x_chunk, frame_first, q_nope, q_r, scale=scale, frame_causal=frame_causal)
    return output_project(out, w["w_o"]), out, q_nope, q_r


# ---------------------------------------------------------------- absorbed form (stage checks)

def absorbed_query(q_nope, q_r, w_uk, t, y, x, split, base) -> np.ndarray:
    """Absorbed query: [W_uk[h]^T q_nope_ih ; R(p_i) qR_ih] -> [Nq, H, d_c + d_rope].
    W_uk[h]^T q . c equals q . (W_uk[h] c), so this query scores latents directly."""
    qa = np.einsum("qhd,hdc->qhc", np.asarray(q_nope, np.float64), np.asarray(w_uk, np.float64),
                   optimize=True)
    qr = rope3d(q_r, t, y, x, split, base)
    return np.concatenate([qa, qr], axis=-1)


def attend_latent(q_abs, c, k_rope, scale: float, block: int = 64, visible=None) -> np.ndarray:
    """Attention in latent space: s = scale * q_abs . [c ; k_rope], softmax over
    keys (those visible[i] marks, when given), output sum_j p_j c_j.
    q_abs [Nq, H, d_c + dr], c [Nk, d_c], k_rope [Nk, dr] (rotated). Returns
    [Nq, H, d_c]; zeros for a query with no key."""
    q_abs = np.asarray(q_abs, np.float64)
    nq, nh, _ = q_abs.shape
    dc = c.shape[-1]
    out = np.zeros((nq, nh, dc))
    if c.shape[0] == 0:
        return out
    kt = np.ascontiguousarray(np.concatenate([c, k_rope], axis=-1).T)  # [dc+dr, Nk]
    for i0 in range(0, nq, block):
        i1 = min(nq, i0 + block)
        s = (q_abs[i0:i1].reshape(-1, q_abs.shape[-1]) @ kt) * scale  # [b*H, Nk]
        vis = None if visible is None else np.repeat(visible[i0:i1], nh, axis=0)
        p = _masked_softmax_rows(s, vis)
        out[i0:i1] = (p @ c).reshape(i1 - i0, nh, dc)
    return out


def up_project(o_lat, w_uv) -> np.ndarray:
    """o_ih = W_uv[h] o_lat_ih: [Nq, H, d_c] -> [Nq, H, d_h]."""
    return np.einsum("hdc,qhc->qhd", np.asarray(w_uv, np.float64), np.asarray(o_lat, np.float64),
                     optimize=True)


def chunk_step_absorbed(cfg_dims: dict, w: dict, ring: RingCache, frame_first: int, q_nope, q_r,
                        scale: float | None = None) -> np.ndarray:
    """Self-check only: the same step through the absorbed query (the ring must
    already hold the chunk)."""
    gy, gx = cfg_dims["grid_y"], cfg_dims["grid_x"]
    split, base = cfg_dims["rope_split"], cfg_dims["rope_base"]
    if scale is None:
        scale = default_scale(cfg_dims["d_head"], cfg_dims["d_rope"])
    c, kr, t, y, x = ring.keys(gy, gx)
    k_rope = rope3d(kr, t, y, x, split, base)
    nq = np.asarray(q_nope).shape[0]
    tq, yq, xq = frame_positions(frame_first + np.arange(nq // (gy * gx)), gy, gx)
    qa = absorbed_query(q_nope, q_r, w["w_uk"], tq, yq, xq, split, base)
    return up_project(attend_latent(qa, c, k_rope, scale), w["w_uv"])


def dims_of(cfg) -> dict:
    """The dimension fields chunk_step needs, read off any object that has them."""
    return dict(d_head=cfg.d_head, d_rope=cfg.d_rope, rope_split=tuple(cfg.rope_split),
                rope_base=cfg.rope_base, grid_y=cfg.grid_y, grid_x=cfg.grid_x)
