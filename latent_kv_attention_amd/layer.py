"""Device state of one latent-KV attention layer for a set of streams.

Holds the weights, the ring cache [B][W][T][d_c + d_rope], the slot->frame
map, RoPE tables and the workspace as torch device tensors, and strings the
C-ABI calls together. Every computation runs in the HIP library; this class
only allocates device memory (once, at construction) and passes pointers.
"""
from __future__ import annotations

import torch

from . import _lib


class LatentLayer:
    def __init__(self, cfg, weights: dict, batch: int | None = None, rope_t_first: int = 0, rope_n_t: int = 256,
                 device: str = "cuda", max_chunk_frames: int | None = None):
        self.cfg = cfg
        self.shape = _lib.make_shape(cfg, batch=batch)
        self.B = self.shape.batch
        self.dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.device = device
        self.T = cfg.grid_y * cfg.grid_x
        for k in ("w_dkv", "w_kr", "w_uk", "w_uv"):
            w = weights[k]
            if w.dtype != self.dtype or w.device.type != "cuda":
                raise ValueError(f"{k} must be a {self.dtype} CUDA tensor")
        self.w = weights
        self.cache = torch.zeros(self.B, cfg.window_frames, self.T, cfg.d_c + cfg.d_rope, dtype=self.dtype,
                                 device=device)
        self.slot_frame = torch.full((self.B, cfg.window_frames), -1, dtype=torch.int32, device=device)
        self.rope_t_first, self.rope_n_t = rope_t_first, rope_n_t
        self.tables = torch.empty(_lib.rope3d_table_floats(self.shape, rope_n_t), dtype=torch.float32,
                                  device=device)
        _lib.rope3d_tables(self.shape, rope_t_first, rope_n_t, self.tables)
        nf = max_chunk_frames or cfg.chunk_frames
        self.max_chunk_frames = nf
        self.workspace = torch.empty(_lib.chunk_attend_workspace_bytes(self.shape, nf), dtype=torch.uint8,
                                     device=device)
        self.heads_workspace = None  # allocated on the first per-head call

    def write(self, x, frame_first: int, n_frames: int, stream=None) -> None:
        """Cache write of frames frame_first .. +n_frames (x [B][n_frames*T][hidden])."""
        _lib.cache_write(self.shape, x, self.w["w_dkv"], self.w["w_kr"], frame_first, n_frames, self.cache,
                         self.slot_frame, stream)

    def attend(self, q_nope, q_r, q_frame_first: int, q_n_frames: int, out=None, stream=None):
        """Attention of the chunk's queries over the window -> out [B][N_q][H][d_head]."""
        if q_n_frames > self.max_chunk_frames:
            raise ValueError("chunk larger than the workspace was sized for")
        if out is None:
            out = torch.empty(self.B, q_n_frames * self.T, self.cfg.n_heads, self.cfg.d_head, dtype=self.dtype,
                              device=self.device)
        _lib.chunk_attend(self.shape, q_nope, q_r, q_frame_first, q_n_frames, self.w["w_uk"], self.w["w_uv"],
                          self.cache, self.slot_frame, self.tables, self.rope_t_first, self.rope_n_t, out,
                          self.workspace, stream)
        return out

    def attend_frame_causal(self, q_nope, q_r, q_frame_first: int, q_n_frames: int, out=None, stream=None):
        """attend() with the frame-causal mask inside the chunk (a query of frame
        f sees keys of frames <= f)."""
        if q_n_frames > self.max_chunk_frames:
            raise ValueError("chunk larger than the workspace was sized for")
        if out is None:
            out = torch.empty(self.B, q_n_frames * self.T, self.cfg.n_heads, self.cfg.d_head, dtype=self.dtype,
                              device=self.device)
        _lib.chunk_attend_frame_causal(self.shape, q_nope, q_r, q_frame_first, q_n_frames, self.w["w_uk"],
                                       self.w["w_uv"], self.cache, self.slot_frame, self.tables, self.rope_t_first,
                                       self.rope_n_t, out, self.workspace, stream)
        return out

    def attend_heads(self, q_nope, q_r, q_frame_first: int, q_n_frames: int, out=None, stream=None):
        """Same as attend(), by the per-head form (keys and values of every head
        expanded for the window, then per-head attention)."""
        if q_n_frames > self.max_chunk_frames:
            raise ValueError("chunk larger than the workspace was sized for")
        if self.heads_workspace is None:
            n = _lib.chunk_attend_heads_workspace_bytes(self.shape, self.max_chunk_frames)
            if n == 0:
                raise ValueError("the per-head form does not support this shape")
            self.heads_workspace = torch.empty(n, dtype=torch.uint8, device=self.device)
        if out is None:
            out = torch.empty(self.B, q_n_frames * self.T, self.cfg.n_heads, self.cfg.d_head, dtype=self.dtype,
                              device=self.device)
        _lib.chunk_attend_heads(self.shape, q_nope, q_r, q_frame_first, q_n_frames, self.w["w_uk"], self.w["w_uv"],
                                self.cache, self.slot_frame, self.tables, self.rope_t_first, self.rope_n_t, out,
                                self.heads_workspace, stream)
        return out
