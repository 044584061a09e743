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
        nf = max_chunk_frames or cfg.chunk_frames
        # RoPE tables: the queries' frames must lie in their t range (the
        # window keys' temporal angles are formed by the attention call for
        # any frame); the range moves with the chunks (ensure_tables)
        self.rope_t_first, self.rope_n_t = rope_t_first, max(rope_n_t, nf)
        self.tables = torch.empty(_lib.rope3d_table_floats(self.shape, self.rope_n_t), dtype=torch.float32,
                                  device=device)
        _lib.rope3d_tables(self.shape, self.rope_t_first, self.rope_n_t, self.tables)
        self.max_chunk_frames = nf
        self.workspace = torch.empty(_lib.chunk_attend_workspace_bytes(self.shape, nf), dtype=torch.uint8,
                                     device=device)
        self.heads_workspace = None  # allocated on the first per-head call
        self.q_buffers = None        # query latent and queries, allocated on the first projection
        self.layer_workspace = None  # (d_cq, workspace, weight struct) of step(), allocated on its first call

    def ensure_tables(self, frame_first: int, n_frames: int, stream=None) -> None:
        """Move the tables' t range so that it covers frames frame_first ..
        frame_first + n_frames - 1 (a rollout runs past any fixed range): the
        range restarts at frame_first, same length, refilled on `stream`."""
        if frame_first >= self.rope_t_first and frame_first + n_frames <= self.rope_t_first + self.rope_n_t:
            return
        if frame_first < 0 or n_frames > self.rope_n_t:
            raise ValueError("query frames outside what the RoPE tables can cover")
        self.rope_t_first = frame_first
        _lib.rope3d_tables(self.shape, self.rope_t_first, self.rope_n_t, self.tables, stream)

    def write(self, x, frame_first: int, n_frames: int, stream=None) -> None:
        """Cache write of frames frame_first .. +n_frames (x [B][n_frames*T][hidden])."""
        _lib.cache_write(self.shape, x, self.w["w_dkv"], self.w["w_kr"], frame_first, n_frames, self.cache,
                         self.slot_frame, stream)

    def attend(self, q_nope, q_r, q_frame_first: int, q_n_frames: int, out=None, stream=None):
        """Attention of the chunk's queries over the window -> out [B][N_q][H][d_head]
        (mla_chunk_attend: the latent or the per-head form, by shape)."""
        if q_n_frames > self.max_chunk_frames:
            raise ValueError("chunk larger than the workspace was sized for")
        if out is None:
            out = torch.empty(self.B, q_n_frames * self.T, self.cfg.n_heads, self.cfg.d_head, dtype=self.dtype,
                              device=self.device)
        self.ensure_tables(q_frame_first, q_n_frames, stream)
        _lib.chunk_attend(self.shape, q_nope, q_r, q_frame_first, q_n_frames, self.w["w_uk"], self.w["w_uv"],
                          self.cache, self.slot_frame, self.tables, self.rope_t_first, self.rope_n_t, out,
                          self.workspace, stream)
        return out

    def attend_latent(self, q_nope, q_r, q_frame_first: int, q_n_frames: int, out=None, stream=None):
        """attend() by the latent form whatever the shape (mla_chunk_attend_latent)."""
        if q_n_frames > self.max_chunk_frames:
            raise ValueError("chunk larger than the workspace was sized for")
        if out is None:
            out = torch.empty(self.B, q_n_frames * self.T, self.cfg.n_heads, self.cfg.d_head, dtype=self.dtype,
                              device=self.device)
        self.ensure_tables(q_frame_first, q_n_frames, stream)
        _lib.chunk_attend_latent(self.shape, q_nope, q_r, q_frame_first, q_n_frames, self.w["w_uk"], self.w["w_uv"],
                                 self.cache, self.slot_frame, self.tables, self.rope_t_first, self.rope_n_t, out,
                                 self.workspace, stream)
        return out

    def _out(self, q_n_frames: int, out):
        if q_n_frames > self.max_chunk_frames:
            raise ValueError("chunk larger than the workspace was sized for")
        if out is None:
            out = torch.empty(self.B, q_n_frames * self.T, self.cfg.n_heads, self.cfg.d_head, dtype=self.dtype,
                              device=self.device)
        return out

    def _heads_ws(self):
        if self.heads_workspace is None:
            n = _lib.chunk_attend_heads_workspace_bytes(self.shape, self.max_chunk_frames)
            if n == 0:
                raise ValueError("the per-head form does not support this shape")
            self.heads_workspace = torch.empty(n, dtype=torch.uint8, device=self.device)
        return self.heads_workspace

    def attend_frame_causal(self, q_nope, q_r, q_frame_first: int, q_n_frames: int, out=None, stream=None):
        """attend() with the frame-causal mask inside the chunk (a query of frame
        f sees keys of frames <= f); the form as attend() takes it."""
        out = self._out(q_n_frames, out)
        self.ensure_tables(q_frame_first, q_n_frames, stream)
        _lib.chunk_attend_frame_causal(self.shape, q_nope, q_r, q_frame_first, q_n_frames, self.w["w_uk"],
                                       self.w["w_uv"], self.cache, self.slot_frame, self.tables, self.rope_t_first,
                                       self.rope_n_t, out, self.workspace, stream)
        return out

    def attend_latent_frame_causal(self, q_nope, q_r, q_frame_first: int, q_n_frames: int, out=None, stream=None):
        """attend_frame_causal() by the latent form whatever the shape."""
        out = self._out(q_n_frames, out)
        self.ensure_tables(q_frame_first, q_n_frames, stream)
        _lib.chunk_attend_latent_frame_causal(self.shape, q_nope, q_r, q_frame_first, q_n_frames, self.w["w_uk"],
                                              self.w["w_uv"], self.cache, self.slot_frame, self.tables,
                                              self.rope_t_first, self.rope_n_t, out, self.workspace, stream)
        return out

    def attend_heads(self, q_nope, q_r, q_frame_first: int, q_n_frames: int, out=None, stream=None):
        """Same as attend(), by the per-head form (keys and values of every head
        expanded for the window, then per-head attention)."""
        out = self._out(q_n_frames, out)
        ws = self._heads_ws()
        self.ensure_tables(q_frame_first, q_n_frames, stream)
        _lib.chunk_attend_heads(self.shape, q_nope, q_r, q_frame_first, q_n_frames, self.w["w_uk"], self.w["w_uv"],
                                self.cache, self.slot_frame, self.tables, self.rope_t_first, self.rope_n_t, out,
                                ws, stream)
        return out

    def attend_heads_frame_causal(self, q_nope, q_r, q_frame_first: int, q_n_frames: int, out=None, stream=None):
        """attend_frame_causal() by the per-head form."""
        out = self._out(q_n_frames, out)
        ws = self._heads_ws()
        self.ensure_tables(q_frame_first, q_n_frames, stream)
        _lib.chunk_attend_heads_frame_causal(self.shape, q_nope, q_r, q_frame_first, q_n_frames, self.w["w_uk"],
                                             self.w["w_uv"], self.cache, self.slot_frame, self.tables,
                                             self.rope_t_first, self.rope_n_t, out, ws, stream)
        return out

    def project_queries(self, x, n_frames: int, stream=None):
        """Query latent and per-head queries of the chunk's tokens x
        [B][n_frames*T][hidden] -> (c_q, q_nope, q_r), views of buffers this
        layer owns (overwritten by the next call). Needs w_dq, w_uq, w_qr."""
        if n_frames > self.max_chunk_frames:
            raise ValueError("chunk larger than the buffers were sized for")
        for k in ("w_dq", "w_uq", "w_qr"):
            if k not in self.w:
                raise ValueError(f"the query path needs {k}")
        d_cq = self.w["w_dq"].shape[0]
        H, n = self.cfg.n_heads, n_frames * self.T
        widths = (d_cq, H * self.cfg.d_head, H * self.cfg.d_rope)
        if self.q_buffers is None or self.q_buffers[0].numel() != self.B * self.max_chunk_frames * self.T * d_cq:
            rows = self.B * self.max_chunk_frames * self.T
            self.q_buffers = tuple(torch.empty(rows * w, dtype=self.dtype, device=self.device) for w in widths)
        # leading elements of the flat buffers, viewed [B][n][...] (contiguous)
        c_q = self.q_buffers[0][:self.B * n * d_cq].view(self.B, n, d_cq)
        q_nope = self.q_buffers[1][:self.B * n * widths[1]].view(self.B, n, H, self.cfg.d_head)
        q_r = self.q_buffers[2][:self.B * n * widths[2]].view(self.B, n, H, self.cfg.d_rope)
        _lib.query_project(self.shape, d_cq, x, n_frames, self.w["w_dq"], self.w["w_uq"], self.w["w_qr"], c_q, q_nope,
                           q_r, stream)
        return c_q, q_nope, q_r

    def absorb_query_weights(self, stream=None):
        """Compute the absorbed query weights [H][Q][d_cq] (W_uk[h]^T W_uq[h]
        stacked over W_qr[h]) once; from then on step() takes the fused query
        path and project_queries_absorbed() is available."""
        d_cq = self.w["w_dq"].shape[0]
        Q = _lib.qabs_dim(self.shape)
        w_qabs = torch.empty(self.cfg.n_heads, Q, d_cq, dtype=self.dtype, device=self.device)
        _lib.query_absorb_weights(self.shape, d_cq, self.w["w_uq"], self.w["w_qr"], self.w["w_uk"], w_qabs, stream)
        self.w = {**self.w, "w_qabs": w_qabs}
        self.layer_workspace = None  # the weight struct now carries w_qabs
        return w_qabs

    def project_queries_absorbed(self, x, q_frame_first: int, n_frames: int, stream=None):
        """(c_q, q_abs) of the chunk's tokens by the fused query path: q_abs
        [B][n_frames*T][H][Q] is the attention's input (scaled, rotated)."""
        if "w_qabs" not in self.w:
            raise ValueError("call absorb_query_weights() first")
        d_cq = self.w["w_dq"].shape[0]
        n = n_frames * self.T
        c_q = torch.empty(self.B, n, d_cq, dtype=self.dtype, device=self.device)
        q_abs = torch.empty(self.B, n, self.cfg.n_heads, _lib.qabs_dim(self.shape), dtype=self.dtype,
                            device=self.device)
        self.ensure_tables(q_frame_first, n_frames, stream)
        _lib.query_project_absorbed(self.shape, d_cq, x, q_frame_first, n_frames, self.w["w_dq"], self.w["w_qabs"],
                                    self.tables, self.rope_t_first, self.rope_n_t, c_q, q_abs, stream)
        return c_q, q_abs

    def project_output(self, o, n_frames: int, out=None, stream=None):
        """u = W_o [o_1; ...; o_H] for the heads' outputs o [B][n_frames*T][H][d_head]."""
        if "w_o" not in self.w:
            raise ValueError("the output projection needs w_o")
        if out is None:
            out = torch.empty(self.B, n_frames * self.T, self.cfg.hidden, dtype=self.dtype, device=self.device)
        _lib.output_project(self.shape, o, n_frames, self.w["w_o"], out, stream)
        return out

    def step(self, x, frame_first: int, n_frames: int, frame_causal: bool = False, out=None, stream=None):
        """The whole layer for one chunk in one library call (mla_layer_step):
        queries from the chunk's tokens, the cache write of the same tokens,
        the attention over the window, and the output projection
        -> u [B][n_frames*T][hidden]. Needs all eight weights; after
        absorb_query_weights() the queries take the fused path."""
        if n_frames > self.max_chunk_frames:
            raise ValueError("chunk larger than the workspace was sized for")
        for k in ("w_dq", "w_uq", "w_qr", "w_o"):
            if k not in self.w:
                raise ValueError(f"the layer step needs {k}")
        d_cq = self.w["w_dq"].shape[0]
        if self.layer_workspace is None or self.layer_workspace[0] != d_cq:
            n = _lib.layer_step_workspace_bytes(self.shape, d_cq, self.max_chunk_frames)
            if n == 0:
                raise ValueError("the layer step does not support this shape")
            self.layer_workspace = (d_cq, torch.empty(n, dtype=torch.uint8, device=self.device),
                                    _lib.layer_weights_struct(self.w))
        if out is None:
            out = torch.empty(self.B, n_frames * self.T, self.cfg.hidden, dtype=self.dtype, device=self.device)
        self.ensure_tables(frame_first, n_frames, stream)
        _lib.layer_step(self.shape, d_cq, self.layer_workspace[2], x, frame_first, n_frames, self.cache,
                        self.slot_frame, self.tables, self.rope_t_first, self.rope_n_t, frame_causal, out,
                        self.layer_workspace[1], stream)
        return out

    def step_composed(self, x, frame_first: int, n_frames: int, frame_causal: bool = False, stream=None):
        """step() as four separate library calls (mla_query_project,
        mla_cache_write, mla_chunk_attend[_frame_causal], mla_output_project)."""
        _, q_nope, q_r = self.project_queries(x, n_frames, stream)
        self.write(x, frame_first, n_frames, stream)
        attend = self.attend_frame_causal if frame_causal else self.attend
        o = attend(q_nope, q_r, frame_first, n_frames, stream=stream)
        return self.project_output(o, n_frames, stream=stream)
