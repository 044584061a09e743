"""The chunk step (cache write, query absorb + rotate, latent attention,
up-projection) captured once in a HIP graph and replayed, for callers that
launch the same step repeatedly without the host launch path: every entry
point launches kernels only on the stream it is given (no allocation, no
memset node, no synchronisation), so the graph holds kernel nodes alone.
Each replay follows eager work that clears the step's outputs and the
chunk's cache rows, and must reproduce the eager step bit for bit; the
attention stage is taken both with a caller workspace and from the
library's fixed scratch (mla_flash_attend_noalloc)."""
import numpy as np
import pytest
import torch

import latent_kv_attention_amd as mla
from harness import chunk_queries, frame_tokens, get_config, layer_weights
from harness.torch_io import to_torch

pytestmark = pytest.mark.gpu

N_T = 64  # temporal rows of the RoPE tables


def _setup(name, seed):
    cfg = get_config(name)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    w = {k: to_torch(v, cfg.dtype, "cuda") for k, v in layer_weights(cfg, seed).items()}
    T, W, nf = cfg.tokens_per_frame, cfg.window_frames, cfg.chunk_frames
    first = W - nf
    shape = mla.make_shape(cfg, batch=1)
    cache = torch.zeros(1, W, T, cfg.d_c + cfg.d_rope, dtype=dt, device="cuda")
    slot_frame = torch.full((1, W), -1, dtype=torch.int32, device="cuda")
    x_pre = to_torch(np.concatenate([frame_tokens(cfg, f, seed) for f in range(first)]), cfg.dtype, "cuda")
    mla.cache_write(shape, x_pre, w["w_dkv"], w["w_kr"], 0, first, cache, slot_frame)
    x = to_torch(np.concatenate([frame_tokens(cfg, first + i, seed) for i in range(nf)]), cfg.dtype, "cuda")
    qn_h, qr_h = chunk_queries(cfg, first, seed)
    tables = torch.empty(mla.rope3d_table_floats(shape, N_T), dtype=torch.float32, device="cuda")
    mla.rope3d_tables(shape, 0, N_T, tables)
    bufs = dict(
        x=x, qn=to_torch(qn_h, cfg.dtype, "cuda"), qr=to_torch(qr_h, cfg.dtype, "cuda"), cache=cache,
        slot_frame=slot_frame, tables=tables,
        q_abs=torch.empty(cfg.n_q, cfg.n_heads, mla.qabs_dim(shape), dtype=dt, device="cuda"),
        o_lat=torch.empty(cfg.n_q, cfg.n_heads, cfg.d_c, dtype=dt, device="cuda"),
        out=torch.empty(cfg.n_q, cfg.n_heads, cfg.d_head, dtype=dt, device="cuda"),
        ws=torch.empty(mla.flash_workspace_bytes(shape, nf, 0), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    return cfg, shape, w, first, bufs


def _step(cfg, shape, w, first, b, noalloc):
    nf = cfg.chunk_frames
    mla.cache_write(shape, b["x"], w["w_dkv"], w["w_kr"], first, nf, b["cache"], b["slot_frame"])
    mla.absorb_q(shape, b["qn"], b["qr"], first, nf, w["w_uk"], b["tables"], 0, N_T, b["q_abs"])
    if noalloc:
        mla.flash_attend_noalloc(shape, b["q_abs"], nf, b["cache"], b["slot_frame"], b["tables"], 0, N_T,
                                 b["o_lat"], 0)
    else:
        mla.flash_attend(shape, b["q_abs"], nf, b["cache"], b["slot_frame"], b["tables"], 0, N_T, b["o_lat"],
                         b["ws"], 0)
    mla.up_v(shape, b["o_lat"], nf, w["w_uv"], b["out"])


@pytest.mark.parametrize("name", ["tiny", "wan_small", "wan"])
@pytest.mark.parametrize("noalloc", [False, True])
def test_chunk_step_graph_replays_match_eager(name, noalloc):
    cfg, shape, w, first, b = _setup(name, seed=11)
    if noalloc and mla.flash_workspace_bytes(shape, cfg.chunk_frames, 0) > mla.NOALLOC_SCRATCH_BYTES:
        pytest.skip("attention workspace larger than the fixed scratch")
    slots = [(first + i) % cfg.window_frames for i in range(cfg.chunk_frames)]
    _step(cfg, shape, w, first, b, noalloc)
    torch.cuda.synchronize()
    ref_out, ref_rows = b["out"].clone(), b["cache"][:, slots].clone()
    assert torch.isfinite(ref_out.float()).all()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(cfg, shape, w, first, b, noalloc)
    for replay in range(3):
        # eager work between replays: clear what the step writes
        b["out"].fill_(float("nan"))
        b["o_lat"].zero_()
        b["q_abs"].zero_()
        b["cache"][:, slots] = 0
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(b["out"], ref_out), f"{name} replay {replay}: output differs from the eager step"
        assert torch.equal(b["cache"][:, slots], ref_rows), f"{name} replay {replay}: cache rows differ"
        assert b["slot_frame"][0, slots].tolist() == [first + i for i in range(cfg.chunk_frames)]
    del g
