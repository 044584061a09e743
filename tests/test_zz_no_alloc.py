"""mla_flash_attend_noalloc (the attention stage with the library's fixed
per-GPU scratch instead of a caller workspace) against mla_flash_attend
with a caller workspace, through the C ABI: two calls in a row, the second
one smaller (the scratch then holds the first call's leftovers), both
bit-identical to the workspace entry point; and the host-side refusal of a
problem larger than the scratch."""
import numpy as np
import pytest
import torch

import latent_kv_attention_amd as mla
from harness import get_config

pytestmark = pytest.mark.gpu


def _inputs(cfg, batch, seed):
    """Seeded device inputs of the attention stage: a full ring (slot s holds
    frame s + 3), absorbed queries (padding columns zero), RoPE tables."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    shape = mla.make_shape(cfg, batch=batch)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    W, T = cfg.window_frames, cfg.tokens_per_frame
    Q = mla.qabs_dim(shape)
    nq = cfg.chunk_frames * T
    cache = torch.randn(batch, W, T, cfg.d_c + cfg.d_rope, generator=g, device="cuda").to(dt)
    slot_frame = (torch.arange(W, dtype=torch.int32, device="cuda") + 3).repeat(batch, 1).contiguous()
    q_abs = torch.zeros(batch, nq, cfg.n_heads, Q, device="cuda", dtype=dt)
    q_abs[..., :cfg.d_c + cfg.d_rope] = (0.2 * torch.randn(batch, nq, cfg.n_heads, cfg.d_c + cfg.d_rope,
                                                           generator=g, device="cuda")).to(dt)
    tables = torch.empty(mla.rope3d_table_floats(shape, 64), dtype=torch.float32, device="cuda")
    mla.rope3d_tables(shape, 0, 64, tables)
    return shape, cache, slot_frame, q_abs, tables


def _both(cfg, batch, seed, kv_splits=0):
    shape, cache, sf, q_abs, tables = _inputs(cfg, batch, seed)
    nq = cfg.chunk_frames * cfg.tokens_per_frame
    out_ws = torch.empty(batch, nq, cfg.n_heads, cfg.d_c, dtype=cache.dtype, device="cuda")
    out_na = torch.full_like(out_ws, float("nan"))
    ws = torch.empty(mla.flash_workspace_bytes(shape, cfg.chunk_frames, kv_splits), dtype=torch.uint8,
                     device="cuda")
    assert 0 < ws.numel() <= mla.NOALLOC_SCRATCH_BYTES
    mla.flash_attend(shape, q_abs, cfg.chunk_frames, cache, sf, tables, 0, 64, out_ws, ws, kv_splits)
    mla.flash_attend_noalloc(shape, q_abs, cfg.chunk_frames, cache, sf, tables, 0, 64, out_na, kv_splits)
    torch.cuda.synchronize()
    return out_ws, out_na


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_noalloc_matches_workspace_entry_point_twice():
    """First the Wan2.1-shaped chunk (4680 queries over 32760 keys, the split
    the benchmark uses: about 53 MB of scratch), then a small Wan-headed
    problem in the same scratch; each bit-identical to mla_flash_attend."""
    for name, batch, seed in (("wan", 1, 1), ("wan_small", 2, 2)):
        cfg = get_config(name)
        out_ws, out_na = _both(cfg, batch, seed)
        print(f"[noalloc] {name} batch={batch} outputs={out_ws.numel()}", flush=True)
        assert torch.isfinite(out_ws.float()).all()
        assert torch.equal(_bits(out_ws), _bits(out_na))


def test_noalloc_fp32_and_one_range_per_row_block():
    cfg = get_config("wan_small_f32")
    out_ws, out_na = _both(cfg, 1, 3, kv_splits=1)
    assert torch.equal(_bits(out_ws), _bits(out_na))


def test_noalloc_refuses_problems_larger_than_its_scratch():
    """Eight Wan-shaped streams need about 70 MB of scratch with the automatic
    split: refused with MLA_ERR_SCRATCH before anything is enqueued."""
    cfg = get_config("wan")
    shape = mla.make_shape(cfg, batch=8)
    assert mla.flash_workspace_bytes(shape, 3, 0) > mla.NOALLOC_SCRATCH_BYTES
    dummy = torch.empty(256, dtype=torch.uint8, device="cuda")
    sf = torch.empty(8, 21, dtype=torch.int32, device="cuda")
    tables = torch.empty(64, dtype=torch.float32, device="cuda")
    with pytest.raises(mla.MlaError) as e:
        mla.flash_attend_noalloc(shape, dummy, 3, dummy, sf, tables, 0, 1, dummy, 0)
    assert e.value.code == 9
