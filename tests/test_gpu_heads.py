"""Parity of the per-head form (mla_chunk_attend_heads) with the fp64 oracle.

The oracle's chunk step reconstructs per-head keys and values explicitly and
attends with the two-part score, which is what this form computes. On the
GPU the expanded keys and values, the scaled queries and the probabilities
are bf16; the gates are the bf16 gates of the latent form.
"""
import numpy as np
import pytest
import torch

import latent_kv_attention_amd as mla
from latent_kv_attention_amd.layer import LatentLayer
from harness import get_config, round_to
from oracle import mla_oracle as O

from .gpu_common import Stream, assert_step_close, device_weights, errors, oracle_step_rows, to_numpy, to_torch

pytestmark = pytest.mark.gpu

HEADS_CONFIGS = ["wan_small", "wan_small_c128r32", "wan_small_c160r64", "wan_small_c192r64"]


@pytest.fixture(scope="module", autouse=True)
def _lib(built_lib):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mla.lib()
    yield


def _step(cfg, seed=0, q_scale=1.0, B=1, fill=None):
    """Prefill the window, write the chunk, attend by the per-head form;
    returns (gpu, oracle) per stream."""
    w, wd = device_weights(cfg, seed)
    W, T = cfg.window_frames, cfg.tokens_per_frame
    fill = W if fill is None else fill
    chunk_first = fill - cfg.chunk_frames
    layer = LatentLayer(cfg, wd, batch=B, rope_n_t=max(64, fill + 1))
    streams = [Stream(cfg, seed=seed, stream=b) for b in range(B)]
    if chunk_first > 0:
        pre = np.stack([s_.xs(0, chunk_first) for s_ in streams])
        layer.write(to_torch(pre, cfg.dtype).contiguous(), 0, chunk_first)
    layer.write(to_torch(np.stack([s_.xs(chunk_first, cfg.chunk_frames) for s_ in streams]), cfg.dtype),
                chunk_first, cfg.chunk_frames)
    qs = [s_.q(chunk_first, q_scale=q_scale) for s_ in streams]
    out = layer.attend_heads(to_torch(np.stack([q[0] for q in qs]), cfg.dtype),
                             to_torch(np.stack([q[1] for q in qs]), cfg.dtype), chunk_first, cfg.chunk_frames)
    torch.cuda.synchronize()
    frames = list(range(max(0, fill - W), fill))
    refs = [oracle_step_rows(cfg, w, {f: s_.x(f) for f in frames}, frames, qs[b][0], qs[b][1], chunk_first)
            for b, s_ in enumerate(streams)]
    return to_numpy(out), np.stack(refs), layer


@pytest.mark.parametrize("name", HEADS_CONFIGS)
def test_heads_full_step(name):
    cfg = get_config(name)
    got, ref, _ = _step(cfg, seed=31)
    assert_step_close(got, ref, cfg.dtype, label=f"{name} per-head step")


def test_heads_sharp_queries():
    cfg = get_config("wan_small")
    got, ref, _ = _step(cfg, seed=32, q_scale=4.0)
    assert_step_close(got, ref, cfg.dtype, label="wan_small per-head step q*4", sharp=True)


def test_heads_batch_and_partial_fill():
    cfg = get_config("wan_small")
    got, ref, _ = _step(cfg, seed=33, B=3, fill=3)
    assert_step_close(got, ref, cfg.dtype, label="wan_small per-head B=3 fill=3")


def test_heads_many_streams_whole_row_blocks():
    """30 streams x 12 heads of one row block each: 360 row blocks, more than
    one per work-group, so the first whole multiple of the work-group count
    goes out as whole row blocks in a round and the rest are shared (pieces
    merged). Every element of every stream against the oracle."""
    cfg = get_config("wan_small")
    got, ref, _ = _step(cfg, seed=34, B=30)
    print(f"[heads] 30 streams, {30 * 12} row blocks", flush=True)
    for b in range(30):
        assert_step_close(got[b], ref[b], cfg.dtype, label=f"wan_small per-head stream {b} of 30")


def test_heads_rollout_ring_eviction():
    """Successive 1-frame chunks over a 3-frame window: eviction from the 4th
    chunk on and t advancing to 9; every step matches the oracle's ring."""
    cfg = get_config("wan_small").with_(window_frames=3, chunk_frames=1)
    w, wd = device_weights(cfg, seed=34)
    layer = LatentLayer(cfg, wd, batch=1, rope_n_t=16)
    st = Stream(cfg, seed=34)
    ring = O.RingCache(3, cfg.tokens_per_frame, cfg.d_c, cfg.d_rope)
    for f in range(10):
        x = st.x(f)
        layer.write(to_torch(x[None], cfg.dtype), f, 1)
        qn, qr = st.q(f)
        out = layer.attend_heads(to_torch(qn[None], cfg.dtype), to_torch(qr[None], cfg.dtype), f, 1)
        torch.cuda.synchronize()
        ref = O.chunk_step(O.dims_of(cfg), w, ring, x, f, qn, qr)
        assert_step_close(to_numpy(out)[0], ref, cfg.dtype, label=f"per-head rollout frame {f}")


def test_heads_wan_full_size_sampled_rows():
    """Wan2.1-1.3B shape, 3-frame chunk over a full 21-frame window, in the
    launch configuration the width sweep times; 64 sampled query rows (all
    heads, full window) against the oracle, including first and last rows and
    the boundaries of the 384-token row blocks and of the last, ragged one."""
    cfg = get_config("wan")
    w, wd = device_weights(cfg, seed=0)
    layer = LatentLayer(cfg, wd, batch=1, rope_n_t=64)
    st = Stream(cfg, seed=0)
    layer.write(to_torch(st.xs(0, 18)[None], cfg.dtype), 0, 18)
    layer.write(to_torch(st.xs(18, 3)[None], cfg.dtype), 18, 3)
    qn, qr = st.q(18)
    out = layer.attend_heads(to_torch(qn[None], cfg.dtype), to_torch(qr[None], cfg.dtype), 18, 3)
    torch.cuda.synchronize()
    got = to_numpy(out)[0]
    rng = np.random.default_rng(1)
    edge = [0, 1, 383, 384, 767, 768, cfg.n_q // 2, 12 * 384 - 1, 12 * 384, cfg.n_q - 1]
    rows = np.unique(np.concatenate([edge, rng.choice(cfg.n_q, 64 - len(edge), replace=False)]))
    xs = {f: st.x(f) for f in range(21)}
    ref = oracle_step_rows(cfg, w, xs, list(range(21)), qn, qr, 18, rows)
    assert_step_close(got[rows], ref, cfg.dtype, label="wan full size per-head, sampled rows")


def test_heads_extreme_logits_use_exact_fallback():
    """Queries scaled by 40 (logit spread far beyond the fixed reference's
    range): rows whose probability sum overflows are listed (the count sits at
    the start of the workspace) and recomputed by the exact kernel. At such
    logits the bf16 storage of the expanded keys and of the scaled queries
    moves scores by whole units, so the oracle here takes the same bf16
    roundings (queries scaled by the float softmax factor in log2 units, keys
    and values, rotated kR) before its fp64 softmax."""
    cfg = get_config("wan_small")
    w, wd = device_weights(cfg, seed=35)
    W, T = cfg.window_frames, cfg.tokens_per_frame
    layer = LatentLayer(cfg, wd, batch=1, rope_n_t=64)
    st = Stream(cfg, seed=35)
    layer.write(to_torch(st.xs(0, W)[None], cfg.dtype), 0, W)
    q_first = W - cfg.chunk_frames
    qn, qr = st.q(q_first, q_scale=40.0)
    out = layer.attend_heads(to_torch(qn[None], cfg.dtype), to_torch(qr[None], cfg.dtype), q_first,
                             cfg.chunk_frames)
    torch.cuda.synchronize()
    n_fallback = int(layer.heads_workspace[:4].view(torch.int32).item())
    got = to_numpy(out)[0]

    # oracle with the kernel's bf16 roundings
    cache = to_numpy(layer.cache)[0]  # [W][T][d_c + d_rope], the stored bf16 values
    sf = to_numpy(layer.slot_frame)[0]
    valid = [s_ for s_ in range(W) if sf[s_] >= 0]
    c = cache[valid, :, :cfg.d_c].reshape(-1, cfg.d_c)
    kr = cache[valid, :, cfg.d_c:].reshape(-1, cfg.d_rope)
    tk, yk, xk = O.frame_positions(sf[valid], cfg.grid_y, cfg.grid_x)
    k_rope = round_to(O.rope3d(kr, tk, yk, xk, cfg.rope_split, cfg.rope_base), "bf16")
    k_nope, v = O.reconstruct(c, w["w_uk"], w["w_uv"])
    k_nope, v = round_to(k_nope, "bf16"), round_to(v, "bf16")
    qscale = float(np.float32(O.default_scale(cfg.d_head, cfg.d_rope) * np.log2(np.e)))
    tq, yq, xq = O.frame_positions(q_first + np.arange(cfg.chunk_frames), cfg.grid_y, cfg.grid_x)
    q_rope = O.rope3d(qr, tq, yq, xq, cfg.rope_split, cfg.rope_base)
    # scores in log2 units; softmax of ln 2 * s is the 2^s weighting
    ref = O.attend(round_to(qn * qscale, "bf16"), round_to(q_rope * qscale, "bf16"), k_nope, k_rope, v,
                   float(np.log(2.0)))
    e = errors(got, ref)
    print(f"[parity] per-head extreme logits fallback rows={n_fallback} {e}", flush=True)
    assert n_fallback > 0
    assert_step_close(got, ref, "bf16", label="per-head extreme logits", sharp=True)


def test_heads_empty_window_gives_zeros():
    cfg = get_config("wan_small")
    w, wd = device_weights(cfg, seed=36)
    layer = LatentLayer(cfg, wd, batch=1, rope_n_t=64)
    qn, qr = Stream(cfg, seed=36).q(0)
    out = layer.attend_heads(to_torch(qn[None], cfg.dtype), to_torch(qr[None], cfg.dtype), 0, cfg.chunk_frames)
    torch.cuda.synchronize()
    assert not to_numpy(out).any()
