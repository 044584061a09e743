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


# ------------------------------------------------------------------ frame-causal per-head form

def _causal_heads_step(cfg, seed, prefill_frames, chunk_first, B=1):
    """Frames written one by one, then the chunk; the per-head form's
    frame-causal attention of the chunk's queries against the oracle's
    frame-causal step, per stream."""
    w, wd = device_weights(cfg, seed)
    layer = LatentLayer(cfg, wd, batch=B, rope_n_t=64)
    streams = [Stream(cfg, seed=seed, stream=b) for b in range(B)]
    rings = [O.RingCache(cfg.window_frames, cfg.tokens_per_frame, cfg.d_c, cfg.d_rope) for _ in range(B)]
    for f in prefill_frames:
        xs = [s_.x(f) for s_ in streams]
        layer.write(to_torch(np.stack(xs), cfg.dtype), f, 1)
        for ring, x in zip(rings, xs):
            ring.write(f, *O.latents(x, w["w_dkv"], w["w_kr"]))
    xcs = [s_.xs(chunk_first, cfg.chunk_frames) for s_ in streams]
    layer.write(to_torch(np.stack(xcs), cfg.dtype), chunk_first, cfg.chunk_frames)
    qs = [s_.q(chunk_first) for s_ in streams]
    out = layer.attend_heads_frame_causal(to_torch(np.stack([q[0] for q in qs]), cfg.dtype),
                                          to_torch(np.stack([q[1] for q in qs]), cfg.dtype), chunk_first,
                                          cfg.chunk_frames)
    torch.cuda.synchronize()
    refs = [O.chunk_step(O.dims_of(cfg), w, rings[b], xcs[b], chunk_first, qs[b][0], qs[b][1], frame_causal=True)
            for b in range(B)]
    return to_numpy(out), np.stack(refs)


@pytest.mark.parametrize("name", HEADS_CONFIGS)
def test_heads_frame_causal_step(name):
    """Two-frame chunk after two earlier frames: queries of the chunk's first
    frame must not see the second frame's keys (the 132 query tokens form one
    384-token row block per head, whose rows see different key prefixes)."""
    cfg = get_config(name).with_(chunk_frames=2, window_frames=4)
    got, ref = _causal_heads_step(cfg, 61, [0, 1], 2)
    assert_step_close(got[0], ref[0], cfg.dtype, label=f"{name} per-head frame-causal step")


def test_heads_frame_causal_row_block_classes():
    """Frames of 416 tokens (16 x 26 grid), 2-frame chunk over a 4-frame
    window, 3 streams: the 832 query tokens of a head form 3 row blocks, the
    first ending in the chunk's first frame (it visits the keys of 3 window
    frames) and the others in its second (all 4), so the units fall into two
    classes; 108 row blocks over the work-groups share their key tiles. Every
    element of every stream against the oracle."""
    cfg = get_config("wan_small").with_(grid_y=16, grid_x=26, chunk_frames=2, window_frames=4)
    got, ref = _causal_heads_step(cfg, 62, [0, 1], 2, B=3)
    for b in range(3):
        assert_step_close(got[b], ref[b], cfg.dtype, label=f"per-head frame-causal classes, stream {b}")


def test_heads_frame_causal_classes_in_rounds():
    """The 16 x 26 grid over a 3-frame window with 8 streams: 288 row blocks
    of two classes, the first 256 dealt whole in a round (work-groups holding
    row blocks of either class), the other 32 shared. Every element of every
    stream against the oracle."""
    cfg = get_config("wan_small").with_(grid_y=16, grid_x=26, chunk_frames=2, window_frames=3)
    got, ref = _causal_heads_step(cfg, 68, [0], 1, B=8)
    for b in range(8):
        assert_step_close(got[b], ref[b], cfg.dtype, label=f"per-head frame-causal rounds, stream {b}")


def test_heads_frame_causal_wrapped_ring():
    """Three-frame chunk into a four-frame ring that already wrapped: the
    window holds frames 3..6 in rotated slots, expanded in frame order; frame
    f sees 3..f."""
    cfg = get_config("wan_small").with_(chunk_frames=3, window_frames=4)
    got, ref = _causal_heads_step(cfg, 63, [0, 1, 2, 3], 4)
    assert_step_close(got[0], ref[0], cfg.dtype, label="per-head frame-causal wrapped ring")


def test_heads_frame_causal_many_streams_whole_row_blocks():
    """30 streams x 12 heads of one row block each under the mask: the first
    256 row blocks go out whole, one per work-group and round, the rest are
    shared; every element of every stream against the oracle."""
    cfg = get_config("wan_small")
    got, ref = _causal_heads_step(cfg, 64, [0, 1], 2, B=30)
    for b in range(30):
        assert_step_close(got[b], ref[b], cfg.dtype, label=f"per-head frame-causal stream {b} of 30")


def test_heads_frame_causal_one_frame_chunk_equals_full():
    """A one-frame chunk sees every window key under the mask, so the
    per-head form's frame-causal call returns the same bits as the plain one;
    over an empty window both return zeros."""
    cfg = get_config("wan_small").with_(chunk_frames=1, window_frames=4)
    w, wd = device_weights(cfg, seed=65)
    st = Stream(cfg, seed=65)
    layer = LatentLayer(cfg, wd, batch=2, rope_n_t=16)
    qn, qr = st.q(3)
    qn_t = to_torch(np.stack([qn, qn]), cfg.dtype)
    qr_t = to_torch(np.stack([qr, qr]), cfg.dtype)
    empty_full = layer.attend_heads(qn_t, qr_t, 3, 1)
    empty_causal = layer.attend_heads_frame_causal(qn_t, qr_t, 3, 1)
    torch.cuda.synchronize()
    assert not to_numpy(empty_full).any() and not to_numpy(empty_causal).any()
    layer.write(to_torch(np.stack([st.xs(0, 4), Stream(cfg, seed=66).xs(0, 4)]), cfg.dtype), 0, 4)
    full = layer.attend_heads(qn_t, qr_t, 3, 1)
    causal = layer.attend_heads_frame_causal(qn_t, qr_t, 3, 1)
    torch.cuda.synchronize()
    assert torch.isfinite(full.float()).all()
    assert torch.equal(full.view(torch.int16), causal.view(torch.int16))


def test_heads_frame_causal_reference_from_unseen_keys():
    """First chunk of a rollout (the window holds only the chunk's frames
    0..2), 30 streams, queries x50 and key 8 of frame 2 scaled x3 in every
    stream. Whole row blocks visit their last key tile first (keys 128..197:
    the last 4 of frame 1, then frame 2), so the rows of frame 0 see none of
    its first 32 keys and take the maximum of those scores, the planted key
    among them, as reference. Rows whose sums leave the bounds are listed
    for the exact pass (count > 0), no row is left at zero, and every output
    matches the oracle's masked softmax taken with the kernel's bf16 roundings
    (as in the unmasked extreme-logit test above)."""
    cfg = get_config("wan_small").with_(chunk_frames=3, window_frames=3)
    B, W, T = 30, 3, cfg.tokens_per_frame
    w, wd = device_weights(cfg, seed=67)
    layer = LatentLayer(cfg, wd, batch=B, rope_n_t=16)
    streams = [Stream(cfg, seed=67, stream=b) for b in range(B)]
    layer.write(to_torch(np.stack([s_.xs(0, 3) for s_ in streams]), cfg.dtype), 0, 3)
    slot = int(np.where(to_numpy(layer.slot_frame)[0] == 2)[0][0])
    layer.cache[:, slot, 8] = (layer.cache[:, slot, 8].float() * 3.0).to(layer.cache.dtype)
    qs = [s_.q(0, q_scale=50.0) for s_ in streams]
    out = layer.attend_heads_frame_causal(to_torch(np.stack([q[0] for q in qs]), cfg.dtype),
                                          to_torch(np.stack([q[1] for q in qs]), cfg.dtype), 0, 3)
    torch.cuda.synchronize()
    n_fallback = int(layer.heads_workspace[:4].view(torch.int32).item())
    got = to_numpy(out)
    cache, sf = to_numpy(layer.cache), to_numpy(layer.slot_frame)
    qscale = float(np.float32(O.default_scale(cfg.d_head, cfg.d_rope) * np.log2(np.e)))
    tq, yq, xq = O.frame_positions(np.arange(3), cfg.grid_y, cfg.grid_x)
    worst = 0.0
    for b in range(B):
        order = np.argsort(sf[b])  # slots in frame order
        c = cache[b][order, :, :cfg.d_c].reshape(-1, cfg.d_c)
        kr = cache[b][order, :, cfg.d_c:].reshape(-1, cfg.d_rope)
        tk, yk, xk = O.frame_positions(sf[b][order], cfg.grid_y, cfg.grid_x)
        k_rope = round_to(O.rope3d(kr, tk, yk, xk, cfg.rope_split, cfg.rope_base), "bf16")
        k_nope, v = O.reconstruct(c, w["w_uk"], w["w_uv"])
        k_nope, v = round_to(k_nope, "bf16"), round_to(v, "bf16")
        qn, qr = qs[b]
        q_rope = O.rope3d(qr, tq, yq, xq, cfg.rope_split, cfg.rope_base)
        ref = O.attend(round_to(qn * qscale, "bf16"), round_to(q_rope * qscale, "bf16"), k_nope, k_rope, v,
                       float(np.log(2.0)), visible=O.frame_causal_mask(tq, tk))
        zero_rows = int((np.abs(got[b]).reshape(-1, cfg.d_head).max(axis=1) == 0).sum())
        assert zero_rows == 0, (b, zero_rows)
        assert_step_close(got[b], ref, "bf16", label=f"per-head causal unseen-reference stream {b}", sharp=True)
        worst = max(worst, errors(got[b], ref)["max_abs"])
    print(f"[parity] per-head causal unseen-reference fallback rows={n_fallback} worst max_abs={worst:.3e}",
          flush=True)
    assert n_fallback > 0
