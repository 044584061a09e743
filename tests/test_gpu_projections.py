"""Parity of the query path (mla_query_project), the output projection
(mla_output_project) and the whole layer built from them with the fp64
oracle.

The projections are plain matrix products with fp32 accumulation and one
rounding of each stored result; the query latent is stored in the element
type before the per-head products read it. The bound used for a product
y = A b whose operand b was rounded (relative error u_b) and whose result is
rounded (u_y) is the standard forward bound
    |y_gpu - y| <= u_b (|A| |b|) + u_y |y| + K * 2^-22 (|A| |b|),
evaluated by the oracle in fp64 (K = contraction length; the last term is
the fp32 accumulation).
"""
import numpy as np
import pytest
import torch

import latent_kv_attention_amd as mla
from latent_kv_attention_amd.layer import LatentLayer
from harness import chunk_queries, get_config, query_weights
from oracle import mla_oracle as O

from .gpu_common import Stream, assert_rounded_close, assert_step_close, device_weights, to_numpy, to_torch

pytestmark = pytest.mark.gpu

PROJ_CONFIGS = ["tiny", "tiny_bf16", "wan_small", "wan_small_f32", "wan_small_c160r64"]


@pytest.fixture(scope="module", autouse=True)
def _lib(built_lib):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mla.lib()
    yield


def _unit(dtype):
    return 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24


def _assert_product_close(got, ref, absprod, dtype, k, rounded_operand, label):
    u = _unit(dtype)
    bound = (u if rounded_operand else 0.0) * absprod + u * np.abs(ref) + k * 2.0 ** -22 * absprod + 1e-30
    bad = np.abs(got - ref) > bound
    print(f"[proj] {label} max_abs={np.abs(got - ref).max():.3e} violations={int(bad.sum())}", flush=True)
    assert not bad.any(), (label, int(bad.sum()))
    assert np.isfinite(got).all()


def _weights(cfg, seed):
    w, wd = device_weights(cfg, seed)
    wq = query_weights(cfg, seed)
    return {**w, **wq}, {**wd, **{k: to_torch(v, cfg.dtype) for k, v in wq.items()}}


def _check_query_path(cfg, seed, x, n_frames, B=1, rows=None):
    """x [B, n, hidden] (host, rounded): GPU query path vs the oracle."""
    w, wd = _weights(cfg, seed)
    layer = LatentLayer(cfg, wd, batch=B, rope_n_t=64, max_chunk_frames=n_frames)
    c_q, qn, qr = layer.project_queries(to_torch(x, cfg.dtype).contiguous(), n_frames)
    torch.cuda.synchronize()
    c_q, qn, qr = to_numpy(c_q), to_numpy(qn), to_numpy(qr)
    xr = x.reshape(-1, cfg.hidden)
    sel = np.arange(xr.shape[0]) if rows is None else rows
    xs = xr[sel]
    c_ref, qn_ref, qr_ref = O.query_project(xs, w["w_dq"], w["w_uq"], w["w_qr"])
    _assert_product_close(c_q.reshape(-1, cfg.q_latent)[sel], c_ref, np.abs(xs) @ np.abs(w["w_dq"]).T, cfg.dtype,
                          cfg.hidden, False, f"{cfg.name} c_q")
    # magnitudes |W_uq| |c_q| for the bound
    ac = np.abs(c_ref)
    an = np.einsum("nc,hdc->nhd", ac, np.abs(w["w_uq"]))
    ar = np.einsum("nc,hdc->nhd", ac, np.abs(w["w_qr"]))
    _assert_product_close(qn.reshape(-1, cfg.n_heads, cfg.d_head)[sel], qn_ref, an, cfg.dtype, cfg.q_latent, True,
                          f"{cfg.name} q_nope")
    _assert_product_close(qr.reshape(-1, cfg.n_heads, cfg.d_rope)[sel], qr_ref, ar, cfg.dtype, cfg.q_latent, True,
                          f"{cfg.name} q_r")


@pytest.mark.parametrize("name", PROJ_CONFIGS)
def test_query_project(name):
    cfg = get_config(name)
    st = Stream(cfg, seed=51)
    x = st.xs(0, cfg.chunk_frames)[None]
    _check_query_path(cfg, 51, x, cfg.chunk_frames)


def test_query_project_batch_ragged_rows_and_narrow_latent():
    """Three streams of a 2-frame chunk (396 rows: ragged against every
    row tile) with a query latent of 40 (a partial K step and a partial
    column tile)."""
    cfg = get_config("wan_small").with_(d_cq=40)
    x = np.stack([Stream(cfg, seed=52, stream=b).xs(0, 2) for b in range(3)])
    _check_query_path(cfg, 52, x, 2, B=3)


def test_query_project_wan_full_size_sampled_rows():
    """Wan2.1-1.3B shape: the 4680 tokens of a 3-frame chunk, d_cq 576; 200
    sampled rows (first and last rows and 128-row tile edges included)."""
    cfg = get_config("wan")
    x = Stream(cfg, seed=53).xs(0, 3)[None]
    rng = np.random.default_rng(3)
    edge = [0, 1, 63, 64, 127, 128, 4607, 4608, cfg.n_q - 1]
    rows = np.unique(np.concatenate([edge, rng.choice(cfg.n_q, 200 - len(edge), replace=False)]))
    _check_query_path(cfg, 53, x, 3, rows=rows)


@pytest.mark.parametrize("name", PROJ_CONFIGS)
def test_output_project(name):
    cfg = get_config(name)
    w, wd = _weights(cfg, 54)
    layer = LatentLayer(cfg, wd, batch=2, rope_n_t=64)
    # seeded stand-ins for the heads' outputs (unit-order entries)
    o = np.stack([chunk_queries(cfg, 0, seed=54, stream=b)[0] for b in range(2)])
    u = layer.project_output(to_torch(o, cfg.dtype).contiguous(), cfg.chunk_frames)
    torch.cuda.synchronize()
    got = to_numpy(u).reshape(-1, cfg.hidden)
    of = o.reshape(-1, cfg.n_heads * cfg.d_head)
    ref = O.output_project(o.reshape(-1, cfg.n_heads, cfg.d_head), w["w_o"])
    _assert_product_close(got, ref, np.abs(of) @ np.abs(w["w_o"]).T, cfg.dtype, cfg.n_heads * cfg.d_head, False,
                          f"{name} u")


def _layer_steps(cfg, seed, n_chunks, frame_causal=False):
    """Chunk after chunk through LatentLayer.step (queries from the tokens,
    cache write, attention, output projection) against O.layer_step."""
    w, wd = _weights(cfg, seed)
    layer = LatentLayer(cfg, wd, batch=1, rope_n_t=64)
    ring = O.RingCache(cfg.window_frames, cfg.tokens_per_frame, cfg.d_c, cfg.d_rope)
    st = Stream(cfg, seed=seed)
    for k in range(n_chunks):
        f0 = k * cfg.chunk_frames
        x = st.xs(f0, cfg.chunk_frames)
        u = layer.step(to_torch(x[None], cfg.dtype), f0, cfg.chunk_frames, frame_causal=frame_causal)
        torch.cuda.synchronize()
        ref, _, _, _ = O.layer_step(O.dims_of(cfg), w, ring, x, f0, frame_causal=frame_causal)
        assert_step_close(to_numpy(u)[0], ref, cfg.dtype, label=f"{cfg.name} layer step chunk {k}")


@pytest.mark.parametrize("name", ["tiny", "wan_small", "wan_small_f32", "wan_small_c128r32"])
def test_layer_step(name):
    cfg = get_config(name)
    n_chunks = cfg.window_frames // cfg.chunk_frames + 2  # the ring wraps
    _layer_steps(cfg, 55, n_chunks)


@pytest.mark.parametrize("fused", [False, True])
def test_layer_step_where_the_per_head_form_is_taken(fused):
    """A 32 x 64 grid with the Wan head shapes: a one-frame chunk has 2048
    queries, so the layer step takes the per-head attention (also when the
    absorbed query weights are set, since the per-head weights are there
    too); chunk after chunk through ring wrap against O.layer_step, and the
    frame-causal step on the same layer (which, with one chunk frame, masks
    nothing) in between."""
    cfg = get_config("wan_small").with_(grid_y=32, grid_x=64, window_frames=3, chunk_frames=1)
    w, wd = _weights(cfg, 58)
    layer = LatentLayer(cfg, wd, batch=1, rope_n_t=64)
    assert mla.chunk_attend_form(layer.shape, 1) == mla.FORM_HEADS
    if fused:
        layer.absorb_query_weights()
    ring = O.RingCache(cfg.window_frames, cfg.tokens_per_frame, cfg.d_c, cfg.d_rope)
    st = Stream(cfg, seed=58)
    for f0 in range(5):
        x = st.xs(f0, 1)
        causal = f0 == 3
        u = layer.step(to_torch(x[None], cfg.dtype), f0, 1, frame_causal=causal)
        torch.cuda.synchronize()
        ref, _, _, _ = O.layer_step(O.dims_of(cfg), w, ring, x, f0, frame_causal=causal)
        assert_step_close(to_numpy(u)[0], ref, cfg.dtype, label=f"per-head layer step fused={fused} frame {f0}")


def test_layer_step_frame_causal_per_head_form():
    """Two-frame chunks of 2048-token frames (32 x 64 grid) over a 3-frame
    ring: the frame-causal layer step takes the per-head form, and the
    queries of a chunk's first frame must not see its second frame; two
    chunks (the second after the ring wrapped) against O.layer_step."""
    cfg = get_config("wan_small").with_(grid_y=32, grid_x=64, window_frames=3, chunk_frames=2)
    w, wd = _weights(cfg, 59)
    layer = LatentLayer(cfg, wd, batch=1, rope_n_t=64)
    assert mla.chunk_attend_form(layer.shape, 2) == mla.FORM_HEADS
    ring = O.RingCache(cfg.window_frames, cfg.tokens_per_frame, cfg.d_c, cfg.d_rope)
    st = Stream(cfg, seed=59)
    for f0 in (0, 2):
        x = st.xs(f0, 2)
        u = layer.step(to_torch(x[None], cfg.dtype), f0, 2, frame_causal=True)
        torch.cuda.synchronize()
        ref, _, _, _ = O.layer_step(O.dims_of(cfg), w, ring, x, f0, frame_causal=True)
        assert_step_close(to_numpy(u)[0], ref, cfg.dtype, label=f"per-head frame-causal layer step frame {f0}")


def test_layer_step_frame_causal():
    cfg = get_config("wan_small").with_(chunk_frames=2, window_frames=4)
    _layer_steps(cfg, 56, 3, frame_causal=True)


@pytest.mark.parametrize("name", ["wan_small", "wan_small_f32"])
@pytest.mark.parametrize("frame_causal", [False, True])
def test_layer_step_single_call_equals_composed_calls(name, frame_causal):
    """mla_layer_step against mla_query_project, mla_cache_write,
    mla_chunk_attend[_frame_causal] and mla_output_project called one by one,
    chunk after chunk through ring wrap, with three streams. The single call
    forms the query latent and the cached rows in one product of x with
    [W_dq ; W_dkv ; W_kR]; its cached rows equal the separate cache write's
    up to the order of the fp32 sums (one rounding each, so within one unit
    of the last place either way), and both match the oracle's latents; the
    slot tables are identical and the layer outputs agree within the step
    gates."""
    cfg = get_config(name).with_(window_frames=4, chunk_frames=2)
    w, wd = _weights(cfg, 57)
    one = LatentLayer(cfg, wd, batch=3, rope_n_t=16)
    four = LatentLayer(cfg, wd, batch=3, rope_n_t=16)
    streams = [Stream(cfg, seed=57, stream=b) for b in range(3)]
    T = cfg.tokens_per_frame
    for k in range(4):
        f0 = 2 * k
        xs = np.stack([s_.xs(f0, 2) for s_ in streams])
        x = to_torch(xs, cfg.dtype)
        u1 = one.step(x, f0, 2, frame_causal=frame_causal)
        u4 = four.step_composed(x, f0, 2, frame_causal=frame_causal)
        torch.cuda.synchronize()
        assert torch.isfinite(u1.float()).all()
        assert torch.equal(one.slot_frame, four.slot_frame)
        c1, c4 = to_numpy(one.cache), to_numpy(four.cache)
        w_cat = np.concatenate([w["w_dkv"], w["w_kr"]])
        for b in range(3):
            for i in range(2):
                xi = xs[b, i * T:(i + 1) * T]
                c, kr = O.latents(xi, w["w_dkv"], w["w_kr"])
                ref = np.concatenate([c, kr], axis=-1)
                slot = (f0 + i) % 4
                # each side: one rounding of an fp32 sum of K products
                bound = 2 * (_unit(cfg.dtype) * np.abs(ref) + cfg.hidden * 2.0 ** -22 * (np.abs(xi) @ np.abs(w_cat).T))
                assert np.all(np.abs(c1[b, slot] - c4[b, slot]) <= bound), f"chunk {k} b={b} frame {f0 + i}"
                assert_rounded_close(c1[b, slot], ref, cfg.dtype, label=f"fused cache write b={b} frame {f0 + i}")
        assert_step_close(to_numpy(u1), to_numpy(u4), cfg.dtype, label=f"{name} single vs composed chunk {k}")


# ------------------------------------------------------------------ fused (absorbed) query path

def _u(dtype):
    return _unit(dtype)


@pytest.mark.parametrize("name", ["tiny", "wan_small", "wan_small_f32", "wan_small_c160r64"])
def test_query_absorb_weights(name):
    """w_qabs[h] = [W_uk[h]^T W_uq[h] ; W_qr[h] ; 0] against the fp64 product
    (one rounding, fp32 sums over d_head)."""
    cfg = get_config(name)
    w, wd = _weights(cfg, 58)
    layer = LatentLayer(cfg, wd, batch=1, rope_n_t=16)
    got = to_numpy(layer.absorb_query_weights())
    torch.cuda.synchronize()
    dc, dr, H = cfg.d_c, cfg.d_rope, cfg.n_heads
    ref = np.zeros(got.shape)
    ref[:, :dc] = np.einsum("hic,hiq->hcq", w["w_uk"], w["w_uq"])
    ref[:, dc:dc + dr] = w["w_qr"]
    absprod = np.zeros(got.shape)
    absprod[:, :dc] = np.einsum("hic,hiq->hcq", np.abs(w["w_uk"]), np.abs(w["w_uq"]))
    _assert_product_close(got, ref, absprod, cfg.dtype, cfg.d_head, False, f"{name} w_qabs")
    assert not got[:, dc + dr:].any()


def _check_absorbed_queries(cfg, seed, B, n_frames, q_frame_first):
    w, wd = _weights(cfg, seed)
    layer = LatentLayer(cfg, wd, batch=B, rope_n_t=64, max_chunk_frames=n_frames)
    layer.absorb_query_weights()
    x = np.stack([Stream(cfg, seed=seed, stream=b).xs(q_frame_first, n_frames) for b in range(B)])
    c_q, q_abs = layer.project_queries_absorbed(to_torch(x, cfg.dtype).contiguous(), q_frame_first, n_frames)
    torch.cuda.synchronize()
    got = to_numpy(q_abs).reshape(-1, cfg.n_heads, q_abs.shape[-1])
    xr = x.reshape(-1, cfg.hidden)
    c_ref, qn, qr = O.query_project(xr, w["w_dq"], w["w_uq"], w["w_qr"])
    n = n_frames * cfg.tokens_per_frame
    tq, yq, xq = O.frame_positions(q_frame_first + np.arange(n_frames), cfg.grid_y, cfg.grid_x)
    tq, yq, xq = (np.tile(a, B) for a in (tq, yq, xq))
    ref = O.absorbed_query(qn, qr, w["w_uk"], tq, yq, xq, cfg.rope_split, cfg.rope_base)
    g = float(np.float32(O.default_scale(cfg.d_head, cfg.d_rope) * np.log2(np.e)))
    dc, dr = cfg.d_c, cfg.d_rope
    # magnitudes: |W_abs| |c_q| per latent column; rotated columns mix a pair
    ac = np.abs(c_ref)
    a_lat = np.einsum("nq,hcq->nhc", ac, np.einsum("hic,hiq->hcq", np.abs(w["w_uk"]), np.abs(w["w_uq"])))
    a_rope = np.einsum("nq,hdq->nhd", ac, np.abs(w["w_qr"]))
    a_rope = np.repeat(a_rope[..., 0::2] + a_rope[..., 1::2], 2, axis=-1)
    absprod = g * np.concatenate([a_lat, a_rope], axis=-1)
    u = _u(cfg.dtype)
    # c_q and the absorbed weight are each rounded once before the fp32 product
    bound = 2.01 * u * absprod + u * np.abs(g * ref) + cfg.q_latent * 2.0 ** -22 * absprod + 1e-30
    d = np.abs(got[..., :dc + dr] - g * ref)
    print(f"[proj] {cfg.name} q_abs fused max_abs={d.max():.3e} violations={int((d > bound).sum())}", flush=True)
    assert not (d > bound).any()
    assert not got[..., dc + dr:].any()
    assert np.isfinite(got).all()


@pytest.mark.parametrize("name", ["tiny", "wan_small", "wan_small_f32", "wan_small_c160r64"])
def test_query_project_absorbed(name):
    cfg = get_config(name)
    _check_absorbed_queries(cfg, 59, B=2, n_frames=cfg.chunk_frames, q_frame_first=5)


def test_query_project_absorbed_wan_full_size():
    cfg = get_config("wan")
    _check_absorbed_queries(cfg, 60, B=1, n_frames=3, q_frame_first=18)


@pytest.mark.parametrize("name", ["tiny", "wan_small", "wan_small_f32"])
def test_layer_step_fused_query_path(name):
    """The whole layer with the fused query path, chunk after chunk through
    ring wrap, against the oracle's layer step."""
    cfg = get_config(name)
    w, wd = _weights(cfg, 61)
    layer = LatentLayer(cfg, wd, batch=1, rope_n_t=64)
    layer.absorb_query_weights()
    ring = O.RingCache(cfg.window_frames, cfg.tokens_per_frame, cfg.d_c, cfg.d_rope)
    st = Stream(cfg, seed=61)
    for k in range(cfg.window_frames // cfg.chunk_frames + 2):
        f0 = k * cfg.chunk_frames
        x = st.xs(f0, cfg.chunk_frames)
        u = layer.step(to_torch(x[None], cfg.dtype), f0, cfg.chunk_frames, frame_causal=(k % 2 == 1))
        torch.cuda.synchronize()
        ref, _, _, _ = O.layer_step(O.dims_of(cfg), w, ring, x, f0, frame_causal=(k % 2 == 1))
        assert_step_close(to_numpy(u)[0], ref, cfg.dtype, label=f"{name} fused layer step chunk {k}")
