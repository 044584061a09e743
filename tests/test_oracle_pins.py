"""Pins for the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: numbers the
pages print (tests/golden/paper_counts.json), closed forms, invariants, a
textbook special case, an independently written dense multi-head attention,
and a pure-Python brute force on the tiny shape.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest

from harness import chunk_queries, frame_tokens, get_config, layer_weights, query_weights
from oracle import mla_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paper_counts.json")


def _dims(cfg):
    return O.dims_of(cfg)


def _ring_step(cfg, seed=0, frames_in_window=None, chunk_first=None, q_scale=1.0):
    """Fill a ring with frames 0..F-1 (chunk = last chunk_frames) and run the oracle step."""
    w = layer_weights(cfg, seed)
    fill = frames_in_window or cfg.window_frames
    chunk_first = fill - cfg.chunk_frames if chunk_first is None else chunk_first
    ring = O.RingCache(cfg.window_frames, cfg.tokens_per_frame, cfg.d_c, cfg.d_rope)
    for f in range(chunk_first):
        c, kr = O.latents(frame_tokens(cfg, f, seed), w["w_dkv"], w["w_kr"])
        ring.write(f, c, kr)
    x_chunk = np.concatenate([frame_tokens(cfg, chunk_first + i, seed) for i in range(cfg.chunk_frames)])
    qn, qr = chunk_queries(cfg, chunk_first, seed, q_scale=q_scale)
    out = O.chunk_step(_dims(cfg), w, ring, x_chunk, chunk_first, qn, qr)
    return out, w, ring, x_chunk, qn, qr, chunk_first


# ------------------------------------------------------------------ counts printed on the pages

def test_scalar_counts_match_pages():
    g = json.load(open(GOLDEN))
    wan = get_config("wan")
    assert O.dense_scalars_per_token(wan.n_heads, wan.d_head) == g["dense_scalars_per_token"]
    assert O.cache_scalars_per_token(wan.d_c, wan.d_rope) == g["latent_scalars_per_token"]
    assert wan.d_c == g["d_c"]
    red = 100.0 * (1.0 - g["latent_scalars_per_token"] / g["dense_scalars_per_token"])
    assert round(red, 1) == g["reduction_percent"]
    assert round(red) == g["reduction_percent_rounded"]
    tiny = get_config("tiny")
    assert O.cache_scalars_per_token(tiny.d_c, tiny.d_rope) == 24
    assert O.dense_scalars_per_token(tiny.n_heads, tiny.d_head) == 32


def test_ring_stores_latent_width_only():
    wan = get_config("wan")
    ring = O.RingCache(wan.window_frames, 4, wan.d_c, wan.d_rope)
    per_token = ring.c.shape[-1] + ring.kr.shape[-1]
    assert per_token == 224
    assert 1.0 - per_token / wan.dense_scalars == pytest.approx(0.927083, abs=1e-6)


# ------------------------------------------------------------------ RoPE

def test_rope_frequencies_closed_form():
    np.testing.assert_allclose(O.rope_inv_freq(8, 10000.0), [1.0, 0.1, 0.01, 0.001], rtol=1e-15)
    np.testing.assert_allclose(O.rope_inv_freq(12, 10000.0), 10000.0 ** (-np.arange(6) / 6.0), rtol=1e-15)


def test_rope_quarter_turn_closed_form():
    # d=2: a single pair rotated by pos radians; pos = pi/2 maps (1, 0) to (0, 1)
    v = np.array([[1.0, 0.0]])
    c, s = O.rope_axis_cos_sin([math.pi / 2], 2, 10000.0)
    r = O.rotate_pairs(v, c, s)
    np.testing.assert_allclose(r, [[0.0, 1.0]], atol=1e-15)


def _textbook_rope_1d(vec, pos, base):
    """1-D RoPE in complex form: z_k = v[2k] + i v[2k+1] times exp(i pos base^(-2k/d))."""
    d = len(vec)
    out = []
    for k in range(d // 2):
        z = complex(vec[2 * k], vec[2 * k + 1]) * cmath.exp(1j * pos * base ** (-2.0 * k / d))
        out += [z.real, z.imag]
    return out


def test_rope3d_blocks_equal_textbook_1d():
    rng = np.random.default_rng(1)
    split, base = (8, 12, 12), 10000.0
    v = rng.standard_normal((5, 32))
    t, y, x = np.array([0, 3, 17, 239, 5]), np.array([0, 29, 4, 11, 1]), np.array([51, 0, 7, 23, 2])
    r = O.rope3d(v, t, y, x, split, base)
    for n in range(5):
        exp = (_textbook_rope_1d(v[n, 0:8], t[n], base) + _textbook_rope_1d(v[n, 8:20], y[n], base)
               + _textbook_rope_1d(v[n, 20:32], x[n], base))
        np.testing.assert_allclose(r[n], exp, rtol=0, atol=1e-12)


def test_rope3d_single_axis_reduces_to_1d():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((4, 16))
    t = np.array([0, 1, 9, 100])
    r = O.rope3d(v, t, np.zeros(4, int), np.zeros(4, int), (16, 0, 0), 10000.0)
    for n in range(4):
        np.testing.assert_allclose(r[n], _textbook_rope_1d(v[n], t[n], 10000.0), atol=1e-12)


def test_rope_identity_norm_group_relative():
    rng = np.random.default_rng(3)
    split, base = (8, 12, 12), 10000.0
    v = rng.standard_normal((6, 32))
    z = np.zeros(6, int)
    np.testing.assert_allclose(O.rope3d(v, z, z, z, split, base), v, atol=0)  # R(0) = I
    t, y, x = rng.integers(0, 240, 6), rng.integers(0, 30, 6), rng.integers(0, 52, 6)
    r = O.rope3d(v, t, y, x, split, base)
    np.testing.assert_allclose(np.linalg.norm(r, axis=1), np.linalg.norm(v, axis=1), rtol=1e-13)
    # group property R(a) R(b) = R(a + b)
    t2, y2, x2 = rng.integers(0, 240, 6), rng.integers(0, 30, 6), rng.integers(0, 52, 6)
    np.testing.assert_allclose(O.rope3d(r, t2, y2, x2, split, base),
                               O.rope3d(v, t + t2, y + y2, x + x2, split, base), atol=1e-12)
    # relative-offset invariance: <R(p) q, R(p') k> unchanged by a common 3-D shift
    q, k = rng.standard_normal((6, 32)), rng.standard_normal((6, 32))
    tp, yp, xp = rng.integers(0, 240, 6), rng.integers(0, 30, 6), rng.integers(0, 52, 6)
    base_dot = np.sum(O.rope3d(q, t, y, x, split, base) * O.rope3d(k, tp, yp, xp, split, base), axis=1)
    for dt, dy, dx in [(7, 0, 0), (0, 3, 0), (0, 0, 11), (113, 5, 40)]:
        sh = np.sum(O.rope3d(q, t + dt, y + dy, x + dx, split, base)
                    * O.rope3d(k, tp + dt, yp + dy, xp + dx, split, base), axis=1)
        np.testing.assert_allclose(sh, base_dot, rtol=1e-11, atol=1e-11)


def test_rope_tables_unit_circle_and_layout():
    split, base = (8, 12, 12), 10000.0
    flat = O.rope_tables_flat(split, base, 3, 21, 30, 52)
    assert flat.size == 2 * (21 * 4 + 30 * 6 + 52 * 6)
    tb = O.rope_tables(split, base, 3, 21, 30, 52)
    for a in "tyx":
        c, s = tb[a]
        np.testing.assert_allclose(c * c + s * s, 1.0, atol=1e-15)
    # row 0 of the t table is position t_first = 3
    np.testing.assert_allclose(tb["t"][0][0], np.cos(3.0 * O.rope_inv_freq(8, base)), atol=1e-15)


# ------------------------------------------------------------------ ring buffer

def test_ring_eviction_closed_form():
    ring = O.RingCache(4, 2, 3, 2)
    for f in range(10):
        ring.write(f, np.full((2, 3), f, float), np.full((2, 2), -f, float))
    assert ring.slot_frame.tolist() == [8, 9, 6, 7]
    assert ring.c[1, 0, 0] == 9 and ring.kr[2, 1, 1] == -6
    with pytest.raises(ValueError):
        ring.write(0, np.zeros((10, 3)), np.zeros((10, 2)))


def test_ring_rewrite_of_a_chunk_replaces_only_its_slots():
    # denoising re-writes the chunk's frames: values written with their own
    # frame index make the state after any run of re-writes readable by hand
    ring = O.RingCache(4, 2, 3, 2)
    for f in range(3):
        ring.write(f, np.full((2, 3), f, float), np.full((2, 2), -f, float))
    for step in range(3):  # chunk = frames 3, 4 (slots 3, 0), re-written per step
        c = np.repeat(np.array([[100.0 * step + 3], [100.0 * step + 4]]), 2, axis=0) * np.ones((4, 3))
        ring.write(3, c, -c[:, :2])
        assert ring.slot_frame.tolist() == [4, 1, 2, 3]
        assert ring.c[0, 0, 0] == 100 * step + 4 and ring.c[3, 1, 2] == 100 * step + 3
        assert ring.c[1, 0, 0] == 1 and ring.c[2, 1, 1] == 2 and ring.kr[2, 0, 0] == -2


def test_ring_slot_layout_does_not_change_output():
    # the same five frames held in rings of different sizes occupy different slots
    cfg = get_config("tiny")
    w = layer_weights(cfg)
    frames = [3, 4, 5, 6, 7]
    outs = []
    for W in (5, 7, 9):
        ring = O.RingCache(W, cfg.tokens_per_frame, cfg.d_c, cfg.d_rope)
        for f in frames[:-1]:
            c, kr = O.latents(frame_tokens(cfg, f), w["w_dkv"], w["w_kr"])
            ring.write(f, c, kr)
        qn, qr = chunk_queries(cfg, 7)
        outs.append(O.chunk_step(_dims(cfg), w, ring, frame_tokens(cfg, 7), 7, qn, qr))
    np.testing.assert_allclose(outs[1], outs[0], atol=1e-13)
    np.testing.assert_allclose(outs[2], outs[0], atol=1e-13)


def test_time_shift_invariance():
    cfg = get_config("tiny")
    w = layer_weights(cfg)
    res = []
    for shift in (0, 40, 233):
        ring = O.RingCache(cfg.window_frames, cfg.tokens_per_frame, cfg.d_c, cfg.d_rope)
        for i in range(2):
            c, kr = O.latents(frame_tokens(cfg, i), w["w_dkv"], w["w_kr"])
            ring.write(i + shift, c, kr)
        qn, qr = chunk_queries(cfg, 2)
        res.append(O.chunk_step(_dims(cfg), w, ring, frame_tokens(cfg, 2), 2 + shift, qn, qr))
    np.testing.assert_allclose(res[1], res[0], atol=1e-12)
    np.testing.assert_allclose(res[2], res[0], atol=1e-12)


# ------------------------------------------------------------------ softmax closed forms

def test_zero_query_gives_uniform_mean():
    cfg = get_config("tiny")
    _, w, ring, _, qn, qr, _ = _ring_step(cfg)
    out = O.chunk_step(_dims(cfg), w, ring, None, 2, np.zeros_like(qn), np.zeros_like(qr), write=False)
    c, _, _, _, _ = ring.keys(cfg.grid_y, cfg.grid_x)
    mean_c = c.mean(axis=0)
    for h in range(cfg.n_heads):
        np.testing.assert_allclose(out[:, h, :], np.broadcast_to(w["w_uv"][h] @ mean_c, out[:, h, :].shape),
                                   atol=1e-13)


def test_single_key_gives_its_value():
    cfg = get_config("tiny").with_(grid_y=1, grid_x=1, window_frames=1)
    w = layer_weights(cfg)
    ring = O.RingCache(1, 1, cfg.d_c, cfg.d_rope)
    x = frame_tokens(cfg, 0)
    qn, qr = chunk_queries(cfg, 0)
    out = O.chunk_step(_dims(cfg), w, ring, x, 0, qn, qr)
    c, _ = O.latents(x, w["w_dkv"], w["w_kr"])
    for h in range(cfg.n_heads):
        np.testing.assert_allclose(out[0, h], w["w_uv"][h] @ c[0], atol=1e-13)


def test_duplicated_keys_leave_output_unchanged():
    rng = np.random.default_rng(4)
    nq, nk, H, dh, dr = 5, 9, 3, 4, 6
    qn, qr = rng.standard_normal((nq, H, dh)), rng.standard_normal((nq, H, dr))
    kn, kr, v = rng.standard_normal((nk, H, dh)), rng.standard_normal((nk, dr)), rng.standard_normal((nk, H, dh))
    a = O.attend(qn, qr, kn, kr, v, 0.3)
    b = O.attend(qn, qr, np.concatenate([kn, kn]), np.concatenate([kr, kr]), np.concatenate([v, v]), 0.3)
    np.testing.assert_allclose(b, a, atol=1e-14)
    perm = rng.permutation(nk)
    c = O.attend(qn, qr, kn[perm], kr[perm], v[perm], 0.3)
    np.testing.assert_allclose(c, a, atol=1e-14)


def test_empty_window_outputs_zero():
    rng = np.random.default_rng(5)
    out = O.attend(rng.standard_normal((3, 2, 4)), rng.standard_normal((3, 2, 2)), np.zeros((0, 2, 4)),
                   np.zeros((0, 2)), np.zeros((0, 2, 4)), 0.5)
    assert out.shape == (3, 2, 4) and not out.any()
    lat = O.attend_latent(rng.standard_normal((3, 2, 6)), np.zeros((0, 4)), np.zeros((0, 2)), 0.5)
    assert lat.shape == (3, 2, 4) and not lat.any()


def test_planted_match_dominates():
    # one key whose score exceeds every other by > 60 takes all the weight
    rng = np.random.default_rng(6)
    H, dh, dr, nk = 2, 4, 2, 7
    kn = rng.standard_normal((nk, H, dh)) * 0.01
    kr = rng.standard_normal((nk, dr)) * 0.01
    v = rng.standard_normal((nk, H, dh))
    kn[3] = 10.0
    qn = np.full((1, H, dh), 10.0)
    qr = np.zeros((1, H, dr))
    out = O.attend(qn, qr, kn, kr, v, 0.5)
    np.testing.assert_allclose(out[0], v[3], atol=1e-12)


# ------------------------------------------------------------------ absorbed == reconstructed

@pytest.mark.parametrize("name", ["tiny", "wan_small"])
def test_absorbed_equals_reconstructed(name):
    cfg = get_config(name)
    out, w, ring, _, qn, qr, cf = _ring_step(cfg, q_scale=2.0)
    ab = O.chunk_step_absorbed(_dims(cfg), w, ring, cf, qn, qr)
    rel = np.linalg.norm(ab - out) / np.linalg.norm(out)
    assert rel < 1e-12


# ------------------------------------------------------------------ reduction to dense MHA

def _naive_mha(x_keys, x_q_nope, qr_rot, kr_rot, WK, WV, n_h, d_h, scale):
    """Independent dense multi-head attention with a decoupled shared rotary key:
    K_h = x W_K[h]^T, V_h = x W_V[h]^T, score = q.K + qR.kR."""
    out = np.zeros((x_q_nope.shape[0], n_h, d_h))
    for h in range(n_h):
        K = x_keys @ WK[h * d_h:(h + 1) * d_h].T
        V = x_keys @ WV[h * d_h:(h + 1) * d_h].T
        for i in range(x_q_nope.shape[0]):
            s = scale * (K @ x_q_nope[i, h] + kr_rot @ qr_rot[i, h])
            p = np.exp(s - s.max())
            out[i, h] = (p / p.sum()) @ V
    return out


def test_mla_with_full_rank_latent_equals_dense_mha():
    cfg = get_config("tiny").with_(hidden=12)
    n_h, d_h = cfg.n_heads, cfg.d_head
    d_c = 2 * n_h * d_h
    cfg = cfg.with_(d_c=d_c)
    rng = np.random.default_rng(7)
    WK = rng.standard_normal((n_h * d_h, cfg.hidden)) / np.sqrt(cfg.hidden)
    WV = rng.standard_normal((n_h * d_h, cfg.hidden)) / np.sqrt(cfg.hidden)
    w_kr = rng.standard_normal((cfg.d_rope, cfg.hidden)) / np.sqrt(cfg.hidden)
    w_uk = np.zeros((n_h, d_h, d_c))
    w_uv = np.zeros((n_h, d_h, d_c))
    for h in range(n_h):
        for d in range(d_h):
            w_uk[h, d, h * d_h + d] = 1.0  # selects head h's key rows of the stacked latent
            w_uv[h, d, n_h * d_h + h * d_h + d] = 1.0  # selects head h's value rows
    w = dict(w_dkv=np.concatenate([WK, WV]), w_kr=w_kr, w_uk=w_uk, w_uv=w_uv)
    ring = O.RingCache(cfg.window_frames, cfg.tokens_per_frame, d_c, cfg.d_rope)
    xs = [rng.standard_normal((cfg.tokens_per_frame, cfg.hidden)) for _ in range(3)]
    for f in range(2):
        c, kr = O.latents(xs[f], w["w_dkv"], w["w_kr"])
        ring.write(f, c, kr)
    qn = rng.standard_normal((cfg.tokens_per_frame, n_h, d_h))
    qr = rng.standard_normal((cfg.tokens_per_frame, n_h, cfg.d_rope))
    out = O.chunk_step(_dims(cfg), w, ring, xs[2], 2, qn, qr)
    xk = np.concatenate(xs)
    t, y, x = O.frame_positions([0, 1, 2], cfg.grid_y, cfg.grid_x)
    kr_rot = O.rope3d(xk @ w_kr.T, t, y, x, cfg.rope_split, cfg.rope_base)
    tq, yq, xq = O.frame_positions([2], cfg.grid_y, cfg.grid_x)
    qr_rot = O.rope3d(qr, tq, yq, xq, cfg.rope_split, cfg.rope_base)
    ref = _naive_mha(xk, qn, qr_rot, kr_rot, WK, WV, n_h, d_h, O.default_scale(d_h, cfg.d_rope))
    np.testing.assert_allclose(out, ref, atol=1e-12)


# ------------------------------------------------------------------ pure-Python brute force

def _brute_force_step(cfg, w, xs_window, frames_window, x_chunk_frames, qn, qr, q_frame_first,
                      frame_causal=False):
    """Triple loop over (query, head, key) with explicit reconstruction, from the
    definitions only (math module, Python floats). frame_causal: a query of
    frame f skips the keys of later frames."""
    gy, gx = cfg.grid_y, cfg.grid_x
    dc, dr, dh, nh = cfg.d_c, cfg.d_rope, cfg.d_head, cfg.n_heads
    split, base = cfg.rope_split, cfg.rope_base
    scale = 1.0 / math.sqrt(dh + dr)

    def rot(vec, t, y, x):
        out, o = [], 0
        for pos, d in ((t, split[0]), (y, split[1]), (x, split[2])):
            for k in range(d // 2):
                a = pos * base ** (-2.0 * k / d)
                v0, v1 = vec[o + 2 * k], vec[o + 2 * k + 1]
                out += [v0 * math.cos(a) - v1 * math.sin(a), v0 * math.sin(a) + v1 * math.cos(a)]
            o += d
        return out

    keys = []  # (k_nope per head, v per head, k_rope)
    for f, xf in zip(frames_window, xs_window):
        for tok in range(gy * gx):
            xv = xf[tok]
            c = [sum(w["w_dkv"][a][b] * xv[b] for b in range(len(xv))) for a in range(dc)]
            kr = [sum(w["w_kr"][a][b] * xv[b] for b in range(len(xv))) for a in range(dr)]
            kn = [[sum(w["w_uk"][h][d][a] * c[a] for a in range(dc)) for d in range(dh)] for h in range(nh)]
            vv = [[sum(w["w_uv"][h][d][a] * c[a] for a in range(dc)) for d in range(dh)] for h in range(nh)]
            keys.append((kn, vv, rot(kr, f, tok // gx, tok % gx), f))
    out = np.zeros((qn.shape[0], nh, dh))
    for i in range(qn.shape[0]):
        f = q_frame_first + i // (gy * gx)
        tok = i % (gy * gx)
        seen = [k for k in keys if not frame_causal or k[3] <= f]
        if not seen:
            continue
        for h in range(nh):
            qrot = rot(list(qr[i, h]), f, tok // gx, tok % gx)
            s = [scale * (sum(qn[i, h, d] * kn[h][d] for d in range(dh))
                          + sum(qrot[d] * krr[d] for d in range(dr))) for kn, _, krr, _ in seen]
            m = max(s)
            e = [math.exp(z - m) for z in s]
            tot = sum(e)
            for d in range(dh):
                out[i, h, d] = sum(e[j] * seen[j][1][h][d] for j in range(len(seen))) / tot
    return out


def test_oracle_matches_brute_force_tiny():
    cfg = get_config("tiny")
    out, w, ring, x_chunk, qn, qr, cf = _ring_step(cfg)
    xs = [frame_tokens(cfg, f) for f in range(3)]
    bf = _brute_force_step(cfg, w, xs, [0, 1, 2], None, qn, qr, cf)
    np.testing.assert_allclose(out, bf, rtol=0, atol=1e-12)


def test_oracle_matches_brute_force_partial_window():
    # window of 3 slots holding frames {3, 4} only after frames 0..2 were evicted
    cfg = get_config("tiny").with_(chunk_frames=1)
    w = layer_weights(cfg, seed=11)
    ring = O.RingCache(3, cfg.tokens_per_frame, cfg.d_c, cfg.d_rope)
    for f in range(5):
        c, kr = O.latents(frame_tokens(cfg, f, seed=11), w["w_dkv"], w["w_kr"])
        ring.write(f, c, kr)
    # window now holds frames 3, 4, 2 -> chunk = frame 5 evicts frame 2
    qn, qr = chunk_queries(cfg, 5, seed=11)
    out = O.chunk_step(_dims(cfg), w, ring, frame_tokens(cfg, 5, seed=11), 5, qn, qr)
    assert sorted(ring.slot_frame.tolist()) == [3, 4, 5]
    xs = [frame_tokens(cfg, f, seed=11) for f in (3, 4, 5)]
    bf = _brute_force_step(cfg, w, xs, [3, 4, 5], None, qn, qr, 5)
    np.testing.assert_allclose(out, bf, rtol=0, atol=1e-12)


def test_oracle_stage_functions_match_brute_force_pieces():
    """absorbed_query / attend_latent / up_project compose to the brute-force output."""
    cfg = get_config("tiny")
    out, w, ring, _, qn, qr, cf = _ring_step(cfg)
    c, kr, t, y, x = ring.keys(cfg.grid_y, cfg.grid_x)
    tq, yq, xq = O.frame_positions([cf], cfg.grid_y, cfg.grid_x)
    qa = O.absorbed_query(qn, qr, w["w_uk"], tq, yq, xq, cfg.rope_split, cfg.rope_base)
    lat = O.attend_latent(qa, c, O.rope3d(kr, t, y, x, cfg.rope_split, cfg.rope_base),
                          O.default_scale(cfg.d_head, cfg.d_rope))
    xs = [frame_tokens(cfg, f) for f in range(3)]
    bf = _brute_force_step(cfg, w, xs, [0, 1, 2], None, qn, qr, cf)
    np.testing.assert_allclose(O.up_project(lat, w["w_uv"]), bf, atol=1e-12)


# ------------------------------------------------------------------ query path and output projection

def _brute_force_layer(cfg, w, wq, xs_window, frames_window, x_chunk, q_frame_first, frame_causal=False):
    """The whole layer by loops: query latent, per-head queries, the brute-force
    attention above, then the output projection summed head by head."""
    nh, dh, dr, dq = cfg.n_heads, cfg.d_head, cfg.d_rope, cfg.q_latent
    n = x_chunk.shape[0]
    qn = np.zeros((n, nh, dh))
    qr = np.zeros((n, nh, dr))
    for i in range(n):
        cq = [sum(wq["w_dq"][a][b] * x_chunk[i][b] for b in range(cfg.hidden)) for a in range(dq)]
        for h in range(nh):
            for d in range(dh):
                qn[i, h, d] = sum(wq["w_uq"][h][d][a] * cq[a] for a in range(dq))
            for d in range(dr):
                qr[i, h, d] = sum(wq["w_qr"][h][d][a] * cq[a] for a in range(dq))
    o = _brute_force_step(cfg, w, xs_window, frames_window, None, qn, qr, q_frame_first, frame_causal)
    u = np.zeros((n, cfg.hidden))
    for i in range(n):
        for j in range(cfg.hidden):
            u[i, j] = sum(wq["w_o"][j][h * dh + d] * o[i, h, d] for h in range(nh) for d in range(dh))
    return u


@pytest.mark.parametrize("frame_causal", [False, True])
def test_layer_step_matches_brute_force(frame_causal):
    cfg = get_config("tiny").with_(chunk_frames=2, d_cq=24)
    w, wq = layer_weights(cfg, seed=21), query_weights(cfg, seed=21)
    ring = O.RingCache(cfg.window_frames, cfg.tokens_per_frame, cfg.d_c, cfg.d_rope)
    c, kr = O.latents(frame_tokens(cfg, 0, seed=21), w["w_dkv"], w["w_kr"])
    ring.write(0, c, kr)
    xc = np.concatenate([frame_tokens(cfg, f, seed=21) for f in (1, 2)])
    u, out, qn, qr = O.layer_step(_dims(cfg), {**w, **wq}, ring, xc, 1, frame_causal=frame_causal)
    assert u.shape == (2 * cfg.tokens_per_frame, cfg.hidden)
    xs = [frame_tokens(cfg, f, seed=21) for f in range(3)]
    bf = _brute_force_layer(cfg, w, wq, xs, [0, 1, 2], xc, 1, frame_causal)
    np.testing.assert_allclose(u, bf, rtol=0, atol=1e-12)


def test_layer_with_full_rank_query_latent_equals_dense_mha_layer():
    """With the identity as query down-projection (d_cq = hidden) and full-rank
    key/value latents, the layer is a dense multi-head attention layer with a
    decoupled rotary key: q_h = W_Q[h] x, qR_h = W_QR[h] x, u = sum_h W_O[h] o_h."""
    cfg = get_config("tiny").with_(hidden=12)
    n_h, d_h, dr = cfg.n_heads, cfg.d_head, cfg.d_rope
    d_c = 2 * n_h * d_h
    cfg = cfg.with_(d_c=d_c, d_cq=cfg.hidden)
    rng = np.random.default_rng(8)
    WK, WV, WQ = (rng.standard_normal((n_h * d_h, cfg.hidden)) / np.sqrt(cfg.hidden) for _ in range(3))
    WQR = rng.standard_normal((n_h * dr, cfg.hidden)) / np.sqrt(cfg.hidden)
    WO = rng.standard_normal((cfg.hidden, n_h * d_h)) / np.sqrt(n_h * d_h)
    w_kr = rng.standard_normal((dr, cfg.hidden)) / np.sqrt(cfg.hidden)
    w_uk = np.zeros((n_h, d_h, d_c))
    w_uv = np.zeros((n_h, d_h, d_c))
    for h in range(n_h):
        for d in range(d_h):
            w_uk[h, d, h * d_h + d] = 1.0
            w_uv[h, d, n_h * d_h + h * d_h + d] = 1.0
    w = dict(w_dkv=np.concatenate([WK, WV]), w_kr=w_kr, w_uk=w_uk, w_uv=w_uv, w_dq=np.eye(cfg.hidden),
             w_uq=WQ.reshape(n_h, d_h, cfg.hidden), w_qr=WQR.reshape(n_h, dr, cfg.hidden), w_o=WO)
    ring = O.RingCache(cfg.window_frames, cfg.tokens_per_frame, d_c, dr)
    xs = [rng.standard_normal((cfg.tokens_per_frame, cfg.hidden)) for _ in range(3)]
    for f in range(2):
        c, kr = O.latents(xs[f], w["w_dkv"], w["w_kr"])
        ring.write(f, c, kr)
    u, _, _, _ = O.layer_step(_dims(cfg), w, ring, xs[2], 2)
    xk = np.concatenate(xs)
    t, y, x = O.frame_positions([0, 1, 2], cfg.grid_y, cfg.grid_x)
    kr_rot = O.rope3d(xk @ w_kr.T, t, y, x, cfg.rope_split, cfg.rope_base)
    tq, yq, xq = O.frame_positions([2], cfg.grid_y, cfg.grid_x)
    qn = np.stack([xs[2] @ WQ[h * d_h:(h + 1) * d_h].T for h in range(n_h)], axis=1)
    qr = np.stack([xs[2] @ WQR[h * dr:(h + 1) * dr].T for h in range(n_h)], axis=1)
    qr_rot = O.rope3d(qr, tq, yq, xq, cfg.rope_split, cfg.rope_base)
    o = _naive_mha(xk, qn, qr_rot, kr_rot, WK, WV, n_h, d_h, O.default_scale(d_h, dr))
    ref = sum(o[:, h] @ WO[:, h * d_h:(h + 1) * d_h].T for h in range(n_h))
    np.testing.assert_allclose(u, ref, atol=1e-12)


# ------------------------------------------------------------------ input generator sanity

def test_bf16_rounding_is_round_to_nearest_even():
    from harness import to_bf16_bits, from_bf16_bits
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0
    assert from_bf16_bits(to_bf16_bits([1.0 + 2 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even -> 1 + 2^-6
    assert from_bf16_bits(to_bf16_bits([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6
    assert from_bf16_bits(to_bf16_bits([-2.5]))[0] == -2.5
    assert to_bf16_bits([1.0])[0] == 0x3F80


# ------------------------------------------------------------------ frame-causal variant

def _causal_ring(cfg, seed, frames_before, chunk_first):
    w = layer_weights(cfg, seed)
    ring = O.RingCache(cfg.window_frames, cfg.tokens_per_frame, cfg.d_c, cfg.d_rope)
    for f in frames_before:
        c, kr = O.latents(frame_tokens(cfg, f, seed), w["w_dkv"], w["w_kr"])
        ring.write(f, c, kr)
    x_chunk = np.concatenate([frame_tokens(cfg, chunk_first + i, seed) for i in range(cfg.chunk_frames)])
    qn, qr = chunk_queries(cfg, chunk_first, seed)
    return w, ring, x_chunk, qn, qr


def test_frame_causal_matches_brute_force():
    """Two-frame chunk: queries of its first frame skip the second frame's keys
    (brute force from the definition, with the skip written out)."""
    cfg = get_config("tiny").with_(chunk_frames=2, window_frames=4)
    w, ring, x_chunk, qn, qr = _causal_ring(cfg, 21, [0, 1], 2)
    out = O.chunk_step(_dims(cfg), w, ring, x_chunk, 2, qn, qr, frame_causal=True)
    xs = [frame_tokens(cfg, f, 21) for f in range(4)]
    bf = _brute_force_step(cfg, w, xs, [0, 1, 2, 3], None, qn, qr, 2, frame_causal=True)
    np.testing.assert_allclose(out, bf, rtol=0, atol=1e-12)


def test_frame_causal_equals_window_without_later_frames():
    """The frame-causal rows of chunk frame f equal the unmasked step of a ring
    that never received the frames after f (a different route: what is in the
    window instead of which scores are masked), here with the ring wrapped:
    after the chunk the window holds frames 3..6."""
    cfg = get_config("tiny").with_(chunk_frames=3, window_frames=4)
    T = cfg.tokens_per_frame
    w, ring, x_chunk, qn, qr = _causal_ring(cfg, 22, [0, 1, 2, 3], 4)
    out = O.chunk_step(_dims(cfg), w, ring, x_chunk, 4, qn, qr, frame_causal=True)
    assert sorted(ring.slot_frame.tolist()) == [3, 4, 5, 6]
    for k in range(3):  # chunk frame 4 + k
        f = 4 + k
        ring_k = O.RingCache(cfg.window_frames, T, cfg.d_c, cfg.d_rope)
        for g in range(3, f + 1):
            c, kr = O.latents(frame_tokens(cfg, g, 22), w["w_dkv"], w["w_kr"])
            ring_k.write(g, c, kr)
        ref = O.chunk_step(_dims(cfg), w, ring_k, None, f, qn[k * T:(k + 1) * T], qr[k * T:(k + 1) * T],
                           write=False)
        np.testing.assert_allclose(out[k * T:(k + 1) * T], ref, rtol=0, atol=1e-12)


def test_frame_causal_single_frame_chunk_is_unmasked():
    cfg = get_config("tiny").with_(chunk_frames=1)
    w, ring, x_chunk, qn, qr = _causal_ring(cfg, 23, [0, 1], 2)
    a = O.chunk_step(_dims(cfg), w, ring, x_chunk, 2, qn, qr, frame_causal=True)
    b = O.chunk_step(_dims(cfg), w, ring, None, 2, qn, qr, write=False)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)

