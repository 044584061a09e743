"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
catch every one: each mutated oracle must fail the brute-force or the
textbook-RoPE comparison."""
import numpy as np
import pytest

from harness import get_config
from oracle import mla_oracle as O

from . import test_oracle_pins as P


def _rot_sign_flip(v, cos, sin):
    out = np.empty(v.shape)
    out[..., 0::2] = v[..., 0::2] * cos + v[..., 1::2] * sin
    out[..., 1::2] = -v[..., 0::2] * sin + v[..., 1::2] * cos
    return out


def _rot_half_split(v, cos, sin):
    h = v.shape[-1] // 2
    out = np.empty(v.shape)
    out[..., :h] = v[..., :h] * cos - v[..., h:] * sin
    out[..., h:] = v[..., :h] * sin + v[..., h:] * cos
    return out


def _freq_wrong_exponent(d, base):
    return np.power(float(base), -np.arange(d // 2, dtype=np.float64) / d)


_orig_attend = O.attend
_orig_reconstruct = O.reconstruct
_orig_rope3d = O.rope3d


def _attend_no_rope(qn, qr, kn, kr, v, scale, block=64, visible=None):
    return _orig_attend(qn, np.zeros_like(qr), kn, np.zeros_like(kr), v, scale, block, visible=visible)


def _attend_wrong_scale(qn, qr, kn, kr, v, scale, block=64, visible=None):
    return _orig_attend(qn, qr, kn, kr, v, scale * np.sqrt(160.0 / 128.0), block, visible=visible)


def _attend_mask_ignored(qn, qr, kn, kr, v, scale, block=64, visible=None):
    return _orig_attend(qn, qr, kn, kr, v, scale, block)


def _causal_strict(q_frames, k_frames):
    return np.asarray(q_frames)[:, None] > np.asarray(k_frames)[None, :]


def _reconstruct_swapped(c, w_uk, w_uv):
    k, v = _orig_reconstruct(c, w_uk, w_uv)
    return v, k


def _rope3d_axes_swapped(v, t, y, x, split, base):
    return _orig_rope3d(v, t, x, y, split, base)


def _attend_softmax_over_heads(qn, qr, kn, kr, v, scale, block=64, visible=None):
    s = (np.einsum("qhd,khd->qhk", qn, kn) + np.einsum("qhr,kr->qhk", qr, kr)) * scale
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return np.einsum("qhk,khd->qhd", p, v)


_orig_query_project = O.query_project


def _query_heads_transposed(x, w_dq, w_uq, w_qr):
    # per-head weights read as [d_h, H, d_cq]: heads and components interleaved
    nh, dh, dq = np.shape(w_uq)
    w_t = np.asarray(w_uq).reshape(dh, nh, dq).transpose(1, 0, 2)
    return _orig_query_project(x, w_dq, w_t, w_qr)


def _query_rope_from_token(x, w_dq, w_uq, w_qr):
    # positional query taken from the content query's first components
    c_q, qn, qr = _orig_query_project(x, w_dq, w_uq, w_qr)
    return c_q, qn, qn[..., :qr.shape[-1]].copy()


def _output_heads_interleaved(o, w_o):
    o = np.asarray(o, np.float64)
    return o.transpose(0, 2, 1).reshape(o.shape[0], -1) @ np.asarray(w_o, np.float64).T


def _output_transposed(o, w_o):
    o = np.asarray(o, np.float64)
    w = np.asarray(w_o, np.float64)
    return o.reshape(o.shape[0], -1) @ w.reshape(w.shape[1], w.shape[0])


MUTATIONS = {
    "rotation_sign": ("rotate_pairs", _rot_sign_flip),
    "half_split_pairs": ("rotate_pairs", _rot_half_split),
    "frequency_exponent": ("rope_inv_freq", _freq_wrong_exponent),
    "dropped_rope_term": ("attend", _attend_no_rope),
    "wrong_scale": ("attend", _attend_wrong_scale),
    "keys_values_swapped": ("reconstruct", _reconstruct_swapped),
    "rope_axes_swapped": ("rope3d", _rope3d_axes_swapped),
    "softmax_axis": ("attend", _attend_softmax_over_heads),
    "causal_mask_ignored": ("attend", _attend_mask_ignored),
    "causal_mask_strict": ("frame_causal_mask", _causal_strict),
    "query_heads_transposed": ("query_project", _query_heads_transposed),
    "query_rope_from_content": ("query_project", _query_rope_from_token),
    "output_heads_interleaved": ("output_project", _output_heads_interleaved),
    "output_weight_transposed": ("output_project", _output_transposed),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = 0
    for check in (P.test_oracle_matches_brute_force_tiny, P.test_rope3d_blocks_equal_textbook_1d,
                  P.test_oracle_matches_brute_force_partial_window, P.test_frame_causal_matches_brute_force,
                  lambda: P.test_layer_step_matches_brute_force(False)):
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"mutation {name} passed every pin"


def test_unmutated_oracle_passes_same_checks():
    cfg = get_config("tiny")
    assert cfg.d_c == 16
    P.test_oracle_matches_brute_force_tiny()
    P.test_rope3d_blocks_equal_textbook_1d()
    P.test_oracle_matches_brute_force_partial_window()
    P.test_frame_causal_matches_brute_force()
    P.test_layer_step_matches_brute_force(False)
