"""Stream state and determinism on the GPU.

The state of a stream is its per-layer ring cache, its slot table and the
index of the next frame: a rollout snapshot taken between chunks and
restored into fresh buffers continues bit for bit like the uninterrupted
run. Every kernel reduces in a fixed order (no atomics in any sum), so the
same call on the same inputs gives the same bits.
"""
import pytest
import torch

import latent_kv_attention_amd as mla
from latent_kv_attention_amd.layer import LatentLayer
from harness import get_config

from .gpu_common import Stream, device_weights, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib(built_lib):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mla.lib()
    yield


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _chunk(layer, st, k, attend="attend"):
    f0 = 3 * k
    layer.write(to_torch(st.xs(f0, 3)[None], layer.cfg.dtype), f0, 3)
    qn, qr = st.q(f0)
    return getattr(layer, attend)(to_torch(qn[None], layer.cfg.dtype), to_torch(qr[None], layer.cfg.dtype), f0, 3)


def test_rollout_snapshot_and_restore_is_bitwise_identical():
    """Wan-shaped rollout through a 21-frame ring: a snapshot after chunk 8
    (the ring has wrapped) restored into a new layer continues through
    chunks 9..11 with bit-identical outputs, cache and slot table."""
    cfg = get_config("wan_rollout")
    w, wd = device_weights(cfg, seed=6)
    st = Stream(cfg, seed=6, pooled=True)
    layer = LatentLayer(cfg, wd, batch=1, rope_n_t=64)
    snap = None
    outs = {}
    for k in range(12):
        out = _chunk(layer, st, k)
        if k >= 9:
            outs[k] = out.clone()
        if k == 8:
            torch.cuda.synchronize()
            snap = (layer.cache.clone(), layer.slot_frame.clone(), 3 * (k + 1))
    torch.cuda.synchronize()
    final = (layer.cache.clone(), layer.slot_frame.clone())

    restored = LatentLayer(cfg, wd, batch=1, rope_n_t=64)
    restored.cache.copy_(snap[0])
    restored.slot_frame.copy_(snap[1])
    assert snap[2] == 27
    for k in range(9, 12):
        out = _chunk(restored, st, k)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(outs[k])), f"chunk {k} differs after restore"
    assert torch.equal(_bits(restored.cache), _bits(final[0]))
    assert torch.equal(restored.slot_frame, final[1])
    print(f"[state] restore after chunk 8: chunks 9-11 bit-identical, slots {final[1].cpu().numpy()[0].tolist()}",
          flush=True)


@pytest.mark.parametrize("attend", ["attend_latent", "attend_latent_frame_causal", "attend_heads",
                                    "attend_heads_frame_causal"])
def test_repeated_calls_are_bitwise_identical(attend):
    """The Wan chunk step (its row blocks split between work-groups and
    merged) repeated on the same inputs gives the same bits, for both forms
    with and without the frame-causal mask."""
    cfg = get_config("wan")
    w, wd = device_weights(cfg, seed=7)
    st = Stream(cfg, seed=7, pooled=True)
    layer = LatentLayer(cfg, wd, batch=1, rope_n_t=64)
    layer.write(to_torch(st.xs(0, 18)[None], cfg.dtype), 0, 18)
    outs = [_chunk(layer, st, 6, attend).clone() for _ in range(3)]
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0].float()).all()
    for o in outs[1:]:
        assert torch.equal(_bits(o), _bits(outs[0]))
