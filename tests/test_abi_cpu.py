"""The C-ABI library loads, exports every symbol include/mla.h declares, and
rejects bad arguments on the host before touching the GPU (no compute calls
here: every call below fails validation, so nothing is enqueued)."""
import ctypes
import os
import re
import subprocess

import pytest

import latent_kv_attention_amd as mla
from harness import get_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert _declared() == sorted(mla.EXPORTS)


def test_library_exports_every_declared_symbol(built_lib):
    out = subprocess.run(["nm", "-D", "--defined-only", built_lib], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\b(mla_[a-z0-9_]+)\b", out))
    missing = set(_declared()) - exported
    assert not missing, missing
    lib = mla.lib()
    for name in _declared():
        assert getattr(lib, name) is not None


def test_abi_version_and_status_strings(built_lib):
    assert mla.abi_version() == 1
    lib = mla.lib()
    for code in range(10):
        s = lib.mla_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert lib.mla_status_string(99) == b"unknown status"


def _shape(name="wan", **kw):
    s = mla.make_shape(get_config(name))
    for k, v in kw.items():
        setattr(s, k, v)
    return s


@pytest.mark.parametrize("field,value,code", [
    ("dtype", 7, 3), ("batch", 0, 2), ("hidden", 12, 2), ("d_head", 12, 2), ("d_head", 512, 2),
    ("window_frames", 0, 2), ("window_frames", 65, 2), ("d_rope_t", 7, 2), ("d_rope_x", 10, 2),
    ("rope_base", 0.0, 2), ("grid_x", 0, 2), ("d_c", 96, 6),
])
def test_shape_validation(built_lib, field, value, code):
    assert mla.shape_check(_shape()) == 0
    assert mla.shape_check(_shape(**{field: value})) == code


SUPPORTED_LATENTS = [(192, 32, (8, 12, 12)), (128, 32, (8, 12, 12)), (160, 64, (16, 24, 24)),
                     (192, 64, (16, 24, 24)), (16, 8, (2, 2, 4))]


def test_latent_widths_with_kernels(built_lib):
    """Every (d_c, d_rope) pair with kernel instantiations passes the shape
    check; other pairs are rejected as unsupported before any launch."""
    for dc, dr, (t, y, x) in SUPPORTED_LATENTS:
        assert mla.shape_check(_shape(d_c=dc, d_rope=dr, d_rope_t=t, d_rope_y=y, d_rope_x=x)) == 0, (dc, dr)
    for dc, dr, (t, y, x) in [(224, 32, (8, 12, 12)), (160, 32, (8, 12, 12)), (128, 64, (16, 24, 24))]:
        assert mla.shape_check(_shape(d_c=dc, d_rope=dr, d_rope_t=t, d_rope_y=y, d_rope_x=x)) == 6, (dc, dr)


def test_host_queries(built_lib):
    wan = _shape()
    assert mla.qabs_dim(wan) == 224
    assert mla.qabs_dim(_shape("tiny")) == 32
    assert mla.qabs_dim(_shape(d_c=100)) == 0
    # tables: 2 * (n_t*4 + 30*6 + 52*6)
    assert mla.rope3d_table_floats(wan, 21) == 2 * (21 * 4 + 30 * 6 + 52 * 6)
    assert mla.rope3d_table_floats(wan, 0) == 0
    ws = mla.chunk_attend_workspace_bytes(wan, 3)
    rows = 3 * 1560 * 12
    assert ws >= rows * 224 * 2 + rows * 192 * 2
    assert mla.flash_workspace_bytes(wan, 3, 4) > mla.flash_workspace_bytes(wan, 3, 1)
    assert mla.flash_workspace_bytes(wan, 3, 17) == 0
    # per-head form: expanded keys and values of every head dominate its workspace
    hws = mla.chunk_attend_heads_workspace_bytes(wan, 3)
    assert hws >= 2 * 12 * 21 * 1560 * 128 * 2 + 12 * rows // 12 * (128 + 32) * 2
    assert mla.chunk_attend_heads_workspace_bytes(_shape("wan_small_f32"), 1) == 0
    assert mla.chunk_attend_heads_workspace_bytes(_shape(d_head=64), 3) == 0


def test_entry_points_reject_bad_arguments_before_launch(built_lib):
    lib = mla.lib()
    s = _shape()
    sp = ctypes.byref(s)
    fake = ctypes.c_void_p(0x100000)  # aligned, never dereferenced: validation fails first
    odd = ctypes.c_void_p(0x100008)
    # NULL pointers
    assert lib.mla_cache_write(sp, None, fake, fake, 0, 3, fake, fake, None) == 1
    assert lib.mla_rope3d_tables(sp, 0, 21, None, None) == 1
    assert lib.mla_up_v(sp, fake, 3, None, fake, None) == 1
    # misalignment
    assert lib.mla_cache_write(sp, odd, fake, fake, 0, 3, fake, fake, None) == 4
    # frame ranges: n_frames > window, negative first frame
    assert lib.mla_cache_write(sp, fake, fake, fake, 0, 22, fake, fake, None) == 8
    assert lib.mla_cache_write(sp, fake, fake, fake, -1, 3, fake, fake, None) == 8
    # query frames outside the RoPE table range
    assert lib.mla_absorb_q(sp, fake, fake, 30, 3, fake, fake, 0, 21, fake, None) == 8
    # workspace too small / splits out of range
    assert lib.mla_flash_attend(sp, fake, 3, fake, fake, fake, 0, 21, fake, 0, fake, 16, None) == 5
    assert lib.mla_flash_attend(sp, fake, 3, fake, fake, fake, 0, 21, fake, 17, fake, 1 << 30, None) == 8
    assert lib.mla_chunk_attend(sp, fake, fake, 0, 3, fake, fake, fake, fake, fake, 0, 21, fake, fake, 16,
                                None) == 5
    # per-head form: workspace too small; shapes it does not cover (fp32, other head widths)
    assert lib.mla_chunk_attend_heads(sp, fake, fake, 0, 3, fake, fake, fake, fake, fake, 0, 21, fake, fake, 16,
                                      None) == 5
    f32 = _shape("wan_small_f32")
    assert lib.mla_chunk_attend_heads(ctypes.byref(f32), fake, fake, 0, 1, fake, fake, fake, fake, fake, 0, 21,
                                      fake, fake, 1 << 40, None) == 6
    # query path and output projection: NULL, alignment, query latent width, frame count
    assert lib.mla_query_project(sp, 576, fake, 3, fake, fake, None, fake, fake, fake, None) == 1
    assert lib.mla_query_project(sp, 576, fake, 3, fake, fake, fake, odd, fake, fake, None) == 4
    assert lib.mla_query_project(sp, 572, fake, 3, fake, fake, fake, fake, fake, fake, None) == 2
    assert lib.mla_query_project(sp, 0, fake, 3, fake, fake, fake, fake, fake, fake, None) == 2
    assert lib.mla_query_project(sp, 576, fake, 0, fake, fake, fake, fake, fake, fake, None) == 8
    assert lib.mla_output_project(sp, fake, 3, None, fake, None) == 1
    assert lib.mla_output_project(sp, fake, 3, fake, odd, None) == 4
    assert lib.mla_output_project(sp, fake, -1, fake, fake, None) == 8
    # unsupported latent width
    bad = _shape(d_c=96)
    assert lib.mla_cache_write(ctypes.byref(bad), fake, fake, fake, 0, 3, fake, fake, None) == 6
    assert lib.mla_shape_check(None) == 1


def test_binding_refuses_host_strided_and_mistyped_tensors():
    """The Python binding passes only dense GPU buffers: a tensor in host
    memory, a strided view or a slot table / RoPE table of another element
    type is refused before the library is called (a host address handed to
    a kernel would fault the GPU)."""
    import torch

    s = mla.make_shape(get_config("wan_small"))
    host = torch.zeros(4, 4)
    with pytest.raises(ValueError, match="GPU tensor"):
        mla.cache_write(s, host, host, host, 0, 1, host, host)
    with pytest.raises(ValueError, match="GPU tensor"):
        mla.layer_weights_struct({"w_dkv": host})
    # the contiguity and dtype checks run on tensors that claim to be on the GPU
    class _Fake:
        is_cuda = True

        def __init__(self, contiguous=True, dtype="torch.bfloat16"):
            self._c, self.dtype = contiguous, dtype

        def is_contiguous(self):
            return self._c

        def stride(self):
            return (1, 4)

        def data_ptr(self):
            return 256

    from latent_kv_attention_amd._lib import _ptr
    with pytest.raises(ValueError, match="contiguous"):
        _ptr(_Fake(contiguous=False))
    with pytest.raises(ValueError, match="int32"):
        _ptr(_Fake(dtype="torch.int64"), "int32")
    with pytest.raises(ValueError, match="float32"):
        _ptr(_Fake(dtype="torch.bfloat16"), "float32")
    assert _ptr(_Fake(dtype="torch.int32"), "int32").value == 256
    assert _ptr(None) is None


def test_ceiling_probe_library_loads_and_checks_arguments():
    """The matrix-core ceiling probe (its own library, used by bench.py) loads,
    counts its FLOPs as documented, and refuses out-of-range launches before
    any HIP call."""
    from latent_kv_attention_amd import build as _build
    if not os.path.exists(_build.CEILING_LIB_PATH):
        _build.build()
    lib = ctypes.CDLL(_build.CEILING_LIB_PATH)
    lib.mla_ceiling_flops.restype = ctypes.c_double
    lib.mla_ceiling_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.mla_ceiling_run.restype = ctypes.c_int32
    lib.mla_ceiling_run.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.mla_ceiling_flops(256, 20000) == 256 * 8 * 20000 * 8 * 2 * 16 * 16 * 32
    fake = ctypes.c_void_p(1 << 20)
    assert lib.mla_ceiling_run(0, 10, fake, None) == 1
    assert lib.mla_ceiling_run(256, 0, fake, None) == 1
    assert lib.mla_ceiling_run(256, 10, None, None) == 1
    # the attention library does not carry the probe
    assert not hasattr(mla.lib(), "mla_ceiling_run")


def test_chunk_attend_form_selection(built_lib):
    """mla_chunk_attend takes the per-head form at the Wan2.1 width for chunks
    of at least 2048 queries per stream, and the latent form for small
    chunks, equal product counts (d_c 128), fp32 and unsupported head widths."""
    def form(name, nf, **kw):
        return mla.chunk_attend_form(mla.make_shape(get_config(name).with_(**kw)), nf)
    assert form("wan", 3) == mla.FORM_HEADS and form("wan", 2) == mla.FORM_HEADS
    assert form("wan", 1) == mla.FORM_LATENT                             # 1560 queries
    assert form("wan", 3, batch=8) == mla.FORM_HEADS
    assert form("wan_small", 2) == mla.FORM_LATENT                       # 132 queries
    assert form("wan_small", 1, grid_y=32, grid_x=64) == mla.FORM_HEADS  # 2048 queries
    assert form("wan_small", 1, grid_y=31, grid_x=66) == mla.FORM_LATENT  # 2046
    assert form("wan", 3, d_c=128) == mla.FORM_LATENT
    assert form("wan", 3, d_c=160, d_rope=64, rope_split=(16, 24, 24)) == mla.FORM_LATENT  # ratio 1.2
    assert form("wan", 3, d_c=192, d_rope=64, rope_split=(16, 24, 24)) == mla.FORM_HEADS
    assert form("wan", 3, dtype="f32") == mla.FORM_LATENT
    assert form("wan", 3, d_head=64) == mla.FORM_LATENT
    assert form("wan", 0) == -1
    s = mla.make_shape(get_config("wan"))
    assert mla.chunk_attend_workspace_bytes(s, 3) >= mla.chunk_attend_heads_workspace_bytes(s, 3)
