"""ctypes binding of libmla355.so (the C ABI declared in include/mla.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI. PyTorch tensors supply device pointers and the
stream. The library must have been built (latent_kv_attention_amd.build);
loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla355.so")

MLA_BF16, MLA_F32 = 0, 1

STATUS = {
    0: "MLA_OK", 1: "MLA_ERR_NULL", 2: "MLA_ERR_SHAPE", 3: "MLA_ERR_DTYPE", 4: "MLA_ERR_ALIGN",
    5: "MLA_ERR_WORKSPACE", 6: "MLA_ERR_UNSUPPORTED", 7: "MLA_ERR_HIP", 8: "MLA_ERR_RANGE", 9: "MLA_ERR_SCRATCH",
}

# every symbol include/mla.h declares
EXPORTS = [
    "mla_abi_version", "mla_status_string", "mla_shape_check", "mla_qabs_dim",
    "mla_rope3d_table_floats", "mla_rope3d_tables", "mla_cache_write", "mla_absorb_q",
    "mla_flash_workspace_bytes", "mla_flash_attend", "mla_flash_attend_frame_causal", "mla_flash_attend_noalloc",
    "mla_up_v",
    "mla_chunk_attend_workspace_bytes", "mla_chunk_attend", "mla_chunk_attend_latent", "mla_chunk_attend_form",
    "mla_chunk_attend_heads_workspace_bytes", "mla_chunk_attend_heads", "mla_chunk_attend_frame_causal",
    "mla_chunk_attend_latent_frame_causal", "mla_chunk_attend_heads_frame_causal",
    "mla_query_project", "mla_output_project", "mla_layer_step_workspace_bytes", "mla_layer_step",
    "mla_query_absorb_weights", "mla_query_project_absorbed",
]


class MlaShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "hidden", "n_heads", "d_head", "d_c", "d_rope", "d_rope_t", "d_rope_y", "d_rope_x",
        "grid_y", "grid_x", "window_frames", "dtype")] + [("rope_base", ctypes.c_float),
                                                          ("softmax_scale", ctypes.c_float)]


class MlaLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_dkv", "w_kr", "w_dq", "w_uq", "w_qr", "w_uk", "w_uv", "w_o",
                                                "w_qabs")]


class MlaError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")
        self.code = code


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t
_SP = ctypes.POINTER(MlaShape)

_SIGS = {
    "mla_abi_version": (_I, []),
    "mla_status_string": (ctypes.c_char_p, [_I]),
    "mla_shape_check": (_I, [_SP]),
    "mla_qabs_dim": (_I, [_SP]),
    "mla_rope3d_table_floats": (_SZ, [_SP, _I]),
    "mla_rope3d_tables": (_I, [_SP, _I, _I, _P, _P]),
    "mla_cache_write": (_I, [_SP, _P, _P, _P, _I, _I, _P, _P, _P]),
    "mla_absorb_q": (_I, [_SP, _P, _P, _I, _I, _P, _P, _I, _I, _P, _P]),
    "mla_flash_workspace_bytes": (_SZ, [_SP, _I, _I]),
    "mla_flash_attend": (_I, [_SP, _P, _I, _P, _P, _P, _I, _I, _P, _I, _P, _SZ, _P]),
    "mla_flash_attend_frame_causal": (_I, [_SP, _P, _I, _I, _P, _P, _P, _I, _I, _P, _I, _P, _SZ, _P]),
    "mla_flash_attend_noalloc": (_I, [_SP, _P, _I, _P, _P, _P, _I, _I, _P, _I, _P]),
    "mla_up_v": (_I, [_SP, _P, _I, _P, _P, _P]),
    "mla_chunk_attend_workspace_bytes": (_SZ, [_SP, _I]),
    "mla_chunk_attend": (_I, [_SP, _P, _P, _I, _I, _P, _P, _P, _P, _P, _I, _I, _P, _P, _SZ, _P]),
    "mla_chunk_attend_latent": (_I, [_SP, _P, _P, _I, _I, _P, _P, _P, _P, _P, _I, _I, _P, _P, _SZ, _P]),
    "mla_chunk_attend_form": (_I, [_SP, _I]),
    "mla_chunk_attend_heads_workspace_bytes": (_SZ, [_SP, _I]),
    "mla_chunk_attend_frame_causal": (_I, [_SP, _P, _P, _I, _I, _P, _P, _P, _P, _P, _I, _I, _P, _P, _SZ, _P]),
    "mla_chunk_attend_heads": (_I, [_SP, _P, _P, _I, _I, _P, _P, _P, _P, _P, _I, _I, _P, _P, _SZ, _P]),
    "mla_chunk_attend_latent_frame_causal": (_I, [_SP, _P, _P, _I, _I, _P, _P, _P, _P, _P, _I, _I, _P, _P, _SZ, _P]),
    "mla_chunk_attend_heads_frame_causal": (_I, [_SP, _P, _P, _I, _I, _P, _P, _P, _P, _P, _I, _I, _P, _P, _SZ, _P]),
    "mla_query_project": (_I, [_SP, _I, _P, _I, _P, _P, _P, _P, _P, _P, _P]),
    "mla_output_project": (_I, [_SP, _P, _I, _P, _P, _P]),
    "mla_layer_step_workspace_bytes": (_SZ, [_SP, _I, _I]),
    "mla_query_absorb_weights": (_I, [_SP, _I, _P, _P, _P, _P, _P]),
    "mla_query_project_absorbed": (_I, [_SP, _I, _P, _I, _I, _P, _P, _P, _I, _I, _P, _P, _P]),
    "mla_layer_step": (_I, [_SP, _I, ctypes.POINTER(MlaLayerWeights), _P, _I, _I, _P, _P, _P, _I, _I, _I, _P, _P,
                            _SZ, _P]),
}


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m latent_kv_attention_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def make_shape(cfg, batch: int | None = None, softmax_scale: float = 0.0) -> MlaShape:
    """mla_shape from any object with the harness config's fields."""
    t, y, x = cfg.rope_split
    return MlaShape(batch=batch if batch is not None else cfg.batch, hidden=cfg.hidden, n_heads=cfg.n_heads,
                    d_head=cfg.d_head, d_c=cfg.d_c, d_rope=cfg.d_rope, d_rope_t=t, d_rope_y=y, d_rope_x=x,
                    grid_y=cfg.grid_y, grid_x=cfg.grid_x, window_frames=cfg.window_frames,
                    dtype=MLA_BF16 if cfg.dtype == "bf16" else MLA_F32, rope_base=cfg.rope_base,
                    softmax_scale=softmax_scale)


def _check(fn, code):
    if code != 0:
        raise MlaError(fn, code)


def _ptr(t, dtype: str | None = None):
    """Device address of a tensor. The kernels read and write dense row-major
    buffers in GPU memory at that address, so a tensor in host memory, a
    strided view or (for the typed arguments: slot table int32, RoPE tables
    float32) another element type is refused here, before any call."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"mla: expected a GPU tensor, got one on {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"mla: expected a contiguous tensor, got strides {tuple(t.stride())}")
    if dtype is not None and str(t.dtype) != "torch." + dtype:
        raise ValueError(f"mla: expected {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def abi_version() -> int:
    return lib().mla_abi_version()


def shape_check(shape: MlaShape) -> int:
    return lib().mla_shape_check(ctypes.byref(shape))


def qabs_dim(shape: MlaShape) -> int:
    return lib().mla_qabs_dim(ctypes.byref(shape))


def rope3d_table_floats(shape: MlaShape, n_t: int) -> int:
    return lib().mla_rope3d_table_floats(ctypes.byref(shape), n_t)


def rope3d_tables(shape: MlaShape, t_first: int, n_t: int, tables, stream=None) -> None:
    _check("mla_rope3d_tables", lib().mla_rope3d_tables(ctypes.byref(shape), t_first, n_t, _ptr(tables, "float32"),
                                                        _stream(stream)))


def cache_write(shape: MlaShape, x, w_dkv, w_kr, frame_first: int, n_frames: int, cache, slot_frame,
                stream=None) -> None:
    _check("mla_cache_write", lib().mla_cache_write(ctypes.byref(shape), _ptr(x), _ptr(w_dkv), _ptr(w_kr),
                                                    frame_first, n_frames, _ptr(cache), _ptr(slot_frame, "int32"),
                                                    _stream(stream)))


def absorb_q(shape: MlaShape, q_nope, q_r, q_frame_first: int, q_n_frames: int, w_uk, tables,
             rope_t_first: int, rope_n_t: int, q_abs, stream=None) -> None:
    _check("mla_absorb_q", lib().mla_absorb_q(ctypes.byref(shape), _ptr(q_nope), _ptr(q_r), q_frame_first,
                                              q_n_frames, _ptr(w_uk), _ptr(tables, "float32"), rope_t_first, rope_n_t,
                                              _ptr(q_abs), _stream(stream)))


def flash_workspace_bytes(shape: MlaShape, q_n_frames: int, kv_splits: int = 0) -> int:
    return lib().mla_flash_workspace_bytes(ctypes.byref(shape), q_n_frames, kv_splits)


def flash_attend(shape: MlaShape, q_abs, q_n_frames: int, cache, slot_frame, tables, rope_t_first: int,
                 rope_n_t: int, o_lat, workspace, kv_splits: int = 0, stream=None) -> None:
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("mla_flash_attend", lib().mla_flash_attend(ctypes.byref(shape), _ptr(q_abs), q_n_frames, _ptr(cache),
                                                      _ptr(slot_frame, "int32"), _ptr(tables, "float32"), rope_t_first, rope_n_t,
                                                      _ptr(o_lat), kv_splits, _ptr(workspace), nbytes,
                                                      _stream(stream)))


def flash_attend_frame_causal(shape: MlaShape, q_abs, q_frame_first: int, q_n_frames: int, cache, slot_frame,
                              tables, rope_t_first: int, rope_n_t: int, o_lat, workspace, kv_splits: int = 0,
                              stream=None) -> None:
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("mla_flash_attend_frame_causal",
           lib().mla_flash_attend_frame_causal(ctypes.byref(shape), _ptr(q_abs), q_frame_first, q_n_frames,
                                               _ptr(cache), _ptr(slot_frame, "int32"), _ptr(tables, "float32"),
                                               rope_t_first, rope_n_t, _ptr(o_lat), kv_splits, _ptr(workspace),
                                               nbytes, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20  # MLA_NOALLOC_SCRATCH_BYTES


def flash_attend_noalloc(shape: MlaShape, q_abs, q_n_frames: int, cache, slot_frame, tables, rope_t_first: int,
                         rope_n_t: int, o_lat, kv_splits: int = 0, stream=None) -> None:
    _check("mla_flash_attend_noalloc",
           lib().mla_flash_attend_noalloc(ctypes.byref(shape), _ptr(q_abs), q_n_frames, _ptr(cache),
                                          _ptr(slot_frame, "int32"), _ptr(tables, "float32"), rope_t_first, rope_n_t,
                                          _ptr(o_lat), kv_splits, _stream(stream)))


def up_v(shape: MlaShape, o_lat, q_n_frames: int, w_uv, out, stream=None) -> None:
    _check("mla_up_v", lib().mla_up_v(ctypes.byref(shape), _ptr(o_lat), q_n_frames, _ptr(w_uv), _ptr(out),
                                      _stream(stream)))


def chunk_attend_workspace_bytes(shape: MlaShape, q_n_frames: int) -> int:
    return lib().mla_chunk_attend_workspace_bytes(ctypes.byref(shape), q_n_frames)


def chunk_attend(shape: MlaShape, q_nope, q_r, q_frame_first: int, q_n_frames: int, w_uk, w_uv, cache,
                 slot_frame, tables, rope_t_first: int, rope_n_t: int, out, workspace, stream=None) -> None:
    nbytes = workspace.numel() * workspace.element_size()
    _check("mla_chunk_attend", lib().mla_chunk_attend(ctypes.byref(shape), _ptr(q_nope), _ptr(q_r), q_frame_first,
                                                      q_n_frames, _ptr(w_uk), _ptr(w_uv), _ptr(cache),
                                                      _ptr(slot_frame, "int32"), _ptr(tables, "float32"), rope_t_first, rope_n_t,
                                                      _ptr(out), _ptr(workspace), nbytes, _stream(stream)))


FORM_LATENT, FORM_HEADS = 0, 1


def chunk_attend_form(shape: MlaShape, q_n_frames: int) -> int:
    """Which form mla_chunk_attend takes: FORM_LATENT or FORM_HEADS (-1: invalid)."""
    return lib().mla_chunk_attend_form(ctypes.byref(shape), q_n_frames)


def chunk_attend_latent(shape: MlaShape, q_nope, q_r, q_frame_first: int, q_n_frames: int, w_uk, w_uv, cache,
                        slot_frame, tables, rope_t_first: int, rope_n_t: int, out, workspace, stream=None) -> None:
    nbytes = workspace.numel() * workspace.element_size()
    _check("mla_chunk_attend_latent",
           lib().mla_chunk_attend_latent(ctypes.byref(shape), _ptr(q_nope), _ptr(q_r), q_frame_first, q_n_frames,
                                         _ptr(w_uk), _ptr(w_uv), _ptr(cache), _ptr(slot_frame, "int32"),
                                         _ptr(tables, "float32"), rope_t_first, rope_n_t, _ptr(out), _ptr(workspace),
                                         nbytes, _stream(stream)))


def chunk_attend_heads_workspace_bytes(shape: MlaShape, q_n_frames: int) -> int:
    return lib().mla_chunk_attend_heads_workspace_bytes(ctypes.byref(shape), q_n_frames)


def chunk_attend_heads(shape: MlaShape, q_nope, q_r, q_frame_first: int, q_n_frames: int, w_uk, w_uv, cache,
                       slot_frame, tables, rope_t_first: int, rope_n_t: int, out, workspace, stream=None) -> None:
    nbytes = workspace.numel() * workspace.element_size()
    _check("mla_chunk_attend_heads",
           lib().mla_chunk_attend_heads(ctypes.byref(shape), _ptr(q_nope), _ptr(q_r), q_frame_first, q_n_frames,
                                        _ptr(w_uk), _ptr(w_uv), _ptr(cache), _ptr(slot_frame, "int32"), _ptr(tables, "float32"),
                                        rope_t_first, rope_n_t, _ptr(out), _ptr(workspace), nbytes,
                                        _stream(stream)))


def _chunk_attend_call(name, shape, q_nope, q_r, q_frame_first, q_n_frames, w_uk, w_uv, cache, slot_frame, tables,
                       rope_t_first, rope_n_t, out, workspace, stream):
    nbytes = workspace.numel() * workspace.element_size()
    _check(name, getattr(lib(), name)(ctypes.byref(shape), _ptr(q_nope), _ptr(q_r), q_frame_first, q_n_frames,
                                      _ptr(w_uk), _ptr(w_uv), _ptr(cache), _ptr(slot_frame, "int32"),
                                      _ptr(tables, "float32"), rope_t_first, rope_n_t, _ptr(out), _ptr(workspace),
                                      nbytes, _stream(stream)))


def chunk_attend_frame_causal(shape: MlaShape, q_nope, q_r, q_frame_first: int, q_n_frames: int, w_uk, w_uv, cache,
                              slot_frame, tables, rope_t_first: int, rope_n_t: int, out, workspace,
                              stream=None) -> None:
    _chunk_attend_call("mla_chunk_attend_frame_causal", shape, q_nope, q_r, q_frame_first, q_n_frames, w_uk, w_uv,
                       cache, slot_frame, tables, rope_t_first, rope_n_t, out, workspace, stream)


def chunk_attend_latent_frame_causal(shape: MlaShape, q_nope, q_r, q_frame_first: int, q_n_frames: int, w_uk, w_uv,
                                     cache, slot_frame, tables, rope_t_first: int, rope_n_t: int, out, workspace,
                                     stream=None) -> None:
    _chunk_attend_call("mla_chunk_attend_latent_frame_causal", shape, q_nope, q_r, q_frame_first, q_n_frames, w_uk,
                       w_uv, cache, slot_frame, tables, rope_t_first, rope_n_t, out, workspace, stream)


def chunk_attend_heads_frame_causal(shape: MlaShape, q_nope, q_r, q_frame_first: int, q_n_frames: int, w_uk, w_uv,
                                    cache, slot_frame, tables, rope_t_first: int, rope_n_t: int, out, workspace,
                                    stream=None) -> None:
    _chunk_attend_call("mla_chunk_attend_heads_frame_causal", shape, q_nope, q_r, q_frame_first, q_n_frames, w_uk,
                       w_uv, cache, slot_frame, tables, rope_t_first, rope_n_t, out, workspace, stream)


def query_project(shape: MlaShape, d_cq: int, x, n_frames: int, w_dq, w_uq, w_qr, c_q, q_nope, q_r,
                  stream=None) -> None:
    _check("mla_query_project",
           lib().mla_query_project(ctypes.byref(shape), d_cq, _ptr(x), n_frames, _ptr(w_dq), _ptr(w_uq), _ptr(w_qr),
                                   _ptr(c_q), _ptr(q_nope), _ptr(q_r), _stream(stream)))


def output_project(shape: MlaShape, o, n_frames: int, w_o, u, stream=None) -> None:
    _check("mla_output_project",
           lib().mla_output_project(ctypes.byref(shape), _ptr(o), n_frames, _ptr(w_o), _ptr(u), _stream(stream)))


def layer_weights_struct(w: dict) -> MlaLayerWeights:
    """A layer's weight tensors (dict of device tensors) as the ABI's struct;
    w_qabs is optional (absent: the unfused query path)."""
    names = ("w_dkv", "w_kr", "w_dq", "w_uq", "w_qr", "w_uk", "w_uv", "w_o", "w_qabs")
    return MlaLayerWeights(*[_ptr(w.get(k)) for k in names])


def layer_step_workspace_bytes(shape: MlaShape, d_cq: int, n_frames: int) -> int:
    return lib().mla_layer_step_workspace_bytes(ctypes.byref(shape), d_cq, n_frames)


def layer_step(shape: MlaShape, d_cq: int, weights: MlaLayerWeights, x, frame_first: int, n_frames: int, cache,
               slot_frame, tables, rope_t_first: int, rope_n_t: int, frame_causal: bool, u, workspace,
               stream=None) -> None:
    nbytes = workspace.numel() * workspace.element_size()
    _check("mla_layer_step",
           lib().mla_layer_step(ctypes.byref(shape), d_cq, ctypes.byref(weights), _ptr(x), frame_first, n_frames,
                                _ptr(cache), _ptr(slot_frame, "int32"), _ptr(tables, "float32"), rope_t_first, rope_n_t,
                                1 if frame_causal else 0, _ptr(u), _ptr(workspace), nbytes, _stream(stream)))


def query_absorb_weights(shape: MlaShape, d_cq: int, w_uq, w_qr, w_uk, w_qabs, stream=None) -> None:
    _check("mla_query_absorb_weights",
           lib().mla_query_absorb_weights(ctypes.byref(shape), d_cq, _ptr(w_uq), _ptr(w_qr), _ptr(w_uk), _ptr(w_qabs),
                                          _stream(stream)))


def query_project_absorbed(shape: MlaShape, d_cq: int, x, q_frame_first: int, n_frames: int, w_dq, w_qabs, tables,
                           rope_t_first: int, rope_n_t: int, c_q, q_abs, stream=None) -> None:
    _check("mla_query_project_absorbed",
           lib().mla_query_project_absorbed(ctypes.byref(shape), d_cq, _ptr(x), q_frame_first, n_frames, _ptr(w_dq),
                                            _ptr(w_qabs), _ptr(tables, "float32"), rope_t_first, rope_n_t, _ptr(c_q),
                                            _ptr(q_abs), _stream(stream)))
