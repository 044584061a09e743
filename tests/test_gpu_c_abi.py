"""The library driven from C alone (tests/c_abi/chunk_step.c: hipMalloc'd
buffers, include/mla.h, no Python in the path) gives the same bits as the
same calls made through the Python binding on the same inputs."""
import os
import subprocess

import numpy as np
import pytest
import torch

import latent_kv_attention_amd as mla
from harness import get_config

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


class _Lcg:
    """The C program's generator: bf16 bit patterns, +-[2^-7, 2)."""

    def __init__(self):
        self.state = 0x2545F4914F6CDD1D

    def bf16(self, n):
        out = np.empty(n, dtype=np.uint16)
        m = (1 << 64) - 1
        st = self.state
        for i in range(n):
            st = (st * 6364136223846793005 + 1442695040888963407) & m
            r = st >> 33
            out[i] = ((r & 1) << 15) | ((120 + ((r >> 1) & 7)) << 7) | ((r >> 4) & 0x7F)
        self.state = st
        return out


def _dev(bits, shape):
    return torch.from_numpy(bits.view(np.int16).reshape(shape).copy()).view(torch.bfloat16).cuda()


def test_chunk_step_from_c_matches_binding(built_lib, tmp_path):
    exe = tmp_path / "chunk_step"
    lib_dir = os.path.dirname(built_lib)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    subprocess.run(["gcc", "-std=c11", "-O1", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(rocm, "include"),
                    os.path.join(ROOT, "tests", "c_abi", "chunk_step.c"), "-o", str(exe), "-L" + lib_dir,
                    "-l:libmla355.so", "-L" + os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + lib_dir,
                    "-Wl,-rpath," + os.path.join(rocm, "lib")], check=True, capture_output=True)
    out_file = tmp_path / "out.bin"
    r = subprocess.run([str(exe), str(out_file)], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    got_c = np.fromfile(out_file, dtype=np.uint16)

    cfg = get_config("wan_small")
    assert (cfg.window_frames, cfg.grid_y, cfg.grid_x) == (5, 6, 11)
    T, H, hid = cfg.tokens_per_frame, cfg.n_heads, cfg.hidden
    g = _Lcg()
    w_dkv = _dev(g.bf16(cfg.d_c * hid), (cfg.d_c, hid))
    w_kr = _dev(g.bf16(cfg.d_rope * hid), (cfg.d_rope, hid))
    w_uk = _dev(g.bf16(H * cfg.d_head * cfg.d_c), (H, cfg.d_head, cfg.d_c))
    w_uv = _dev(g.bf16(H * cfg.d_head * cfg.d_c), (H, cfg.d_head, cfg.d_c))
    x_pre = _dev(g.bf16(3 * T * hid), (1, 3 * T, hid))
    x_chunk = _dev(g.bf16(2 * T * hid), (1, 2 * T, hid))
    qn = _dev(g.bf16(2 * T * H * cfg.d_head), (1, 2 * T, H, cfg.d_head))
    qr = _dev(g.bf16(2 * T * H * cfg.d_rope), (1, 2 * T, H, cfg.d_rope))
    shape = mla.make_shape(cfg, batch=1)
    tables = torch.empty(mla.rope3d_table_floats(shape, 16), dtype=torch.float32, device="cuda")
    mla.rope3d_tables(shape, 0, 16, tables)
    cache = torch.zeros(1, 5, T, cfg.d_c + cfg.d_rope, dtype=torch.bfloat16, device="cuda")
    slot = torch.full((1, 5), -1, dtype=torch.int32, device="cuda")
    mla.cache_write(shape, x_pre, w_dkv, w_kr, 0, 3, cache, slot)
    mla.cache_write(shape, x_chunk, w_dkv, w_kr, 3, 2, cache, slot)
    out = torch.empty(1, 2 * T, H, cfg.d_head, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mla.chunk_attend_workspace_bytes(shape, 2), dtype=torch.uint8, device="cuda")
    mla.chunk_attend(shape, qn, qr, 3, 2, w_uk, w_uv, cache, slot, tables, 0, 16, out, ws)
    torch.cuda.synchronize()
    got_py = out.view(torch.int16).cpu().numpy().reshape(-1).view(np.uint16)
    assert got_c.size == got_py.size
    assert np.isfinite(out.float().cpu().numpy()).all()
    assert np.array_equal(got_c, got_py)
