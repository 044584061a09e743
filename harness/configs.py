"""Named workload shapes for the latent-KV chunk-attention step.

Shapes come from the VideoMLA pages: Wan2.1-1.3B with 12 heads of 128, a
192-d content latent and a 32-d positional key (224 cached scalars per token
instead of 3072; ai-papers.net blog, architecture paragraph under Fig. 1), and
a fixed-size sliding-window cache (chatpaper.ai, English abstract). The frame
grid (30x52), window (21 frames), chunk (3 frames), RoPE axis split and the
tiny parity shape are workload choices stated alongside each config.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class MLAConfig:
    name: str
    hidden: int
    n_heads: int
    d_head: int
    d_c: int
    d_rope: int
    rope_split: tuple  # (d_t, d_y, d_x): per-axis rotary widths, in this order
    grid_y: int
    grid_x: int
    window_frames: int
    chunk_frames: int
    dtype: str  # "f32" or "bf16"
    batch: int = 1
    layers: int = 1
    rope_base: float = 10000.0
    # frames held in the window when the chunk attends (chunk included)
    window_fill: int = 0
    # query latent width; 0 selects 3 * d_c (the pages leave it open)
    d_cq: int = 0
    note: str = field(default="", compare=False)

    @property
    def q_latent(self) -> int:
        return self.d_cq or 3 * self.d_c

    @property
    def tokens_per_frame(self) -> int:
        return self.grid_y * self.grid_x

    @property
    def n_q(self) -> int:
        return self.chunk_frames * self.tokens_per_frame

    @property
    def n_k(self) -> int:
        fill = self.window_fill or self.window_frames
        return fill * self.tokens_per_frame

    @property
    def cached_scalars(self) -> int:
        return self.d_c + self.d_rope

    @property
    def dense_scalars(self) -> int:
        return 2 * self.n_heads * self.d_head

    def with_(self, **kw) -> "MLAConfig":
        return replace(self, **kw)


_WAN = dict(hidden=1536, n_heads=12, d_head=128, d_c=192, d_rope=32,
            rope_split=(8, 12, 12), grid_y=30, grid_x=52, window_frames=21,
            chunk_frames=3, dtype="bf16")

CONFIGS = {
    # tiny fp32 single layer: chunk = frame 2 attending to frames {0, 1, 2}
    "tiny": MLAConfig(name="tiny", hidden=16, n_heads=2, d_head=8, d_c=16, d_rope=8,
                      rope_split=(2, 2, 4), grid_y=4, grid_x=4, window_frames=3,
                      chunk_frames=1, dtype="f32",
                      note="n_h=2 d_h=8 d_c=16 d_rope=8 (2/2/4), grid 4x4, 16 q x 48 k, fp32"),
    # Wan2.1-1.3B-shaped single layer: 4680 queries x 32760 window keys
    "wan": MLAConfig(name="wan", **_WAN,
                     note="hidden 1536, 12x128 heads, d_c 192, d_rope 32, grid 30x52, "
                          "3-frame chunk over a 21-frame window (4680 q x 32760 k), bf16"),
    # 30 layers x 7 chunks while the window fills from 3 to 21 frames
    "wan_fill30": MLAConfig(name="wan_fill30", layers=30, **_WAN,
                            note="30-layer chunk step, window filling 3 -> 21 frames over 7 chunks"),
    # batch of 8 independent streams, each with a full 21-frame window
    "wan_batch8": MLAConfig(name="wan_batch8", batch=8, layers=30, **_WAN,
                            note="8 independent streams, full 21-frame window each"),
    # 80 chunks = 240 latent frames; the ring evicts from the 8th chunk on
    "wan_rollout": MLAConfig(name="wan_rollout", layers=30, **_WAN,
                             note="80 successive 3-frame chunks, ring evicting, t advancing to 239"),
    # Wan head shapes on a small grid: several tiles with ragged tails, fast on CPU
    "wan_small": MLAConfig(name="wan_small", hidden=1536, n_heads=12, d_head=128, d_c=192,
                           d_rope=32, rope_split=(8, 12, 12), grid_y=6, grid_x=11,
                           window_frames=5, chunk_frames=2, dtype="bf16",
                           note="Wan head shapes, 6x11 grid, 2-frame chunk over 5 frames"),
    # tiny head shapes in bf16 (same kernels as tiny, bf16 instantiation)
    "tiny_bf16": MLAConfig(name="tiny_bf16", hidden=16, n_heads=2, d_head=8, d_c=16, d_rope=8,
                           rope_split=(2, 2, 4), grid_y=4, grid_x=4, window_frames=3,
                           chunk_frames=1, dtype="bf16"),
    # Wan head shapes in fp32 (the fp32 instantiation at the real latent widths)
    "wan_small_f32": MLAConfig(name="wan_small_f32", hidden=1536, n_heads=12, d_head=128,
                               d_c=192, d_rope=32, rope_split=(8, 12, 12), grid_y=5, grid_x=7,
                               window_frames=4, chunk_frames=1, dtype="f32"),
}

# Other latent widths on the small Wan-headed grid: a smaller latent, the same
# 224 cached scalars with more positional channels, and a larger latent (the
# pages' ablations vary the latent size and the content/positional split).
for _dc, _dr, _split in ((128, 32, (8, 12, 12)), (160, 64, (16, 24, 24)), (192, 64, (16, 24, 24))):
    for _dt in ("bf16", "f32"):
        _n = f"wan_small_c{_dc}r{_dr}" + ("_f32" if _dt == "f32" else "")
        CONFIGS[_n] = CONFIGS["wan_small"].with_(name=_n, d_c=_dc, d_rope=_dr, rope_split=_split, dtype=_dt)


def get_config(name: str) -> MLAConfig:
    return CONFIGS[name]
