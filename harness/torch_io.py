"""Moving rounded float64 arrays to torch tensors and back (no arithmetic of
the method: bf16 values travel as their exact bit patterns)."""
from __future__ import annotations

import numpy as np
import torch

from .gen import from_bf16_bits, to_bf16_bits


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_torch(a, dtype: str, device="cuda") -> torch.Tensor:
    """float64 values already rounded to `dtype` -> tensor of that dtype (exact)."""
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        bits = to_bf16_bits(a).view(np.int16)
        return torch.from_numpy(bits).view(torch.bfloat16).to(device)
    if dtype == "f32":
        return torch.from_numpy(a.astype(np.float32)).to(device)
    raise ValueError(dtype)


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Tensor -> float64 array (exact for bf16 and float32)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return from_bf16_bits(t.view(torch.int16).numpy().view(np.uint16))
    return t.double().numpy()
