"""GPU-side helpers of the parity tests: upload / download of bfloat16 bit patterns."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda:0"


def up(a, dev=DEV) -> torch.Tensor:
    """uint16 bfloat16 bits (numpy) -> int16 tensor on the GPU (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(dev)


def down(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


def lib():
    """The HIP binding; fails loudly when the library is not built."""
    import skinny_gemm_attention_amd as sga

    return sga
