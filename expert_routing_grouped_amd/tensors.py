"""numpy <-> torch device plumbing for the seeded inputs (bf16 arrays travel as uint16 bit patterns)."""
from __future__ import annotations

import numpy as np
import torch


def to_device(a: np.ndarray, device) -> torch.Tensor:
    """float32/int32 arrays keep their dtype; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """bf16 tensors come back as uint16 bit patterns, everything else as its numpy dtype."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
