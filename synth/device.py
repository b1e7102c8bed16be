"""Copy a synthetic case onto a torch device (layout only, no arithmetic)."""
from __future__ import annotations

import numpy as np
import torch


def to_tensor(a: np.ndarray, device) -> torch.Tensor:
    """float32 arrays stay float32; uint16 arrays are bfloat16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    if a.dtype == np.int32:
        return torch.from_numpy(a).to(device)
    raise TypeError(a.dtype)


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Inverse of to_tensor (bfloat16 comes back as uint16 bit patterns)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
