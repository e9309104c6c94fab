"""Device-memory plumbing around the library (torch is used for memory and
streams only): upload of generator storage arrays, download to storage
arrays, and allocation of the buffers one shard / one expert group needs.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (TP_BF16, TP_F32, TP_ACT_SWIGLU, tp_mlp_shard_bwd_workspace,
               tp_grouped_expert_bwd_workspace)


def torch_dtype(dtype: int):
    return torch.bfloat16 if dtype == TP_BF16 else torch.float32


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """float32 array -> float32 tensor; uint16 (bf16 bits) -> bfloat16 tensor."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Inverse of to_device: bf16 tensors come back as uint16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def empty(shape, dtype: int, device="cuda") -> torch.Tensor:
    return torch.empty(shape, dtype=torch_dtype(dtype), device=device)


class ShardBuffers:
    """Outputs and workspace of one shard's forward and backward."""

    def __init__(self, desc: dict, device="cuda", save=True, backward=True):
        N = desc["S"] * desc["B"]
        H, Ft, dt = desc["H"], desc["F_shard"], desc["dtype"]
        sw = desc["act"] == TP_ACT_SWIGLU
        self.Z = empty((N, 2 * Ft if sw else Ft), dt, device) if save else None
        self.H = empty((N, Ft), dt, device)
        self.Y = empty((N, H), dt, device)
        if backward:
            self.dX = empty((N, H), dt, device)
            self.dA = torch.empty((H, Ft), dtype=torch.float32, device=device)
            self.dA_up = torch.empty((H, Ft), dtype=torch.float32, device=device) if sw else None
            self.dB = torch.empty((Ft, H), dtype=torch.float32, device=device)
            self.ws_bytes = tp_mlp_shard_bwd_workspace(desc)
            self.ws = torch.empty(max(16, self.ws_bytes), dtype=torch.uint8, device=device)


class ExpertBuffers:
    """Outputs and workspace of one grouped expert forward and backward."""

    def __init__(self, desc: dict, offsets, device="cuda", save=True, backward=True):
        R = int(offsets[-1])
        H, F, E = desc["H"], desc["F"], desc["E"]
        self.Z = empty((R, 2 * F), TP_BF16, device) if save else None
        self.H = empty((R, F), TP_BF16, device)
        self.Y = empty((R, H), TP_BF16, device)
        if backward:
            self.dX = empty((R, H), TP_BF16, device)
            self.dWg = torch.empty((E, H, F), dtype=torch.float32, device=device)
            self.dWu = torch.empty((E, H, F), dtype=torch.float32, device=device)
            self.dWd = torch.empty((E, F, H), dtype=torch.float32, device=device)
            self.ws_bytes = tp_grouped_expert_bwd_workspace(desc, offsets)
            self.ws = torch.empty(max(16, self.ws_bytes), dtype=torch.uint8, device=device)
