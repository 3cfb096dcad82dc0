"""Helpers shared by the GPU tests: storage <-> device tensors, plans for both
paths from the same synthetic arrays."""

from __future__ import annotations

import numpy as np

import synthetic as S
from oracle import transform as T


def torch_mod():
    import torch
    return torch


def to_dev(arr: np.ndarray, dtype: str):
    torch = torch_mod()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.cuda()


def from_dev(t) -> np.ndarray:
    torch = torch_mod()
    t = t.detach()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def torch_dtype(dtype: str):
    torch = torch_mod()
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def orc_plan(side: S.SidePlan) -> T.Plan:
    return T.Plan(side.d, side.radix, side.mode, side.blocks,
                  None if side.signs is None else side.signs.astype(np.float64))


def lib_plan(side: S.SidePlan):
    import butterfly_rotation_quantization_amd as brq
    return brq.Plan(side.d, side.radix, side.mode, side.blocks, side.signs)


def method_for(d: int) -> str:
    """Dense formation up to d = 4096, the factor-by-factor definition above
    (the two are pinned equal in the oracle tests)."""
    return "dense" if d <= 4096 else "factored"


def announce(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
