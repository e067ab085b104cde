"""Shared test helpers: run workloads through the C ABI on the GPU and through
the oracle on the CPU.  (Test infrastructure; the oracle and the HIP path
never import each other -- only this test layer touches both.)"""
from __future__ import annotations

import numpy as np


def torch_dev(a: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype == "u8":
        t = t.to(torch.uint8)
    return t.cuda()


def empty_dev(shape, dtype: str):
    import torch
    td = {"f32": torch.float32, "bf16": torch.bfloat16, "u8": torch.uint8}[dtype]
    return torch.empty(tuple(shape), dtype=td, device="cuda")


def host64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()
