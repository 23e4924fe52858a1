"""Device helpers for the GPU tests (numpy <-> torch on cuda:0)."""
from __future__ import annotations

import sys

import numpy as np
import pytest


def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def to_dev(a: np.ndarray, kind: str = "f32"):
    """Storage array -> device tensor: 'f32' float32, 'bf16' from uint16 bits, 'i8' int8."""
    torch, dev = torch_dev()
    if kind == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    if kind == "i8":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).to(dev)
    if kind == "f64":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def ws_tensor(nbytes: int):
    torch, dev = torch_dev()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()
