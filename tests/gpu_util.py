"""Helpers shared by the GPU tests: host<->device marshalling of seeded cases."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda:0"


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f32_dev(a) -> torch.Tensor:
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def say(msg: str):
    """Name the case before each GPU step so a fault can be traced to it."""
    print(msg, flush=True)
