"""GPU-side helpers for the parity tests: upload seeded inputs, cache the
large configurations within one pytest process, sample rows."""
from __future__ import annotations

import functools
import os
import sys

import numpy as np

from synth import make_config_inputs


def torch_dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype: str):
    """Upload a host array: bf16 bit patterns (uint16) or float32."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch_dev())


def upload(inp):
    names = ("x", "Wg", "W1", "W3", "W2")
    return {k: to_dev(getattr(inp, k), inp.dtype) for k in names if getattr(inp, k) is not None}


@functools.lru_cache(maxsize=2)
def config_inputs(name: str, router_only: bool = False):
    return make_config_inputs(name, router_only=router_only)


def sample_rows(T: int, count: int, seed: int = 99) -> np.ndarray:
    """A seeded row sample that always includes the first and last token."""
    if T <= count:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    rows = rng.choice(T, size=count - 2, replace=False)
    return np.unique(np.concatenate([[0, T - 1], rows]))


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def cpu_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1
