"""Shared helpers for the test suite: moving generator output to the GPU and
reading kernel results back as float64 NumPy arrays.  No arithmetic of the
method lives here."""
from __future__ import annotations

import re
import sys

import numpy as np
import torch

from activation_sparse_feedforward_amd import twell as T
from activation_sparse_feedforward_amd import workloads as W

HEADER = __import__("os").path.join(__import__("os").path.dirname(__file__), "..", "include", "twell.h")


def header_symbols():
    """Function names declared in include/twell.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:twell_status|const char\*)\s+(twell_\w+)\s*\(", text, re.M)))


def gpu_available() -> bool:
    return torch.cuda.is_available()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(raw: np.ndarray, dtype: str) -> torch.Tensor:
    """Storage array from the generator -> contiguous GPU tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32)).cuda()


def host64(t: torch.Tensor) -> np.ndarray:
    """GPU tensor -> float64 NumPy (exact for bf16 and fp32)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def desc_for(w: W.Workload, **over) -> T.Desc:
    kw = dict(T=w.T, d_model=w.d_model, d_ff=w.d_ff, tile_n=w.tile_n, slots=w.slots, dtype=w.dtype)
    kw.update(over)
    return T.Desc(**kw)


def poison_(t: torch.Tensor):
    """Fill an output buffer with a non-zero byte pattern so unwritten entries show up."""
    t.view(torch.uint8).fill_(0xA5)
    return t
