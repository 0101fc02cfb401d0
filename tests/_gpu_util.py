"""Helpers for the GPU parity tests: move generator output to the device and
back, and build both sides' frequency tables independently (the library's
host call for the GPU path, the oracle for the expected values)."""

import math
import sys

import numpy as np
import torch

from oracle import freqs as ofreqs
from yarn_scaled_rope_amd import ops
from yarn_scaled_rope_amd import workloads as wl

BF16_TOL = 2e-2   # max-abs bound for bf16 inputs with fp32 accumulation
F32_TOL = 1e-5    # max-abs bound for the fp32 path


def say(msg: str):
    """Name the case before each GPU step, flushed, so that a run that dies
    on the device still says what it was doing."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def lib_theta(d, base, s, L, method="yarn"):
    """GPU-side table and scale from the library's own host call."""
    _, f64, t = ops.yarn_rope_freqs(d, base, s, L, 1.0, 32.0, method)
    return torch.from_numpy(f64).cuda(), t / math.sqrt(d)


def oracle_theta(d, base, s, L, method="yarn"):
    th = ofreqs.theta_for(method, d, base, s, L)
    return th, ofreqs.softmax_scale(d, ofreqs.temperature_for(method, s))


def max_abs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


class LazyF64:
    """Index-on-demand fp64 view of stored inputs (float32 arrays or bf16
    bits): the full workloads are too large to widen to fp64 at once, and the
    oracle only slices them."""

    def __init__(self, arr, dtype):
        self.arr, self.dtype = arr, dtype
        self.shape = arr.shape

    def __getitem__(self, idx):
        return wl.as_f64(self.arr[idx], self.dtype)

    def __array__(self, dtype=None, copy=None):
        raise TypeError("materialising the whole input is not intended")
