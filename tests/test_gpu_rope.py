"""rope_apply on the GPU against the oracle rotation."""

import numpy as np
import pytest
import torch

from oracle import rope as orope
from tests._gpu_util import BF16_TOL, F32_TOL, lib_theta, max_abs, oracle_theta, say, to_dev, to_f64
from yarn_scaled_rope_amd import ops
from yarn_scaled_rope_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,T,H,D,base,s,L", [
    ("f32", 1000, 3, 64, 10000.0, 4.0, 64),
    ("f32", 333, 2, 128, 500000.0, 8.0, 16384),
    ("bf16", 777, 8, 128, 500000.0, 8.0, 16384),
    ("bf16", 65, 5, 64, 10000.0, 4.0, 4096),
])
def test_rope_apply_matches_oracle(dtype, T, H, D, base, s, L):
    rng = np.random.Generator(np.random.PCG64(100 + T))
    x32 = rng.standard_normal((T, H, D), dtype=np.float32)
    x = wl.round_to_bf16_bits(x32) if dtype == "bf16" else x32
    pos = rng.integers(0, 131073, size=T).astype(np.int32)
    pos[:3] = [0, 1, 131072]
    th_dev, _ = lib_theta(D, base, s, L)
    th_ref, _ = oracle_theta(D, base, s, L)
    say(f"rope_apply {dtype} T={T} H={H} D={D}")
    xd = to_dev(x, dtype)
    ops.rope_apply(xd, torch.from_numpy(pos).cuda(), th_dev)
    torch.cuda.synchronize()
    got = to_f64(xd)
    ref = orope.rotate(wl.as_f64(x, dtype), pos, th_ref)
    err = max_abs(got, ref)
    if dtype == "f32":
        assert err <= F32_TOL, err
    else:
        assert err <= BF16_TOL, err
        # the kernel rounds its fp32 rotation to bf16 once: every element is
        # within one bf16 ulp of the exact value
        mag = np.maximum(np.abs(ref), 1e-30)
        ulp = 2.0 ** (np.floor(np.log2(mag)) - 7)
        assert np.all(np.abs(got - ref) <= ulp + 1e-6)


def test_rope_apply_position_zero_is_identity():
    D = 128
    th_dev, _ = lib_theta(D, 500000.0, 8.0, 16384)
    x = torch.randn(50, 4, D, device="cuda")
    ref = x.clone()
    say("rope_apply identity at position 0")
    ops.rope_apply(x, torch.zeros(50, dtype=torch.int32, device="cuda"), th_dev)
    torch.cuda.synchronize()
    assert torch.equal(x, ref)


def test_rope_apply_empty():
    th_dev, _ = lib_theta(64, 10000.0, 4.0, 64)
    x = torch.empty(0, 2, 64, device="cuda")
    ops.rope_apply(x, torch.empty(0, dtype=torch.int32, device="cuda"), th_dev)
