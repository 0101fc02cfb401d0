"""Pins of the oracle's E4M3 decoding (CPU only): every code against torch's
float8_e4m3fn (an independent library implementation of the OCP format),
the values the format's definition fixes by hand (1, 448, the smallest normal
and subnormal, signed zero, NaN codes), monotonicity over the positive codes,
and the per-head scale of the cache."""

import math

import numpy as np
import torch

from oracle import fp8


def test_every_code_matches_library_decoding():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.e4m3_to_f64(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(lib)
    assert np.all(both_nan | (ours == lib))
    assert int(np.isnan(ours).sum()) == 2


def test_hand_values():
    v = fp8.e4m3_to_f64([0x38, 0x7E, 0x08, 0x01, 0x00, 0x80, 0xB8, 0x07, 0x3C, 0x7F, 0xFF])
    assert v[0] == 1.0                      # exponent 7, mantissa 0
    assert v[1] == 448.0                    # largest finite: 2^8 * 1.75
    assert v[2] == 2.0 ** -6                # smallest normal
    assert v[3] == 2.0 ** -9                # smallest subnormal: 1/8 * 2^-6
    assert v[4] == 0.0 and math.copysign(1.0, v[5]) == -1.0 and v[5] == 0.0
    assert v[6] == -1.0
    assert v[7] == 7.0 / 8.0 * 2.0 ** -6    # largest subnormal
    assert v[8] == 1.5
    assert np.isnan(v[9]) and np.isnan(v[10])


def test_positive_codes_increase():
    v = fp8.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)


def test_dequantize_applies_the_head_scale():
    rng = np.random.Generator(np.random.PCG64(5))
    codes = rng.integers(0, 0x7E, size=(2, 3, 4, 8), dtype=np.uint8)
    scale = np.array([0.5, 1.0, 2.0 ** -6, 3.0], dtype=np.float32)
    out = fp8.dequantize_cache(codes, scale)
    for h in range(4):
        assert np.array_equal(out[:, :, h], fp8.e4m3_to_f64(codes[:, :, h]) * float(scale[h]))
