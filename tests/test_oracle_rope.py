"""Pins of the oracle's rotation (CPU only): the complex-number form of RoPE,
orthogonality, identity at position 0, composition, the relative-position
property and a pure-Python 2x2 brute force."""

import numpy as np
import pytest

from oracle import bruteforce, freqs, rope


def _rng(seed=0):
    return np.random.Generator(np.random.PCG64(seed))


def test_matches_complex_multiplication():
    """Pair (x_{2i}, x_{2i+1}) read as x_{2i} + j x_{2i+1} is multiplied by
    exp(j m theta_i); this fixes both the sign of the rotation and the
    adjacent-pair layout."""
    rng = _rng(1)
    T, H, D = 37, 3, 16
    x = rng.standard_normal((T, H, D))
    pos = rng.integers(0, 131072, size=T)
    th = freqs.yarn_theta(D, 500000.0, 8.0, 16384)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    zr = z * np.exp(1j * pos[:, None, None] * th[None, None, :])
    out = rope.rotate(x, pos, th)
    assert np.allclose(out[..., 0::2], zr.real, rtol=0, atol=1e-12)
    assert np.allclose(out[..., 1::2], zr.imag, rtol=0, atol=1e-12)


def test_rotation_of_unit_vectors():
    # theta = (1, 1/2, 1/4, 1/8) (base 16, d 8).  At m = 3 the unit vector
    # e_0 of pair 0 turns counter-clockwise by 3 rad, e_1 of pair 1 by 1.5 rad;
    # pairs that start at zero stay zero.
    th = freqs.rope_theta(8, 16.0)
    x = np.array([[1.0, 0.0, 0.0, 1.0, 0.0, 0.0, 0.0, 0.0]])
    out = rope.rotate(x, [3], th)
    assert out[0, 0] == pytest.approx(np.cos(3.0), abs=1e-15)
    assert out[0, 1] == pytest.approx(np.sin(3.0), abs=1e-15)     # +sin: counter-clockwise
    assert out[0, 2] == pytest.approx(-np.sin(1.5), abs=1e-15)    # (0,1) -> (-sin, cos)
    assert out[0, 3] == pytest.approx(np.cos(1.5), abs=1e-15)
    assert np.all(out[0, 4:] == 0.0)


def test_position_zero_is_identity():
    rng = _rng(2)
    x = rng.standard_normal((5, 2, 64))
    th = freqs.yarn_theta(64, 10000.0, 4.0, 64)
    assert np.array_equal(rope.rotate(x, np.zeros(5, int), th), x)


def test_norm_preserved_per_pair():
    rng = _rng(3)
    x = rng.standard_normal((50, 4, 128))
    pos = rng.integers(0, 131073, size=50)
    out = rope.rotate(x, pos, freqs.yarn_theta(128, 500000.0, 8.0, 16384))
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = out[..., 0::2] ** 2 + out[..., 1::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-12, atol=1e-12)


def test_composition():
    rng = _rng(4)
    x = rng.standard_normal((20, 1, 32))
    th = freqs.yarn_theta(32, 10000.0, 4.0, 512)
    a = rng.integers(0, 5000, size=20)
    b = rng.integers(0, 5000, size=20)
    two = rope.rotate(rope.rotate(x, a, th), b, th)
    one = rope.rotate(x, a + b, th)
    assert np.allclose(two, one, rtol=0, atol=1e-10)


@pytest.mark.parametrize("c", [1, 17, 4096, 100000])
def test_relative_position_property(c):
    rng = _rng(5)
    D = 64
    th = freqs.yarn_theta(D, 10000.0, 4.0, 64)
    q = rng.standard_normal((1, D))
    k = rng.standard_normal((1, D))
    for m, n in [(0, 0), (5, 2), (100, 3), (7, 7)]:
        d0 = rope.rotate(q, [m], th)[0] @ rope.rotate(k, [n], th)[0]
        d1 = rope.rotate(q, [m + c], th)[0] @ rope.rotate(k, [n + c], th)[0]
        assert d0 == pytest.approx(d1, abs=1e-9)


def test_bruteforce_matches_vectorised():
    rng = _rng(6)
    D = 8
    th = freqs.yarn_theta(D, 10000.0, 4.0, 64)
    x = rng.standard_normal((9, D))
    pos = rng.integers(0, 300, size=9)
    out = rope.rotate(x, pos, th)
    for t in range(9):
        bf = bruteforce.rotate_vector(list(x[t]), int(pos[t]), list(th))
        assert np.allclose(out[t], bf, rtol=0, atol=1e-13)
