"""Rotary position embedding applied to query/key feature pairs, in fp64.
Test infrastructure only (see the package docstring).

"Arch 03 -- Long Context", RoPE slide; "Long-context models", "Position enters
attention": at position m the pair (x_{2i}, x_{2i+1}) is multiplied by
R = [[cos(m*theta_i), -sin(m*theta_i)], [sin(m*theta_i), cos(m*theta_i)]], the
same matrix for queries and keys.  Pairs are adjacent features (2i, 2i+1) and
every feature of the head is rotated.
"""

import numpy as np


def rotation_angles(positions, theta) -> np.ndarray:
    """phi[t, i] = m_t * theta_i in fp64."""
    m = np.asarray(positions, dtype=np.float64).reshape(-1)
    th = np.asarray(theta, dtype=np.float64).reshape(-1)
    return m[:, None] * th[None, :]


def rotate(x, positions, theta) -> np.ndarray:
    """Rotate x of shape [T, H, D] (or [T, D]) whose row t sits at position
    positions[t].  Returns a new fp64 array."""
    x = np.asarray(x, dtype=np.float64)
    squeeze = x.ndim == 2
    if squeeze:
        x = x[:, None, :]
    phi = rotation_angles(positions, theta)          # [T, D/2]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    even = x[..., 0::2]
    odd = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = even * c - odd * s
    out[..., 1::2] = even * s + odd * c
    return out[:, 0, :] if squeeze else out
