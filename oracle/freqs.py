"""Rotary frequencies (plain RoPE, PI, NTK-aware, YaRN) and the YaRN logit
temperature, in fp64.  Test infrastructure only (see the package docstring).

Reading adopted where the pages disagree or are silent (each is listed again in
the design notes):
  * Ramp variable: the wavelength ratio r_i = L / lambda_i, lambda_i = 2*pi/theta_i,
    L = original (training) context length; alpha = 1, beta = 32 as in the YaRN
    steps table of the "Arch 03 -- Long Context" deck.
  * Orientation: pairs that turn many times over the original context
    (r >= beta, high frequency) keep theta unchanged; pairs that turn at most
    alpha times (r <= alpha, low frequency) are interpolated like PI
    (theta / s); in between, a ramp linear in r.  This follows the YaRN slide's
    wavelength groups (short wavelength: no interpolation; long wavelength:
    PI) and the NTK-aware slide's remark that PI hurts the fast-turning pairs
    most.  The code listing on "LLM context window mechanics" uses an
    index-space ramp with the opposite wording; it is not followed.
  * Temperature: t = 0.1 * ln(s) + 1 multiplies the logits once.
"""

import math

import numpy as np

METHODS = ("plain", "pi", "ntk", "yarn")


def rope_theta(head_dim: int, base: float) -> np.ndarray:
    """Base RoPE frequencies theta_i = base^(-2i/d), i = 0 .. d/2-1.

    "Arch 03 -- Long Context", RoPE slide (one frequency per feature pair
    (2i, 2i+1)); "LLM context window mechanics", "The position wall".
    """
    d = int(head_dim)
    return np.array([float(base) ** (-(2.0 * i) / d) for i in range(d // 2)],
                    dtype=np.float64)


def wavelength(theta: np.ndarray) -> np.ndarray:
    """lambda_i = 2*pi / theta_i ("Arch 03 -- Long Context", YaRN slide)."""
    return (2.0 * math.pi) / np.asarray(theta, dtype=np.float64)


def yarn_gamma(r: float, alpha: float, beta: float) -> float:
    """Ramp weight toward the unscaled frequency as a function of the number of
    turns r a pair makes over the original context: 0 at or below alpha (PI),
    1 at or above beta (unscaled), linear in between ("Arch 03 -- Long
    Context", YaRN slide: three wavelength groups, linear ramp between)."""
    if r <= alpha:
        return 0.0
    if r >= beta:
        return 1.0
    return (r - alpha) / (beta - alpha)


def yarn_theta(head_dim: int, base: float, factor: float,
               original_max_position: float, alpha: float = 1.0,
               beta: float = 32.0) -> np.ndarray:
    """YaRN-scaled frequencies theta'_i.

    For each pair: r_i = L / lambda_i; gamma_i = ramp(r_i); theta'_i is theta_i/s
    where gamma_i = 0, theta_i where gamma_i = 1, and
    theta_i/s + gamma_i * (theta_i - theta_i/s) in the ramp ("Arch 03 -- Long
    Context", YaRN slide and steps table; Position Interpolation slide for the
    theta/s end).  The pure regions are assigned directly so that they are
    exact, and s = 1 returns theta bit for bit.
    """
    theta = rope_theta(head_dim, base)
    lam = wavelength(theta)
    out = np.empty_like(theta)
    for i in range(theta.size):
        r = float(original_max_position) / lam[i]
        g = yarn_gamma(r, alpha, beta)
        interp = theta[i] / factor
        if g == 0.0:
            out[i] = interp
        elif g == 1.0:
            out[i] = theta[i]
        else:
            out[i] = interp + g * (theta[i] - interp)
    return out


def pi_theta(head_dim: int, base: float, factor: float) -> np.ndarray:
    """Position Interpolation: every theta_i divided by s = L_target / L_train
    ("Arch 03 -- Long Context", Position Interpolation slide)."""
    return rope_theta(head_dim, base) / float(factor)


def ntk_base(head_dim: int, base: float, factor: float) -> float:
    """NTK-aware scaling raises the base to base * s^(d/(d-2))
    ("Arch 03 -- Long Context", NTK-aware slide)."""
    d = float(head_dim)
    return float(base) * float(factor) ** (d / (d - 2.0))


def ntk_theta(head_dim: int, base: float, factor: float) -> np.ndarray:
    """Frequencies of plain RoPE over the NTK-aware base."""
    return rope_theta(head_dim, ntk_base(head_dim, base, factor))


def dynamic_ntk_factor(seq_len: int, original_max_position: float) -> float:
    """Dynamic NTK: the factor follows the current sequence, s = length /
    training length, and no scaling applies below the training length
    (s = max(1, length / L)) ("Arch 03 -- Long Context", NTK-aware slide)."""
    return max(1.0, float(seq_len) / float(original_max_position))


def dynamic_ntk_theta(head_dim: int, base: float, seq_len: int,
                      original_max_position: float) -> np.ndarray:
    """NTK-aware frequencies for the factor Dynamic NTK picks at seq_len."""
    return ntk_theta(head_dim, base, dynamic_ntk_factor(seq_len, original_max_position))


def attention_temperature(factor: float) -> float:
    """YaRN logit temperature t = 0.1 * ln(s) + 1 (natural log)
    ("Arch 03 -- Long Context", YaRN slide; "LLM context window mechanics",
    "The position wall")."""
    return 0.1 * math.log(float(factor)) + 1.0


def theta_for(method: str, head_dim: int, base: float, factor: float,
              original_max_position: float, alpha: float = 1.0,
              beta: float = 32.0) -> np.ndarray:
    """Dispatch by method name: 'plain', 'pi', 'ntk' or 'yarn'."""
    if method == "plain":
        return rope_theta(head_dim, base)
    if method == "pi":
        return pi_theta(head_dim, base, factor)
    if method == "ntk":
        return ntk_theta(head_dim, base, factor)
    if method == "yarn":
        return yarn_theta(head_dim, base, factor, original_max_position,
                          alpha, beta)
    raise ValueError(f"unknown method {method!r}")


def temperature_for(method: str, factor: float) -> float:
    """Only YaRN rescales the logits; the other methods leave them at 1."""
    return attention_temperature(factor) if method == "yarn" else 1.0


def softmax_scale(head_dim: int, temperature: float) -> float:
    """Scale applied to q~.k~: the 1/sqrt(d) of scaled dot-product attention
    ("Arch 03 -- Long Context", attention slide) times the temperature t."""
    return float(temperature) / math.sqrt(float(head_dim))


def to_fp32(theta: np.ndarray) -> np.ndarray:
    """Round an fp64 table to fp32, round-to-nearest-even (numpy's cast)."""
    return np.asarray(theta, dtype=np.float64).astype(np.float32)


def fp32_midpoint_distance(theta: np.ndarray) -> np.ndarray:
    """Relative distance of each fp64 value from the nearest fp32 rounding
    midpoint.  A value far from every midpoint rounds to the same fp32 number
    however the last fp64 bits come out, so two libms that differ by a few
    fp64 ulps still produce the same fp32 table."""
    x = np.asarray(theta, dtype=np.float64)
    f = x.astype(np.float32)
    up = np.nextafter(f, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(f, np.float32(-np.inf)).astype(np.float64)
    f64 = f.astype(np.float64)
    mid_up = (f64 + up) / 2.0
    mid_dn = (f64 + dn) / 2.0
    d = np.minimum(np.abs(x - mid_up), np.abs(x - mid_dn))
    return d / np.abs(x)
