"""Pure-Python brute force for tiny cases: an independent second statement of
rotation and causal attention, written with explicit loops, explicit 2x2
matrices and the textbook (unshifted) softmax.  Test infrastructure only; it
exists to pin the vectorised oracle.  Keep n and d small: it is O(n^2 d) in
Python.

"Arch 03 -- Long Context": RoPE slide (R_{m,i} as a 2x2 matrix on pair
(2i, 2i+1)), attention slide (softmax(Q K^T / sqrt(d)) V), ALiBi slide (causal
rule i - j >= 0).
"""

import math


def rotation_matrix(angle):
    return [[math.cos(angle), -math.sin(angle)],
            [math.sin(angle), math.cos(angle)]]


def rotate_vector(x, m, theta):
    """x: list of d floats at position m; theta: list of d/2 frequencies."""
    out = [0.0] * len(x)
    for i, th in enumerate(theta):
        r = rotation_matrix(m * th)
        a, b = x[2 * i], x[2 * i + 1]
        out[2 * i] = r[0][0] * a + r[0][1] * b
        out[2 * i + 1] = r[1][0] * a + r[1][1] * b
    return out


def causal_attention(q, k, v, seq_lens, theta, scale):
    """q: nested lists [T][Hq][D]; k, v: [T][Hkv][D]; seq_lens: lengths of the
    packed sequences.  Returns (out [T][Hq][D], lse [Hq][T])."""
    T = len(q)
    hq = len(q[0])
    hkv = len(k[0])
    d = len(q[0][0])
    g = hq // hkv
    out = [[[0.0] * d for _ in range(hq)] for _ in range(T)]
    lse = [[0.0] * T for _ in range(hq)]
    start = 0
    for n in seq_lens:
        for h in range(hq):
            hk = h // g
            for m in range(n):
                qm = rotate_vector(q[start + m][h], m, theta) if theta else q[start + m][h]
                weights = []
                for j in range(m + 1):
                    kj = rotate_vector(k[start + j][hk], j, theta) if theta else k[start + j][hk]
                    dot = 0.0
                    for c in range(d):
                        dot += qm[c] * kj[c]
                    weights.append(math.exp(scale * dot))
                total = sum(weights)
                lse[h][start + m] = math.log(total)
                for c in range(d):
                    acc = 0.0
                    for j in range(m + 1):
                        acc += weights[j] * v[start + j][hk][c]
                    out[start + m][h][c] = acc / total
        start += n
    return out, lse
