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


def sees(m, j, window=0, sinks=0):
    """Position j is visible from position m: j <= m, and when a window of W
    tokens is set, j is one of the W most recent positions or one of the
    first S ("Arch 03", sliding window; StreamingLLM sinks)."""
    if j > m:
        return False
    if window <= 0:
        return True
    return j > m - window or j < sinks


def causal_attention(q, k, v, seq_lens, theta, scale, window=0, sinks=0):
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
                    if not sees(m, j, window, sinks):
                        weights.append(0.0)
                        continue
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


def chunk_attention(q, k_cache, v_cache, q_lens, ctx_lens, theta, scale, window=0, sinks=0):
    """Chunked prefill, brute force.  q: [Tq][Hq][D] packed by q_lens (new
    tokens, unrotated); k_cache, v_cache: [B][Lmax][Hkv][D] with keys already
    rotated.  New token i of sequence b sits at position ctx_lens[b] + i and
    attends to cache rows j <= that position (window / sinks applied).
    Returns (out [Tq][Hq][D], lse [Hq][Tq])."""
    Tq = len(q)
    hq = len(q[0])
    hkv = len(k_cache[0][0])
    d = len(q[0][0])
    g = hq // hkv
    out = [[[0.0] * d for _ in range(hq)] for _ in range(Tq)]
    lse = [[0.0] * Tq for _ in range(hq)]
    start = 0
    for b, n in enumerate(q_lens):
        for i in range(n):
            m = ctx_lens[b] + i
            for h in range(hq):
                hk = h // g
                qm = rotate_vector(q[start + i][h], m, theta) if theta else q[start + i][h]
                weights = []
                for j in range(m + 1):
                    if not sees(m, j, window, sinks):
                        weights.append(0.0)
                        continue
                    dot = 0.0
                    for c in range(d):
                        dot += qm[c] * k_cache[b][j][hk][c]
                    weights.append(math.exp(scale * dot))
                total = sum(weights)
                lse[h][start + i] = math.log(total)
                for c in range(d):
                    acc = 0.0
                    for j in range(m + 1):
                        acc += weights[j] * v_cache[b][j][hk][c]
                    out[start + i][h][c] = acc / total
        start += n
    return out, lse
