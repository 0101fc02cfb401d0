"""Dense causal softmax attention over YaRN-rotated queries and keys, in fp64.
Test infrastructure only (see the package docstring).

Definitions followed:
  * Scaled dot-product attention softmax(Q K^T / sqrt(d)) V ("Arch 03 -- Long
    Context", attention slide), with the YaRN temperature t multiplying the
    logits once, so z = (t / sqrt(d)) * q~ . k~ (YaRN slide).  The caller
    passes the whole factor as ``scale``.
  * Causal visibility: key n is visible to query m iff m - n >= 0 (the ALiBi
    slide of the same deck states the rule), diagonal included.
  * Queries and keys are rotated at their 0-based position inside their own
    sequence; a packed ragged batch is described by cu_seqlens (sequence b
    owns rows cu_seqlens[b] .. cu_seqlens[b+1]-1) and positions restart at 0
    for every sequence.
  * Grouped-query attention: query head h reads key/value head
    floor(h / (Hq / Hkv)) (contiguous groups); the pages give only head
    counts ("LLM context window mechanics", "The memory wall"; "Long
    Context", worked scale), the contiguous grouping is the reading adopted.
  * LSE is the natural log of the sum of exp(z) over the visible keys; it is
    the row state that partial results merge by ("Long-context models",
    "Context parallelism distributes exact attention": row maxima, sums and
    output accumulators combine blockwise).
  * Decode: one new query per sequence, rotated at its position (by default
    the cache length L_b), attends to cache entries 0 .. L_b-1 with no mask.
    Cached keys are taken as already rotated.
  * Sliding window and sinks (optional): with a window of W tokens a query
    at position m sees only the W most recent positions m-W+1 .. m ("Arch 03
    -- Long Context", sliding-window slide); S sink tokens, positions
    0 .. S-1, stay visible to every later query (StreamingLLM: keep the first
    tokens and the last W; "Long context (engineering 100k+ tokens)",
    attention sinks).  Positions are the original ones; W = 0 means no window.
  * Chunked prefill: new tokens of a sequence whose first ctx_b tokens are
    already cached sit at positions ctx_b + i and attend to cache entries
    0 .. ctx_b + i (the chunk's own keys are in the cache too), so the causal
    boundary moves to the bottom-right of the (chunk x cache) score block.

Row blocking below only bounds memory: every row is still computed from its
definition over its full set of visible keys, and rows are independent.
"""

import numpy as np

from .rope import rotate

_ROW_BLOCK = 1024


def visible(m, n, window: int = 0, sinks: int = 0):
    """Key position n is visible to query position m (broadcasting arrays):
    causal (n <= m), and inside the window of the W most recent positions or
    among the first S positions when a window is set."""
    m = np.asarray(m)
    n = np.asarray(n)
    ok = n <= m
    if window > 0:
        ok = ok & ((n > m - window) | (n < sinks))
    return ok


def attend(z: np.ndarray, v: np.ndarray):
    """Softmax over the last axis of logits z [R, N] (-inf = not visible),
    applied to values v [N, D].  Returns (out [R, D], lse [R])."""
    z = np.asarray(z, dtype=np.float64)
    zmax = np.max(z, axis=1, keepdims=True)
    e = np.exp(z - zmax)
    total = np.sum(e, axis=1)
    lse = zmax[:, 0] + np.log(total)
    out = (e @ np.asarray(v, dtype=np.float64)) / total[:, None]
    return out, lse


def _sequence_bounds(cu_seqlens):
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    return [(cu[b], cu[b + 1]) for b in range(len(cu) - 1)]


def _group(hq: int, hkv: int) -> int:
    if hq % hkv != 0:
        raise ValueError("query heads must be a multiple of key/value heads")
    return hq // hkv


def prefill(q, k, v, cu_seqlens, theta, scale, window: int = 0, sinks: int = 0):
    """Causal prefill over a packed ragged batch.

    q: [T, Hq, D]; k, v: [T, Hkv, D] (unrotated; theta=None means q and k
    are already rotated).  Returns out [T, Hq, D] and lse [Hq, T], fp64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    T, hq, d = q.shape
    hkv = k.shape[1]
    g = _group(hq, hkv)
    out = np.zeros((T, hq, d), dtype=np.float64)
    lse = np.zeros((hq, T), dtype=np.float64)
    for s0, s1 in _sequence_bounds(cu_seqlens):
        n = s1 - s0
        if n <= 0:
            continue
        pos = np.arange(n)
        qs = np.asarray(q[s0:s1], dtype=np.float64)
        ks = np.asarray(k[s0:s1], dtype=np.float64)
        vs = np.asarray(v[s0:s1], dtype=np.float64)
        if theta is not None:
            qs = rotate(qs, pos, theta)
            ks = rotate(ks, pos, theta)
        for h in range(hq):
            hk = h // g
            kh = ks[:, hk, :]
            vh = vs[:, hk, :]
            for r0 in range(0, n, _ROW_BLOCK):
                r1 = min(n, r0 + _ROW_BLOCK)
                z = scale * (qs[r0:r1, h, :] @ kh[:r1].T)     # [R, r1]
                rows = np.arange(r0, r1)[:, None]
                cols = np.arange(r1)[None, :]
                z[~visible(rows, cols, window, sinks)] = -np.inf
                o, l = attend(z, vh[:r1])
                out[s0 + r0:s0 + r1, h, :] = o
                lse[h, s0 + r0:s0 + r1] = l
    return out, lse


def prefill_rows(q, k, v, cu_seqlens, theta, scale, rows, window: int = 0, sinks: int = 0):
    """Causal prefill evaluated only at the requested (token, head) pairs,
    each over its full causal prefix.  ``rows`` is an iterable of
    (global token index, query head).  Returns (out [R, D], lse [R]) in the
    order given."""
    # q, k, v are only sliced here, so any array-like with numpy indexing and
    # .shape will do (large inputs can be widened slice by slice)
    hq = q.shape[1]
    hkv = k.shape[1]
    g = _group(hq, hkv)
    bounds = _sequence_bounds(cu_seqlens)
    starts = np.array([b[0] for b in bounds])
    rows = [(int(t), int(h)) for t, h in rows]
    # group requests by (sequence, kv head) so each key block is rotated once
    groups = {}
    for idx, (t, h) in enumerate(rows):
        b = int(np.searchsorted(starts, t, side="right") - 1)
        while bounds[b][1] <= t:      # skip empty sequences
            b += 1
        groups.setdefault((b, h // g), []).append(idx)
    out = np.zeros((len(rows), q.shape[2]), dtype=np.float64)
    lse = np.zeros(len(rows), dtype=np.float64)
    for (b, hk), idxs in groups.items():
        s0, s1 = bounds[b]
        last = max(rows[i][0] for i in idxs) - s0
        kk = np.asarray(k[s0:s0 + last + 1, hk, :], dtype=np.float64)
        vv = np.asarray(v[s0:s0 + last + 1, hk, :], dtype=np.float64)
        if theta is not None:
            kk = rotate(kk, np.arange(last + 1), theta)
        # the rows of one group share their keys: form their logits together,
        # each row over its own causal prefix (later keys set to -inf)
        for c0 in range(0, len(idxs), 256):
            part = idxs[c0:c0 + 256]
            pos = np.array([rows[i][0] - s0 for i in part])
            qr = np.stack([np.asarray(q[rows[i][0], rows[i][1], :], dtype=np.float64)
                           for i in part])
            if theta is not None:
                qr = rotate(qr, pos, theta)
            span = int(pos.max()) + 1
            z = scale * (qr @ kk[:span].T)
            z[~visible(pos[:, None], np.arange(span)[None, :], window, sinks)] = -np.inf
            o, l = attend(z, vv[:span])
            out[part] = o
            lse[part] = l
    return out, lse


def decode(q, k_cache, v_cache, seqlens, theta, scale, q_pos=None, window: int = 0,
           sinks: int = 0):
    """One new query per sequence over a contiguous per-sequence cache.

    q: [B, Hq, D] (unrotated); k_cache, v_cache: [B, Lmax, Hkv, D] with keys
    already rotated; seqlens: [B] cache lengths L_b >= 1.  The query of
    sequence b is rotated at q_pos[b] (default L_b) and attends to the cache
    rows 0 .. L_b-1 that the window / sinks leave visible from that position
    (all of them without a window).  Returns out [B, Hq, D] and lse [B, Hq],
    fp64."""
    q = np.asarray(q)
    B, hq, d = q.shape
    hkv = k_cache.shape[2]
    g = _group(hq, hkv)
    out = np.zeros((B, hq, d), dtype=np.float64)
    lse = np.zeros((B, hq), dtype=np.float64)
    for b in range(B):
        L = int(seqlens[b])
        m = L if q_pos is None else int(q_pos[b])
        qr = np.asarray(q[b], dtype=np.float64)
        if theta is not None:
            qr = rotate(qr[None, :, :], [m], theta)[0]
        for hk in range(hkv):
            kk = np.asarray(k_cache[b, :L, hk, :], dtype=np.float64)
            vv = np.asarray(v_cache[b, :L, hk, :], dtype=np.float64)
            heads = list(range(hk * g, (hk + 1) * g))
            z = scale * (qr[heads] @ kk.T)                 # [g, L]
            if window > 0:
                z[:, ~((np.arange(L) > m - window) | (np.arange(L) < sinks))] = -np.inf
            o, l = attend(z, vv)
            out[b, heads] = o
            lse[b, heads] = l
    return out, lse


def prefill_chunk(q, k_cache, v_cache, cu_seqlens_q, ctx_lens, theta, scale, window: int = 0,
                  sinks: int = 0, rows=None):
    """Prefill of new tokens against a per-sequence cache (chunked prefill).

    q: [Tq, Hq, D] unrotated, packed by cu_seqlens_q; k_cache, v_cache:
    [B, Lmax, Hkv, D] holding, for sequence b, ctx_lens[b] earlier tokens and
    then the n_b new ones (keys already rotated).  Token i of the chunk sits
    at position ctx_b + i and attends to the visible cache rows 0 .. ctx_b + i.
    Returns out [Tq, Hq, D] and lse [Hq, Tq], fp64; with ``rows`` (an
    iterable of (token, query head)) only those are evaluated and
    (out [R, D], lse [R]) come back in that order."""
    hq, d = q.shape[1], q.shape[2]
    hkv = k_cache.shape[2]
    g = _group(hq, hkv)
    bounds = _sequence_bounds(cu_seqlens_q)
    if rows is None:
        want = [(t, h) for s0, s1 in bounds for t in range(s0, s1) for h in range(hq)]
    else:
        want = [(int(t), int(h)) for t, h in rows]
    starts = np.array([b[0] for b in bounds])
    groups = {}
    for idx, (t, h) in enumerate(want):
        b = int(np.searchsorted(starts, t, side="right") - 1)
        while bounds[b][1] <= t:
            b += 1
        groups.setdefault((b, h // g), []).append(idx)
    out_r = np.zeros((len(want), d), dtype=np.float64)
    lse_r = np.zeros(len(want), dtype=np.float64)
    for (b, hk), idxs in groups.items():
        s0 = bounds[b][0]
        ctx = int(ctx_lens[b])
        pos_all = np.array([ctx + want[i][0] - s0 for i in idxs])
        span = int(pos_all.max()) + 1
        kk = np.asarray(k_cache[b, :span, hk, :], dtype=np.float64)
        vv = np.asarray(v_cache[b, :span, hk, :], dtype=np.float64)
        for c0 in range(0, len(idxs), 256):
            part = idxs[c0:c0 + 256]
            pos = pos_all[c0:c0 + 256]
            qr = np.stack([np.asarray(q[want[i][0], want[i][1], :], dtype=np.float64)
                           for i in part])
            if theta is not None:
                qr = rotate(qr, pos, theta)
            z = scale * (qr @ kk.T)
            z[~visible(pos[:, None], np.arange(span)[None, :], window, sinks)] = -np.inf
            o, l = attend(z, vv)
            out_r[part] = o
            lse_r[part] = l
    if rows is not None:
        return out_r, lse_r
    Tq = q.shape[0]
    out = np.zeros((Tq, hq, d), dtype=np.float64)
    lse = np.zeros((hq, Tq), dtype=np.float64)
    for i, (t, h) in enumerate(want):
        out[t, h] = out_r[i]
        lse[h, t] = lse_r[i]
    return out, lse


def merge(outs, lses):
    """Combine partial results computed over disjoint key sets.

    outs: [P, ..., D], lses: [P, ...].  The merged LSE is the log of the sum
    of exp(lse_p); the merged output weights each partial by
    exp(lse_p - lse) ("Long-context models", "Context parallelism distributes
    exact attention")."""
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    top = np.max(lses, axis=0)
    w = np.exp(lses - top[None])
    total = np.sum(w, axis=0)
    lse = top + np.log(total)
    out = np.sum(w[..., None] * outs, axis=0) / total[..., None]
    return out, lse


def causal_probs(q, k, theta, scale):
    """Full attention probabilities [Hq, n, n] of one sequence (small n only),
    for the row-sum and causality checks."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n, hq, _ = q.shape
    g = _group(hq, k.shape[1])
    pos = np.arange(n)
    if theta is not None:
        q = rotate(q, pos, theta)
        k = rotate(k, pos, theta)
    p = np.zeros((hq, n, n))
    for h in range(hq):
        z = scale * (q[:, h, :] @ k[:, h // g, :].T)
        z[np.triu(np.ones((n, n), dtype=bool), 1)] = -np.inf
        zmax = z.max(axis=1, keepdims=True)
        e = np.exp(z - zmax)
        p[h] = e / e.sum(axis=1, keepdims=True)
    return p
