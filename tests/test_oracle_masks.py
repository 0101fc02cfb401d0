"""Pins of the oracle's sliding-window / sink visibility and of chunked
prefill (CPU only): pure-Python brute force on tiny ragged inputs, the
single-token window, windows at least as long as the sequence, the all-zero
query (log of the visible count and the mean of the visible values, with the
count and the index set written in closed form), chunked prefill against full
prefill (empty prefix and two-chunk composition), the last chunk row against
decode, and the row-sampled forms against the dense ones."""

import math

import numpy as np
import pytest

from oracle import attention, bruteforce, freqs, rope


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _theta_scale(D=8, base=10000.0, s=4.0, L=16):
    th = freqs.yarn_theta(D, base, s, L)
    return th, freqs.softmax_scale(D, freqs.attention_temperature(s))


def _nested(a):
    return np.asarray(a, dtype=np.float64).tolist()


def _visible_count(m, W, S):
    """Positions a query at m sees: min(m+1, W) recent ones plus the sinks
    that lie before the window."""
    if W <= 0:
        return m + 1
    return min(m + 1, W) + min(S, max(0, m - W + 1))


def _visible_set(m, W, S):
    if W <= 0:
        return list(range(m + 1))
    lo = max(0, m - W + 1)
    return list(range(min(S, lo))) + list(range(lo, m + 1))


@pytest.mark.parametrize("window,sinks", [(1, 0), (3, 0), (3, 2), (5, 1), (4, 7)])
def test_prefill_window_sinks_matches_brute_force(window, sinks):
    rng = _rng(40 + window * 10 + sinks)
    lens = [7, 12]
    T, hq, hkv, D = sum(lens), 4, 2, 8
    th, sc = _theta_scale(D)
    q = rng.standard_normal((T, hq, D))
    k = rng.standard_normal((T, hkv, D))
    v = rng.standard_normal((T, hkv, D))
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, lse = attention.prefill(q, k, v, cu, th, sc, window=window, sinks=sinks)
    bo, bl = bruteforce.causal_attention(_nested(q), _nested(k), _nested(v), lens, list(th), sc,
                                         window=window, sinks=sinks)
    assert np.allclose(out, np.array(bo), rtol=0, atol=1e-12)
    assert np.allclose(lse, np.array(bl), rtol=0, atol=1e-12)


def test_single_token_window_returns_own_value():
    rng = _rng(50)
    n, hq, hkv, D = 11, 2, 1, 8
    th, sc = _theta_scale(D)
    q = rng.standard_normal((n, hq, D))
    k = rng.standard_normal((n, hkv, D))
    v = rng.standard_normal((n, hkv, D))
    out, lse = attention.prefill(q, k, v, [0, n], th, sc, window=1)
    qr = rope.rotate(q, np.arange(n), th)
    kr = rope.rotate(k, np.arange(n), th)
    for h in range(hq):
        assert np.array_equal(out[:, h], v[:, 0])
        z = sc * np.einsum("td,td->t", qr[:, h], kr[:, 0])
        assert np.allclose(lse[h], z, rtol=0, atol=1e-13)


def test_window_as_long_as_the_sequence_is_plain_causal():
    rng = _rng(51)
    n, hq, hkv, D = 17, 4, 2, 8
    th, sc = _theta_scale(D)
    q = rng.standard_normal((n, hq, D))
    k = rng.standard_normal((n, hkv, D))
    v = rng.standard_normal((n, hkv, D))
    ref = attention.prefill(q, k, v, [0, n], th, sc)
    for W, S in ((n, 0), (n + 5, 3)):
        got = attention.prefill(q, k, v, [0, n], th, sc, window=W, sinks=S)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


@pytest.mark.parametrize("window,sinks", [(1, 0), (4, 0), (4, 2), (6, 3), (9, 9)])
def test_zero_query_counts_visible_keys(window, sinks):
    rng = _rng(52)
    n, D = 30, 8
    th, sc = _theta_scale(D)
    q = np.zeros((n, 2, D))
    k = rng.standard_normal((n, 1, D))
    v = rng.standard_normal((n, 1, D))
    out, lse = attention.prefill(q, k, v, [0, n], th, sc, window=window, sinks=sinks)
    for m in range(n):
        cnt = _visible_count(m, window, sinks)
        idx = _visible_set(m, window, sinks)
        assert len(idx) == cnt
        for h in range(2):
            assert lse[h, m] == pytest.approx(math.log(cnt), abs=1e-13)
            assert np.allclose(out[m, h], v[idx, 0].mean(axis=0), rtol=0, atol=1e-13)


def _cache_from_sequences(k_seq, v_seq, th, Lmax):
    """Rotated-key caches [B, Lmax, Hkv, D] from per-sequence K, V (positions
    from 0), tails filled with NaN so that over-reads show."""
    B = len(k_seq)
    hkv, D = k_seq[0].shape[1], k_seq[0].shape[2]
    kc = np.full((B, Lmax, hkv, D), np.nan)
    vc = np.full((B, Lmax, hkv, D), np.nan)
    for b in range(B):
        L = k_seq[b].shape[0]
        kc[b, :L] = rope.rotate(k_seq[b], np.arange(L), th) if th is not None else k_seq[b]
        vc[b, :L] = v_seq[b]
    return kc, vc


@pytest.mark.parametrize("window,sinks", [(0, 0), (3, 0), (4, 2)])
def test_chunk_matches_brute_force(window, sinks):
    rng = _rng(60 + window)
    ctx, qlens = [0, 5, 2], [4, 6, 1]
    hq, hkv, D, Lmax = 4, 2, 8, 13
    th, sc = _theta_scale(D)
    k_seq = [rng.standard_normal((c + n, hkv, D)) for c, n in zip(ctx, qlens)]
    v_seq = [rng.standard_normal((c + n, hkv, D)) for c, n in zip(ctx, qlens)]
    kc, vc = _cache_from_sequences(k_seq, v_seq, th, Lmax)
    q = rng.standard_normal((sum(qlens), hq, D))
    cu = np.concatenate([[0], np.cumsum(qlens)])
    out, lse = attention.prefill_chunk(q, kc, vc, cu, ctx, th, sc, window=window, sinks=sinks)
    kcb = np.nan_to_num(kc, nan=1e300)  # the brute force must not touch the tails
    vcb = np.nan_to_num(vc, nan=1e300)
    bo, bl = bruteforce.chunk_attention(_nested(q), _nested(kcb), _nested(vcb), qlens, ctx,
                                        list(th), sc, window=window, sinks=sinks)
    assert np.allclose(out, np.array(bo), rtol=0, atol=1e-12)
    assert np.allclose(lse, np.array(bl), rtol=0, atol=1e-12)


@pytest.mark.parametrize("window,sinks", [(0, 0), (5, 2)])
def test_chunk_with_empty_prefix_is_prefill(window, sinks):
    rng = _rng(61)
    lens = [9, 14]
    hq, hkv, D = 4, 2, 16
    th, sc = _theta_scale(D)
    k_seq = [rng.standard_normal((n, hkv, D)) for n in lens]
    v_seq = [rng.standard_normal((n, hkv, D)) for n in lens]
    q = rng.standard_normal((sum(lens), hq, D))
    kc, vc = _cache_from_sequences(k_seq, v_seq, th, max(lens))
    cu = np.concatenate([[0], np.cumsum(lens)])
    got = attention.prefill_chunk(q, kc, vc, cu, [0, 0], th, sc, window=window, sinks=sinks)
    ref = attention.prefill(q, np.concatenate(k_seq), np.concatenate(v_seq), cu, th, sc,
                            window=window, sinks=sinks)
    assert np.allclose(got[0], ref[0], rtol=0, atol=1e-13)
    assert np.allclose(got[1], ref[1], rtol=0, atol=1e-13)


@pytest.mark.parametrize("window,sinks", [(0, 0), (6, 0), (6, 3)])
def test_two_chunks_compose_to_prefill(window, sinks):
    rng = _rng(62)
    n, n1, hq, hkv, D = 21, 8, 4, 1, 16
    th, sc = _theta_scale(D)
    q = rng.standard_normal((n, hq, D))
    k = rng.standard_normal((n, hkv, D))
    v = rng.standard_normal((n, hkv, D))
    ref_o, ref_l = attention.prefill(q, k, v, [0, n], th, sc, window=window, sinks=sinks)
    kc, vc = _cache_from_sequences([k], [v], th, n)
    o1, l1 = attention.prefill_chunk(q[:n1], kc, vc, [0, n1], [0], th, sc, window=window,
                                     sinks=sinks)
    o2, l2 = attention.prefill_chunk(q[n1:], kc, vc, [0, n - n1], [n1], th, sc, window=window,
                                     sinks=sinks)
    assert np.allclose(np.concatenate([o1, o2]), ref_o, rtol=0, atol=1e-13)
    assert np.allclose(np.concatenate([l1, l2], axis=1), ref_l, rtol=0, atol=1e-13)


@pytest.mark.parametrize("window,sinks", [(0, 0), (7, 0), (7, 4)])
def test_last_chunk_row_is_decode(window, sinks):
    rng = _rng(63)
    ctx, qlens = [10, 3], [5, 8]
    hq, hkv, D, Lmax = 4, 2, 16, 16
    th, sc = _theta_scale(D)
    k_seq = [rng.standard_normal((c + n, hkv, D)) for c, n in zip(ctx, qlens)]
    v_seq = [rng.standard_normal((c + n, hkv, D)) for c, n in zip(ctx, qlens)]
    kc, vc = _cache_from_sequences(k_seq, v_seq, th, Lmax)
    q = rng.standard_normal((sum(qlens), hq, D))
    cu = np.concatenate([[0], np.cumsum(qlens)])
    out, lse = attention.prefill_chunk(q, kc, vc, cu, ctx, th, sc, window=window, sinks=sinks)
    last = cu[1:] - 1
    L = np.array(ctx) + np.array(qlens)
    do, dl = attention.decode(q[last], kc, vc, L, th, sc, q_pos=L - 1, window=window, sinks=sinks)
    assert np.allclose(out[last], do, rtol=0, atol=1e-13)
    assert np.allclose(lse[:, last].T, dl, rtol=0, atol=1e-13)


def test_chunk_rows_equal_dense():
    rng = _rng(64)
    ctx, qlens = [6, 0], [7, 9]
    hq, hkv, D, Lmax = 4, 2, 8, 13
    th, sc = _theta_scale(D)
    k_seq = [rng.standard_normal((c + n, hkv, D)) for c, n in zip(ctx, qlens)]
    v_seq = [rng.standard_normal((c + n, hkv, D)) for c, n in zip(ctx, qlens)]
    kc, vc = _cache_from_sequences(k_seq, v_seq, th, Lmax)
    q = rng.standard_normal((sum(qlens), hq, D))
    cu = np.concatenate([[0], np.cumsum(qlens)])
    out, lse = attention.prefill_chunk(q, kc, vc, cu, ctx, th, sc, window=4, sinks=1)
    rows = [(3, 1), (0, 0), (15, 3), (7, 2), (8, 0)]
    ro, rl = attention.prefill_chunk(q, kc, vc, cu, ctx, th, sc, window=4, sinks=1, rows=rows)
    for i, (t, h) in enumerate(rows):
        assert np.allclose(ro[i], out[t, h], rtol=0, atol=1e-14)
        assert rl[i] == pytest.approx(lse[h, t], abs=1e-14)


def test_prefill_rows_with_window_equal_dense():
    rng = _rng(65)
    lens = [20, 13]
    T, hq, hkv, D = sum(lens), 4, 2, 8
    th, sc = _theta_scale(D)
    q = rng.standard_normal((T, hq, D))
    k = rng.standard_normal((T, hkv, D))
    v = rng.standard_normal((T, hkv, D))
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, lse = attention.prefill(q, k, v, cu, th, sc, window=5, sinks=2)
    rows = [(0, 0), (19, 3), (20, 1), (32, 2), (11, 0)]
    ro, rl = attention.prefill_rows(q, k, v, cu, th, sc, rows, window=5, sinks=2)
    for i, (t, h) in enumerate(rows):
        assert np.allclose(ro[i], out[t, h], rtol=0, atol=1e-14)
        assert rl[i] == pytest.approx(lse[h, t], abs=1e-14)


@pytest.mark.parametrize("window,sinks", [(4, 0), (4, 2)])
def test_decode_window_zero_query_counts(window, sinks):
    """Decode at position m = L over cache rows < L: the window keeps rows
    > L - W (W - 1 cache rows, the query's own slot is not in the cache) plus
    the sinks before them."""
    rng = _rng(66)
    B, Lmax, D = 3, 20, 8
    th, sc = _theta_scale(D)
    L = np.array([20, 9, 2])
    q = np.zeros((B, 2, D))
    kc = rng.standard_normal((B, Lmax, 1, D))
    vc = rng.standard_normal((B, Lmax, 1, D))
    out, lse = attention.decode(q, kc, vc, L, th, sc, window=window, sinks=sinks)
    for b in range(B):
        m = int(L[b])
        idx = [j for j in _visible_set(m, window, sinks) if j < m]
        assert lse[b, 0] == pytest.approx(math.log(len(idx)), abs=1e-13)
        assert np.allclose(out[b, 1], vc[b, idx, 0].mean(axis=0), rtol=0, atol=1e-13)
