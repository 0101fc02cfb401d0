"""Pins of the oracle's attention (CPU only): softmax normalisation and
causality, the first row, the all-zero-query closed form, brute force on tiny
inputs, GQA as repeated heads, the split/merge identity, decode against a
prefill row, and shift invariance."""

import math

import numpy as np
import pytest

from oracle import attention, bruteforce, freqs, rope


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _theta_scale(D=8, base=10000.0, s=4.0, L=16):
    th = freqs.yarn_theta(D, base, s, L)
    return th, freqs.softmax_scale(D, freqs.attention_temperature(s))


def test_probabilities_rows_sum_to_one_and_are_causal():
    rng = _rng(10)
    n, hq, hkv, D = 23, 4, 2, 16
    th, sc = _theta_scale(D)
    q = rng.standard_normal((n, hq, D))
    k = rng.standard_normal((n, hkv, D))
    p = attention.causal_probs(q, k, th, sc)
    assert np.allclose(p.sum(axis=2), 1.0, rtol=0, atol=1e-14)
    assert np.all(p[:, np.triu_indices(n, 1)[0], np.triu_indices(n, 1)[1]] == 0.0)
    assert np.all(p[:, np.tril_indices(n)[0], np.tril_indices(n)[1]] > 0.0)


def test_first_row_is_first_value():
    rng = _rng(11)
    n, hq, hkv, D = 9, 4, 2, 8
    th, sc = _theta_scale(D)
    q = rng.standard_normal((n, hq, D))
    k = rng.standard_normal((n, hkv, D))
    v = rng.standard_normal((n, hkv, D))
    out, lse = attention.prefill(q, k, v, [0, n], th, sc)
    for h in range(hq):
        assert np.array_equal(out[0, h], v[0, h // 2])
        # position 0 is not rotated, so z_00 is the plain scaled product
        assert lse[h, 0] == pytest.approx(sc * float(q[0, h] @ k[0, h // 2]), abs=1e-14)


def test_zero_query_gives_running_mean_and_log_count():
    rng = _rng(12)
    n, D = 40, 16
    th, sc = _theta_scale(D)
    q = np.zeros((n, 2, D))
    k = rng.standard_normal((n, 1, D))
    v = rng.standard_normal((n, 1, D))
    out, lse = attention.prefill(q, k, v, [0, n], th, sc)
    mean = np.cumsum(v[:, 0, :], axis=0) / np.arange(1, n + 1)[:, None]
    for h in range(2):
        assert np.allclose(out[:, h, :], mean, rtol=0, atol=1e-13)
        assert np.allclose(lse[h], np.log(np.arange(1, n + 1)), rtol=0, atol=1e-13)


@pytest.mark.parametrize("lens", [(5,), (1, 7, 4), (16,)])
def test_bruteforce_matches_vectorised(lens):
    rng = _rng(13)
    T = sum(lens)
    hq, hkv, D = 4, 2, 8
    th, sc = _theta_scale(D)
    q = rng.standard_normal((T, hq, D))
    k = rng.standard_normal((T, hkv, D))
    v = rng.standard_normal((T, hkv, D))
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, lse = attention.prefill(q, k, v, cu, th, sc)
    bo, bl = bruteforce.causal_attention(q.tolist(), k.tolist(), v.tolist(), list(lens), list(th), sc)
    assert np.allclose(out, np.array(bo), rtol=0, atol=1e-12)
    assert np.allclose(lse, np.array(bl), rtol=0, atol=1e-12)


def test_gqa_equals_repeated_heads():
    rng = _rng(14)
    n, hq, hkv, D = 31, 8, 2, 16
    th, sc = _theta_scale(D)
    q = rng.standard_normal((n, hq, D))
    k = rng.standard_normal((n, hkv, D))
    v = rng.standard_normal((n, hkv, D))
    g = hq // hkv
    out_g, lse_g = attention.prefill(q, k, v, [0, n], th, sc)
    out_m, lse_m = attention.prefill(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), [0, n], th, sc)
    assert np.allclose(out_g, out_m, rtol=0, atol=1e-14)
    assert np.allclose(lse_g, lse_m, rtol=0, atol=1e-14)


def test_ragged_batch_equals_separate_sequences():
    rng = _rng(15)
    lens = (3, 11, 1, 6)
    hq, hkv, D = 2, 1, 8
    th, sc = _theta_scale(D)
    T = sum(lens)
    q = rng.standard_normal((T, hq, D))
    k = rng.standard_normal((T, hkv, D))
    v = rng.standard_normal((T, hkv, D))
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, lse = attention.prefill(q, k, v, cu, th, sc)
    for b, n in enumerate(lens):
        s0 = cu[b]
        o1, l1 = attention.prefill(q[s0:s0 + n], k[s0:s0 + n], v[s0:s0 + n], [0, n], th, sc)
        assert np.array_equal(out[s0:s0 + n], o1)
        assert np.array_equal(lse[:, s0:s0 + n], l1)


def test_prefill_rows_matches_dense():
    rng = _rng(16)
    lens = (70, 1, 33)
    hq, hkv, D = 4, 2, 16
    th, sc = _theta_scale(D, s=8.0, L=32)
    T = sum(lens)
    q = rng.standard_normal((T, hq, D))
    k = rng.standard_normal((T, hkv, D))
    v = rng.standard_normal((T, hkv, D))
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, lse = attention.prefill(q, k, v, cu, th, sc)
    rows = [(0, 0), (69, 3), (70, 1), (71, 2), (103, 0), (40, 2)]
    ro, rl = attention.prefill_rows(q, k, v, cu, th, sc, rows)
    for i, (t, h) in enumerate(rows):
        assert np.allclose(ro[i], out[t, h], rtol=0, atol=1e-13)
        assert rl[i] == pytest.approx(lse[h, t], abs=1e-13)


def test_causality_future_keys_do_not_matter():
    rng = _rng(17)
    n, D = 20, 8
    th, sc = _theta_scale(D)
    q = rng.standard_normal((n, 2, D))
    k = rng.standard_normal((n, 1, D))
    v = rng.standard_normal((n, 1, D))
    out, lse = attention.prefill(q, k, v, [0, n], th, sc)
    k2, v2 = k.copy(), v.copy()
    k2[12:] = rng.standard_normal(k2[12:].shape)
    v2[12:] = 100.0
    out2, lse2 = attention.prefill(q, k2, v2, [0, n], th, sc)
    assert np.array_equal(out[:12], out2[:12]) and np.array_equal(lse[:, :12], lse2[:, :12])
    assert not np.allclose(out[12:], out2[12:])


@pytest.mark.parametrize("parts", [(1,), (3, 17, 10), (29, 1)])
def test_split_merge_identity(parts):
    rng = _rng(18)
    D = 16
    nk = sum(parts)
    q = rng.standard_normal((3, D))
    kk = rng.standard_normal((nk, D))
    vv = rng.standard_normal((nk, D))
    z = 0.3 * q @ kk.T
    full_o, full_l = attention.attend(z, vv)
    outs, lses = [], []
    s = 0
    for p in parts:
        o, l = attention.attend(z[:, s:s + p], vv[s:s + p])
        outs.append(o)
        lses.append(l)
        s += p
    mo, ml = attention.merge(outs, lses)
    assert np.allclose(mo, full_o, rtol=0, atol=1e-13)
    assert np.allclose(ml, full_l, rtol=0, atol=1e-13)


def test_decode_equals_prefill_last_row():
    rng = _rng(19)
    L, hq, hkv, D = 45, 8, 2, 16
    th, sc = _theta_scale(D, base=500000.0, s=8.0, L=16)
    q = rng.standard_normal((L, hq, D))
    k = rng.standard_normal((L, hkv, D))
    v = rng.standard_normal((L, hkv, D))
    out, lse = attention.prefill(q, k, v, [0, L], th, sc)
    kc = rope.rotate(k, np.arange(L), th)[None]          # cache of rotated keys
    vc = v[None]
    do, dl = attention.decode(q[L - 1][None], kc, vc, [L], th, sc, q_pos=[L - 1])
    assert np.allclose(do[0], out[L - 1], rtol=0, atol=1e-13)
    assert np.allclose(dl[0], lse[:, L - 1], rtol=0, atol=1e-13)


def test_decode_shift_invariance():
    rng = _rng(20)
    L, hq, hkv, D = 30, 4, 1, 32
    th, sc = _theta_scale(D, base=500000.0, s=8.0, L=64)
    q = rng.standard_normal((1, hq, D))
    k = rng.standard_normal((L, hkv, D))
    v = rng.standard_normal((1, L, hkv, D))
    o0, l0 = attention.decode(q, rope.rotate(k, np.arange(L), th)[None], v, [L], th, sc)
    c = 77777
    o1, l1 = attention.decode(q, rope.rotate(k, np.arange(L) + c, th)[None], v, [L], th, sc, q_pos=[L + c])
    assert np.allclose(o0, o1, rtol=0, atol=1e-9)
    assert np.allclose(l0, l1, rtol=0, atol=1e-9)


def test_decode_ignores_cache_rows_past_length():
    rng = _rng(21)
    B, Lmax, hq, hkv, D = 3, 12, 2, 1, 8
    th, sc = _theta_scale(D)
    q = rng.standard_normal((B, hq, D))
    kc = rng.standard_normal((B, Lmax, hkv, D))
    vc = rng.standard_normal((B, Lmax, hkv, D))
    lens = np.array([1, 5, 12])
    for b in range(B):
        kc[b, lens[b]:] = np.nan
        vc[b, lens[b]:] = np.nan
    o, l = attention.decode(q, kc, vc, lens, th, sc)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    # a single cached entry: the output is that value
    assert np.array_equal(o[0, 0], vc[0, 0, 0])


def test_temperature_multiplies_logits_once():
    # with all keys equal except one, the probability ratio is exp(scale * delta):
    # doubling the temperature doubles log of the ratio.
    D = 8
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = 1.0
    kc = np.zeros((1, 2, 1, D))
    kc[0, 1, 0, 0] = 1.0
    vc = np.zeros((1, 2, 1, D))
    vc[0, 1, 0, 0] = 1.0
    th = np.zeros(D // 2)          # no rotation, isolates the scale
    t = freqs.attention_temperature(8.0)
    sc = freqs.softmax_scale(D, t)
    o, _ = attention.decode(q, kc, vc, [2], th, sc)
    p1 = o[0, 0, 0]
    assert math.log(p1 / (1 - p1)) == pytest.approx(t / math.sqrt(D), rel=1e-12)
