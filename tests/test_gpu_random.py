"""Seeded random configurations of every path against the oracle, in full:
ragged prefill (bf16, windows, sinks, GQA groups, head_dim 64/128, bf16 or
fp32 output), chunked prefill against a cache, and bf16 / FP8 decode with
windows, sinks and query positions placed inside the cache.  Each case draws
its shapes from its own seed (printed before it runs), so a failure names a
reproducible configuration; the sizes keep the fp64 oracle to a second or so
per case."""

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import fp8 as ofp8
from tests._gpu_util import BF16_TOL, LazyF64, lib_theta, oracle_theta, say, to_dev, to_f64
from yarn_scaled_rope_amd import ops
from yarn_scaled_rope_amd import workloads as wl

pytestmark = pytest.mark.gpu

GROUPS = [(4, 1), (8, 2), (6, 3), (4, 4), (16, 2)]


def _close(got, ref, tol=BF16_TOL):
    """max |got - ref| <= tol where both are finite; -inf exactly where the
    oracle has -inf (a query that sees no key)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    assert np.all(np.isfinite(got[fin]))
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    assert err <= tol, err
    return err


def _window(rng):
    w = int(rng.choice([0, 0, 1, 2, 64, int(rng.integers(3, 600))]))
    s = int(rng.choice([0, int(rng.integers(1, 80))])) if w else 0
    if w == 1 and s == 0:
        s = 1
    return w, s


@pytest.mark.parametrize("seed", range(8))
def test_random_prefill(seed):
    rng = np.random.Generator(np.random.PCG64(500 + seed))
    B = int(rng.integers(1, 5))
    lens = tuple(int(x) for x in rng.integers(1, 700, size=B))
    hq, hkv = GROUPS[int(rng.integers(len(GROUPS)))]
    D = int(rng.choice([64, 128]))
    window, sinks = _window(rng)
    out_dtype = ops.YR_F32 if rng.integers(2) else ops.YR_BF16
    say(f"random prefill seed={seed}: lens={lens} hq={hq} hkv={hkv} D={D} W={window} S={sinks} "
        f"out={'f32' if out_dtype == ops.YR_F32 else 'bf16'}")
    cfg = wl.PrefillConfig("t", 600 + seed, lens, hq, hkv, D, "bf16", 500000.0, 8.0, 16384)
    inp = wl.make_prefill(cfg)
    th_dev, scale = lib_theta(D, cfg.base, cfg.factor, cfg.original_max_position)
    out, lse = ops.attn_prefill_fwd(to_dev(inp["q"], "bf16"), to_dev(inp["k"], "bf16"),
                                    to_dev(inp["v"], "bf16"),
                                    torch.from_numpy(inp["cu_seqlens"]).cuda(), max(lens), th_dev,
                                    scale, out_dtype=out_dtype, window=window, sinks=sinks)
    torch.cuda.synchronize()
    th, sc = oracle_theta(D, cfg.base, cfg.factor, cfg.original_max_position)
    ro, rl = oatt.prefill(wl.as_f64(inp["q"], "bf16"), wl.as_f64(inp["k"], "bf16"),
                          wl.as_f64(inp["v"], "bf16"), inp["cu_seqlens"], th, sc,
                          window=window, sinks=sinks)
    print(f"max-abs out {_close(to_f64(out), ro):.3e} lse {_close(lse.cpu().numpy(), rl):.3e}")


@pytest.mark.parametrize("seed", range(6))
def test_random_chunk(seed):
    rng = np.random.Generator(np.random.PCG64(700 + seed))
    B = int(rng.integers(1, 4))
    ctx = tuple(int(x) for x in rng.integers(0, 1500, size=B))
    qlens = tuple(int(x) for x in rng.integers(1, 400, size=B))
    lmax = max(c + n for c, n in zip(ctx, qlens)) + int(rng.integers(0, 100))
    hq, hkv = GROUPS[int(rng.integers(len(GROUPS)))]
    D = int(rng.choice([64, 128]))
    window, sinks = _window(rng)
    say(f"random chunk seed={seed}: ctx={ctx} qlens={qlens} Lmax={lmax} hq={hq} hkv={hkv} D={D} "
        f"W={window} S={sinks}")
    cfg = wl.ChunkConfig("t", 800 + seed, ctx, qlens, lmax, hq, hkv, D, "bf16", 500000.0, 8.0,
                         16384)
    inp = wl.make_chunk(cfg)
    th_dev, scale = lib_theta(D, cfg.base, cfg.factor, cfg.original_max_position)
    out, lse = ops.attn_prefill_chunk(
        to_dev(inp["q"], "bf16"), to_dev(inp["k_cache"], "bf16"), to_dev(inp["v_cache"], "bf16"),
        torch.from_numpy(inp["cu_seqlens_q"]).cuda(), torch.from_numpy(inp["ctx_lens"]).cuda(),
        max(qlens), th_dev, scale, window=window, sinks=sinks, out_dtype=ops.YR_F32)
    torch.cuda.synchronize()
    th, sc = oracle_theta(D, cfg.base, cfg.factor, cfg.original_max_position)
    ro, rl = oatt.prefill_chunk(LazyF64(inp["q"], "bf16"), LazyF64(inp["k_cache"], "bf16"),
                                LazyF64(inp["v_cache"], "bf16"), inp["cu_seqlens_q"],
                                inp["ctx_lens"], th, sc, window=window, sinks=sinks)
    print(f"max-abs out {_close(to_f64(out), ro):.3e} lse {_close(lse.cpu().numpy(), rl):.3e}")


class _LazyFP8:
    def __init__(self, codes, scale):
        self.codes, self.scale = codes, np.asarray(scale, dtype=np.float64)
        self.shape = codes.shape

    def __getitem__(self, idx):
        b, rows, h, d = idx
        return ofp8.e4m3_to_f64(self.codes[b, rows, h, d]) * self.scale[h]


class _Rows:
    """The caches of the sequences in idx only (the oracle slices [b, :L, h, :])."""

    def __init__(self, cache, idx):
        self.cache, self.idx = cache, idx
        self.shape = (len(idx),) + tuple(cache.shape[1:])

    def __getitem__(self, key):
        b, rows, h, d = key
        return self.cache[int(self.idx[b]), rows, h, d]


@pytest.mark.parametrize("seed", range(8))
def test_random_decode(seed):
    rng = np.random.Generator(np.random.PCG64(900 + seed))
    B = int(rng.integers(1, 6))
    lmax = int(rng.integers(2, 3000))
    hq, hkv = GROUPS[int(rng.integers(len(GROUPS)))]
    D = int(rng.choice([64, 128]))
    window, sinks = _window(rng)
    fp8 = bool(seed % 2)
    cfg = wl.DecodeConfig("t", 1000 + seed, 0, 0, 0, hq, hkv, D, "bf16", 500000.0, 8.0, 16384)
    make = wl.make_decode_fp8 if fp8 else wl.make_decode
    inp = make(cfg, seed=1000 + seed, batch=B, max_cache_len=lmax, min_cache_len=1)
    L = inp["seqlens"]
    # half the queries at their cache length, the rest anywhere up to past it
    q_pos = np.where(rng.integers(2, size=B) == 0, L,
                     rng.integers(0, L + 1 + (window or 1))).astype(np.int32)
    say(f"random decode seed={seed}: {'fp8' if fp8 else 'bf16'} seqlens={L.tolist()} "
        f"q_pos={q_pos.tolist()} Lmax={lmax} hq={hq} hkv={hkv} D={D} W={window} S={sinks}")
    th_dev, scale = lib_theta(D, cfg.base, cfg.factor, cfg.original_max_position)
    qp = torch.from_numpy(q_pos).cuda()
    sl = torch.from_numpy(L).cuda()
    if fp8:
        out, lse = ops.attn_decode_fp8(
            to_dev(inp["q"], "bf16"), torch.from_numpy(inp["k_cache"]).cuda(),
            torch.from_numpy(inp["v_cache"]).cuda(), torch.from_numpy(inp["k_scale"]).cuda(),
            torch.from_numpy(inp["v_scale"]).cuda(), sl, th_dev, scale, q_pos=qp,
            out_dtype=ops.YR_F32, window=window, sinks=sinks)
        kc, vc = (_LazyFP8(inp["k_cache"], inp["k_scale"]),
                  _LazyFP8(inp["v_cache"], inp["v_scale"]))
    else:
        out, lse = ops.attn_decode(to_dev(inp["q"], "bf16"), to_dev(inp["k_cache"], "bf16"),
                                   to_dev(inp["v_cache"], "bf16"), sl, th_dev, scale, q_pos=qp,
                                   out_dtype=ops.YR_F32, window=window, sinks=sinks)
        kc, vc = LazyF64(inp["k_cache"], "bf16"), LazyF64(inp["v_cache"], "bf16")
    torch.cuda.synchronize()
    th, sc = oracle_theta(D, cfg.base, cfg.factor, cfg.original_max_position)
    # a query that sees no cache row (placed past its window, no sinks before
    # it): out = 0, lse = -inf; the oracle's softmax over nothing is left out
    n = [np.arange(int(x)) for x in L]
    seen = np.array([window == 0 or bool(np.any((n[b] > int(q_pos[b]) - window) | (n[b] < sinks)))
                     for b in range(B)])
    got, gl = to_f64(out), lse.cpu().numpy().astype(np.float64)
    assert np.all(got[~seen] == 0.0) and np.all(np.isneginf(gl[~seen]))
    if not seen.any():
        return
    idx = np.flatnonzero(seen)
    ro, rl = oatt.decode(wl.as_f64(inp["q"], "bf16")[idx], _Rows(kc, idx), _Rows(vc, idx), L[idx],
                         th, sc, q_pos=q_pos[idx].tolist(), window=window, sinks=sinks)
    print(f"{len(idx)} of {B} queries see keys: max-abs out {_close(got[idx], ro):.3e} "
          f"lse {_close(gl[idx], rl):.3e}")
