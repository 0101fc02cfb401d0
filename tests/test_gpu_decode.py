"""attn_decode on the GPU against the oracle: small caches in full, the full
16-sequence 32K-128K workload in full, NaN-poisoned cache tails, the
decode/prefill cross-check, bad seqlens, and determinism."""

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from tests._gpu_util import (BF16_TOL, F32_TOL, LazyF64, lib_theta, max_abs, oracle_theta, say,
                             to_dev, to_f64)
from yarn_scaled_rope_amd import ops
from yarn_scaled_rope_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _run(inp, cfg, out_dtype=None, q_pos=None):
    dt = inp["dtype"]
    th_dev, scale = lib_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    q = to_dev(inp["q"], dt)
    kc = to_dev(inp["k_cache"], dt)
    vc = to_dev(inp["v_cache"], dt)
    sl = torch.from_numpy(inp["seqlens"]).cuda()
    qp = None if q_pos is None else torch.from_numpy(np.asarray(q_pos, dtype=np.int32)).cuda()
    out, lse = ops.attn_decode(q, kc, vc, sl, th_dev, scale, q_pos=qp, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to_f64(out), lse.cpu().numpy().astype(np.float64)


def _oracle(inp, cfg, q_pos=None):
    th, scale = oracle_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    dt = inp["dtype"]
    return oatt.decode(wl.as_f64(inp["q"], dt), LazyF64(inp["k_cache"], dt),
                       LazyF64(inp["v_cache"], dt), inp["seqlens"], th, scale, q_pos=q_pos)


def _cfg(dtype, hq, hkv, D):
    return wl.DecodeConfig("t", 80, 0, 0, 0, hq, hkv, D, dtype, 500000.0, 8.0, 16384)


@pytest.mark.parametrize("dtype,B,lmax,lmin,hq,hkv,D,out_dtype", [
    ("bf16", 5, 300, 1, 8, 2, 128, ops.YR_BF16),
    ("bf16", 3, 5000, 1000, 32, 8, 128, ops.YR_F32),
    ("bf16", 4, 2100, 1, 4, 4, 64, ops.YR_BF16),
    ("bf16", 2, 700, 600, 16, 2, 128, ops.YR_BF16),
    ("bf16", 6, 70, 1, 16, 1, 64, ops.YR_F32),
    ("bf16", 3, 1100, 1, 2, 2, 128, ops.YR_F32),
    ("bf16", 2, 4500, 2000, 32, 1, 128, ops.YR_BF16),
    ("f32", 4, 3000, 1, 8, 2, 128, ops.YR_F32),
    ("f32", 3, 257, 1, 4, 1, 64, ops.YR_F32),
])
def test_decode_small_full(dtype, B, lmax, lmin, hq, hkv, D, out_dtype):
    cfg = _cfg(dtype, hq, hkv, D)
    inp = wl.make_decode(cfg, seed=90 + B, batch=B, max_cache_len=lmax, min_cache_len=lmin)
    say(f"decode {dtype} B={B} Lmax={lmax} hq={hq} hkv={hkv} D={D} seqlens={list(inp['seqlens'])}")
    out, lse = _run(inp, cfg, out_dtype=out_dtype)
    ro, rl = _oracle(inp, cfg)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    tol = F32_TOL if dtype == "f32" else BF16_TOL
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    print(f"max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= tol and e_lse <= tol


def test_decode_workload_full():
    cfg = wl.DECODE_B16
    inp = wl.make_decode(cfg)
    say(f"decode {cfg.name} full, seqlens={list(inp['seqlens'])}")
    out, lse = _run(inp, cfg)
    ro, rl = _oracle(inp, cfg)
    assert np.all(np.isfinite(out))
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    print(f"{cfg.name}: max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


@pytest.mark.parametrize("hq,hkv,D,use_qpos", [
    (32, 8, 128, False),
    (48, 12, 128, True),
    (16, 4, 64, False),
    (32, 8, 64, True),   # eight KV heads per workgroup
])
def test_decode_balanced_split(hq, hkv, D, use_qpos):
    """Caches of >= 512K keys in all take the balanced split over one
    workgroup per CU (head-per-wave form, four or eight KV heads per
    workgroup):
    lengths of 1, 31, 32, 33 keys beside full and odd ones, so that pieces
    start and end inside sequences and some sequences fit inside one piece."""
    B, lmax = 10, 60000
    cfg = _cfg("bf16", hq, hkv, D)
    inp = wl.make_decode(cfg, seed=77 + hkv, batch=B, max_cache_len=lmax, min_cache_len=lmax)
    lens = np.array([1, 31, 32, 33, lmax, lmax - 1, 1000, 20000, 7, 45001], dtype=np.int32)
    for name in ("k_cache", "v_cache"):
        for b in range(B):
            inp[name][b, lens[b]:] = wl.BF16_NAN_BITS
    inp["seqlens"] = lens
    q_pos = None
    if use_qpos:
        q_pos = [int(x) for x in np.maximum(lens // 2, 0)]
    say(f"decode balanced split hq={hq} hkv={hkv} D={D} seqlens={lens.tolist()} q_pos={q_pos}")
    out, lse = _run(inp, cfg, out_dtype=ops.YR_F32, q_pos=q_pos)
    ro, rl = _oracle(inp, cfg, q_pos=q_pos)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    print(f"max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


@pytest.mark.parametrize("B,lmax,hq,hkv,window,sinks", [
    (300, 2048, 32, 8, 0, 0),      # two head groups per sequence
    (1024, 600, 16, 4, 0, 0),      # one head group, many short sequences
    (140, 4096, 32, 8, 4000, 4),   # windows that reach 512K visible keys in all
])
def test_decode_balanced_split_large_batch(B, lmax, hq, hkv, window, sinks):
    """Batches of hundreds of sequences take the balanced split too (each
    workgroup finds its first piece from chunk sums over its threads, the
    merge its pieces the same way): lengths from 1 key up, with 1, 31, 32
    and 33 among them, against the oracle in full."""
    cfg = _cfg("bf16", hq, hkv, 128)
    # every cache row drawn, then lengths of 1 .. lmax (rows past them NaN)
    inp = wl.make_decode(cfg, seed=83 + B, batch=B, max_cache_len=lmax, min_cache_len=lmax)
    lens = np.random.Generator(np.random.PCG64(84 + B)).integers(
        1, lmax, size=B, endpoint=True).astype(np.int32)
    lens[:4] = [1, 31, 32, 33]
    lens[4] = lmax
    for name in ("k_cache", "v_cache"):
        for b in range(B):
            inp[name][b, lens[b]:] = wl.BF16_NAN_BITS
    inp["seqlens"] = lens
    say(f"decode balanced split B={B} lmax={lmax} hq={hq} hkv={hkv} window={window} "
        f"sum(L)={int(lens.sum())}")
    th_dev, scale = lib_theta(128, cfg.base, cfg.factor, cfg.original_max_position)
    out, lse = ops.attn_decode(to_dev(inp["q"], "bf16"), to_dev(inp["k_cache"], "bf16"),
                               to_dev(inp["v_cache"], "bf16"), torch.from_numpy(lens).cuda(),
                               th_dev, scale, out_dtype=ops.YR_F32, window=window, sinks=sinks)
    torch.cuda.synchronize()
    th, sc = oracle_theta(128, cfg.base, cfg.factor, cfg.original_max_position)
    ro, rl = oatt.decode(wl.as_f64(inp["q"], "bf16"), LazyF64(inp["k_cache"], "bf16"),
                         LazyF64(inp["v_cache"], "bf16"), lens, th, sc, window=window,
                         sinks=sinks)
    got, gl = to_f64(out), lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(gl))
    e_out, e_lse = max_abs(got, ro), max_abs(gl, rl)
    print(f"max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


@pytest.mark.parametrize("window,sinks,lmax", [(4096, 4, 60000), (100, 0, 60000), (1, 3, 60000),
                                               (60000, 4, 70000), (70000, 2, 60000)])
def test_decode_balanced_split_window(window, sinks, lmax):
    """Windows and sinks on large caches: short windows take the shared form
    in chunks; windows whose visible rows reach 512K keys in all take the
    balanced split, where a sequence contributes its visible rows only, sinks
    first; query positions at, inside and past the cache."""
    B, hq, hkv, D = 10, 32, 8, 128
    cfg = _cfg("bf16", hq, hkv, D)
    inp = wl.make_decode(cfg, seed=79, batch=B, max_cache_len=lmax, min_cache_len=lmax)
    lens = np.array([1, 31, 32, 33, lmax, lmax - 1, 1000, 20000, 7, 45001], dtype=np.int32)
    for name in ("k_cache", "v_cache"):
        for b in range(B):
            inp[name][b, lens[b]:] = wl.BF16_NAN_BITS
    inp["seqlens"] = lens
    q_pos = [int(L) if b % 3 == 0 else int(L) // 2 if b % 3 == 1 else int(L) + 50
             for b, L in enumerate(lens)]
    say(f"decode balanced split window={window} sinks={sinks} seqlens={lens.tolist()} "
        f"q_pos={q_pos}")
    th_dev, scale = lib_theta(D, cfg.base, cfg.factor, cfg.original_max_position)
    out, lse = ops.attn_decode(to_dev(inp["q"], "bf16"), to_dev(inp["k_cache"], "bf16"),
                               to_dev(inp["v_cache"], "bf16"),
                               torch.from_numpy(lens).cuda(), th_dev, scale,
                               q_pos=torch.tensor(q_pos, dtype=torch.int32, device="cuda"),
                               out_dtype=ops.YR_F32, window=window, sinks=sinks)
    torch.cuda.synchronize()
    got, gl = to_f64(out), lse.cpu().numpy().astype(np.float64)
    # queries that see no row (past the window, no sinks before it): 0 / -inf
    seen = np.array([window == 0 or bool(np.any((np.arange(L) > q - window) | (np.arange(L) < sinks)))
                     for L, q in zip(lens.tolist(), q_pos)])
    assert np.all(got[~seen] == 0.0) and np.all(np.isneginf(gl[~seen]))
    idx = np.flatnonzero(seen)
    th, sc = oracle_theta(D, cfg.base, cfg.factor, cfg.original_max_position)
    ro, rl = oatt.decode(wl.as_f64(inp["q"], "bf16")[idx], _Rows(LazyF64(inp["k_cache"], "bf16"), idx),
                         _Rows(LazyF64(inp["v_cache"], "bf16"), idx), lens[idx], th, sc,
                         q_pos=[q_pos[i] for i in idx], window=window, sinks=sinks)
    e_out, e_lse = max_abs(got[idx], ro), max_abs(gl[idx], rl)
    print(f"{len(idx)} of {B} see rows: max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


class _Rows:
    """The caches of the sequences in idx only (the oracle slices [b, :L, h, :])."""

    def __init__(self, cache, idx):
        self.cache, self.idx = cache, idx
        self.shape = (len(idx),) + tuple(cache.shape[1:])

    def __getitem__(self, key):
        b, rows, h, d = key
        return self.cache[int(self.idx[b]), rows, h, d]


def test_decode_matches_prefill_last_row():
    """Decode at q_pos = L-1 over the keys rotated by rope_apply equals row
    L-1 of prefill over the same unrotated inputs."""
    L, hq, hkv, D = 1500, 8, 2, 128
    cfg = wl.PrefillConfig("t", 81, (L,), hq, hkv, D, "bf16", 500000.0, 8.0, 64)
    inp = wl.make_prefill(cfg)
    th_dev, scale = lib_theta(D, cfg.base, cfg.factor, cfg.original_max_position)
    q, k, v = to_dev(inp["q"], "bf16"), to_dev(inp["k"], "bf16"), to_dev(inp["v"], "bf16")
    say("decode vs prefill last row")
    pout, plse = ops.attn_prefill_fwd(q, k, v, torch.from_numpy(inp["cu_seqlens"]).cuda(), L,
                                      th_dev, scale, out_dtype=ops.YR_F32)
    kr = k.clone()
    ops.rope_apply(kr, torch.arange(L, dtype=torch.int32, device="cuda"), th_dev)
    dout, dlse = ops.attn_decode(q[L - 1:L].contiguous(), kr[None].contiguous(), v[None].contiguous(),
                                 torch.tensor([L], dtype=torch.int32, device="cuda"), th_dev, scale,
                                 q_pos=torch.tensor([L - 1], dtype=torch.int32, device="cuda"),
                                 out_dtype=ops.YR_F32)
    torch.cuda.synchronize()
    # both sides round q~ and k~ to bf16 identically; they differ only in how
    # P is rounded (prefill feeds bf16 P to the matrix cores) and summed
    assert max_abs(to_f64(dout[0]), to_f64(pout[L - 1])) <= BF16_TOL
    assert max_abs(dlse[0].cpu().numpy(), plse[:, L - 1].cpu().numpy()) <= 1e-3


def test_decode_bad_seqlens_sets_flag():
    B, lmax, hq, hkv, D = 3, 512, 8, 2, 128
    th_dev, scale = lib_theta(D, 500000.0, 8.0, 16384)
    q = torch.randn(B, hq, D, device="cuda").to(torch.bfloat16)
    kc = torch.randn(B, lmax, hkv, D, device="cuda").to(torch.bfloat16)
    vc = torch.randn(B, lmax, hkv, D, device="cuda").to(torch.bfloat16)
    ws = torch.empty(ops.attn_decode_workspace_bytes(B, lmax, hq, D), dtype=torch.uint8,
                     device="cuda")
    for sl, bit in (([5, 512, 1], 0), ([0, 10, 10], ops.YR_DEVERR_SEQLENS),
                    ([5, 513, 7], ops.YR_DEVERR_SEQLENS), ([5, -3, 7], ops.YR_DEVERR_SEQLENS)):
        say(f"decode device flag seqlens={sl}")
        out, _ = ops.attn_decode(q, kc, vc, torch.tensor(sl, dtype=torch.int32, device="cuda"),
                                 th_dev, scale, workspace=ws)
        assert ops.read_device_error(ws) == bit
    say("decode device flag q_pos<0")
    ops.attn_decode(q, kc, vc, torch.tensor([5, 6, 7], dtype=torch.int32, device="cuda"), th_dev,
                    scale, q_pos=torch.tensor([1, -1, 2], dtype=torch.int32, device="cuda"),
                    workspace=ws)
    assert ops.read_device_error(ws) == ops.YR_DEVERR_QPOS


def test_decode_deterministic():
    cfg = _cfg("bf16", 32, 8, 128)
    inp = wl.make_decode(cfg, seed=5, batch=4, max_cache_len=9000, min_cache_len=3000)
    say("decode determinism")
    a = _run(inp, cfg)
    b = _run(inp, cfg)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
