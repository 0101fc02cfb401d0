"""Sliding-window / sink prefill and decode and chunked prefill (new tokens
against a cache) on the GPU against the oracle: full element-by-element
checks at sizes the oracle finishes in seconds (ragged sequences, 1-token
windows, windows longer than the sequence, sinks spanning more than one key
tile, NaN-poisoned cache tails), sampled rows of the 4 x 4K-chunk workload,
the full 16-sequence decode with a 4096-token window and 4 sinks, and the
cross-kernel identities (a chunk with no prefix equals packed prefill; the
last chunk row equals decode)."""

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from tests._gpu_util import (BF16_TOL, F32_TOL, LazyF64, lib_theta, max_abs, oracle_theta, say,
                             to_dev, to_f64)
from yarn_scaled_rope_amd import ops
from yarn_scaled_rope_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _tol(dtype):
    return F32_TOL if dtype == "f32" else BF16_TOL


# ------------------------------------------------------------ windowed prefill
@pytest.mark.parametrize("dtype,lens,hq,hkv,D,window,sinks", [
    ("bf16", (1, 300, 700), 8, 2, 128, 64, 0),
    ("bf16", (1, 300, 700), 8, 2, 128, 100, 4),
    ("bf16", (513, 1000), 4, 4, 64, 1, 0),
    ("bf16", (2000,), 8, 1, 128, 257, 70),     # sinks over more than one key tile
    ("bf16", (777,), 8, 2, 128, 5000, 3),      # window longer than the sequence
    # windows of several key tiles over long sequences: the rotated window
    # sweep puts the unmasked tiles in one run of the list for some q-tiles
    # and in two (wrapped) for others
    ("bf16", (3000, 1500), 4, 2, 64, 700, 4),
    ("bf16", (4100,), 8, 8, 128, 1500, 0),
    ("f32", (1, 130, 400), 4, 2, 64, 50, 2),
    ("f32", (300,), 2, 2, 128, 1, 0),
])
def test_prefill_window_full(dtype, lens, hq, hkv, D, window, sinks):
    cfg = wl.PrefillConfig("t", 81, lens, hq, hkv, D, dtype, 500000.0, 8.0, 64)
    inp = wl.make_prefill(cfg)
    say(f"windowed prefill {dtype} lens={lens} hq={hq} hkv={hkv} D={D} W={window} S={sinks}")
    th_dev, scale = lib_theta(D, cfg.base, cfg.factor, cfg.original_max_position)
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    out, lse = ops.attn_prefill_fwd(to_dev(inp["q"], dtype), to_dev(inp["k"], dtype),
                                    to_dev(inp["v"], dtype), cu, max(lens), th_dev, scale,
                                    out_dtype=ops.YR_F32, window=window, sinks=sinks)
    torch.cuda.synchronize()
    th, sc = oracle_theta(D, cfg.base, cfg.factor, cfg.original_max_position)
    ro, rl = oatt.prefill(wl.as_f64(inp["q"], dtype), wl.as_f64(inp["k"], dtype),
                          wl.as_f64(inp["v"], dtype), inp["cu_seqlens"], th, sc,
                          window=window, sinks=sinks)
    e_out, e_lse = max_abs(to_f64(out), ro), max_abs(lse.cpu().numpy(), rl)
    print(f"max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= _tol(dtype) and e_lse <= _tol(dtype)


def test_prefill_window_16k_sampled():
    cfg = wl.LLAMA2_7B_16K_SWA
    inp = wl.make_prefill(cfg)
    say(f"windowed prefill {cfg.name}, sampled rows")
    th_dev, scale = lib_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    out, lse = ops.attn_prefill_fwd(to_dev(inp["q"], "bf16"), to_dev(inp["k"], "bf16"),
                                    to_dev(inp["v"], "bf16"), cu, cfg.max_seqlen, th_dev, scale,
                                    out_dtype=ops.YR_F32, window=cfg.window, sinks=cfg.sinks)
    torch.cuda.synchronize()
    rows = wl.sample_rows(cfg.seq_lens, cfg.hq, cfg.hkv, n_random=24)
    # rows just past the window edge, where the sinks and the window part
    rows += [(r, h) for r in (cfg.window - 1, cfg.window, cfg.window + 1, cfg.window + 63)
             for h in (0, 17)]
    th, sc = oracle_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    ro, rl = oatt.prefill_rows(LazyF64(inp["q"], "bf16"), LazyF64(inp["k"], "bf16"),
                               LazyF64(inp["v"], "bf16"), inp["cu_seqlens"], th, sc, rows,
                               window=cfg.window, sinks=cfg.sinks)
    o = to_f64(out)
    l = lse.cpu().numpy()
    go = np.stack([o[t, h] for t, h in rows])
    gl = np.array([l[h, t] for t, h in rows])
    e_out, e_lse = max_abs(go, ro), max_abs(gl, rl)
    print(f"{len(rows)} rows: max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


# ------------------------------------------------------------ chunked prefill
def _chunk_run(inp, cfg, window=0, sinks=0, out_dtype=ops.YR_F32, ws=None):
    dt = inp["dtype"]
    th_dev, scale = lib_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    cu = torch.from_numpy(inp["cu_seqlens_q"]).cuda()
    ctx = torch.from_numpy(inp["ctx_lens"]).cuda()
    out, lse = ops.attn_prefill_chunk(to_dev(inp["q"], dt), to_dev(inp["k_cache"], dt),
                                      to_dev(inp["v_cache"], dt), cu, ctx, max(inp["chunk_lens"]),
                                      th_dev, scale, window=window, sinks=sinks,
                                      out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    return out, lse


def _chunk_oracle(inp, cfg, window=0, sinks=0, rows=None):
    dt = inp["dtype"]
    th, sc = oracle_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    return oatt.prefill_chunk(LazyF64(inp["q"], dt), LazyF64(inp["k_cache"], dt),
                              LazyF64(inp["v_cache"], dt), inp["cu_seqlens_q"], inp["ctx_lens"],
                              th, sc, window=window, sinks=sinks, rows=rows)


@pytest.mark.parametrize("dtype,ctx,qlens,lmax,hq,hkv,D,window,sinks,out_dtype", [
    ("bf16", (0, 300, 1000), (200, 65, 513), 2048, 8, 2, 128, 0, 0, ops.YR_BF16),
    ("bf16", (5, 700), (1, 300), 1024, 8, 8, 64, 0, 0, ops.YR_F32),
    ("bf16", (1500, 40), (400, 600), 2048, 8, 2, 128, 256, 4, ops.YR_BF16),
    ("bf16", (3000,), (257,), 4096, 16, 2, 128, 1000, 0, ops.YR_F32),
    ("f32", (0, 200), (130, 70), 512, 4, 2, 64, 0, 0, ops.YR_F32),
    ("f32", (333,), (129,), 512, 4, 1, 128, 100, 2, ops.YR_F32),
])
def test_chunk_full(dtype, ctx, qlens, lmax, hq, hkv, D, window, sinks, out_dtype):
    cfg = wl.ChunkConfig("t", 82, ctx, qlens, lmax, hq, hkv, D, dtype, 500000.0, 8.0, 16384)
    inp = wl.make_chunk(cfg)
    say(f"chunk {dtype} ctx={ctx} qlens={qlens} Lmax={lmax} hq={hq} hkv={hkv} D={D} "
        f"W={window} S={sinks}")
    out, lse = _chunk_run(inp, cfg, window, sinks, out_dtype)
    ro, rl = _chunk_oracle(inp, cfg, window, sinks)
    o = to_f64(out)
    assert np.all(np.isfinite(o))
    e_out, e_lse = max_abs(o, ro), max_abs(lse.cpu().numpy(), rl)
    print(f"max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= _tol(dtype) and e_lse <= _tol(dtype)


def test_chunk_workload_sampled():
    cfg = wl.CHUNK_4X4K
    inp = wl.make_chunk(cfg)
    say(f"chunk {cfg.name}, sampled rows")
    out, lse = _chunk_run(inp, cfg)
    rows = wl.sample_rows(cfg.chunk_lens, cfg.hq, cfg.hkv, n_random=12)
    ro, rl = _chunk_oracle(inp, cfg, rows=rows)
    o = to_f64(out)
    l = lse.cpu().numpy()
    go = np.stack([o[t, h] for t, h in rows])
    gl = np.array([l[h, t] for t, h in rows])
    e_out, e_lse = max_abs(go, ro), max_abs(gl, rl)
    print(f"{len(rows)} rows: max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


@pytest.mark.parametrize("window,sinks", [(0, 0), (300, 4)])
def test_chunk_without_prefix_equals_packed_prefill(window, sinks):
    """The same keys, once packed ([T, Hkv, D], pre-rotated) and once in a
    cache with ctx_lens = 0: the two entry points run the same tile schedule
    and must agree bit for bit."""
    lens, hq, hkv, D = (700, 129), 8, 2, 128
    pcfg = wl.PrefillConfig("t", 83, lens, hq, hkv, D, "bf16", 500000.0, 8.0, 16384)
    inp = wl.make_prefill(pcfg)
    say(f"chunk vs packed prefill lens={lens} W={window} S={sinks}")
    th_dev, scale = lib_theta(D, pcfg.base, pcfg.factor, pcfg.original_max_position)
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    q = to_dev(inp["q"], "bf16")
    kr = ops.rope_apply_packed(to_dev(inp["k"], "bf16"), cu, max(lens), th_dev)
    v = to_dev(inp["v"], "bf16")
    o1, l1 = ops.attn_prefill_fwd(q, kr, v, cu, max(lens), th_dev, scale, k_rotated=True,
                                  window=window, sinks=sinks)
    lmax = max(lens)
    kc = torch.zeros((len(lens), lmax, hkv, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for b, (s0, s1) in enumerate(zip(inp["cu_seqlens"][:-1], inp["cu_seqlens"][1:])):
        kc[b, :s1 - s0] = kr[s0:s1]
        vc[b, :s1 - s0] = v[s0:s1]
    ctx = torch.zeros(len(lens), dtype=torch.int32, device="cuda")
    o2, l2 = ops.attn_prefill_chunk(q, kc, vc, cu, ctx, max(lens), th_dev, scale, window=window,
                                    sinks=sinks)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("window,sinks", [(0, 0), (500, 4)])
def test_last_chunk_row_equals_decode(window, sinks):
    cfg = wl.ChunkConfig("t", 84, (1200, 37, 0), (300, 90, 64), 2048, 16, 2, 128, "bf16",
                         500000.0, 8.0, 16384)
    inp = wl.make_chunk(cfg)
    say(f"chunk last row vs decode W={window} S={sinks}")
    out, lse = _chunk_run(inp, cfg, window, sinks)
    th_dev, scale = lib_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    last = inp["cu_seqlens_q"][1:] - 1
    L = (inp["ctx_lens"] + np.asarray(inp["chunk_lens"])).astype(np.int32)
    qd = to_dev(inp["q"], "bf16")[torch.from_numpy(last.astype(np.int64)).cuda()].contiguous()
    do, dl = ops.attn_decode(qd, to_dev(inp["k_cache"], "bf16"), to_dev(inp["v_cache"], "bf16"),
                             torch.from_numpy(L).cuda(), th_dev, scale,
                             q_pos=torch.from_numpy(L - 1).cuda(), out_dtype=ops.YR_F32,
                             window=window, sinks=sinks)
    torch.cuda.synchronize()
    e_out = max_abs(to_f64(out)[last], to_f64(do))
    e_lse = max_abs(lse.cpu().numpy()[:, last].T, dl.cpu().numpy())
    print(f"max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


def test_chunk_bad_ctx_sets_flag():
    cfg = wl.ChunkConfig("t", 85, (10, 20), (30, 40), 128, 4, 2, 64, "bf16", 500000.0, 8.0, 16384)
    inp = wl.make_chunk(cfg)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    # a negative prefix (clamped to 0: rows that hold data), and a prefix that
    # pushes the chunk past the cache (clamped to Lmax - n: sequence 1 then
    # reads NaN padding, sequence 0 stays finite)
    for bad, finite_rows in (((-3, 20), 70), ((10, 100), 30)):
        inp2 = dict(inp, ctx_lens=np.asarray(bad, dtype=np.int32))
        say(f"chunk bad ctx {bad}")
        out, _ = _chunk_run(inp2, cfg, ws=ws)
        assert ops.read_device_error(ws) & ops.YR_DEVERR_CTX_LENS
        assert torch.isfinite(out[:finite_rows]).all()
    _chunk_run(inp, cfg, ws=ws)
    assert ops.read_device_error(ws) == 0


@pytest.mark.parametrize("window,sinks", [(0, 0), (100, 3)])
def test_chunk_with_empty_chunks(window, sinks):
    """Sequences with no new token (n_b = 0) among others: they produce
    nothing, the others match the oracle."""
    cfg = wl.ChunkConfig("t", 89, (500, 0, 40, 1000), (0, 130, 0, 7), 1200, 8, 2, 128, "bf16",
                         500000.0, 8.0, 16384)
    inp = wl.make_chunk(cfg)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    say(f"chunk with empty chunks ctx={cfg.ctx_lens} qlens={cfg.chunk_lens} W={window} S={sinks}")
    out, lse = _chunk_run(inp, cfg, window, sinks, ws=ws)
    assert ops.read_device_error(ws) == 0
    ro, rl = _chunk_oracle(inp, cfg, window, sinks)
    e_out, e_lse = max_abs(to_f64(out), ro), max_abs(lse.cpu().numpy(), rl)
    print(f"max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


def test_chunk_without_new_tokens():
    """Tq = 0: the call succeeds with empty q / out (NULL data pointers) and
    still checks ctx_lens on the device."""
    cfg = wl.ChunkConfig("t", 90, (10, 20), (0, 0), 64, 4, 2, 64, "bf16", 500000.0, 8.0, 16384)
    inp = wl.make_chunk(cfg)
    th_dev, scale = lib_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    q = torch.empty((0, cfg.hq, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    kc, vc = to_dev(inp["k_cache"], "bf16"), to_dev(inp["v_cache"], "bf16")
    cu = torch.zeros(3, dtype=torch.int32, device="cuda")
    say("chunk with no new tokens")
    for ctx, flagged in (((10, 20), 0), ((10, 65), ops.YR_DEVERR_CTX_LENS)):
        cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
        out, lse = ops.attn_prefill_chunk(q, kc, vc, cu, cl, 1, th_dev, scale, workspace=ws)
        assert tuple(out.shape) == (0, cfg.hq, cfg.head_dim) and tuple(lse.shape) == (cfg.hq, 0)
        assert ops.read_device_error(ws) == flagged


# ------------------------------------------------------------ windowed decode
def _decode_run(inp, cfg, window, sinks, q_pos=None, out_dtype=ops.YR_F32):
    dt = inp["dtype"]
    th_dev, scale = lib_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    qp = None if q_pos is None else torch.from_numpy(np.asarray(q_pos, dtype=np.int32)).cuda()
    out, lse = ops.attn_decode(to_dev(inp["q"], dt), to_dev(inp["k_cache"], dt),
                               to_dev(inp["v_cache"], dt), torch.from_numpy(inp["seqlens"]).cuda(),
                               th_dev, scale, q_pos=qp, out_dtype=out_dtype, window=window,
                               sinks=sinks)
    torch.cuda.synchronize()
    return to_f64(out), lse.cpu().numpy().astype(np.float64)


def _decode_oracle(inp, cfg, window, sinks, q_pos=None):
    th, sc = oracle_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    dt = inp["dtype"]
    return oatt.decode(wl.as_f64(inp["q"], dt), LazyF64(inp["k_cache"], dt),
                       LazyF64(inp["v_cache"], dt), inp["seqlens"], th, sc, q_pos=q_pos,
                       window=window, sinks=sinks)


@pytest.mark.parametrize("dtype,B,lmax,lmin,hq,hkv,D,window,sinks", [
    ("bf16", 5, 3000, 1, 8, 2, 128, 2, 0),
    ("bf16", 5, 3000, 1, 8, 2, 128, 700, 4),
    ("bf16", 4, 5000, 2500, 32, 8, 128, 2100, 40),   # window across chunk edges
    ("bf16", 3, 900, 1, 16, 1, 64, 64, 1),
    ("bf16", 5, 3000, 1, 8, 2, 128, 5000, 2),  # window past the cache: chunks over [0, L)
    ("f32", 4, 3000, 1, 8, 2, 128, 500, 3),
    ("f32", 3, 257, 1, 4, 1, 64, 2, 0),
])
def test_decode_window_full(dtype, B, lmax, lmin, hq, hkv, D, window, sinks):
    cfg = wl.DecodeConfig("t", 86, 0, 0, 0, hq, hkv, D, dtype, 500000.0, 8.0, 16384)
    inp = wl.make_decode(cfg, seed=86 + B, batch=B, max_cache_len=lmax, min_cache_len=lmin)
    say(f"windowed decode {dtype} B={B} seqlens={list(inp['seqlens'])} hq={hq} hkv={hkv} D={D} "
        f"W={window} S={sinks}")
    out, lse = _decode_run(inp, cfg, window, sinks)
    ro, rl = _decode_oracle(inp, cfg, window, sinks)
    assert np.all(np.isfinite(out))
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    print(f"max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= _tol(dtype) and e_lse <= _tol(dtype)


def test_decode_window_q_pos_and_empty():
    """Queries placed by q_pos: inside the cache, and past every visible row
    (no sinks): the latter give out = 0 and lse = -inf."""
    cfg = wl.DecodeConfig("t", 87, 0, 0, 0, 8, 2, 128, "bf16", 500000.0, 8.0, 16384)
    inp = wl.make_decode(cfg, seed=87, batch=3, max_cache_len=2000, min_cache_len=1500)
    L = inp["seqlens"]
    q_pos = np.array([L[0] - 1, L[1] // 2, L[2] + 5000], dtype=np.int32)
    say(f"windowed decode q_pos={list(q_pos)} seqlens={list(L)}")
    out, lse = _decode_run(inp, cfg, 300, 0, q_pos=q_pos)
    ro, rl = _decode_oracle(inp, cfg, 300, 0, q_pos=q_pos[:2].tolist() + [0])
    assert max_abs(out[:2], ro[:2]) <= BF16_TOL and max_abs(lse[:2], rl[:2]) <= BF16_TOL
    assert np.all(out[2] == 0.0) and np.all(np.isneginf(lse[2]))


def test_decode_window_q_pos_sinks():
    """Queries placed well inside the cache with sinks: the visible rows run
    past the usual window length, so the last chunk of the visible rows takes
    the long tail."""
    cfg = wl.DecodeConfig("t", 88, 0, 0, 0, 8, 2, 128, "bf16", 500000.0, 8.0, 16384)
    inp = wl.make_decode(cfg, seed=88, batch=3, max_cache_len=4000, min_cache_len=3000)
    L = inp["seqlens"]
    q_pos = np.array([L[0] // 3, 10, L[2] - 1], dtype=np.int32)
    say(f"windowed decode q_pos={list(q_pos)} seqlens={list(L)} W=256 S=7")
    out, lse = _decode_run(inp, cfg, 256, 7, q_pos=q_pos)
    ro, rl = _decode_oracle(inp, cfg, 256, 7, q_pos=q_pos.tolist())
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    print(f"max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


def test_decode_window_workload_full():
    cfg = wl.DECODE_B16_SWA
    inp = wl.make_decode(wl.DECODE_B16)    # the decode workload's inputs, windowed
    say(f"windowed decode {cfg.name} full, seqlens={list(inp['seqlens'])}")
    out, lse = _decode_run(inp, cfg, cfg.window, cfg.sinks, out_dtype=ops.YR_BF16)
    ro, rl = _decode_oracle(inp, cfg, cfg.window, cfg.sinks)
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    print(f"{cfg.name}: max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL
