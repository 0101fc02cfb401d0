"""Inputs whose element offsets pass 2^31, against the oracle: a packed
prefill batch whose queries and outputs hold 2.6e9 elements (the checked rows
all lie past element 2^31), the rotation of those queries in place, and
caches of 2^21 - 100 rows per sequence for decode and chunked prefill, so that
the second sequence's rows start 100 rows before element (FP8: byte) 2^31 and
run past it.  An offset computed in 32 bits anywhere on these paths reads or
writes the wrong rows.

To keep the host side short, the prefill queries are drawn only for the
checked tokens (every other query row is zero, which the kernel processes like
any other), and the caches only for each sequence's rows (the rest hold NaN,
which no visible result may touch)."""

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import fp8 as ofp8
from oracle import rope as orope
from tests._gpu_util import (BF16_TOL, LazyF64, lib_theta, max_abs, oracle_theta, say, to_dev,
                             to_f64)
from yarn_scaled_rope_amd import ops
from yarn_scaled_rope_amd import workloads as wl

pytestmark = pytest.mark.gpu

LMAX = (1 << 21) - 100        # cache rows per sequence: 1024-element rows
SEQLENS = (1500, 40000)       # the second sequence crosses element 2^31 at its row 100


@pytest.mark.timeout(400)
def test_prefill_offsets_past_2_to_31():
    lens = (65536, 65536, 30000)
    hq, hkv, D = 128, 8, 128
    T = sum(lens)
    assert T * hq * D > (1 << 31)
    rng = np.random.Generator(np.random.PCG64(4242))
    s2 = lens[0] + lens[1]           # first token of the third sequence
    assert s2 * hq * D >= (1 << 31)
    toks = sorted({lens[0] - 1, s2 - 1, 70000, s2, s2 + 1, s2 + 255, s2 + 256, s2 + 257,
                   T - 1, *(int(x) for x in rng.integers(s2, T, size=40))})
    cfg = wl.PrefillConfig("offsets", 31, lens, hq, hkv, D, "bf16", 500000.0, 8.0, 16384)
    inp = wl.make_prefill(cfg, q_tokens=toks)
    say(f"prefill past 2^31 elements: lens={lens} hq={hq} hkv={hkv} D={D}, {len(toks)} tokens "
        f"x {hq} heads checked")
    th_dev, scale = lib_theta(D, cfg.base, cfg.factor, cfg.original_max_position)
    out, lse = ops.attn_prefill_fwd(to_dev(inp["q"], "bf16"), to_dev(inp["k"], "bf16"),
                                    to_dev(inp["v"], "bf16"),
                                    torch.from_numpy(inp["cu_seqlens"]).cuda(), max(lens),
                                    th_dev, scale)
    torch.cuda.synchronize()
    tix = torch.tensor(toks, dtype=torch.long, device=out.device)
    got_o = to_f64(out.index_select(0, tix)).reshape(len(toks) * hq, D)
    got_l = lse.index_select(1, tix).t().contiguous().cpu().numpy().astype(np.float64).reshape(-1)
    del out, lse
    torch.cuda.empty_cache()
    rows = [(t, h) for t in toks for h in range(hq)]
    th, sc = oracle_theta(D, cfg.base, cfg.factor, cfg.original_max_position)
    ro, rl = oatt.prefill_rows(LazyF64(inp["q"], "bf16"), LazyF64(inp["k"], "bf16"),
                               LazyF64(inp["v"], "bf16"), inp["cu_seqlens"], th, sc, rows)
    e_out, e_lse = max_abs(got_o, ro), max_abs(got_l, rl)
    print(f"{len(rows)} (row, head) pairs, max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert np.all(np.isfinite(got_o))
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL

    # the same queries rotated in place by rope_apply_packed: each checked
    # element within one bf16 ulp of the exact rotation at its position
    say("rope_apply_packed in place past 2^31 elements")
    qd = to_dev(inp["q"], "bf16")
    ops.rope_apply_packed(qd, torch.from_numpy(inp["cu_seqlens"]).cuda(), max(lens), th_dev,
                          dst=qd)
    torch.cuda.synchronize()
    got = to_f64(qd.index_select(0, tix))
    del qd
    torch.cuda.empty_cache()
    starts = inp["cu_seqlens"][np.searchsorted(inp["cu_seqlens"], toks, side="right") - 1]
    ref = orope.rotate(wl.as_f64(inp["q"][toks], "bf16"), np.asarray(toks) - starts, th)
    mag = np.maximum(np.abs(ref), 1e-30)
    ulp = 2.0 ** (np.floor(np.log2(mag)) - 7)
    print(f"rotation max-abs {max_abs(got, ref):.3e}")
    assert np.all(np.abs(got - ref) <= ulp + 1e-6)


def _decode_cfg():
    return wl.DecodeConfig("offsets", 32, 0, 0, 0, 32, 8, 128, "bf16", 500000.0, 8.0, 16384)


@pytest.mark.timeout(400)
def test_decode_offsets_past_2_to_31():
    cfg = _decode_cfg()
    assert LMAX * cfg.hkv * cfg.head_dim < (1 << 31) <= (LMAX + 100) * cfg.hkv * cfg.head_dim
    inp = wl.make_decode(cfg, seed=4343, batch=2, max_cache_len=LMAX, seqlens=SEQLENS)
    th_dev, scale = lib_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    th, sc = oracle_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    q = to_dev(inp["q"], "bf16")
    kc = to_dev(inp["k_cache"], "bf16")
    vc = to_dev(inp["v_cache"], "bf16")
    sl = torch.from_numpy(inp["seqlens"]).cuda()
    for window, sinks in ((0, 0), (4096, 4)):
        say(f"decode past 2^31 elements: Lmax={LMAX} seqlens={SEQLENS} W={window} S={sinks}")
        out, lse = ops.attn_decode(q, kc, vc, sl, th_dev, scale, window=window, sinks=sinks)
        torch.cuda.synchronize()
        ro, rl = oatt.decode(wl.as_f64(inp["q"], "bf16"), LazyF64(inp["k_cache"], "bf16"),
                             LazyF64(inp["v_cache"], "bf16"), inp["seqlens"], th, sc,
                             window=window, sinks=sinks)
        got_o, got_l = to_f64(out), lse.cpu().numpy().astype(np.float64)
        e_out, e_lse = max_abs(got_o, ro), max_abs(got_l, rl)
        print(f"W={window}: max-abs out {e_out:.3e} lse {e_lse:.3e}")
        assert np.all(np.isfinite(got_o))
        assert e_out <= BF16_TOL and e_lse <= BF16_TOL


class _LazyFP8:
    """Exact values of an E4M3 cache [B, L, Hkv, D] with per-KV-head scales,
    decoded slice by slice."""

    def __init__(self, codes, scale):
        self.codes, self.scale = codes, np.asarray(scale, dtype=np.float64)
        self.shape = codes.shape

    def __getitem__(self, idx):
        b, rows, h, d = idx
        return ofp8.e4m3_to_f64(self.codes[b, rows, h, d]) * self.scale[h]


@pytest.mark.timeout(400)
def test_decode_fp8_offsets_past_2_to_31():
    cfg = _decode_cfg()
    inp = wl.make_decode_fp8(cfg, seed=4444, batch=2, max_cache_len=LMAX, seqlens=SEQLENS)
    say(f"FP8 decode past 2^31 bytes: Lmax={LMAX} seqlens={SEQLENS}")
    th_dev, scale = lib_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    out, lse = ops.attn_decode_fp8(
        to_dev(inp["q"], "bf16"), torch.from_numpy(inp["k_cache"]).cuda(),
        torch.from_numpy(inp["v_cache"]).cuda(), torch.from_numpy(inp["k_scale"]).cuda(),
        torch.from_numpy(inp["v_scale"]).cuda(), torch.from_numpy(inp["seqlens"]).cuda(),
        th_dev, scale, out_dtype=ops.YR_F32)
    torch.cuda.synchronize()
    th, sc = oracle_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    ro, rl = oatt.decode(wl.as_f64(inp["q"], "bf16"), _LazyFP8(inp["k_cache"], inp["k_scale"]),
                         _LazyFP8(inp["v_cache"], inp["v_scale"]), inp["seqlens"], th, sc)
    got_o, got_l = to_f64(out), lse.cpu().numpy().astype(np.float64)
    e_out, e_lse = max_abs(got_o, ro), max_abs(got_l, rl)
    print(f"max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert np.all(np.isfinite(got_o))
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


@pytest.mark.timeout(400)
def test_chunk_offsets_past_2_to_31():
    ctx, qlens = (1000, 30000), (300, 700)
    cfg = wl.ChunkConfig("offsets", 33, ctx, qlens, LMAX, 32, 8, 128, "bf16", 500000.0, 8.0,
                         16384)
    inp = wl.make_chunk(cfg, seed=4545)
    th_dev, scale = lib_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    th, sc = oracle_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    q = to_dev(inp["q"], "bf16")
    kc = to_dev(inp["k_cache"], "bf16")
    vc = to_dev(inp["v_cache"], "bf16")
    cu = torch.from_numpy(inp["cu_seqlens_q"]).cuda()
    cl = torch.from_numpy(inp["ctx_lens"]).cuda()
    for window, sinks in ((0, 0), (4096, 4)):
        say(f"chunked prefill past 2^31 elements: Lmax={LMAX} ctx={ctx} chunks={qlens} "
            f"W={window} S={sinks}")
        out, lse = ops.attn_prefill_chunk(q, kc, vc, cu, cl, max(qlens), th_dev, scale,
                                          window=window, sinks=sinks, out_dtype=ops.YR_F32)
        torch.cuda.synchronize()
        ro, rl = oatt.prefill_chunk(LazyF64(inp["q"], "bf16"), LazyF64(inp["k_cache"], "bf16"),
                                    LazyF64(inp["v_cache"], "bf16"), inp["cu_seqlens_q"],
                                    inp["ctx_lens"], th, sc, window=window, sinks=sinks)
        got_o, got_l = to_f64(out), lse.cpu().numpy().astype(np.float64)
        e_out, e_lse = max_abs(got_o, ro), max_abs(got_l, rl)
        print(f"W={window}: max-abs out {e_out:.3e} lse {e_lse:.3e}")
        assert np.all(np.isfinite(got_o))
        assert e_out <= BF16_TOL and e_lse <= BF16_TOL
