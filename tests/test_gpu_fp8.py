"""attn_decode_fp8 (E4M3 cache, per-KV-head scales) on the GPU against the
oracle over the exactly decoded cache: small caches in full (head_dim 64 and
128, 1 to 32 query heads per KV head, windows with sinks, NaN codes past every
sequence), four cache-length-128K sequences of the decode workload's shape, the
balanced split over short and full caches, and the cross-check with the bf16 decode over the same values (exact in
bf16)."""

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import fp8 as ofp8
from tests._gpu_util import BF16_TOL, lib_theta, max_abs, oracle_theta, say, to_dev, to_f64
from yarn_scaled_rope_amd import ops
from yarn_scaled_rope_amd import workloads as wl

pytestmark = pytest.mark.gpu


class LazyFP8:
    """Index-on-demand exact values of an E4M3 cache [B, L, Hkv, D] with
    per-KV-head scales (the oracle only slices it)."""

    def __init__(self, codes, scale):
        self.codes, self.scale = codes, np.asarray(scale, dtype=np.float64)
        self.shape = codes.shape

    def __getitem__(self, idx):
        b, rows, h, d = idx
        return ofp8.e4m3_to_f64(self.codes[b, rows, h, d]) * self.scale[h]


def _run(inp, cfg, window=0, sinks=0, out_dtype=ops.YR_F32):
    th_dev, scale = lib_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    out, lse = ops.attn_decode_fp8(
        to_dev(inp["q"], "bf16"), torch.from_numpy(inp["k_cache"]).cuda(),
        torch.from_numpy(inp["v_cache"]).cuda(), torch.from_numpy(inp["k_scale"]).cuda(),
        torch.from_numpy(inp["v_scale"]).cuda(), torch.from_numpy(inp["seqlens"]).cuda(),
        th_dev, scale, out_dtype=out_dtype, window=window, sinks=sinks)
    torch.cuda.synchronize()
    return to_f64(out), lse.cpu().numpy().astype(np.float64)


def _oracle(inp, cfg, window=0, sinks=0):
    th, sc = oracle_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    return oatt.decode(wl.as_f64(inp["q"], "bf16"), LazyFP8(inp["k_cache"], inp["k_scale"]),
                       LazyFP8(inp["v_cache"], inp["v_scale"]), inp["seqlens"], th, sc,
                       window=window, sinks=sinks)


def _cfg(hq, hkv, D):
    return wl.DecodeConfig("t", 91, 0, 0, 0, hq, hkv, D, "bf16", 500000.0, 8.0, 16384)


@pytest.mark.parametrize("B,lmax,lmin,hq,hkv,D,window,sinks", [
    (5, 300, 1, 8, 2, 128, 0, 0),
    (3, 5000, 1000, 32, 8, 128, 0, 0),
    (4, 2100, 1, 4, 4, 64, 0, 0),
    (2, 4500, 2000, 32, 1, 128, 0, 0),
    (6, 70, 1, 16, 1, 64, 0, 0),
    (4, 5000, 2500, 32, 8, 128, 2100, 40),
    (3, 3000, 100, 8, 2, 64, 300, 4),
])
def test_decode_fp8_small_full(B, lmax, lmin, hq, hkv, D, window, sinks):
    cfg = _cfg(hq, hkv, D)
    inp = wl.make_decode_fp8(cfg, seed=91 + B + D, batch=B, max_cache_len=lmax, min_cache_len=lmin)
    say(f"fp8 decode B={B} seqlens={list(inp['seqlens'])} hq={hq} hkv={hkv} D={D} "
        f"W={window} S={sinks}")
    out, lse = _run(inp, cfg, window, sinks)
    ro, rl = _oracle(inp, cfg, window, sinks)
    assert np.all(np.isfinite(out))
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    print(f"max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


def test_decode_fp8_long_caches():
    cfg = wl.DecodeConfig("t", 92, 4, 131072, 100000, 32, 8, 128, "bf16", 500000.0, 8.0, 16384)
    inp = wl.make_decode_fp8(cfg)
    say(f"fp8 decode 4 long caches, seqlens={list(inp['seqlens'])}")
    out, lse = _run(inp, cfg, out_dtype=ops.YR_BF16)
    ro, rl = _oracle(inp, cfg)
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    print(f"max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


@pytest.mark.parametrize("hq,hkv,D,window,sinks", [(32, 8, 128, 0, 0), (16, 4, 64, 0, 0),
                                                  (32, 8, 64, 0, 0), (32, 8, 128, 3000, 4),
                                                  (32, 8, 128, 60000, 4)])
def test_decode_fp8_balanced_split(hq, hkv, D, window, sinks):
    """Caches of >= 512K keys in all take the balanced split (head-per-wave
    form, one workgroup per CU): very short, full and odd lengths."""
    B, lmax = 10, 60000
    cfg = _cfg(hq, hkv, D)
    inp = wl.make_decode_fp8(cfg, seed=95 + D, batch=B, max_cache_len=lmax, min_cache_len=lmax)
    lens = np.array([1, 31, 32, 33, lmax, lmax - 1, 1000, 20000, 7, 45001], dtype=np.int32)
    for name in ("k_cache", "v_cache"):
        for b in range(B):
            inp[name][b, lens[b]:] = wl.E4M3_NAN_CODE
    inp["seqlens"] = lens
    say(f"fp8 decode balanced split hq={hq} hkv={hkv} D={D} W={window} S={sinks} "
        f"seqlens={lens.tolist()}")
    out, lse = _run(inp, cfg, window, sinks)
    ro, rl = _oracle(inp, cfg, window, sinks)
    assert np.all(np.isfinite(out))
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    print(f"max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


def test_decode_fp8_matches_bf16_decode_of_the_same_values():
    cfg = _cfg(16, 4, 128)
    inp = wl.make_decode_fp8(cfg, seed=93, batch=4, max_cache_len=6000, min_cache_len=3000)
    say(f"fp8 vs bf16 decode, seqlens={list(inp['seqlens'])}")
    out8, lse8 = _run(inp, cfg)
    # the same cache values in bf16 (code * scale has at most 8 significant bits)
    kv = [ofp8.dequantize_cache(inp[c], inp[s]).astype(np.float32)
          for c, s in (("k_cache", "k_scale"), ("v_cache", "v_scale"))]
    bits = [wl.round_to_bf16_bits(np.nan_to_num(x, nan=0.0)) for x in kv]
    assert all(np.array_equal(wl.bf16_bits_to_f32(b), np.nan_to_num(x, nan=0.0))
               for b, x in zip(bits, kv))
    th_dev, scale = lib_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    o16, l16 = ops.attn_decode(to_dev(inp["q"], "bf16"), to_dev(bits[0], "bf16"),
                               to_dev(bits[1], "bf16"), torch.from_numpy(inp["seqlens"]).cuda(),
                               th_dev, scale, out_dtype=ops.YR_F32)
    torch.cuda.synchronize()
    e_out = max_abs(out8, to_f64(o16))
    e_lse = max_abs(lse8, l16.cpu().numpy())
    print(f"fp8 vs bf16: max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= 2e-3 and e_lse <= 2e-3
