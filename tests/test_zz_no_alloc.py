"""attn_decode_noalloc (the library's fixed per-device scratch instead of a
workspace) against attn_decode, through the C ABI: two calls in a row, the
second on a smaller input, each bit-identical to attn_decode on the same
inputs and within the bf16 bound of the oracle."""

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from tests._gpu_util import BF16_TOL, F32_TOL, lib_theta, max_abs, oracle_theta, say, to_dev, to_f64
from yarn_scaled_rope_amd import ops
from yarn_scaled_rope_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _case(dtype, B, lmax, lmin, hq, hkv, seed, window=0, sinks=0):
    cfg = wl.DecodeConfig("t", 81, 0, 0, 0, hq, hkv, 128, dtype, 500000.0, 8.0, 16384)
    inp = wl.make_decode(cfg, seed=seed, batch=B, max_cache_len=lmax, min_cache_len=lmin)
    th_dev, scale = lib_theta(128, cfg.base, cfg.factor, cfg.original_max_position)
    dev = dict(q=to_dev(inp["q"], dtype), kc=to_dev(inp["k_cache"], dtype),
               vc=to_dev(inp["v_cache"], dtype), sl=torch.from_numpy(inp["seqlens"]).cuda())
    return cfg, inp, dev, th_dev, scale


@pytest.mark.parametrize("first,second", [
    # balanced split (>= 512K keys in all), then a short batch in chunks
    (("bf16", 8, 131072, 65536, 32, 8, 5, 0, 0), ("bf16", 3, 3000, 100, 32, 8, 6, 0, 0)),
    # windowed (shared form), then a smaller plain call
    (("bf16", 6, 20000, 9000, 16, 4, 7, 4096, 4), ("bf16", 2, 700, 1, 16, 4, 8, 0, 0)),
    # the fp32 path, then a smaller fp32 call
    (("f32", 4, 5000, 1000, 8, 2, 9, 0, 0), ("f32", 2, 300, 1, 8, 2, 10, 0, 0)),
])
def test_noalloc_matches_attn_decode_twice(first, second):
    for args in (first, second):
        dtype, B, lmax, lmin, hq, hkv, seed, window, sinks = args
        cfg, inp, d, th_dev, scale = _case(dtype, B, lmax, lmin, hq, hkv, seed, window, sinks)
        say(f"decode_noalloc {dtype} B={B} Lmax={lmax} hq={hq} hkv={hkv} W={window} "
            f"seqlens={list(inp['seqlens'])}")
        ref_o, ref_l = ops.attn_decode(d["q"], d["kc"], d["vc"], d["sl"], th_dev, scale,
                                       window=window, sinks=sinks)
        out = torch.full_like(d["q"], float("nan"))
        lse = torch.full((B, hq), float("nan"), dtype=torch.float32, device="cuda")
        err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        ops.attn_decode_noalloc(d["q"], d["kc"], d["vc"], d["sl"], th_dev, scale, out, lse=lse,
                                dev_error=err, window=window, sinks=sinks)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        th, sc = oracle_theta(128, cfg.base, cfg.factor, cfg.original_max_position)
        ro, rl = oatt.decode(wl.as_f64(inp["q"], dtype), wl.as_f64(inp["k_cache"], dtype),
                             wl.as_f64(inp["v_cache"], dtype), inp["seqlens"], th, sc,
                             window=window, sinks=sinks)
        tol = F32_TOL if dtype == "f32" else BF16_TOL
        e_out, e_lse = max_abs(to_f64(out), ro), max_abs(lse.cpu().numpy(), rl)
        print(f"noalloc vs oracle: out {e_out:.3e} lse {e_lse:.3e}")
        assert e_out <= tol and e_lse <= tol


def test_noalloc_flags_bad_seqlens_and_rejects_large_splits():
    cfg, inp, d, th_dev, scale = _case("bf16", 3, 1000, 10, 8, 2, 11)
    bad = torch.tensor([10, 2000, 5], dtype=torch.int32, device="cuda")   # 2000 > Lmax
    out = torch.empty_like(d["q"])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("decode_noalloc out-of-range seqlens")
    ops.attn_decode_noalloc(d["q"], d["kc"], d["vc"], bad, th_dev, scale, out, dev_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) == ops.YR_DEVERR_SEQLENS
    # a split larger than the fixed scratch (4096 sequences of at most 64
    # keys, 32 query heads: 131072 partial rows) is refused before anything is
    # read or launched, so the buffer pointers below are never dereferenced
    import ctypes
    lib = ops.load_library()
    p = ctypes.c_void_p(d["q"].data_ptr())
    st = lib.attn_decode_noalloc(p, p, p, ops.YR_BF16, ctypes.c_void_p(d["sl"].data_ptr()), None,
                                 4096, 64, 32, 8, 128, ctypes.c_void_p(th_dev.data_ptr()), scale,
                                 0, 0, p, ops.YR_BF16, None, None, None)
    assert st == ops.YR_ERR_WORKSPACE
    assert b"fixed" in lib.yr_last_error()
