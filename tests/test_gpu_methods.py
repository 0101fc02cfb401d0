"""The kernels with the other frequency rules ("Arch 03 -- Long Context":
plain RoPE, Position Interpolation, NTK-aware and Dynamic NTK slides) and
YaRN at s = 1, against the oracle with the same rule: prefill (bf16 and fp32
paths) and decode.  YaRN at s = 1 must give plain RoPE attention bit for bit
(equal tables, temperature 1)."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import freqs as ofreqs
from tests._gpu_util import BF16_TOL, F32_TOL, lib_theta, max_abs, oracle_theta, say, to_dev, to_f64
from yarn_scaled_rope_amd import ops
from yarn_scaled_rope_amd import workloads as wl

pytestmark = pytest.mark.gpu

RULES = [("plain", 1.0), ("pi", 4.0), ("ntk", 8.0), ("yarn", 1.0), ("yarn", 16.0)]


def _tables(rule, s, D, base, L):
    """(device table, scale) from the library; (table, scale) from the oracle."""
    if rule == "dynamic_ntk":
        _, f64, fac = ops.yarn_rope_dynamic_ntk_freqs(D, base, s, L)
        th = ofreqs.dynamic_ntk_theta(D, base, s, L)
        assert fac == ofreqs.dynamic_ntk_factor(s, L)
        return (torch.from_numpy(f64).cuda(), 1.0 / math.sqrt(D)), (th, 1.0 / math.sqrt(D))
    return lib_theta(D, base, s, L, rule), oracle_theta(D, base, s, L, rule)


@pytest.mark.parametrize("rule,s", RULES + [("dynamic_ntk", 3000)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_frequency_rules(rule, s, dtype):
    lens, hq, hkv, D, base, L = (300, 77, 1, 129), 8, 2, 128, 10000.0, 1024
    cfg = wl.PrefillConfig("t", 120, lens, hq, hkv, D, dtype, base, 1.0, L)
    inp = wl.make_prefill(cfg)
    (th_dev, scale), (th, sc) = _tables(rule, s, D, base, L)
    say(f"prefill {dtype} rule={rule} s={s}")
    out, lse = ops.attn_prefill_fwd(to_dev(inp["q"], dtype), to_dev(inp["k"], dtype),
                                    to_dev(inp["v"], dtype),
                                    torch.from_numpy(inp["cu_seqlens"]).cuda(), max(lens), th_dev,
                                    scale)
    torch.cuda.synchronize()
    ro, rl = oatt.prefill(wl.as_f64(inp["q"], dtype), wl.as_f64(inp["k"], dtype),
                          wl.as_f64(inp["v"], dtype), inp["cu_seqlens"], th, sc)
    tol = F32_TOL if dtype == "f32" else BF16_TOL
    e_out, e_lse = max_abs(to_f64(out), ro), max_abs(lse.cpu().numpy(), rl)
    print(f"{rule} s={s}: out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= tol and e_lse <= tol


@pytest.mark.parametrize("rule,s", RULES + [("dynamic_ntk", 100000)])
def test_decode_frequency_rules(rule, s):
    D, base, L = 128, 500000.0, 16384
    cfg = wl.DecodeConfig("t", 121, 0, 0, 0, 16, 4, D, "bf16", base, 1.0, L)
    inp = wl.make_decode(cfg, seed=121, batch=4, max_cache_len=3000, min_cache_len=1)
    (th_dev, scale), (th, sc) = _tables(rule, s, D, base, L)
    say(f"decode rule={rule} s={s} seqlens={list(inp['seqlens'])}")
    out, lse = ops.attn_decode(to_dev(inp["q"], "bf16"), to_dev(inp["k_cache"], "bf16"),
                               to_dev(inp["v_cache"], "bf16"),
                               torch.from_numpy(inp["seqlens"]).cuda(), th_dev, scale)
    torch.cuda.synchronize()
    ro, rl = oatt.decode(wl.as_f64(inp["q"], "bf16"), wl.as_f64(inp["k_cache"], "bf16"),
                         wl.as_f64(inp["v_cache"], "bf16"), inp["seqlens"], th, sc)
    e_out, e_lse = max_abs(to_f64(out), ro), max_abs(lse.cpu().numpy(), rl)
    print(f"{rule} s={s}: out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


def test_yarn_at_s1_is_plain_rope_attention_bitwise():
    lens, hq, hkv, D = (400, 33), 8, 2, 128
    cfg = wl.PrefillConfig("t", 122, lens, hq, hkv, D, "bf16", 500000.0, 1.0, 16384)
    inp = wl.make_prefill(cfg)
    q, k, v = (to_dev(inp[x], "bf16") for x in ("q", "k", "v"))
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    ty, sy = lib_theta(D, 500000.0, 1.0, 16384, "yarn")
    tp, sp = lib_theta(D, 500000.0, 1.0, 16384, "plain")
    assert torch.equal(ty, tp) and sy == sp
    say("prefill yarn s=1 vs plain")
    a = ops.attn_prefill_fwd(q, k, v, cu, 400, ty, sy)
    b = ops.attn_prefill_fwd(q, k, v, cu, 400, tp, sp)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
