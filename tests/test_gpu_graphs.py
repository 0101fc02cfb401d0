"""The entry points captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: the library only launches kernels on the caller's stream (no
allocation, memset or synchronisation), so a captured call must give the
same bits as the same call made eagerly.  Each test captures once, then
replays several times with new inputs written eagerly between the replays,
and compares every replay with an eager call on the same inputs."""

import numpy as np
import pytest
import torch

from tests._gpu_util import lib_theta, say, to_dev
from yarn_scaled_rope_amd import ops
from yarn_scaled_rope_amd import workloads as wl

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(fn):
    """Warm up on a side stream (the pattern torch documents for capture),
    then capture fn() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("k_rotated,window,sinks", [(False, 0, 0), (True, 0, 0), (False, 300, 4)])
def test_prefill_graph_replays_match_eager(k_rotated, window, sinks):
    lens = (700, 129, 1)
    hq, hkv, D = 8, 2, 128
    cfg = wl.PrefillConfig("graph", 41, lens, hq, hkv, D, "bf16", 500000.0, 8.0, 16384)
    inputs = [wl.make_prefill(cfg, seed=900 + r) for r in range(REPLAYS + 1)]
    th_dev, scale = lib_theta(D, cfg.base, cfg.factor, cfg.original_max_position)
    T = sum(lens)
    cu = torch.from_numpy(inputs[0]["cu_seqlens"]).cuda()
    q, k, v = (to_dev(inputs[0][n], "bf16") for n in ("q", "k", "v"))
    out = torch.empty_like(q)
    lse = torch.empty((hq, T), dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.attn_prefill_workspace_bytes(T, hkv, D, ops.YR_BF16), dtype=torch.uint8,
                     device="cuda")
    say(f"prefill graph capture k_rotated={k_rotated} W={window} S={sinks}")

    def call():
        ops.attn_prefill_fwd(q, k, v, cu, max(lens), th_dev, scale, out=out, lse=lse,
                             workspace=ws, k_rotated=k_rotated, window=window, sinks=sinks)

    g = _capture(call)
    for r in range(1, REPLAYS + 1):
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            t.copy_(to_dev(inputs[r][n], "bf16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        ref_o, ref_l = ops.attn_prefill_fwd(q, k, v, cu, max(lens), th_dev, scale,
                                            k_rotated=k_rotated, window=window, sinks=sinks)
        torch.cuda.synchronize()
        assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l), f"replay {r}"
        assert not torch.equal(got_o, out.new_zeros(out.shape))


@pytest.mark.parametrize("B,lmax,lmin,window,sinks,noalloc", [
    (8, 131072, 65536, 0, 0, False),   # balanced split + merge
    (5, 3000, 100, 0, 0, False),       # chunks + merge
    (6, 20000, 9000, 4096, 4, False),  # windowed (shared form)
    (8, 131072, 65536, 0, 0, True),    # the entry point that allocates nothing
])
def test_decode_graph_replays_match_eager(B, lmax, lmin, window, sinks, noalloc):
    hq, hkv, D = 32, 8, 128
    cfg = wl.DecodeConfig("graph", 42, 0, 0, 0, hq, hkv, D, "bf16", 500000.0, 8.0, 16384)
    inp = wl.make_decode(cfg, seed=950, batch=B, max_cache_len=lmax, min_cache_len=lmin)
    rng = np.random.Generator(np.random.PCG64(951))
    queries = [wl.round_to_bf16_bits(rng.standard_normal((B, hq, D), dtype=np.float32))
               for _ in range(REPLAYS)]
    th_dev, scale = lib_theta(D, cfg.base, cfg.factor, cfg.original_max_position)
    q = to_dev(inp["q"], "bf16")
    kc, vc = to_dev(inp["k_cache"], "bf16"), to_dev(inp["v_cache"], "bf16")
    sl = torch.from_numpy(inp["seqlens"]).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.attn_decode_workspace_bytes(B, lmax, hq, D), dtype=torch.uint8,
                     device="cuda")
    say(f"decode graph capture B={B} Lmax={lmax} W={window} S={sinks} noalloc={noalloc}")

    def call():
        if noalloc:
            ops.attn_decode_noalloc(q, kc, vc, sl, th_dev, scale, out, lse=lse, window=window,
                                    sinks=sinks)
        else:
            ops.attn_decode(q, kc, vc, sl, th_dev, scale, out=out, lse=lse, workspace=ws,
                            window=window, sinks=sinks)

    g = _capture(call)
    for r in range(REPLAYS):
        q.copy_(to_dev(queries[r], "bf16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        ref_o, ref_l = ops.attn_decode(q, kc, vc, sl, th_dev, scale, window=window, sinks=sinks)
        torch.cuda.synchronize()
        assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l), f"replay {r}"
        assert torch.isfinite(got_o.float()).all()
