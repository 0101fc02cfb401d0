"""Concurrent calls with separate outputs and workspaces: prefill and decode
issued on two streams at once, and several host threads calling the library
on their own streams, each result bit-identical to the same call made alone
on the default stream."""

import threading

import pytest
import torch

from tests._gpu_util import lib_theta, say, to_dev
from yarn_scaled_rope_amd import ops
from yarn_scaled_rope_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _prefill_inputs():
    cfg = wl.PrefillConfig("conc", 43, (900, 300, 17), 16, 4, 128, "bf16", 500000.0, 8.0, 16384)
    inp = wl.make_prefill(cfg)
    th, scale = lib_theta(128, cfg.base, cfg.factor, cfg.original_max_position)
    d = dict(q=to_dev(inp["q"], "bf16"), k=to_dev(inp["k"], "bf16"), v=to_dev(inp["v"], "bf16"),
             cu=torch.from_numpy(inp["cu_seqlens"]).cuda(), ms=max(cfg.seq_lens), th=th,
             scale=scale, T=sum(cfg.seq_lens), hq=cfg.hq, hkv=cfg.hkv)
    return d


def _decode_inputs(seed, B=8, lmax=70000, lmin=30000):
    cfg = wl.DecodeConfig("conc", 44, 0, 0, 0, 32, 8, 128, "bf16", 500000.0, 8.0, 16384)
    inp = wl.make_decode(cfg, seed=seed, batch=B, max_cache_len=lmax, min_cache_len=lmin)
    th, scale = lib_theta(128, cfg.base, cfg.factor, cfg.original_max_position)
    return dict(q=to_dev(inp["q"], "bf16"), kc=to_dev(inp["k_cache"], "bf16"),
                vc=to_dev(inp["v_cache"], "bf16"), sl=torch.from_numpy(inp["seqlens"]).cuda(),
                th=th, scale=scale, B=B, lmax=lmax)


def _prefill(p, stream=None, ws=None, out=None, lse=None):
    return ops.attn_prefill_fwd(p["q"], p["k"], p["v"], p["cu"], p["ms"], p["th"], p["scale"],
                                out=out, lse=lse, workspace=ws, stream=stream)


def _decode(d, stream=None, ws=None, out=None, lse=None):
    return ops.attn_decode(d["q"], d["kc"], d["vc"], d["sl"], d["th"], d["scale"], out=out,
                           lse=lse, workspace=ws, stream=stream)


def test_prefill_and_decode_on_two_streams():
    p = _prefill_inputs()
    d = _decode_inputs(960)
    say("prefill and decode on two streams")
    ref_p = _prefill(p)
    ref_d = _decode(d)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    # buffers allocated up front, on the default stream, before either stream runs
    ws1 = torch.empty(ops.attn_prefill_workspace_bytes(p["T"], p["hkv"], 128, ops.YR_BF16),
                      dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(ops.attn_decode_workspace_bytes(d["B"], d["lmax"], 32, 128),
                      dtype=torch.uint8, device="cuda")
    po = [torch.empty_like(ref_p[0]) for _ in range(3)]
    pl = [torch.empty_like(ref_p[1]) for _ in range(3)]
    do = [torch.empty_like(ref_d[0]) for _ in range(3)]
    dl = [torch.empty_like(ref_d[1]) for _ in range(3)]
    torch.cuda.synchronize()
    for i in range(3):   # interleaved launches, no synchronisation between them
        _prefill(p, stream=s1, ws=ws1, out=po[i], lse=pl[i])
        _decode(d, stream=s2, ws=ws2, out=do[i], lse=dl[i])
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(po[i], ref_p[0]) and torch.equal(pl[i], ref_p[1]), i
        assert torch.equal(do[i], ref_d[0]) and torch.equal(dl[i], ref_d[1]), i


def test_host_threads_on_their_own_streams():
    cases = [_decode_inputs(970 + i, B=4, lmax=40000, lmin=20000) for i in range(4)]
    say("decode from 4 host threads, one stream each")
    refs = [_decode(c) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    wss = [torch.empty(ops.attn_decode_workspace_bytes(c["B"], c["lmax"], 32, 128),
                       dtype=torch.uint8, device="cuda") for c in cases]
    outs = [[torch.empty_like(r[0]) for _ in range(5)] for r in refs]
    lses = [[torch.empty_like(r[1]) for _ in range(5)] for r in refs]
    torch.cuda.synchronize()
    errors = []
    barrier = threading.Barrier(len(cases))

    def worker(i):
        try:
            barrier.wait()
            for j in range(5):
                _decode(cases[i], stream=streams[i], ws=wss[i], out=outs[i][j], lse=lses[i][j])
            streams[i].synchronize()
        except Exception as e:   # reported in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, r in enumerate(refs):
        for j in range(5):
            assert torch.equal(outs[i][j], r[0]) and torch.equal(lses[i][j], r[1]), (i, j)
