"""Prefill launches large enough to hand out the tail of their work items
through the work queues in the workspace header (at least 8192 (q-tile,
sequence, head) items): windowed and plain prefill with 128 query heads over
16K tokens, and chunked prefill of more sequences than the ranked map takes
(so the packed map and its queues serve it), each on sampled rows against the
oracle; the same bits with the items permuted, from a workspace header full
of stale values, on a second call with the same workspace, and on every
replay of a captured graph."""

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from tests._gpu_util import BF16_TOL, LazyF64, lib_theta, max_abs, oracle_theta, say, to_dev, to_f64
from yarn_scaled_rope_amd import ops
from yarn_scaled_rope_amd import workloads as wl

pytestmark = pytest.mark.gpu

# 16384 tokens = 64 q-tiles of 256 rows; with 128 query heads, 8192 items
CFG = wl.PrefillConfig("t", 91, (16384,), 128, 8, 64, "bf16", 500000.0, 8.0, 4096)


@pytest.fixture(scope="module")
def big():
    inp = wl.make_prefill(CFG)
    th_dev, scale = lib_theta(CFG.head_dim, CFG.base, CFG.factor, CFG.original_max_position)
    dev = {"q": to_dev(inp["q"], "bf16"), "k": to_dev(inp["k"], "bf16"),
           "v": to_dev(inp["v"], "bf16"), "cu": torch.from_numpy(inp["cu_seqlens"]).cuda(),
           "theta": th_dev, "scale": scale}
    return inp, dev


def _call(dev, window=0, sinks=0, workspace=None, permuted=False):
    out, lse = ops.attn_prefill_fwd(dev["q"], dev["k"], dev["v"], dev["cu"], CFG.max_seqlen,
                                    dev["theta"], dev["scale"], out_dtype=ops.YR_F32,
                                    window=window, sinks=sinks, workspace=workspace,
                                    permuted_order=permuted)
    torch.cuda.synchronize()
    return out, lse


def _rows():
    # rows of every KV group at the edges, random rows, and the first and last
    # row of every q-tile for one group: the queued tail is the items of the
    # lowest q-tiles (rows below ~5,400), the statically mapped part the rest
    rows = _subset(wl.sample_rows(CFG.seq_lens, CFG.hq, CFG.hkv, n_random=8), 2000)
    rows += wl.tile_edge_rows(CFG.seq_lens, CFG.hq, CFG.hkv, 3, 256)
    return sorted(set(rows))


def _subset(rows, n, seed=3):
    """A seeded subset of n rows (the oracle's time is per row)."""
    rows = sorted(set(rows))
    if len(rows) <= n:
        return rows
    pick = np.random.Generator(np.random.PCG64(seed)).choice(len(rows), n, replace=False)
    return [rows[i] for i in sorted(pick)]


@pytest.mark.parametrize("window,sinks", [(0, 0), (4096, 4)])
def test_queued_prefill_sampled(big, window, sinks):
    inp, dev = big
    say(f"prefill 16K x 128 heads (8192 items, queued tail) W={window} S={sinks}")
    out, lse = _call(dev, window, sinks)
    rows = _rows()
    th, sc = oracle_theta(CFG.head_dim, CFG.base, CFG.factor, CFG.original_max_position)
    ro, rl = oatt.prefill_rows(LazyF64(inp["q"], "bf16"), LazyF64(inp["k"], "bf16"),
                               LazyF64(inp["v"], "bf16"), inp["cu_seqlens"], th, sc, rows,
                               window=window, sinks=sinks)
    o, l = to_f64(out), lse.cpu().numpy()
    e_out = max_abs(np.stack([o[t, h] for t, h in rows]), ro)
    e_lse = max_abs(np.array([l[h, t] for t, h in rows]), rl)
    print(f"{len(rows)} rows: max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert np.all(np.isfinite(o))
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


def test_queued_prefill_order_and_stale_header(big):
    """Permuted items, a header of stale counter values, and a second call on
    the same workspace all give the bits of a call on a fresh workspace."""
    _, dev = big
    say("prefill 16K x 128 heads: permuted, stale header, repeated call")
    # the library rotates the keys into the workspace, after the header
    nbytes = ops.attn_prefill_workspace_bytes(CFG.seq_lens[0], CFG.hkv, CFG.head_dim, ops.YR_BF16)
    ref = _call(dev, 4096, 4, workspace=torch.zeros(nbytes, dtype=torch.uint8, device="cuda"))
    perm = _call(dev, 4096, 4, permuted=True)
    stale = torch.full((nbytes,), 0x7f, dtype=torch.uint8, device="cuda")
    stale[:4] = 0  # the device error word
    first = _call(dev, 4096, 4, workspace=stale)
    again = _call(dev, 4096, 4, workspace=stale)
    for got in (perm, first, again):
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    assert ops.read_device_error(stale) == 0


def test_queued_chunk_packed_map():
    """72 sequences (more than the ranked map of chunked prefill takes): the
    packed map with its queued tail serves the chunk, 128 query heads."""
    rng = np.random.Generator(np.random.PCG64(5))
    ctx = tuple(int(x) for x in rng.integers(0, 700, 72))
    lens = tuple(int(x) for x in rng.integers(1, 300, 72))
    cfg = wl.ChunkConfig("t", 92, ctx, lens, 1024, 128, 8, 128, "bf16", 500000.0, 8.0, 16384)
    inp = wl.make_chunk(cfg)
    n_items = cfg.hq * sum((n + 255) // 256 for n in lens)
    assert n_items >= 8192
    say(f"chunked prefill, 72 sequences, {n_items} items (queued tail)")
    th_dev, scale = lib_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    cu = torch.from_numpy(inp["cu_seqlens_q"]).cuda()
    ctx_d = torch.from_numpy(inp["ctx_lens"]).cuda()
    out, lse = ops.attn_prefill_chunk(to_dev(inp["q"], "bf16"), to_dev(inp["k_cache"], "bf16"),
                                      to_dev(inp["v_cache"], "bf16"), cu, ctx_d, max(lens),
                                      th_dev, scale, out_dtype=ops.YR_F32)
    torch.cuda.synchronize()
    rows = _subset(wl.sample_rows(lens, cfg.hq, cfg.hkv, n_random=2), 3000)
    th, sc = oracle_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    ro, rl = oatt.prefill_chunk(LazyF64(inp["q"], "bf16"), LazyF64(inp["k_cache"], "bf16"),
                                LazyF64(inp["v_cache"], "bf16"), inp["cu_seqlens_q"],
                                inp["ctx_lens"], th, sc, rows=rows)
    o, l = to_f64(out), lse.cpu().numpy()
    e_out = max_abs(np.stack([o[t, h] for t, h in rows]), ro)
    e_lse = max_abs(np.array([l[h, t] for t, h in rows]), rl)
    print(f"{len(rows)} rows: max-abs out {e_out:.3e} lse {e_lse:.3e}")
    assert e_out <= BF16_TOL and e_lse <= BF16_TOL


def test_queued_prefill_graph_replays_match_eager(big):
    """A queued launch captured in a HIP graph: the counter reset is a kernel
    node, so every replay starts from zeroed queues.  Three replays with new
    queries written eagerly between them, each against an eager call."""
    _, dev = big
    say("prefill 16K x 128 heads (queued tail) in a graph, 3 replays")
    q0 = dev["q"].clone()
    q = dev["q"].clone()
    T = CFG.seq_lens[0]
    out = torch.empty((T, CFG.hq, CFG.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((CFG.hq, T), dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.attn_prefill_workspace_bytes(T, CFG.hkv, CFG.head_dim, ops.YR_BF16),
                     dtype=torch.uint8, device="cuda")

    def call():
        ops.attn_prefill_fwd(q, dev["k"], dev["v"], dev["cu"], CFG.max_seqlen, dev["theta"],
                             dev["scale"], out=out, out_dtype=ops.YR_F32, lse=lse, workspace=ws,
                             window=4096, sinks=4)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for r in range(1, 4):
        q.copy_(q0.roll(shifts=97 * r, dims=0))  # other rows at every position
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        ref_o, ref_l = ops.attn_prefill_fwd(q, dev["k"], dev["v"], dev["cu"], CFG.max_seqlen,
                                            dev["theta"], dev["scale"], out_dtype=ops.YR_F32,
                                            window=4096, sinks=4)
        torch.cuda.synchronize()
        assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l), f"replay {r}"
