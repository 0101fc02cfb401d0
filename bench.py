#!/usr/bin/env python3
"""Benchmark of the YaRN-RoPE causal attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the prefill hot path over the largest single-GPU
workload, the Llama-3-70B-shaped ragged batch (4 sequences of 131072, 65537,
32000 and 4097 tokens, 64 query / 8 KV heads, head_dim 128, bf16, YaRN s=8
over 16384, base 5e5): the key rotation pass (rope_apply_packed) and the
attention kernel (queries rotated on load, causal online softmax on bf16 MFMA,
out + LSE).  The frequency table (host, fp64, once per model) is timed
separately.  W untimed steps, then exactly K steps between two device
synchronisations; the JSON line's `value` is the algorithmic causal FLOPs of
one step over the wall time of one step.

The same run times, under `secondary`, the 128K Llama-3-8B GQA prefill and
the 16K Llama-2-7B prefill with the same step; the decode hot path (split-K
sweep + LSE merge) over the 16-sequence 32K-128K cache workload as `decode`;
under `next`, chunked prefill (4 chunks of 4096 new tokens after 28K-124K
cached ones), a 4096-token sliding window with 4 sink tokens on the 16K
prefill and the decode inputs, and decode over an FP8 (E4M3) copy of the
decode cache; and the fp64 CPU checker on bounded samples of the same inputs
as `cpu_baseline` (per row).

Roofline: each kernel's own duration comes from HIP events on the launch
stream around its launch inside every timed step.  `traffic` is filled from a
counter summary under profiles/ when one exists for the current kernel source
(FETCH_SIZE + WRITE_SIZE per dispatch, scaled by the same counters on a plain
copy of known size); otherwise it is null.

Other modes:
    --workload NAME           time another prefill workload as the main line
    --secondary a,b           prefill workloads of the secondary rows
                              ("none" for none)
    --copy-probe              also run a 1 GiB device copy (counter calibration)
    --no-next                 skip the lines of the next rows
    --summarize DIR --out F   turn rocprofv3 output (kernel stats and / or
                              counter CSVs under DIR, or several DIRs joined
                              by commas) into a short text summary, with the
                              matrix-core utilisation, MFMA FLOPs and shader
                              clock of each dispatch when the counters for
                              them are there
    --counters-json FETCH_DIR WRITE_DIR [--command "c1 ;; c2"] [--counters-row ROW]
                              HBM bytes per launch of the prefill and decode
                              kernels from FETCH_SIZE / WRITE_SIZE runs of
                              `bench.py --copy-probe`, into profiles/; with
                              --counters-row, of one next row's kernels from
                              runs of `bench.py --only-next ROW --copy-probe`
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0       # HBM3E
METRIC = "causal prefill TFLOP/s + % bf16 MFMA peak; decode KV GB/s + % HBM peak"
ATTN_SOURCES = ["yarn_scaled_rope_amd/csrc/prefill_bf16.hip",
                "yarn_scaled_rope_amd/csrc/device_common.h"]
DECODE_SOURCES = ["yarn_scaled_rope_amd/csrc/decode.hip",
                  "yarn_scaled_rope_amd/csrc/device_common.h"]


def source_digest(paths) -> str:
    """Digest of the kernel sources with comments and whitespace removed, so
    that a counter summary stays valid across comment-only edits."""
    import re
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


# The kernels of each next row, for its counter summary: (kind, workload,
# the row kernel's name up to its distinguishing template arguments, the
# kernel launched after each of its dispatches in the same call or None,
# sources, note).  In a run of `--only-next ROW` (with --no-decode for the
# 256-sequence row, whose split kernel is the decode line's) the row kernel's
# dispatches are that row's alone.
NEXT_COUNTER_ROWS = {
    "chunked_prefill": ("prefill_bf16", "llama3_8b_chunked_prefill_4x4k",
                        "prefill_bf16_kernel<128, false, true, true>", None, ATTN_SOURCES,
                        "one attn_prefill_chunk launch"),
    "window_prefill": ("prefill_bf16", "llama2_7b_prefill_16k_window4k_sinks4",
                       "prefill_bf16_kernel<128, false, true, true>", None, ATTN_SOURCES,
                       "one windowed attn_prefill_fwd launch (keys pre-rotated)"),
    "window_decode": ("decode", "decode_b16_gqa_window4k_sinks4",
                      "decode_mfma_kernel<128, 4, 1, false, true, true, false>",
                      "decode_merge_kernel", DECODE_SOURCES,
                      "split + merge kernels of one windowed attn_decode call"),
    "fp8_decode": ("decode", "decode_b16_gqa_32k_128k_fp8_e4m3",
                   "decode_mfma_kernel<128, 8, 2, true, false, false, true>",
                   "decode_merge_kernel", DECODE_SOURCES,
                   "split + merge kernels of one attn_decode_fp8 call"),
    "large_batch_decode": ("decode", "decode_b256_gqa_512_4k",
                           "decode_mfma_kernel<128, 4, 2, false, false, false, true>",
                           "decode_merge_kernel", DECODE_SOURCES,
                           "split + merge kernels of one attn_decode call"),
}


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def traffic_from_profiles(kind: str, workload: str, digest: str):
    """HBM bytes per launch from a committed counter summary, or None when
    there is none for this kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("source_digest") != digest:
        return None
    return d.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ prefill
def bench_prefill(args, torch, ops, wl, name=None, steps=None, warmup=None):
    cfg = wl.PREFILL_CONFIGS[name or args.workload]
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    if cfg.dtype != "bf16":
        raise SystemExit("bench times the bf16 path; the fp32 workload is a parity case")
    D, hq, hkv = cfg.head_dim, cfg.hq, cfg.hkv
    t0 = time.perf_counter()
    for _ in range(100):
        _, f64, t = ops.yarn_rope_freqs(D, cfg.base, cfg.factor, cfg.original_max_position)
    a1_us = (time.perf_counter() - t0) / 100 * 1e6
    theta = torch.from_numpy(f64).cuda()
    scale = t / math.sqrt(D)

    log(f"generating {cfg.name} inputs")
    inp = wl.make_prefill(cfg)
    import numpy as np

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = up(inp["q"]), up(inp["k"]), up(inp["v"])
    del inp["q"], inp["k"], inp["v"]
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    T = q.shape[0]
    maxlen = cfg.max_seqlen
    krot = torch.empty_like(k)
    out = torch.empty((T, hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((hq, T), dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    dev_err = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        ops.rope_apply_packed(k, cu, maxlen, theta, dst=krot, dev_error=dev_err, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        ops.attn_prefill_fwd(q, krot, v, cu, maxlen, theta, scale, out=out, lse=lse, workspace=ws,
                             k_rotated=True, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    log(f"prefill {cfg.name} warmup x{warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if int(dev_err.item()) != 0 or ops.read_device_error(ws) != 0:
        raise SystemExit("device range check failed")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    log(f"prefill {cfg.name} timed x{steps}")
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    rope_ms = sum(e[0].elapsed_time(e[1]) for e in events) / steps
    attn_ms = sum(e[1].elapsed_time(e[2]) for e in events) / steps
    ms_per_step = wall / steps * 1e3
    flops = wl.prefill_causal_flops(cfg.seq_lens, hq, D)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (attn_ms * 1e-3) / 1e12
    digest = source_digest(ATTN_SOURCES)
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_from_profiles("prefill_bf16", cfg.name, digest),
            "kernel": "prefill_bf16_kernel<128,false,true,false>", "kernel_ms": round(attn_ms, 4),
            "flops_per_launch": flops}
    extra = {"rope_pass_ms": round(rope_ms, 4), "freqs_host_us": round(a1_us, 2),
             "wall_ms_per_step": round(ms_per_step, 4), "source_digest": digest}
    conf = {"workload": cfg.name, "batch": len(cfg.seq_lens), "seq_lens": list(cfg.seq_lens),
            "hq": hq, "hkv": hkv, "head_dim": D, "rope": "yarn", "rope_base": cfg.base,
            "factor": cfg.factor, "original_max_position": cfg.original_max_position,
            "out_dtype": "bf16", "seed": 1000 + cfg.index}
    state = {"inp": inp, "q": q, "k": k, "v": v, "krot": krot, "cu": cu, "theta": theta,
             "theta_host": f64, "scale": scale, "maxlen": maxlen}
    return value, ms_per_step, roof, extra, conf, state


# ------------------------------------------------------------------ decode
def bench_decode(args, torch, ops, wl):
    import numpy as np
    cfg = wl.DECODE_B16
    D = cfg.head_dim
    _, f64, t = ops.yarn_rope_freqs(D, cfg.base, cfg.factor, cfg.original_max_position)
    theta = torch.from_numpy(f64).cuda()
    scale = t / math.sqrt(D)
    log(f"generating {cfg.name} inputs")
    inp = wl.make_decode(cfg)

    def up(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

    q = up(inp["q"])
    kc = up(inp["k_cache"])
    del inp["k_cache"]
    vc = up(inp["v_cache"])
    del inp["v_cache"]
    sl = torch.from_numpy(inp["seqlens"]).cuda()
    out = torch.empty((cfg.batch, cfg.hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((cfg.batch, cfg.hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(ops.attn_decode_workspace_bytes(cfg.batch, cfg.max_cache_len, cfg.hq, D),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    steps = args.decode_steps
    log(f"decode warmup x{args.warmup} timed x{steps}")
    for _ in range(args.warmup):
        ops.attn_decode(q, kc, vc, sl, theta, scale, out=out, lse=lse, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    if ops.read_device_error(ws) != 0:
        raise SystemExit("device range check failed (decode)")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        ops.attn_decode(q, kc, vc, sl, theta, scale, out=out, lse=lse, workspace=ws, stream=stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    call_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    nbytes = wl.decode_kv_bytes(inp["seqlens"], cfg.hkv, D)
    gbs = nbytes / (wall / steps) / 1e9
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    digest = source_digest(DECODE_SOURCES)
    res = {"metric": "decode KV GB/s", "value": round(gbs, 2), "unit": "GB/s",
           "ms_per_step": round(wall / steps * 1e3, 4), "steps": steps,
           "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
           "config": {"workload": cfg.name, "batch": cfg.batch, "seqlens": [int(x) for x in inp["seqlens"]],
                      "kv_bytes": int(nbytes), "hq": cfg.hq, "hkv": cfg.hkv, "head_dim": D,
                      "rope": "yarn", "rope_base": cfg.base, "factor": cfg.factor,
                      "original_max_position": cfg.original_max_position,
                      "seed": 1000 + cfg.index},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                        "traffic": traffic_from_profiles("decode", cfg.name, digest),
                        "kernel": "decode_mfma_kernel<128,4,2,false,false,false,true> + decode_merge_kernel<128,false> (one call)",
                        "kernel_ms": round(call_ms, 4), "bytes_per_launch": int(nbytes)},
           "source_digest": digest}
    state = {"seqlens": inp["seqlens"], "sl": sl, "q": q, "kc": kc, "vc": vc, "theta": theta,
             "scale": scale, "ws": ws}
    return res, state


# ------------------------------------------------------------------ next rows
QUEUED_TIMING = ("calls back to back after an unsynchronised burst of untimed calls "
                 "(the device stays busy at its working clock; host issue time excluded)")


def _queued_ms(torch, fns, warmup: int, steps: int, stream) -> float:
    """Mean duration (ms) of one call when `steps` calls run back to back on
    the stream, call i being fns[i % len(fns)].  One call and a device
    synchronisation absorb first-call costs; then `warmup` more calls go out
    with no synchronisation, so the device is busy (at the clock it holds
    under this load, not ramping up from idle) while the host queues the
    timed calls behind them, and the host's time to issue a call (the Python
    binding and the launches) does not open gaps between them."""
    fns[0]()
    torch.cuda.synchronize()
    for i in range(max(warmup, 4)):
        fns[i % len(fns)]()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        fns[i % len(fns)]()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _event_ms(torch, fn, warmup: int, steps: int, stream) -> float:
    """Mean duration (ms) of fn() between HIP events on the launch stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        fn()
        e[1].record(stream)
    torch.cuda.synchronize()
    return sum(e[0].elapsed_time(e[1]) for e in ev) / steps


def bench_next(args, torch, ops, wl, pstate, dstate):
    """Chunked prefill (4 chunks of 4096 tokens after 28K..124K cached
    tokens), a 4096-token window with 4 sinks on the prefill and decode
    inputs already resident, FP8-cache decode and a 256-sequence decode.
    Each line: algorithmic work / mean call time.  --only-next restricts the
    rows (for profiling one of them)."""
    import numpy as np
    stream = torch.cuda.current_stream()
    res = {}
    only = set(args.only_next.split(",")) if args.only_next else None

    def want(row):
        return only is None or row in only

    if want("chunked_prefill"):
        cfg = wl.CHUNK_4X4K
        D = cfg.head_dim
        _, f64, t = ops.yarn_rope_freqs(D, cfg.base, cfg.factor, cfg.original_max_position)
        theta = torch.from_numpy(f64).cuda()
        scale = t / math.sqrt(D)
        log(f"generating {cfg.name} inputs")
        inp = wl.make_chunk(cfg)

        def up(a):
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

        # host copy of sequence 0 (its cached rows and new tokens) for the oracle
        # sample, before the full caches are dropped
        n0, ctx0 = int(cfg.chunk_lens[0]), int(cfg.ctx_lens[0])
        chunk_host = {"q": np.array(inp["q"][:n0]), "k": np.array(inp["k_cache"][0:1, :ctx0 + n0]),
                      "v": np.array(inp["v_cache"][0:1, :ctx0 + n0]), "n": n0, "ctx": ctx0}
        q, kc = up(inp["q"]), up(inp["k_cache"])
        del inp["k_cache"]
        vc = up(inp["v_cache"])
        del inp["v_cache"]
        cu = torch.from_numpy(inp["cu_seqlens_q"]).cuda()
        ctx = torch.from_numpy(inp["ctx_lens"]).cuda()
        out = torch.empty((q.shape[0], cfg.hq, D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((cfg.hq, q.shape[0]), dtype=torch.float32, device="cuda")
        ws = torch.empty(256, dtype=torch.uint8, device="cuda")
        nq = max(cfg.chunk_lens)
        log("chunked prefill timed")
        ms = _event_ms(torch, lambda: ops.attn_prefill_chunk(q, kc, vc, cu, ctx, nq, theta, scale,
                                                             out=out, lse=lse, workspace=ws,
                                                             stream=stream),
                       args.warmup, max(5, args.steps // 2), stream)
        if ops.read_device_error(ws) != 0:
            raise SystemExit("device range check failed (chunked prefill)")
        flops = wl.prefill_visible_flops(cfg.chunk_lens, cfg.hq, D, ctx_lens=cfg.ctx_lens)
        tf = flops / (ms * 1e-3) / 1e12
        res["chunked_prefill"] = {
            "metric": "chunked prefill TFLOP/s", "value": round(tf, 2), "unit": "TFLOP/s",
            "ms_per_call": round(ms, 4), "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "flops_per_launch": flops,
            "config": {"workload": cfg.name, "ctx_lens": list(cfg.ctx_lens),
                       "chunk_lens": list(cfg.chunk_lens), "max_cache_len": cfg.max_cache_len,
                       "hq": cfg.hq, "hkv": cfg.hkv, "head_dim": D, "seed": 1000 + cfg.index}}
        del q, kc, vc, out, lse

    if want("window_prefill"):
        pc = wl.LLAMA2_7B_16K_SWA
        p = pstate
        out = torch.empty_like(p["q"])
        ws = torch.empty(256, dtype=torch.uint8, device="cuda")
        log("windowed prefill timed")
        ms = _queued_ms(torch, [lambda: ops.attn_prefill_fwd(p["q"], p["krot"], p["v"], p["cu"],
                                                             p["maxlen"], p["theta"], p["scale"],
                                                             out=out, want_lse=False, workspace=ws,
                                                             k_rotated=True, window=pc.window,
                                                             sinks=pc.sinks, stream=stream)],
                        args.warmup, args.steps, stream)
        flops = wl.prefill_visible_flops(pc.seq_lens, pc.hq, pc.head_dim, pc.window, pc.sinks)
        tf = flops / (ms * 1e-3) / 1e12
        res["window_prefill"] = {
            "metric": "windowed prefill TFLOP/s", "value": round(tf, 2), "unit": "TFLOP/s",
            "ms_per_call": round(ms, 4), "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "flops_per_launch": flops, "timing": QUEUED_TIMING,
            "config": {"workload": pc.name, "inputs": "those of the prefill line",
                       "window": pc.window, "sinks": pc.sinks}}

    fp8_state = None
    if dstate is not None and (want("window_decode") or want("fp8_decode")):
        dc = wl.DECODE_B16_SWA
        d = dstate
        out = torch.empty_like(d["q"])
        log("windowed decode timed")
        # The visible rows of one call (268 MB) would fit the 256 MB last-level
        # cache, so consecutive calls take the windows of 8 cache lengths
        # 4096 rows apart (disjoint rows, 2.1 GB in all): every call reads
        # its window from HBM.  Every sequence stays longer than window + sinks.
        shifts = [dc.window * k for k in range(8)]
        assert int(d["seqlens"].min()) - shifts[-1] >= dc.window + dc.sinks
        sls = [torch.from_numpy((d["seqlens"] - sh).astype(np.int32)).cuda() for sh in shifts]

        def wcall(sl):
            return lambda: ops.attn_decode(d["q"], d["kc"], d["vc"], sl, d["theta"], d["scale"],
                                           out=out, want_lse=False, workspace=d["ws"],
                                           window=dc.window, sinks=dc.sinks, stream=stream)
        ms = _queued_ms(torch, [wcall(sl) for sl in sls], args.warmup, max(args.decode_steps, 40),
                        stream)
        nb = [wl.decode_visible_bytes(d["seqlens"] - sh, dc.hkv, dc.head_dim, dc.window,
                                      dc.sinks) for sh in shifts]
        nbytes = sum(nb) / len(nb)
        gbs = nbytes / (ms * 1e-3) / 1e9
        res["window_decode"] = {
            "metric": "windowed decode KV GB/s", "value": round(gbs, 2), "unit": "GB/s",
            "ms_per_call": round(ms, 4), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "bytes_per_launch": int(nbytes),
            "timing": QUEUED_TIMING + ", windows of 8 cache lengths 4096 rows apart in turn",
            "config": {"workload": dc.name, "inputs": "those of the decode line",
                       "window": dc.window, "sinks": dc.sinks}}
        # FP8 (E4M3) copy of the same cache, one scale per KV head (amax / 448
        # of its valid rows), quantised on the device
        log("fp8 decode: quantising the cache")
        scales, codes = [], []
        L = torch.from_numpy(d["seqlens"].astype(np.int64)).cuda()
        valid = (torch.arange(d["kc"].shape[1], device="cuda")[None, :] < L[:, None])
        for c in (d["kc"], d["vc"]):
            amax = torch.stack([c[:, :, h].float().abs().masked_fill(~valid[:, :, None], 0).amax()
                                for h in range(c.shape[2])])
            sc = (amax / 448.0).clamp_min(1e-12).float().contiguous()
            q8 = torch.empty(c.shape, dtype=torch.uint8, device="cuda")
            for b in range(c.shape[0]):  # per sequence, to bound the temporaries
                q8[b] = (c[b].float() / sc[None, :, None]).nan_to_num(0.0).to(
                    torch.float8_e4m3fn).view(torch.uint8)
            scales.append(sc)
            codes.append(q8)
        out = torch.empty_like(d["q"])
        log("fp8 decode timed")
        # 2.7 GB per call, far past the last-level cache: calls back to back
        ms = _queued_ms(torch, [lambda: ops.attn_decode_fp8(d["q"], codes[0], codes[1], scales[0],
                                                            scales[1], d["sl"], d["theta"],
                                                            d["scale"], out=out, want_lse=False,
                                                            workspace=d["ws"], stream=stream)],
                        args.warmup, args.decode_steps, stream)
        nbytes = wl.decode_kv_bytes(d["seqlens"], wl.DECODE_B16.hkv, wl.DECODE_B16.head_dim, 1)
        gbs = nbytes / (ms * 1e-3) / 1e9
        res["fp8_decode"] = {
            "metric": "FP8-cache decode KV GB/s", "value": round(gbs, 2), "unit": "GB/s",
            "ms_per_call": round(ms, 4), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "bytes_per_launch": int(nbytes), "timing": QUEUED_TIMING,
            "config": {"workload": wl.DECODE_B16.name + "_fp8_e4m3",
                       "inputs": "the decode line's cache, as E4M3 codes with per-KV-head "
                                 "scales amax/448"}}
        fp8_state = {"codes": codes, "scales": scales}
    if want("large_batch_decode"):
        # many sequences: the balanced split over a 256-sequence batch
        lb = wl.DECODE_B256
        log(f"generating {lb.name} inputs")
        linp = wl.make_decode(lb)

        def upb(a):
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

        lq, lkc, lvc = upb(linp["q"]), upb(linp["k_cache"]), upb(linp["v_cache"])
        lsl = torch.from_numpy(linp["seqlens"]).cuda()
        _, lf64, lt = ops.yarn_rope_freqs(lb.head_dim, lb.base, lb.factor, lb.original_max_position)
        lth = torch.from_numpy(lf64).cuda()
        lws = torch.empty(ops.attn_decode_workspace_bytes(lb.batch, lb.max_cache_len, lb.hq,
                                                          lb.head_dim), dtype=torch.uint8,
                          device="cuda")
        lout = torch.empty_like(lq)
        log("large-batch decode timed")
        lscale = lt / math.sqrt(lb.head_dim)
        # 2.5 GB per call: calls back to back, as the FP8 row
        ms = _queued_ms(torch, [lambda: ops.attn_decode(lq, lkc, lvc, lsl, lth, lscale, out=lout,
                                                        want_lse=False, workspace=lws,
                                                        stream=stream)],
                        args.warmup, args.decode_steps, stream)
        if ops.read_device_error(lws) != 0:
            raise SystemExit("device range check failed (large-batch decode)")
        nbytes = wl.decode_kv_bytes(linp["seqlens"], lb.hkv, lb.head_dim)
        gbs = nbytes / (ms * 1e-3) / 1e9
        res["large_batch_decode"] = {
            "metric": "decode KV GB/s", "value": round(gbs, 2), "unit": "GB/s",
            "ms_per_call": round(ms, 4), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "bytes_per_launch": int(nbytes), "timing": QUEUED_TIMING,
            "config": {"workload": lb.name, "batch": lb.batch, "sum_seqlens": int(linp["seqlens"].sum()),
                       "hq": lb.hq, "hkv": lb.hkv, "head_dim": lb.head_dim, "seed": 1000 + lb.index}}
        del lkc, lvc
        # keep the host copies of the 32 sequences the CPU baseline reads
        linp["k_cache"] = np.array(linp["k_cache"][:32])
        linp["v_cache"] = np.array(linp["v_cache"][:32])
    if not args.no_cpu_baseline and only is None:
        log("timing the fp64 CPU oracle on bounded samples of the next rows")
        cpu_next(res, chunk_host, pstate, dstate, fp8_state, wl, torch, args.cpu_next_seconds)
        from oracle import attention as oatt
        from oracle import freqs as ofreqs
        th = ofreqs.yarn_theta(lb.head_dim, lb.base, lb.factor, lb.original_max_position)
        sc = ofreqs.softmax_scale(lb.head_dim, ofreqs.attention_temperature(lb.factor))
        q64 = wl.as_f64(linp["q"][:32], "bf16")
        kc64, vc64 = wl.as_f64(linp["k_cache"], "bf16"), wl.as_f64(linp["v_cache"], "bf16")
        passes, t0 = 0, time.perf_counter()
        while True:
            oatt.decode(q64, kc64, vc64, linp["seqlens"][:32], th, sc)
            passes += 1
            if time.perf_counter() - t0 >= args.cpu_next_seconds:
                break
        dt = time.perf_counter() - t0
        nb = wl.decode_kv_bytes(linp["seqlens"][:32], lb.hkv, lb.head_dim) * passes
        res["large_batch_decode"]["cpu_baseline"] = {
            "value": round(nb / dt / 1e9, 3), "unit": "GB/s", "cores": int(oracle_threads()),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"fp64 decode of sequences 0-31 of the same {lb.name} inputs, "
                      f"{passes} whole passes"}
    del fp8_state
    # the roofline object of each row, in the main line's form; traffic from
    # the row's counter summary when it matches the kernel sources
    for name, row in res.items():
        hbm = row["unit"] == "GB/s"
        kind, wname, _, _, srcs, _ = NEXT_COUNTER_ROWS[name]
        row["roofline"] = {"bound": "hbm" if hbm else "mfma", "achieved": row["value"],
                           "peak": PEAK_HBM_GBS if hbm else PEAK_BF16_TFLOPS,
                           "unit": row["unit"],
                           "frac": row["frac_hbm_peak" if hbm else "frac_mfma_peak"],
                           "traffic": traffic_from_profiles(kind, wname, source_digest(srcs))}
    return res


def cpu_next(res, chunk_host, pstate, dstate, fp8_state, wl, torch, seconds):
    """The fp64 oracle, as it stands, beside each next row: a bounded sample of
    the same inputs (about `seconds` of host work each), in the row's unit."""
    import numpy as np
    from oracle import attention as oatt
    from oracle import fp8 as ofp8
    from oracle import freqs as ofreqs
    threads = oracle_threads()

    def entry(value, unit, dt, sample):
        return {"value": round(value, 5 if unit == "TFLOP/s" else 3), "unit": unit,
                "cores": int(threads), "kind": "oracle", "seconds": round(dt, 2),
                "sample": sample}

    # chunked prefill: query heads of sequence 0's chunk, all its rows
    cfg = wl.CHUNK_4X4K
    th = ofreqs.yarn_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    sc = ofreqs.softmax_scale(cfg.head_dim, ofreqs.attention_temperature(cfg.factor))
    h = chunk_host
    q = wl.as_f64(h["q"], "bf16")
    kc, vc = wl.as_f64(h["k"], "bf16"), wl.as_f64(h["v"], "bf16")
    cu = np.array([0, h["n"]], dtype=np.int32)
    ctx = np.array([h["ctx"]], dtype=np.int32)
    heads, flops, t0 = 0, 0, time.perf_counter()
    while heads < cfg.hq and time.perf_counter() - t0 < seconds:
        oatt.prefill_chunk(q, kc, vc, cu, ctx, th, sc, rows=[(t, heads) for t in range(h["n"])])
        flops += wl.prefill_visible_flops([h["n"]], 1, cfg.head_dim, ctx_lens=[h["ctx"]])
        heads += 1
    dt = time.perf_counter() - t0
    res["chunked_prefill"]["cpu_baseline"] = entry(
        flops / dt / 1e12, "TFLOP/s", dt,
        f"fp64 chunked prefill of sequence 0 ({h['n']} new tokens after {h['ctx']} cached), "
        f"query heads 0-{heads - 1}, same inputs")

    # windowed prefill: the first query heads of the prefill inputs, all rows
    pc = wl.LLAMA2_7B_16K_SWA
    th = ofreqs.yarn_theta(pc.head_dim, pc.base, pc.factor, pc.original_max_position)
    sc = ofreqs.softmax_scale(pc.head_dim, ofreqs.attention_temperature(pc.factor))
    g = pc.hq // pc.hkv
    qh = pstate["q"].view(torch.int16).cpu().numpy()
    kh = pstate["k"].view(torch.int16).cpu().numpy()
    vh = pstate["v"].view(torch.int16).cpu().numpy()
    heads, flops, t0 = 0, 0, time.perf_counter()
    while heads < pc.hq and time.perf_counter() - t0 < seconds:
        hk = heads // g
        oatt.prefill(wl.as_f64(qh[:, heads:heads + 1].view("uint16"), "bf16"),
                     wl.as_f64(kh[:, hk:hk + 1].view("uint16"), "bf16"),
                     wl.as_f64(vh[:, hk:hk + 1].view("uint16"), "bf16"),
                     pstate["inp"]["cu_seqlens"], th, sc, window=pc.window, sinks=pc.sinks)
        flops += wl.prefill_visible_flops(pc.seq_lens, 1, pc.head_dim, pc.window, pc.sinks)
        heads += 1
    dt = time.perf_counter() - t0
    res["window_prefill"]["cpu_baseline"] = entry(
        flops / dt / 1e12, "TFLOP/s", dt,
        f"fp64 windowed prefill of query heads 0-{heads - 1}, all {pc.total_tokens} rows, "
        f"same inputs")
    if dstate is None:
        return

    # decode rows: sequences 0-3 of the decode inputs, whole passes
    dc = wl.DECODE_B16
    th = ofreqs.yarn_theta(dc.head_dim, dc.base, dc.factor, dc.original_max_position)
    sc = ofreqs.softmax_scale(dc.head_dim, ofreqs.attention_temperature(dc.factor))
    nseq = min(4, len(dstate["seqlens"]))
    lens = [int(x) for x in dstate["seqlens"][:nseq]]

    def host_bf16(t):
        return wl.as_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16), "bf16")

    qs = [host_bf16(dstate["q"][b:b + 1]) for b in range(nseq)]
    sw = wl.DECODE_B16_SWA
    kv = [(host_bf16(dstate["kc"][b:b + 1, :lens[b]]), host_bf16(dstate["vc"][b:b + 1, :lens[b]]))
          for b in range(nseq)]
    passes, t0 = 0, time.perf_counter()
    while True:
        for b in range(nseq):
            oatt.decode(qs[b], kv[b][0], kv[b][1], dstate["seqlens"][b:b + 1], th, sc,
                        window=sw.window, sinks=sw.sinks)
        passes += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    nbytes = wl.decode_visible_bytes(dstate["seqlens"][:nseq], sw.hkv, sw.head_dim, sw.window,
                                     sw.sinks) * passes
    res["window_decode"]["cpu_baseline"] = entry(
        nbytes / dt / 1e9, "GB/s", dt,
        f"fp64 windowed decode of sequences 0-{nseq - 1} (cache lengths {lens}), {passes} "
        f"whole passes, same inputs")
    del kv

    codes, scales = fp8_state["codes"], fp8_state["scales"]
    ks, vs = scales[0].cpu().numpy(), scales[1].cpu().numpy()
    c8 = [(codes[0][b:b + 1, :lens[b]].cpu().numpy(), codes[1][b:b + 1, :lens[b]].cpu().numpy())
          for b in range(nseq)]
    passes, t0 = 0, time.perf_counter()
    while True:
        for b in range(nseq):
            oatt.decode(qs[b], ofp8.dequantize_cache(c8[b][0], ks),
                        ofp8.dequantize_cache(c8[b][1], vs), dstate["seqlens"][b:b + 1], th, sc)
        passes += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    nbytes = wl.decode_kv_bytes(lens, dc.hkv, dc.head_dim, 1) * passes
    res["fp8_decode"]["cpu_baseline"] = entry(
        nbytes / dt / 1e9, "GB/s", dt,
        f"fp64 decode of sequences 0-{nseq - 1} from their E4M3 caches (decoding included), "
        f"{passes} whole passes, same inputs")


# ------------------------------------------------------------------ CPU baseline
def oracle_threads() -> int:
    """Threads the oracle's BLAS calls use (the host cores it runs on)."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return len(os.sched_getaffinity(0))


class _HostBf16:
    """fp64 view of a device bf16 tensor, copied to the host once and widened
    slice by slice (the oracle only slices its inputs)."""

    def __init__(self, t, wl, torch):
        import numpy as np
        self.bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        self.shape = self.bits.shape
        self.wl = wl

    def __getitem__(self, idx):
        return self.wl.as_f64(self.bits[idx], "bf16")


def cpu_baseline_rows(cfg_name, state, wl, torch, target_s: float, seed: int = 11):
    """The fp64 oracle, as it stands, on seeded random query rows of the same
    prefill inputs (each row over its full causal prefix, all query heads of
    KV head 0), in batches of 64 rows until about target_s seconds of work.
    FLOPs counted: 4 * D * (position + 1) per (row, head)."""
    import numpy as np
    from oracle import attention as oatt
    from oracle import freqs as ofreqs
    cfg = wl.PREFILL_CONFIGS[cfg_name]
    th = ofreqs.yarn_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    sc = ofreqs.softmax_scale(cfg.head_dim, ofreqs.attention_temperature(cfg.factor))
    q, k, v = (_HostBf16(state[x], wl, torch) for x in ("q", "k", "v"))
    cu = state["inp"]["cu_seqlens"]
    T = int(cu[-1])
    g = cfg.hq // cfg.hkv
    rng = np.random.Generator(np.random.PCG64(seed))
    starts = np.asarray(cu[:-1], dtype=np.int64)
    nrows, flops, elapsed = 0, 0, 0.0
    while elapsed < target_s and nrows < T:
        toks = rng.integers(0, T, size=64)
        rows = [(int(t), h) for t in toks for h in range(g)]
        pos = toks - starts[np.searchsorted(starts, toks, side="right") - 1]
        t0 = time.perf_counter()
        oatt.prefill_rows(q, k, v, cu, th, sc, rows)
        elapsed += time.perf_counter() - t0
        flops += int(4 * cfg.head_dim * g * int(np.sum(pos + 1)))
        nrows += len(toks)
    return {"value": round(flops / elapsed / 1e12, 5), "unit": "TFLOP/s",
            "cores": int(oracle_threads()), "kind": "oracle", "seconds": round(elapsed, 2),
            "sample": f"fp64 causal prefill of {nrows} seeded random query rows of the same "
                      f"{cfg.name} inputs (rows of every sequence, each over its full causal "
                      f"prefix), all {g} query heads of KV head 0"}


def cpu_baseline_decode(state, wl, torch, seconds: float = 10.0, nseq: int = 4):
    """The fp64 oracle on the first `nseq` sequences of the decode workload
    (inputs copied back from device memory and widened once), repeated in
    whole passes until at least `seconds` have elapsed."""
    import numpy as np
    from oracle import attention as oatt
    from oracle import freqs as ofreqs
    cfg = wl.DECODE_B16
    th = ofreqs.yarn_theta(cfg.head_dim, cfg.base, cfg.factor, cfg.original_max_position)
    sc = ofreqs.softmax_scale(cfg.head_dim, ofreqs.attention_temperature(cfg.factor))

    def host(t):
        return wl.as_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16), "bf16")

    seqs = []
    for b in range(min(nseq, len(state["seqlens"]))):
        L = int(state["seqlens"][b])
        seqs.append((host(state["q"][b:b + 1]), host(state["kc"][b:b + 1, :L]),
                     host(state["vc"][b:b + 1, :L]), state["seqlens"][b:b + 1]))
    lens = [int(x[3][0]) for x in seqs]
    passes = 0
    t0 = time.perf_counter()
    while True:
        for q, kc, vc, sl in seqs:
            oatt.decode(q, kc, vc, sl, th, sc)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    nbytes = wl.decode_kv_bytes(lens, cfg.hkv, cfg.head_dim) * passes
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": oracle_threads(),
            "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"fp64 decode of sequences 0-{len(seqs) - 1} (cache lengths {lens}) of the "
                      f"same inputs, {passes} whole passes"}


# ------------------------------------------------------------------ rocprof summaries
N_SIMD = 1024   # 256 CUs x 4 SIMDs
N_XCD = 8       # GRBM_GUI_ACTIVE counts once per XCD


def summarize(dirnames: str, out_path: str, command: str):
    """Condense rocprofv3 CSV output under one or more directories (comma
    separated) into a short text file: kernel statistics, dispatch durations
    by kernel and grid size (one kernel serves several workloads), the mean
    of every counter per dispatch by kernel and grid size, and per kernel and
    grid the figures the counters allow -- matrix-core busy fraction
    SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE / XCDs), MFMA FLOPs
    SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 per dispatch, and with a kernel trace
    of the same dispatches the shader clock GRBM_GUI_ACTIVE / XCDs / duration
    and the MFMA rate."""
    import csv
    dirs = [d for d in dirnames.split(",") if d]
    lines = ["# rocprofv3 summary", f"# command: {command}", ""]
    durations = {}
    for dirname in dirs:
        for p in glob.glob(os.path.join(dirname, "**", "*kernel_stats.csv"), recursive=True):
            rows = list(csv.DictReader(open(p)))
            lines.append(f"## kernel stats ({os.path.relpath(p, dirname)})")
            lines.append("name | calls | total_ns | avg_ns | min_ns | max_ns | pct")
            for r in rows:
                lines.append(f"{r.get('Name', '')[:110]} | {r.get('Calls')} | "
                             f"{r.get('TotalDurationNs')} | {r.get('AverageNs')} | {r.get('MinNs')} | "
                             f"{r.get('MaxNs')} | {r.get('Percentage')}")
            lines.append("")
        for p in glob.glob(os.path.join(dirname, "**", "*kernel_trace.csv"), recursive=True):
            groups = {}
            for r in csv.DictReader(open(p)):
                try:
                    dur = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
                except (KeyError, ValueError):
                    continue
                key = (r.get("Kernel_Name", "")[:110], r.get("Grid_Size", r.get("Grid_Size_X", "")))
                groups.setdefault(key, []).append(dur)
            if not groups:
                continue
            lines.append(f"## dispatches by kernel and grid size ({os.path.relpath(p, dirname)})")
            lines.append("name | grid size (threads) | calls | avg_ns | min_ns | max_ns")
            for (name, grid), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
                durations[(name, grid)] = sum(d) / len(d)
                lines.append(f"{name} | {grid} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.0f} | "
                             f"{max(d):.0f}")
            lines.append("")
    derived = []
    for dirname in dirs:
        for p in glob.glob(os.path.join(dirname, "**", "*counter_collection.csv"), recursive=True):
            per = {}
            for r in csv.DictReader(open(p)):
                key = (r.get("Kernel_Name", "")[:110], r.get("Grid_Size", ""),
                       r.get("Counter_Name", ""), r.get("Dispatch_Id", ""))
                per[key] = per.get(key, 0.0) + float(r.get("Counter_Value", 0) or 0)
            agg = {}
            for (kname, grid, cname, _), val in per.items():
                agg.setdefault((kname, grid, cname), []).append(val)
            lines.append(f"## counters ({os.path.relpath(p, dirname)}): mean per dispatch")
            lines.append("kernel | grid size | counter | dispatches | mean | min | max")
            for (kname, grid, cname), vals in sorted(agg.items()):
                lines.append(f"{kname} | {grid} | {cname} | {len(vals)} | "
                             f"{sum(vals) / len(vals):.6g} | {min(vals):.6g} | {max(vals):.6g}")
            lines.append("")
            for kname, grid in sorted({(k, g) for k, g, _ in agg}):
                m = {c: sum(v) / len(v) for (k, g, c), v in agg.items() if k == kname and g == grid}
                busy, gui = m.get("SQ_VALU_MFMA_BUSY_CYCLES"), m.get("GRBM_GUI_ACTIVE")
                mops = m.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
                if not busy or not gui:
                    continue
                cyc = gui / N_XCD
                d = {"kernel": kname, "grid": grid, "kernel_cycles": cyc,
                     "mfma_busy_frac": busy / (N_SIMD * cyc)}
                if mops:
                    d["mfma_flops_per_dispatch"] = mops * 512
                dur = durations.get((kname, grid))
                if dur:
                    d["duration_ms"] = dur / 1e6
                    d["shader_clock_ghz"] = cyc / dur
                    if mops:
                        d["mfma_tflops"] = mops * 512 / (dur * 1e-9) / 1e12
                        d["frac_of_peak"] = d["mfma_tflops"] / PEAK_BF16_TFLOPS
                derived.append(d)
    if derived:
        lines.append("## matrix-core utilisation (derived, mean per dispatch)")
        lines.append(f"# busy frac = SQ_VALU_MFMA_BUSY_CYCLES / ({N_SIMD} SIMDs x GRBM_GUI_ACTIVE/"
                     f"{N_XCD}); FLOPs = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; clock = "
                     f"GRBM_GUI_ACTIVE/{N_XCD} / kernel-trace duration of the same kernel and grid; "
                     f"peak {PEAK_BF16_TFLOPS} TFLOP/s")
        lines.append("kernel | grid | mfma busy | kernel cycles | MFMA FLOP/dispatch | duration ms | "
                     "clock GHz | MFMA TFLOP/s | frac of peak")

        def f(d, k, fmt):
            return format(d[k], fmt) if k in d else "-"
        for d in derived:
            lines.append(f"{d['kernel']} | {d['grid']} | {d['mfma_busy_frac']:.3f} | "
                         f"{d['kernel_cycles']:.4g} | {f(d, 'mfma_flops_per_dispatch', '.4g')} | "
                         f"{f(d, 'duration_ms', '.4f')} | {f(d, 'shader_clock_ghz', '.3f')} | "
                         f"{f(d, 'mfma_tflops', '.1f')} | {f(d, 'frac_of_peak', '.4f')}")
        lines.append("")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out_path)


def counters_json(fetch_dir: str, write_dir: str, workload: str, commands, row=None):
    """Per-launch HBM bytes of the prefill and decode kernels from two
    rocprofv3 --pmc runs of `bench.py --copy-probe` (FETCH_SIZE, WRITE_SIZE;
    KiB per dispatch).  Each counter is scaled by what it reads for the 1 GiB
    device copy of the probe (WRITE_SIZE of that copy picks it out; FETCH_SIZE
    is taken from the same kernel in the other run).  Writes
    profiles/{kind}_{workload}_hbm_counters.json for both kernels, or with
    `row` for that next row's kernels only (NEXT_COUNTER_ROWS): the row
    kernel's dispatches, plus the dispatch right after each of them when the
    row has a second kernel."""
    import csv

    def load(d, counter):
        out = []  # (dispatch id, kernel name, value) in dispatch order
        acc = {}
        for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(p)):
                if r.get("Counter_Name") != counter:
                    continue
                i = int(r["Dispatch_Id"])
                k, v = acc.get(i, (r["Kernel_Name"], 0.0))
                acc[i] = (k, v + float(r["Counter_Value"] or 0))
        for i in sorted(acc):
            out.append((i, acc[i][0], acc[i][1]))
        return out

    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    gib_kib = (1 << 30) / 1024
    copy = min((x for x in write if "yr::" not in x[1]), key=lambda x: abs(x[2] - gib_kib))
    copy_fetch = [x[2] for x in fetch if x[1] == copy[1]]
    copy_fetch = max(copy_fetch)  # the 1 GiB copy is the largest dispatch of that kernel
    scale_fetch, scale_write = gib_kib / copy_fetch, gib_kib / copy[2]

    def mean(rows, key):
        v = [x[2] for x in rows if key in x[1]]
        return sum(v) / len(v) if v else None

    def follower_mean(rows, key, nxt):
        # the dispatch that follows each `key` dispatch, when it is `nxt`
        v = [rows[i + 1][2] for i in range(len(rows) - 1)
             if key in rows[i][1] and nxt in rows[i + 1][1]]
        return sum(v) / len(v) if v else None

    if row is not None:
        kind, wname, key, nxt, srcs, note = NEXT_COUNTER_ROWS[row]
        keys = [key] + ([nxt] if nxt else [])
        f_kib = [mean(fetch, key)] + ([follower_mean(fetch, key, nxt)] if nxt else [])
        w_kib = [mean(write, key)] + ([follower_mean(write, key, nxt)] if nxt else [])
        if any(x is None for x in f_kib + w_kib):
            raise SystemExit(f"no dispatches of {keys} in the counter files")
        names = [k.split("<")[0] for k in keys]
        per_kernel = {n: int(round((fk * scale_fetch + wk * scale_write) * 1024))
                      for n, fk, wk in zip(names, f_kib, w_kib)}
        d = {"kernel": " + ".join(keys), "workload": wname, "source_digest": source_digest(srcs),
             "fetch_kib_per_dispatch_raw": dict(zip(names, f_kib)),
             "write_kib_per_dispatch_raw": dict(zip(names, w_kib)),
             "copy_probe": {"kernel": copy[1][:100], "bytes_read": 1 << 30, "bytes_written": 1 << 30,
                            "fetch_kib": copy_fetch, "write_kib": copy[2]},
             "scale_fetch": scale_fetch, "scale_write": scale_write,
             "hbm_bytes_per_launch": sum(per_kernel.values()), "bytes_per_kernel": per_kernel,
             "commands": list(commands), "note": note}
        path = os.path.join(ROOT, "profiles", f"{kind}_{wname}_hbm_counters.json")
        with open(path, "w") as fh:
            json.dump(d, fh, indent=1)
        print(path)
        return

    kinds = {
        "prefill_bf16": (workload, ["prefill_bf16_kernel"], ATTN_SOURCES,
                         "one attn_prefill_fwd launch (keys pre-rotated)"),
        "decode": ("decode_b16_gqa_32k_128k", ["decode_mfma_kernel", "decode_merge_kernel"],
                   DECODE_SOURCES, "split + merge kernels of one attn_decode call"),
    }
    written = []
    for kind, (wname, keys, srcs, note) in kinds.items():
        f_kib = [mean(fetch, k) for k in keys]
        w_kib = [mean(write, k) for k in keys]
        if any(x is None for x in f_kib + w_kib):
            continue
        per_kernel = {k: int(round((fk * scale_fetch + wk * scale_write) * 1024))
                      for k, fk, wk in zip(keys, f_kib, w_kib)}
        d = {"kernel": " + ".join(keys), "workload": wname, "source_digest": source_digest(srcs),
             "fetch_kib_per_dispatch_raw": dict(zip(keys, f_kib)),
             "write_kib_per_dispatch_raw": dict(zip(keys, w_kib)),
             "copy_probe": {"kernel": copy[1][:100], "bytes_read": 1 << 30, "bytes_written": 1 << 30,
                            "fetch_kib": copy_fetch, "write_kib": copy[2]},
             "scale_fetch": scale_fetch, "scale_write": scale_write,
             "hbm_bytes_per_launch": sum(per_kernel.values()), "bytes_per_kernel": per_kernel,
             "commands": list(commands), "note": note}
        path = os.path.join(ROOT, "profiles", f"{kind}_{wname}_hbm_counters.json")
        with open(path, "w") as fh:
            json.dump(d, fh, indent=1)
        written.append(path)
    print("\n".join(written))


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=None)
    ap.add_argument("--workload", default="llama3_70b_ragged_prefill")
    ap.add_argument("--secondary", default="llama3_8b_gqa_prefill_128k,llama2_7b_prefill_16k")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true")
    ap.add_argument("--only-next", default=None,
                    help="comma-separated next rows to run (chunked_prefill, window_prefill, "
                         "window_decode, fp8_decode, large_batch_decode); default all")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-next-seconds", type=float, default=3.0)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--summarize", default=None)
    ap.add_argument("--counters-json", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None)
    ap.add_argument("--out", default=None)
    ap.add_argument("--command", default="")
    ap.add_argument("--counters-row", default=None, choices=sorted(NEXT_COUNTER_ROWS))
    args = ap.parse_args()

    if args.counters_json:
        counters_json(args.counters_json[0], args.counters_json[1], args.workload,
                      args.command.split(" ;; ") if args.command else [], args.counters_row)
        return 0
    if args.summarize:
        summarize(args.summarize, args.out or "summary.txt", args.command)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2
    if args.decode_steps is None:
        args.decode_steps = max(args.steps, 20)

    import torch
    from yarn_scaled_rope_amd import ops
    from yarn_scaled_rope_amd import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    ops.load_library()
    torch.cuda.set_device(0)

    value, ms, roof, extra, conf, pstate = bench_prefill(args, torch, ops, wl)
    line = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic", "config": conf, "roofline": roof,
            "frac_mfma_peak_wall": round(value / PEAK_BF16_TFLOPS, 4)}
    line.update(extra)
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle on sampled rows of the main workload")
        line["cpu_baseline"] = cpu_baseline_rows(args.workload, pstate, wl, torch,
                                                 args.cpu_seconds)
    del pstate
    torch.cuda.empty_cache()
    # secondary prefill rows (same step, fewer steps for the long ones); the
    # 16K state is kept for the windowed-prefill row
    swa_state = None
    names = [] if args.secondary == "none" else [n for n in args.secondary.split(",") if n]
    if names:
        line["secondary"] = {}
    for name in names:
        cfg = wl.PREFILL_CONFIGS[name]
        big = max(cfg.seq_lens) > 32768
        st = max(3, args.steps // 4) if big else args.steps
        v2, ms2, roof2, extra2, conf2, state2 = bench_prefill(args, torch, ops, wl, name=name,
                                                              steps=st)
        row = {"metric": "causal prefill TFLOP/s", "value": round(v2, 2), "unit": "TFLOP/s",
               "steps": st, "ms_per_step": round(ms2, 4),
               "frac_mfma_peak_wall": round(v2 / PEAK_BF16_TFLOPS, 4), "config": conf2,
               "roofline": roof2}
        row.update(extra2)
        line["secondary"][name] = row
        if name == wl.LLAMA2_7B_16K.name:
            swa_state = state2
        else:
            del state2
        torch.cuda.empty_cache()
    if args.copy_probe:
        a = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        line["copy_probe_bytes"] = {"read": a.numel() * 2, "written": b.numel() * 2}
        del a, b
    dstate = None
    if not args.no_decode:
        dres, dstate = bench_decode(args, torch, ops, wl)
        line["decode"] = dres
    if not args.no_next:
        if swa_state is None:
            *_, swa_state = bench_prefill(args, torch, ops, wl, name=wl.LLAMA2_7B_16K.name,
                                          steps=1, warmup=1)
        line["next"] = bench_next(args, torch, ops, wl, swa_state, dstate)
    if not args.no_cpu_baseline and not args.no_decode:
        line["decode"]["cpu_baseline"] = cpu_baseline_decode(dstate, wl, torch)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
