"""The figures the benchmark divides by (algorithmic FLOPs of prefill,
visible K/V bytes of decode) against a brute-force count of visible
(query, key) pairs with the oracle's visibility rule, and the rocprofv3
post-processing of bench.py (matrix-core busy fraction, MFMA FLOPs, shader
clock, HBM bytes scaled by a copy of known size) on synthetic counter files
whose answers are known.  CPU only."""

import csv
import importlib
import json
import os
import sys

import numpy as np
import pytest

from oracle.bruteforce import sees
from yarn_scaled_rope_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    return importlib.import_module("bench")


def _pairs(lens, ctx=None, window=0, sinks=0):
    """Visible (query, key) pairs by enumeration: query i of sequence b sits
    at position ctx_b + i and may see key positions 0 .. ctx_b + n_b - 1."""
    total = 0
    for b, n in enumerate(lens):
        p0 = 0 if ctx is None else ctx[b]
        for i in range(n):
            m = p0 + i
            total += sum(1 for j in range(p0 + n) if sees(m, j, window, sinks))
    return total


@pytest.mark.parametrize("lens,hq,D", [((1, 5, 17), 3, 8), ((64, 65, 1), 8, 128), ((200,), 2, 64)])
def test_causal_flops_count_every_visible_pair(lens, hq, D):
    want = 4 * D * hq * _pairs(lens)
    assert wl.prefill_causal_flops(lens, hq, D) == want
    assert wl.prefill_visible_flops(lens, hq, D) == want


@pytest.mark.parametrize("lens,ctx,window,sinks", [
    ((40, 7), None, 8, 0),
    ((40, 7), None, 8, 3),
    ((33,), None, 1, 2),          # a window of one: the query itself and the sinks
    ((10, 20), (0, 15), 0, 0),    # chunks after cached prefixes
    ((10, 20), (5, 50), 12, 4),   # chunks with a window and sinks
])
def test_windowed_and_chunk_flops_count_every_visible_pair(lens, ctx, window, sinks):
    hq, D = 4, 16
    want = 4 * D * hq * _pairs(lens, ctx, window, sinks)
    assert wl.prefill_visible_flops(lens, hq, D, window, sinks, ctx_lens=ctx) == want


@pytest.mark.parametrize("window,sinks,use_qpos", [(0, 0, False), (16, 0, False), (16, 4, False),
                                                   (16, 4, True), (1000, 4, False)])
def test_decode_bytes_count_every_visible_row(window, sinks, use_qpos):
    rng = np.random.default_rng(7)
    seqlens = rng.integers(1, 90, size=9)
    q_pos = rng.integers(0, 120, size=9) if use_qpos else None
    hkv, D = 2, 32
    # decode reads every cache row 0 .. L-1 the window and sinks leave
    # visible from the query's position m (default L), as oracle.decode does:
    # the rows are the past by construction, so only the window rule applies
    rows = 0
    for b, L in enumerate(seqlens):
        m = int(L) if q_pos is None else int(q_pos[b])
        rows += sum(1 for j in range(int(L)) if window <= 0 or j > m - window or j < sinks)
    want = 2 * hkv * D * 2 * rows
    assert wl.decode_visible_bytes(seqlens, hkv, D, window, sinks, q_pos=q_pos) == want
    if window == 0 and not use_qpos:
        assert wl.decode_kv_bytes(seqlens, hkv, D) == want


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def test_summarize_derives_busy_fraction_flops_and_clock(tmp_path):
    bench = _bench()
    name = "void yr::(anonymous namespace)::prefill_bf16_kernel<128, false, true, false>(args)"
    # two dispatches of 2 ms each on the trace
    _write_csv(str(tmp_path / "trace" / "run_kernel_trace.csv"), [
        {"Kernel_Name": name, "Start_Timestamp": 0, "End_Timestamp": 2_000_000,
         "Grid_Size_X": 1048576},
        {"Kernel_Name": name, "Start_Timestamp": 5_000_000, "End_Timestamp": 7_000_000,
         "Grid_Size_X": 1048576},
    ])
    # one dispatch's counters: 8 XCDs x 3.6e6 cycles; busy 1024 SIMDs x 1.8e6
    gui = 8 * 3.6e6
    busy = 1024 * 1.8e6
    mops = 2.2e12 / 512
    rows = []
    for cname, val in (("GRBM_GUI_ACTIVE", gui), ("SQ_VALU_MFMA_BUSY_CYCLES", busy),
                       ("SQ_INSTS_VALU_MFMA_MOPS_BF16", mops)):
        rows.append({"Dispatch_Id": 1, "Kernel_Name": name, "Grid_Size": 1048576,
                     "Counter_Name": cname, "Counter_Value": val})
    _write_csv(str(tmp_path / "mfma" / "run_counter_collection.csv"), rows)
    out = tmp_path / "summary.txt"
    bench.summarize(f"{tmp_path / 'mfma'},{tmp_path / 'trace'}", str(out), "synthetic")
    text = out.read_text().splitlines()
    i = next(k for k, l in enumerate(text) if l.startswith("## matrix-core utilisation"))
    fields = [x.strip() for x in text[i + 3].split("|")]
    assert fields[1] == "1048576"
    assert float(fields[2]) == pytest.approx(0.5, abs=1e-3)            # busy / (1024 x cycles)
    assert float(fields[3]) == pytest.approx(3.6e6, rel=1e-3)          # GRBM / 8
    assert float(fields[4]) == pytest.approx(2.2e12, rel=1e-3)         # MOPS x 512
    assert float(fields[5]) == pytest.approx(2.0, rel=1e-6)            # ms
    assert float(fields[6]) == pytest.approx(1.8, rel=1e-3)            # 3.6e6 cycles / 2 ms
    assert float(fields[7]) == pytest.approx(1100.0, rel=1e-3)         # 2.2e12 / 2 ms
    assert float(fields[8]) == pytest.approx(1100.0 / 2516.6, rel=1e-3)


def test_counters_json_scales_by_the_copy_and_sums_kernels(tmp_path, monkeypatch):
    bench = _bench()
    # a private tree: the digest reads the kernel sources, the output goes to profiles/
    for rel in set(bench.ATTN_SOURCES + bench.DECODE_SOURCES):
        p = tmp_path / rel
        p.parent.mkdir(parents=True, exist_ok=True)
        p.write_text("// placeholder\nint x;\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    gib_kib = (1 << 30) / 1024
    copy = "__amd_rocclr_copyBuffer"
    pre = "void yr::(anonymous namespace)::prefill_bf16_kernel<128, false, true, false>(x)"
    dec = "void yr::(anonymous namespace)::decode_mfma_kernel<128, 4, 2, false, false, false, true>(x)"
    mrg = "void yr::(anonymous namespace)::decode_merge_kernel<128, false, false>(x)"
    # FETCH_SIZE of the copy reads half its bytes (scale 2); WRITE_SIZE all of them (scale 1)
    fetch = [(1, copy, gib_kib / 2), (2, pre, 1000.0), (3, pre, 3000.0), (4, dec, 500.0),
             (5, mrg, 10.0), (6, copy, 0.5)]
    write = [(1, copy, gib_kib), (2, pre, 100.0), (3, pre, 300.0), (4, dec, 1.0), (5, mrg, 2.0),
             (6, copy, 0.25)]
    for d, rows, cname in (("fetch", fetch, "FETCH_SIZE"), ("write", write, "WRITE_SIZE")):
        _write_csv(str(tmp_path / d / "run_counter_collection.csv"),
                   [{"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": cname, "Counter_Value": v}
                    for i, k, v in rows])
    bench.counters_json(str(tmp_path / "fetch"), str(tmp_path / "write"), "synthetic_prefill",
                        ["synthetic"])
    p = json.load(open(tmp_path / "profiles" / "prefill_bf16_synthetic_prefill_hbm_counters.json"))
    assert p["scale_fetch"] == pytest.approx(2.0) and p["scale_write"] == pytest.approx(1.0)
    # mean over the two prefill dispatches: fetch 2000 KiB x 2 + write 200 KiB
    assert p["hbm_bytes_per_launch"] == int(round((2000 * 2 + 200) * 1024))
    assert p["source_digest"] == bench.source_digest(bench.ATTN_SOURCES)
    d = json.load(open(tmp_path / "profiles" / "decode_decode_b16_gqa_32k_128k_hbm_counters.json"))
    assert d["bytes_per_kernel"]["decode_mfma_kernel"] == int(round((500 * 2 + 1) * 1024))
    assert d["bytes_per_kernel"]["decode_merge_kernel"] == int(round((10 * 2 + 2) * 1024))
    assert d["hbm_bytes_per_launch"] == sum(d["bytes_per_kernel"].values())


def test_counters_json_of_a_next_row_pairs_each_split_with_its_merge(tmp_path, monkeypatch):
    bench = _bench()
    for rel in set(bench.ATTN_SOURCES + bench.DECODE_SOURCES):
        p = tmp_path / rel
        p.parent.mkdir(parents=True, exist_ok=True)
        p.write_text("// placeholder\nint x;\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    gib_kib = (1 << 30) / 1024
    copy = "__amd_rocclr_copyBuffer"
    main = "void yr::(anonymous namespace)::decode_mfma_kernel<128, 4, 2, false, false, false, true>(x)"
    win = "void yr::(anonymous namespace)::decode_mfma_kernel<128, 4, 1, false, true, true, false>(x)"
    mrg = "void yr::(anonymous namespace)::decode_merge_kernel<128, false, false>(x)"
    # the decode line's split + merge, then two windowed calls: only the merges
    # that follow a windowed split count for the row
    fetch = [(1, copy, gib_kib), (2, main, 9000.0), (3, mrg, 700.0), (4, win, 100.0),
             (5, mrg, 7.0), (6, win, 300.0), (7, mrg, 9.0)]
    write = [(1, copy, gib_kib), (2, main, 5.0), (3, mrg, 70.0), (4, win, 1.0), (5, mrg, 2.0),
             (6, win, 3.0), (7, mrg, 4.0)]
    for d, rows, cname in (("fetch", fetch, "FETCH_SIZE"), ("write", write, "WRITE_SIZE")):
        _write_csv(str(tmp_path / d / "run_counter_collection.csv"),
                   [{"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": cname, "Counter_Value": v}
                    for i, k, v in rows])
    bench.counters_json(str(tmp_path / "fetch"), str(tmp_path / "write"), "unused", ["synthetic"],
                        row="window_decode")
    p = json.load(open(tmp_path / "profiles" / "decode_decode_b16_gqa_window4k_sinks4_hbm_counters.json"))
    assert p["scale_fetch"] == pytest.approx(1.0) and p["scale_write"] == pytest.approx(1.0)
    assert p["bytes_per_kernel"]["decode_mfma_kernel"] == int(round((200 + 2) * 1024))
    assert p["bytes_per_kernel"]["decode_merge_kernel"] == int(round((8 + 3) * 1024))
    assert p["hbm_bytes_per_launch"] == sum(p["bytes_per_kernel"].values())
    assert p["source_digest"] == bench.source_digest(bench.DECODE_SOURCES)
    # and the row's roofline reads it back for the same sources
    kind, wname, _, _, srcs, _ = bench.NEXT_COUNTER_ROWS["window_decode"]
    assert bench.traffic_from_profiles(kind, wname, bench.source_digest(srcs)) == \
        p["hbm_bytes_per_launch"]
    assert bench.traffic_from_profiles(kind, wname, "0" * 16) is None


def test_next_counter_rows_name_the_bench_rows():
    bench = _bench()
    assert set(bench.NEXT_COUNTER_ROWS) == {"chunked_prefill", "window_prefill", "window_decode",
                                            "fp8_decode", "large_batch_decode"}
    names = {r[1] for r in bench.NEXT_COUNTER_ROWS.values()}
    assert {wl.CHUNK_4X4K.name, wl.LLAMA2_7B_16K_SWA.name, wl.DECODE_B16_SWA.name,
            wl.DECODE_B256.name, wl.DECODE_B16.name + "_fp8_e4m3"} == names
