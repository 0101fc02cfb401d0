"""Host-side checks of the input generator (CPU only)."""

import numpy as np
import torch

from yarn_scaled_rope_amd import workloads as wl


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.Generator(np.random.PCG64(0))
    x = rng.standard_normal(200000, dtype=np.float32) * np.float32(3.0)
    # include exact ties (low 16 bits == 0x8000) of both parities
    ties = (np.arange(64, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x3F808000)
    x = np.concatenate([x, ties.view(np.float32)])
    ours = wl.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = wl.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_chunked_draw_equals_single_draw(monkeypatch):
    a = wl._draw(np.random.Generator(np.random.PCG64(5)), (1000, 3), "bf16")
    monkeypatch.setattr(wl, "_CHUNK", 77)
    b = wl._draw(np.random.Generator(np.random.PCG64(5)), (1000, 3), "bf16")
    assert np.array_equal(a, b)


def test_prefill_inputs_shapes_and_determinism():
    cfg = wl.TINY_F32
    a = wl.make_prefill(cfg)
    b = wl.make_prefill(cfg)
    assert a["q"].shape == (256, 4, 64) and a["k"].shape == (256, 2, 64)
    assert a["q"].dtype == np.float32
    assert np.array_equal(a["q"], b["q"]) and list(a["cu_seqlens"]) == [0, 256]
    c = wl.make_prefill(wl.LLAMA3_70B_RAGGED, seq_lens=(5, 1, 3))
    assert c["q"].dtype == np.uint16 and list(c["cu_seqlens"]) == [0, 5, 6, 9]


def test_decode_inputs_nan_tails():
    d = wl.make_decode(wl.DECODE_B16, batch=3, max_cache_len=40, min_cache_len=10)
    assert d["k_cache"].shape == (3, 40, 8, 128)
    for b, L in enumerate(d["seqlens"]):
        assert 10 <= L <= 40
        assert np.all(np.isnan(wl.bf16_bits_to_f32(d["k_cache"][b, L:])))
        assert np.all(np.isfinite(wl.bf16_bits_to_f32(d["v_cache"][b, :L])))


def test_prefill_sparse_q_draws_only_the_named_rows():
    cfg = wl.PrefillConfig("t", 3, (40, 25), 4, 2, 64, "bf16", 10000.0, 1.0, 64)
    a = wl.make_prefill(cfg, q_tokens=[64, 3, 3, 41])
    nz = np.flatnonzero(np.any(a["q"] != 0, axis=(1, 2)))
    assert list(nz) == [3, 41, 64]
    # the rows are drawn in ascending token order, before k and v
    rng = np.random.Generator(np.random.PCG64(1000 + cfg.index))
    want = wl._draw(rng, (3, 4, 64), "bf16")
    assert np.array_equal(a["q"][[3, 41, 64]], want)
    assert np.array_equal(a["k"], wl._draw(rng, (65, 2, 64), "bf16"))


def test_decode_given_seqlens():
    d = wl.make_decode(wl.DECODE_B16, batch=2, max_cache_len=50, seqlens=[7, 50])
    assert list(d["seqlens"]) == [7, 50]
    assert np.all(np.isnan(wl.bf16_bits_to_f32(d["k_cache"][0, 7:])))
    assert np.all(np.isfinite(wl.bf16_bits_to_f32(d["k_cache"][1])))
    f = wl.make_decode_fp8(wl.DECODE_B16, batch=2, max_cache_len=30, seqlens=[30, 0])
    assert list(f["seqlens"]) == [30, 0]
    assert np.all(f["v_cache"][1] == wl.E4M3_NAN_CODE)


def test_sample_rows_cover_edges_and_tails():
    rows = wl.sample_rows((300, 65), 8, 2, n_random=5)
    toks = {t for t, _ in rows}
    assert {0, 1, 2, 3, 127, 128, 129, 297, 298, 299} <= toks
    assert set(range(300, 365)) <= toks          # second sequence is all tail
    heads = {(t, h) for t, h in rows if t == 0}
    assert heads == {(0, h) for h in range(8)}
