"""The pages' printed worked values, recomputed (CPU only).  They pin the work
counters that throughput is quoted on and the NTK base rule."""

import json
import os

import pytest

from oracle import freqs
from yarn_scaled_rope_amd import workloads as wl

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")))
UNITS = {"GB": 1e9, "GiB": 2.0 ** 30, "TiB": 2.0 ** 40}


@pytest.mark.parametrize("e", GOLDEN["kv_cache"], ids=lambda e: e["what"])
def test_kv_cache_bytes(e):
    got = wl.kv_cache_bytes(e["n_layers"], e["n_kv_heads"], e["head_dim"], e["seq_len"],
                            1, e["dtype_bytes"]) / UNITS[e["unit"]]
    assert abs(got - e["printed"]) / e["printed"] <= e["rel_tol"], got


@pytest.mark.parametrize("e", GOLDEN["attention_flops_one_head"], ids=lambda e: e["what"])
def test_attention_flops(e):
    got = wl.dense_attention_flops(e["seq_len"], e["head_dim"], 1)
    assert abs(got - e["printed"]) / e["printed"] <= e["rel_tol"], got


@pytest.mark.parametrize("e", GOLDEN["score_matrix_bytes"], ids=lambda e: e["what"])
def test_score_matrix_bytes(e):
    got = wl.score_matrix_bytes(e["seq_len"], e["heads"], e["dtype_bytes"]) / UNITS[e["unit"]]
    assert abs(got - e["printed"]) / e["printed"] <= e["rel_tol"], got


@pytest.mark.parametrize("e", GOLDEN["model_prefill_flops"], ids=lambda e: e["what"])
def test_model_prefill_flops(e):
    got = wl.dense_attention_flops(e["seq_len"], e["head_dim"], e["heads"]) * e["n_layers"]
    assert abs(got - e["printed"]) / e["printed"] <= e["rel_tol"], got


@pytest.mark.parametrize("e", GOLDEN["ntk_base"], ids=lambda e: e["what"])
def test_ntk_base(e):
    got = freqs.ntk_base(e["head_dim"], e["base"], e["factor"])
    assert abs(got - e["printed"]) / e["printed"] <= e["rel_tol"], got


def test_causal_count_is_half_dense_plus_diagonal():
    # 4 D Hq n(n+1)/2 = (dense 4 n^2 D Hq + diagonal 4 n D Hq) / 2
    for n, hq, d in [(4096, 1, 128), (16384, 32, 128), (1, 4, 64)]:
        causal = wl.prefill_causal_flops([n], hq, d)
        assert 2 * causal == wl.dense_attention_flops(n, d, hq) + 4 * n * d * hq


def test_workload_work_figures():
    # Llama-2-7B 16K prefill, Llama-3-8B 128K, Llama-3-70B ragged
    assert wl.prefill_causal_flops((16384,), 32, 128) == pytest.approx(2.199e12, rel=1e-3)
    assert wl.prefill_causal_flops((131072,), 32, 128) == pytest.approx(1.407e14, rel=1e-3)
    assert wl.prefill_causal_flops((131072, 65537, 32000, 4097), 64, 128) == pytest.approx(3.689e14, rel=1e-3)
    assert wl.mean_decode_bytes(wl.DECODE_B16) == pytest.approx(5.37e9, rel=1e-3)
    assert wl.decode_kv_bytes([1], 8, 128) == 4096
