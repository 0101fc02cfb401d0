"""The Python binding rejects malformed arguments before anything reaches the
library or the device (CPU only): wrong dtypes, shapes and element counts of
every tensor argument raise YarnAttnError naming the argument, and well-formed
host tensors are then refused only because they are not device tensors."""

import pytest
import torch

from yarn_scaled_rope_amd import ops

D, HQ, HKV, T, B, LMAX = 128, 8, 2, 40, 3, 64


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def f64(n=D // 2):
    return torch.zeros(n, dtype=torch.float64)


def raises(fn, fragment):
    with pytest.raises(ops.YarnAttnError) as e:
        fn()
    assert fragment in str(e.value), str(e.value)
    assert "device tensor" not in str(e.value) or fragment == "device tensor"


# ---- decode ---------------------------------------------------------------
def dec(**kw):
    a = dict(q=bf(B, HQ, D), k_cache=bf(B, LMAX, HKV, D), v_cache=bf(B, LMAX, HKV, D),
             seqlens=i32(B), inv_freq_f64=f64(), softmax_scale=0.1)
    a.update(kw)
    return lambda: ops.attn_decode(**a)


@pytest.mark.parametrize("kw,frag", [
    (dict(k_cache=f32(B, LMAX, HKV, D), v_cache=f32(B, LMAX, HKV, D)), "caches must be"),
    (dict(v_cache=bf(B, LMAX, HKV, 64)), "caches must be"),
    (dict(seqlens=i32(B + 1)), "seqlens"),
    (dict(seqlens=torch.zeros(B, dtype=torch.int64)), "seqlens"),
    (dict(q_pos=i32(B - 1)), "q_pos"),
    (dict(inv_freq_f64=f64(D)), "inv_freq_f64"),
    (dict(inv_freq_f64=torch.zeros(D // 2, dtype=torch.float32)), "inv_freq_f64"),
    (dict(out=bf(B, HQ, D), out_dtype=ops.YR_F32), "out"),
    (dict(out=bf(B, HQ + 1, D)), "out"),
    (dict(lse=f32(HQ, B)), "lse"),
    (dict(lse=bf(B, HQ)), "lse"),
    (dict(out_dtype=7), "out_dtype"),
    (dict(q=bf(B, HQ)), "q must be a 3-d"),
])
def test_decode_rejects(kw, frag):
    raises(dec(**kw), frag)


def test_decode_well_formed_host_tensors_need_the_device():
    raises(dec(), "device tensor")
    raises(dec(q=f32(B, HQ, D), k_cache=f32(B, LMAX, HKV, D), v_cache=f32(B, LMAX, HKV, D),
               out=f32(B, HQ, D), lse=f32(B, HQ), q_pos=i32(B)), "device tensor")


def dec8(**kw):
    a = dict(q=bf(B, HQ, D), k_cache=torch.zeros(B, LMAX, HKV, D, dtype=torch.uint8),
             v_cache=torch.zeros(B, LMAX, HKV, D, dtype=torch.uint8), k_scale=f32(HKV),
             v_scale=f32(HKV), seqlens=i32(B), inv_freq_f64=f64(), softmax_scale=0.1)
    a.update(kw)
    return lambda: ops.attn_decode_fp8(**a)


@pytest.mark.parametrize("kw,frag", [
    (dict(k_cache=bf(B, LMAX, HKV, D)), "caches must be"),
    (dict(k_scale=f32(HKV + 1)), "k_scale"),
    (dict(v_scale=f32(HKV - 1)), "v_scale"),
    (dict(q=f32(B, HQ, D)), "q must be"),
    (dict(out=f32(B, HQ, D)), "out"),
    (dict(lse=f32(B)), "lse"),
    (dict(seqlens=i32(2 * B)), "seqlens"),
])
def test_decode_fp8_rejects(kw, frag):
    raises(dec8(**kw), frag)


# ---- prefill ----------------------------------------------------------------
def pre(**kw):
    a = dict(q=bf(T, HQ, D), k=bf(T, HKV, D), v=bf(T, HKV, D),
             cu_seqlens=torch.tensor([0, 10, T], dtype=torch.int32), max_seqlen=30,
             inv_freq_f64=f64(), softmax_scale=0.1)
    a.update(kw)
    return lambda: ops.attn_prefill_fwd(**a)


@pytest.mark.parametrize("kw,frag", [
    (dict(k=f32(T, HKV, D)), "k and v"),
    (dict(v=bf(T + 1, HKV, D)), "k and v"),
    (dict(cu_seqlens=torch.tensor([0, T], dtype=torch.int64)), "cu_seqlens"),
    (dict(cu_seqlens=i32(1)), "cu_seqlens"),
    (dict(inv_freq_f64=f64(D // 2 + 1)), "inv_freq_f64"),
    (dict(out=bf(T, HQ, D), out_dtype=ops.YR_F32), "out"),
    (dict(out=bf(T, HQ, 64)), "out"),
    (dict(lse=f32(T, HQ)), "lse"),
    (dict(lse=torch.zeros(HQ, T, dtype=torch.float64)), "lse"),
])
def test_prefill_rejects(kw, frag):
    raises(pre(**kw), frag)


def chk(**kw):
    a = dict(q=bf(T, HQ, D), k_cache=bf(B, LMAX, HKV, D), v_cache=bf(B, LMAX, HKV, D),
             cu_seqlens_q=torch.tensor([0, 10, 20, T], dtype=torch.int32), ctx_lens=i32(B),
             max_seqlen_q=20, inv_freq_f64=f64(), softmax_scale=0.1)
    a.update(kw)
    return lambda: ops.attn_prefill_chunk(**a)


@pytest.mark.parametrize("kw,frag", [
    (dict(ctx_lens=i32(B + 1)), "ctx_lens"),
    (dict(cu_seqlens_q=i32(B)), "cu_seqlens_q"),
    (dict(out=bf(T, HQ, D + 2)), "out"),
    (dict(lse=f32(HQ, T + 1)), "lse"),
    (dict(v_cache=f32(B, LMAX, HKV, D)), "caches must be"),
])
def test_chunk_rejects(kw, frag):
    raises(chk(**kw), frag)


# ---- rope -------------------------------------------------------------------
def test_rope_rejects():
    x = bf(T, HKV, D)
    raises(lambda: ops.rope_apply(x, i32(T + 1), f64()), "positions")
    raises(lambda: ops.rope_apply(x, i32(T), f64(3)), "inv_freq_f64")
    raises(lambda: ops.rope_apply(x, i32(T), f64()), "device tensor")
    cu = torch.tensor([0, T], dtype=torch.int32)
    raises(lambda: ops.rope_apply_packed(x, cu, T, f64(), dst=bf(T, HKV, 64)), "dst")
    raises(lambda: ops.rope_apply_packed(x, cu, T, f64(), dst=f32(T, HKV, D)), "dst")
    raises(lambda: ops.rope_apply_packed(x, cu, T, f64(),
                                         dev_error=torch.zeros(1, dtype=torch.int64)), "dev_error")
    raises(lambda: ops.rope_apply_packed(x, cu, T, f64()), "device tensor")
