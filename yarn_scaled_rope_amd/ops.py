"""ctypes binding of libyarnattn.so with the C entry-point names.

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's kernels.  The
library is loaded on first use (after torch, so that both share one HIP
runtime); if it is missing, every call raises -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

YR_OK = 0
YR_ERR_INVALID = 1
YR_ERR_NULL = 2
YR_ERR_UNSUPPORTED = 3
YR_ERR_WORKSPACE = 4
YR_ERR_HIP = 5
YR_ERR_DEVICE_RANGE = 6

YR_F32 = 0
YR_BF16 = 1
YR_FP8_E4M3 = 2

YR_ROPE_PLAIN = 0
YR_ROPE_PI = 1
YR_ROPE_NTK = 2
YR_ROPE_YARN = 3
METHODS = {"plain": YR_ROPE_PLAIN, "pi": YR_ROPE_PI, "ntk": YR_ROPE_NTK, "yarn": YR_ROPE_YARN}

YR_PREFILL_K_ROTATED = 1
YR_PREFILL_PERMUTED_ORDER = 2

YR_DEVERR_CU_SEQLENS = 1
YR_DEVERR_SEQLENS = 2
YR_DEVERR_QPOS = 4
YR_DEVERR_CTX_LENS = 8

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libyarnattn.so")

_lib = None


class YarnAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


def _declare(lib):
    vp, i, ll, d, f, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_double,
                           ctypes.c_float, ctypes.c_size_t)
    sig = {
        "yarn_rope_freqs": (i, [i, d, d, ll, d, d, i, vp, vp, vp]),
        "yarn_rope_dynamic_ntk_freqs": (i, [i, d, ll, ll, vp, vp, vp]),
        "rope_apply": (i, [vp, i, ll, i, i, vp, vp, vp]),
        "rope_apply_packed": (i, [vp, vp, i, vp, i, i, ll, i, i, vp, vp, vp]),
        "attn_prefill_workspace_bytes": (sz, [ll, i, i, i]),
        "attn_prefill_fwd": (i, [vp, vp, vp, i, vp, i, i, ll, i, i, i, vp, i, f, i, i, vp, i, vp, vp,
                                 sz, vp]),
        "attn_prefill_chunk": (i, [vp, vp, vp, i, vp, vp, i, i, ll, i, i, i, i, vp, f, i, i, vp, i,
                                   vp, vp, sz, vp]),
        "attn_decode_workspace_bytes": (sz, [i, i, i, i]),
        "attn_decode": (i, [vp, vp, vp, i, vp, vp, i, i, i, i, i, vp, f, i, i, vp, i, vp, vp, sz, vp]),
        "attn_decode_fp8": (i, [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp, f, i, i, vp, i, vp, vp,
                                sz, vp]),
        "attn_decode_noalloc": (i, [vp, vp, vp, i, vp, vp, i, i, i, i, i, vp, f, i, i, vp, i, vp, vp,
                                    vp]),
        "yr_read_device_error": (i, [vp, vp, vp]),
        "yr_status_string": (ctypes.c_char_p, [i]),
        "yr_last_error": (ctypes.c_char_p, []),
        "yr_version": (i, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load_library(path: Optional[str] = None):
    """Load (once) and return the ctypes handle.  Raises if the library is not
    built: there is no CPU or PyTorch fallback."""
    global _lib
    if _lib is None:
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise YarnAttnError(-1, f"{p} is missing; build it with "
                                    "`python -m yarn_scaled_rope_amd.build`")
        _lib = _declare(ctypes.CDLL(p))
    return _lib


def _check(status: int):
    if status != YR_OK:
        lib = load_library()
        raise YarnAttnError(status, f"{lib.yr_status_string(status).decode()}: "
                                    f"{lib.yr_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return YR_F32
    if t.dtype == torch.bfloat16:
        return YR_BF16
    raise YarnAttnError(YR_ERR_UNSUPPORTED, f"dtype {t.dtype}")


def _torch_dtype(code: int):
    return torch.float32 if code == YR_F32 else torch.bfloat16


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, numel=None):
    """Host-side checks of one tensor argument (no device access): contiguous,
    of the given dtype, shape and / or element count."""
    if not isinstance(t, torch.Tensor):
        raise YarnAttnError(YR_ERR_INVALID, f"{name} must be a tensor")
    if not t.is_contiguous():
        raise YarnAttnError(YR_ERR_INVALID, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise YarnAttnError(YR_ERR_INVALID, f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise YarnAttnError(YR_ERR_INVALID, f"{name} must have shape {tuple(shape)}, "
                                            f"got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise YarnAttnError(YR_ERR_INVALID, f"{name} must have {numel} elements, got {t.numel()}")


def _ndim(t: torch.Tensor, name: str, n: int):
    if not isinstance(t, torch.Tensor) or t.dim() != n:
        raise YarnAttnError(YR_ERR_INVALID, f"{name} must be a {n}-d tensor")


def _on_device(**tensors):
    """Every given tensor lives in device memory (checked after the shapes, so
    that argument errors are reported the same with or without a GPU)."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise YarnAttnError(YR_ERR_INVALID, f"{name} must be a device tensor")


def _table(inv_freq_f64, D: int):
    if inv_freq_f64 is not None:
        _need(inv_freq_f64, "inv_freq_f64", torch.float64, numel=D // 2)


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


# ------------------------------------------------------------------ freqs
def yarn_rope_freqs(head_dim: int, base: float, factor: float = 1.0,
                    original_max_position: int = 1, alpha: float = 1.0, beta: float = 32.0,
                    method: str = "yarn"):
    """Host call: returns (fp32 table, fp64 table, attention factor t)."""
    lib = load_library()
    f32 = np.zeros(head_dim // 2, dtype=np.float32)
    f64 = np.zeros(head_dim // 2, dtype=np.float64)
    t = ctypes.c_double(0.0)
    _check(lib.yarn_rope_freqs(int(head_dim), float(base), float(factor),
                               int(original_max_position), float(alpha), float(beta),
                               METHODS[method], f32.ctypes.data_as(ctypes.c_void_p),
                               f64.ctypes.data_as(ctypes.c_void_p), ctypes.byref(t)))
    return f32, f64, t.value


def yarn_rope_dynamic_ntk_freqs(head_dim: int, base: float, seq_len: int,
                                original_max_position: int):
    """Host call: Dynamic NTK table for a sequence of seq_len tokens.  Returns
    (fp32 table, fp64 table, factor s)."""
    lib = load_library()
    f32 = np.zeros(head_dim // 2, dtype=np.float32)
    f64 = np.zeros(head_dim // 2, dtype=np.float64)
    s = ctypes.c_double(0.0)
    _check(lib.yarn_rope_dynamic_ntk_freqs(int(head_dim), float(base), int(seq_len),
                                           int(original_max_position),
                                           f32.ctypes.data_as(ctypes.c_void_p),
                                           f64.ctypes.data_as(ctypes.c_void_p), ctypes.byref(s)))
    return f32, f64, s.value


# ------------------------------------------------------------------ rope
def rope_apply(x: torch.Tensor, positions: torch.Tensor, inv_freq_f64: torch.Tensor, stream=None):
    """Rotate x [T, H, D] in place at positions[T] (int32)."""
    _ndim(x, "x", 3)
    _need(x, "x")
    T, H, D = x.shape
    _need(positions, "positions", torch.int32, numel=T)
    if inv_freq_f64 is None:
        raise YarnAttnError(YR_ERR_NULL, "inv_freq_f64 is required")
    _table(inv_freq_f64, D)
    _dtype_code(x)
    _on_device(x=x, positions=positions, inv_freq_f64=inv_freq_f64)
    lib = load_library()
    _check(lib.rope_apply(_ptr(x), _dtype_code(x), T, H, D, _ptr(positions), _ptr(inv_freq_f64),
                          _stream(stream)))
    return x


def rope_apply_packed(src: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                      inv_freq_f64: torch.Tensor, dst: Optional[torch.Tensor] = None,
                      dev_error: Optional[torch.Tensor] = None, stream=None):
    """Rotate the rows of a packed batch [T, H, D] at their in-sequence
    positions into dst (a new tensor by default; may be src)."""
    _ndim(src, "src", 3)
    _need(src, "src")
    T, H, D = src.shape
    _dtype_code(src)
    _ndim(cu_seqlens, "cu_seqlens", 1)
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.numel() < 2:
        raise YarnAttnError(YR_ERR_INVALID, "cu_seqlens needs B+1 >= 2 entries")
    if inv_freq_f64 is None:
        raise YarnAttnError(YR_ERR_NULL, "inv_freq_f64 is required")
    _table(inv_freq_f64, D)
    if dst is not None:
        _need(dst, "dst", src.dtype, shape=src.shape)
    if dev_error is not None:
        _need(dev_error, "dev_error", torch.int32)
        if dev_error.numel() < 1:
            raise YarnAttnError(YR_ERR_INVALID, "dev_error needs one element")
    _on_device(src=src, cu_seqlens=cu_seqlens, inv_freq_f64=inv_freq_f64, dst=dst,
               dev_error=dev_error)
    if dst is None:
        dst = torch.empty_like(src)
    lib = load_library()
    _check(lib.rope_apply_packed(_ptr(src), _ptr(dst), _dtype_code(src), _ptr(cu_seqlens),
                                 cu_seqlens.numel() - 1, int(max_seqlen), T, H, D,
                                 _ptr(inv_freq_f64), _ptr(dev_error), _stream(stream)))
    return dst


# ------------------------------------------------------------------ prefill
def attn_prefill_workspace_bytes(T: int, hkv: int, head_dim: int, in_dtype: int) -> int:
    return int(load_library().attn_prefill_workspace_bytes(T, hkv, head_dim, in_dtype))


def attn_prefill_fwd(q, k, v, cu_seqlens, max_seqlen: int, inv_freq_f64, softmax_scale: float,
                     out=None, out_dtype=None, lse=None, workspace=None, want_lse=True,
                     k_rotated=False, window: int = 0, sinks: int = 0, stream=None,
                     permuted_order=False):
    """Causal prefill.  q [T, Hq, D], k/v [T, Hkv, D] unrotated (or rotated,
    with inv_freq_f64=None; or only k rotated, with k_rotated=True);
    cu_seqlens int32 [B+1]; optional sliding window / sinks.  Returns
    (out, lse)."""
    _ndim(q, "q", 3)
    _ndim(k, "k", 3)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n)
    T, hq, D = q.shape
    hkv = k.shape[1]
    if k.shape != (T, hkv, D) or v.shape != (T, hkv, D) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise YarnAttnError(YR_ERR_INVALID, "k and v must be [T, Hkv, D] of q's dtype")
    in_code = _dtype_code(q)
    _ndim(cu_seqlens, "cu_seqlens", 1)
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.numel() < 2:
        raise YarnAttnError(YR_ERR_INVALID, "cu_seqlens needs B+1 >= 2 entries")
    _table(inv_freq_f64, D)
    out_code = (YR_F32 if in_code == YR_F32 else YR_BF16) if out_dtype is None else out_dtype
    if out_code not in (YR_F32, YR_BF16):
        raise YarnAttnError(YR_ERR_UNSUPPORTED, f"out_dtype {out_code}")
    if out is not None:
        _need(out, "out", _torch_dtype(out_code), shape=(T, hq, D))
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(hq, T))
    key_pass = inv_freq_f64 is not None and not k_rotated
    if workspace is not None:
        _need(workspace, "workspace")
    _on_device(q=q, k=k, v=v, cu_seqlens=cu_seqlens, inv_freq_f64=inv_freq_f64, out=out, lse=lse,
               workspace=workspace)
    if out is None:
        out = torch.empty((T, hq, D), dtype=_torch_dtype(out_code), device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((hq, T), dtype=torch.float32, device=q.device)
    need = attn_prefill_workspace_bytes(T, hkv, D, in_code) if key_pass else 256
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    B = cu_seqlens.numel() - 1
    lib = load_library()
    _check(lib.attn_prefill_fwd(_ptr(q), _ptr(k), _ptr(v), in_code, _ptr(cu_seqlens), B,
                                int(max_seqlen), T, hq, hkv, D, _ptr(inv_freq_f64),
                                (YR_PREFILL_K_ROTATED if k_rotated else 0) |
                                (YR_PREFILL_PERMUTED_ORDER if permuted_order else 0),
                                float(softmax_scale), int(window), int(sinks), _ptr(out), out_code,
                                _ptr(lse), _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return out, lse


def attn_prefill_chunk(q, k_cache, v_cache, cu_seqlens_q, ctx_lens, max_seqlen_q: int,
                       inv_freq_f64, softmax_scale: float, window: int = 0, sinks: int = 0,
                       out=None, out_dtype=None, lse=None, workspace=None, want_lse=True,
                       stream=None):
    """Chunked prefill: new tokens q [Tq, Hq, D] (packed by cu_seqlens_q)
    against caches [B, Lmax, Hkv, D] that already hold ctx_lens[b] earlier
    tokens followed by the chunk's rotated keys and values.  Returns
    (out, lse)."""
    _ndim(q, "q", 3)
    _ndim(k_cache, "k_cache", 4)
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n)
    Tq, hq, D = q.shape
    B, lmax, hkv, _ = k_cache.shape
    if k_cache.shape != (B, lmax, hkv, D) or v_cache.shape != k_cache.shape or \
            k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise YarnAttnError(YR_ERR_INVALID, "caches must be [B, Lmax, Hkv, D] of q's dtype")
    in_code = _dtype_code(q)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, numel=B + 1)
    _need(ctx_lens, "ctx_lens", torch.int32, numel=B)
    _table(inv_freq_f64, D)
    out_code = (YR_F32 if in_code == YR_F32 else YR_BF16) if out_dtype is None else out_dtype
    if out_code not in (YR_F32, YR_BF16):
        raise YarnAttnError(YR_ERR_UNSUPPORTED, f"out_dtype {out_code}")
    if out is not None:
        _need(out, "out", _torch_dtype(out_code), shape=(Tq, hq, D))
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(hq, Tq))
    if workspace is not None:
        _need(workspace, "workspace")
    _on_device(q=q, k_cache=k_cache, v_cache=v_cache, cu_seqlens_q=cu_seqlens_q,
               ctx_lens=ctx_lens, inv_freq_f64=inv_freq_f64, out=out, lse=lse,
               workspace=workspace)
    if out is None:
        out = torch.empty((Tq, hq, D), dtype=_torch_dtype(out_code), device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((hq, Tq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(256, dtype=torch.uint8, device=q.device)
    lib = load_library()
    _check(lib.attn_prefill_chunk(_ptr(q), _ptr(k_cache), _ptr(v_cache), in_code,
                                  _ptr(cu_seqlens_q), _ptr(ctx_lens), B, int(max_seqlen_q), Tq,
                                  lmax, hq, hkv, D, _ptr(inv_freq_f64), float(softmax_scale),
                                  int(window), int(sinks), _ptr(out), out_code, _ptr(lse),
                                  _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return out, lse


# ------------------------------------------------------------------ decode
def attn_decode_workspace_bytes(B: int, max_cache_len: int, hq: int, head_dim: int) -> int:
    return int(load_library().attn_decode_workspace_bytes(B, max_cache_len, hq, head_dim))


def _decode_checks(q, k_cache, v_cache, seqlens, q_pos, inv_freq_f64, out, out_code, lse,
                   workspace, cache_dtype):
    """Shapes and dtypes of a decode call (host side, before any launch)."""
    _ndim(q, "q", 3)
    _ndim(k_cache, "k_cache", 4)
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n)
    B, hq, D = q.shape
    _, lmax, hkv, _ = k_cache.shape
    if k_cache.shape != (B, lmax, hkv, D) or v_cache.shape != k_cache.shape:
        raise YarnAttnError(YR_ERR_INVALID, "caches must be [B, Lmax, Hkv, D]")
    if k_cache.dtype != cache_dtype or v_cache.dtype != cache_dtype:
        raise YarnAttnError(YR_ERR_INVALID, f"caches must be {cache_dtype}")
    _need(seqlens, "seqlens", torch.int32, numel=B)
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int32, numel=B)
    _table(inv_freq_f64, D)
    if out_code not in (YR_F32, YR_BF16):
        raise YarnAttnError(YR_ERR_UNSUPPORTED, f"out_dtype {out_code}")
    if out is not None:
        _need(out, "out", _torch_dtype(out_code), shape=(B, hq, D))
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(B, hq))
    if workspace is not None:
        _need(workspace, "workspace")
    _on_device(q=q, k_cache=k_cache, v_cache=v_cache, seqlens=seqlens, q_pos=q_pos,
               inv_freq_f64=inv_freq_f64, out=out, lse=lse, workspace=workspace)
    return B, hq, D, lmax, hkv


def attn_decode(q, k_cache, v_cache, seqlens, inv_freq_f64, softmax_scale: float, q_pos=None,
                out=None, out_dtype=None, lse=None, workspace=None, want_lse=True,
                window: int = 0, sinks: int = 0, stream=None):
    """One query per sequence over a contiguous cache.  q [B, Hq, D];
    caches [B, Lmax, Hkv, D] of q's dtype; seqlens int32 [B]; optional
    sliding window / sinks.  Returns (out, lse)."""
    _ndim(q, "q", 3)
    in_code = _dtype_code(q)
    out_code = (YR_F32 if in_code == YR_F32 else YR_BF16) if out_dtype is None else out_dtype
    B, hq, D, lmax, hkv = _decode_checks(q, k_cache, v_cache, seqlens, q_pos, inv_freq_f64, out,
                                         out_code, lse, workspace, q.dtype)
    if out is None:
        out = torch.empty((B, hq, D), dtype=_torch_dtype(out_code), device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(attn_decode_workspace_bytes(B, lmax, hq, D), dtype=torch.uint8,
                                device=q.device)
    lib = load_library()
    _check(lib.attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), in_code, _ptr(seqlens),
                           _ptr(q_pos), B, lmax, hq, hkv, D, _ptr(inv_freq_f64),
                           float(softmax_scale), int(window), int(sinks), _ptr(out), out_code,
                           _ptr(lse), _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return out, lse


def attn_decode_noalloc(q, k_cache, v_cache, seqlens, inv_freq_f64, softmax_scale: float,
                        out, lse=None, q_pos=None, dev_error=None, window: int = 0,
                        sinks: int = 0, stream=None):
    """attn_decode without a workspace: the library's fixed per-device scratch
    holds the partials, and nothing is allocated (the caller passes `out`,
    and `lse` if wanted).  Calls that may overlap on one device race on that
    scratch.  Returns (out, lse)."""
    _ndim(q, "q", 3)
    in_code = _dtype_code(q)
    if out is None:
        raise YarnAttnError(YR_ERR_NULL, "out is required (nothing is allocated)")
    out_code = _dtype_code(out)
    _decode_checks(q, k_cache, v_cache, seqlens, q_pos, inv_freq_f64, out, out_code, lse, None,
                   q.dtype)
    if dev_error is not None:
        _need(dev_error, "dev_error", torch.int32)
        _on_device(dev_error=dev_error)
    B, hq, D = q.shape
    _, lmax, hkv, _ = k_cache.shape
    lib = load_library()
    _check(lib.attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), in_code, _ptr(seqlens),
                                   _ptr(q_pos), B, lmax, hq, hkv, D, _ptr(inv_freq_f64),
                                   float(softmax_scale), int(window), int(sinks), _ptr(out),
                                   out_code, _ptr(lse), _ptr(dev_error), _stream(stream)))
    return out, lse


def attn_decode_fp8(q, k_cache, v_cache, k_scale, v_scale, seqlens, inv_freq_f64,
                    softmax_scale: float, q_pos=None, out=None, out_dtype=None, lse=None,
                    workspace=None, want_lse=True, window: int = 0, sinks: int = 0, stream=None):
    """attn_decode over an FP8 (E4M3) cache: q bf16 [B, Hq, D]; caches uint8
    [B, Lmax, Hkv, D] of E4M3 codes standing for code * k_scale[h] /
    code * v_scale[h] (float32 [Hkv]).  Returns (out, lse)."""
    _ndim(q, "q", 3)
    _need(q, "q", torch.bfloat16)
    _ndim(k_cache, "k_cache", 4)
    _need(k_scale, "k_scale", torch.float32, numel=k_cache.shape[2])
    _need(v_scale, "v_scale", torch.float32, numel=k_cache.shape[2])
    out_code = YR_BF16 if out_dtype is None else out_dtype
    B, hq, D, lmax, hkv = _decode_checks(q, k_cache, v_cache, seqlens, q_pos, inv_freq_f64, out,
                                         out_code, lse, workspace, torch.uint8)
    _on_device(k_scale=k_scale, v_scale=v_scale)
    if out is None:
        out = torch.empty((B, hq, D), dtype=_torch_dtype(out_code), device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(attn_decode_workspace_bytes(B, lmax, hq, D), dtype=torch.uint8,
                                device=q.device)
    lib = load_library()
    _check(lib.attn_decode_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                               _ptr(v_scale), _ptr(seqlens), _ptr(q_pos), B, lmax, hq, hkv, D,
                               _ptr(inv_freq_f64), float(softmax_scale), int(window), int(sinks),
                               _ptr(out), out_code, _ptr(lse), _ptr(workspace),
                               _nbytes(workspace), _stream(stream)))
    return out, lse


def read_device_error(workspace: torch.Tensor, stream=None) -> int:
    """Synchronise and return the device error bits of a workspace."""
    flags = ctypes.c_int(0)
    lib = load_library()
    st = lib.yr_read_device_error(_ptr(workspace), _stream(stream), ctypes.byref(flags))
    if st not in (YR_OK, YR_ERR_DEVICE_RANGE):
        _check(st)
    return flags.value
