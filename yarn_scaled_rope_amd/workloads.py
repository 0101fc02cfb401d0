"""Seeded synthetic workloads and algorithmic work counts.

This module holds no part of the attention method: it draws the inputs (the
same bits go to the GPU library and to the CPU checker) and counts the
algorithmic work that throughput is quoted on.

Input recipe: ``numpy.random.Generator(PCG64(1000 + index))``; for the decode
workload the cache lengths are drawn first; then Q, K and V are drawn as
float32 standard normals in their storage layouts, in that order, and rounded
once to bfloat16 (round to nearest, ties to even) except for the fp32
workload.  The decode cache draws K rows of sequence 0, 1, ... then V rows in
the same order; cache rows past a sequence's length are NaN so any read
beyond ``seqlens`` shows up in the output.

Shapes follow the attention layers of the models the pages use for their
worked figures (Llama-2-7B, Llama-3-8B at 128K, Llama-3-70B, GQA with 8 KV
heads).
"""

from __future__ import annotations

import dataclasses

import numpy as np

BF16_NAN_BITS = 0x7FC0
_CHUNK = 1 << 24          # elements per generation chunk (bounds host memory)


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    index: int
    seq_lens: tuple
    hq: int
    hkv: int
    head_dim: int
    dtype: str                 # "f32" or "bf16" (input storage type)
    base: float
    factor: float
    original_max_position: int
    window: int = 0            # sliding window (0 = plain causal)
    sinks: int = 0

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def max_seqlen(self) -> int:
        return int(max(self.seq_lens))


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    index: int
    batch: int
    max_cache_len: int
    min_cache_len: int
    hq: int
    hkv: int
    head_dim: int
    dtype: str
    base: float
    factor: float
    original_max_position: int
    window: int = 0
    sinks: int = 0


@dataclasses.dataclass(frozen=True)
class ChunkConfig:
    """Chunked prefill: chunk_lens[b] new tokens after ctx_lens[b] cached ones,
    caches [B, max_cache_len, Hkv, D]."""
    name: str
    index: int
    ctx_lens: tuple
    chunk_lens: tuple
    max_cache_len: int
    hq: int
    hkv: int
    head_dim: int
    dtype: str
    base: float
    factor: float
    original_max_position: int
    window: int = 0
    sinks: int = 0


TINY_F32 = PrefillConfig("tiny_fp32_prefill", 0, (256,), 4, 2, 64, "f32",
                         10000.0, 4.0, 64)
LLAMA2_7B_16K = PrefillConfig("llama2_7b_prefill_16k", 1, (16384,), 32, 32,
                              128, "bf16", 10000.0, 4.0, 4096)
LLAMA3_8B_128K = PrefillConfig("llama3_8b_gqa_prefill_128k", 2, (131072,),
                               32, 8, 128, "bf16", 500000.0, 8.0, 16384)
DECODE_B16 = DecodeConfig("decode_b16_gqa_32k_128k", 3, 16, 131072, 32768,
                          32, 8, 128, "bf16", 500000.0, 8.0, 16384)
LLAMA3_70B_RAGGED = PrefillConfig("llama3_70b_ragged_prefill", 4,
                                  (131072, 65537, 32000, 4097), 64, 8, 128,
                                  "bf16", 500000.0, 8.0, 16384)

# Chunked prefill: 4 sequences, each a 4096-token chunk after a cached prefix
# of 28K .. 124K tokens (Llama-3-8B GQA attention layer).
CHUNK_4X4K = ChunkConfig("llama3_8b_chunked_prefill_4x4k", 5, (28672, 61440, 94208, 126976),
                         (4096, 4096, 4096, 4096), 131072, 32, 8, 128, "bf16", 500000.0, 8.0,
                         16384)
# Sliding window of 4096 tokens plus 4 sink tokens ("effective context = 4 +
# last 4096") on the 16K MHA prefill and on the 16-sequence decode.
LLAMA2_7B_16K_SWA = PrefillConfig("llama2_7b_prefill_16k_window4k_sinks4", 6, (16384,), 32, 32,
                                  128, "bf16", 10000.0, 4.0, 4096, window=4096, sinks=4)
DECODE_B16_SWA = DecodeConfig("decode_b16_gqa_window4k_sinks4", 7, 16, 131072, 32768, 32, 8,
                              128, "bf16", 500000.0, 8.0, 16384, window=4096, sinks=4)

# Many sequences: 256 caches of 512 .. 4096 tokens (Llama-3-8B GQA layer),
# a serving batch of many short caches.
DECODE_B256 = DecodeConfig("decode_b256_gqa_512_4k", 9, 256, 4096, 512, 32, 8, 128, "bf16",
                           500000.0, 8.0, 16384)

PREFILL_CONFIGS = {c.name: c for c in (TINY_F32, LLAMA2_7B_16K, LLAMA3_8B_128K,
                                       LLAMA3_70B_RAGGED, LLAMA2_7B_16K_SWA)}
DECODE_CONFIGS = {c.name: c for c in (DECODE_B16, DECODE_B16_SWA, DECODE_B256)}
CHUNK_CONFIGS = {CHUNK_4X4K.name: CHUNK_4X4K}


# ---------------------------------------------------------------- bf16 bits
def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.
    Inputs are finite standard normals, so no NaN/Inf handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def as_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """The exact fp64 values of stored inputs."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def _draw(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """Standard normals of the given shape, stored as float32 (fp32 workloads)
    or bf16 bits; drawn in row-major chunks from the one generator."""
    n = int(np.prod(shape))
    if dtype == "f32":
        return rng.standard_normal(n, dtype=np.float32).reshape(shape)
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = round_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def cu_seqlens_of(seq_lens) -> np.ndarray:
    cu = np.zeros(len(seq_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(seq_lens, dtype=np.int64))
    return cu


def make_prefill(cfg: PrefillConfig, seed: int | None = None, seq_lens=None, q_tokens=None):
    """Packed ragged prefill inputs: q [T, Hq, D], k, v [T, Hkv, D].

    q_tokens (optional): only these token rows of q are drawn (in ascending
    order, before k and v); every other row of q is zero.  For batches whose
    q is too large to draw in full when only a few rows are checked."""
    lens = tuple(cfg.seq_lens if seq_lens is None else seq_lens)
    rng = np.random.Generator(np.random.PCG64(1000 + cfg.index if seed is None else seed))
    T = int(sum(lens))
    if q_tokens is None:
        q = _draw(rng, (T, cfg.hq, cfg.head_dim), cfg.dtype)
    else:
        toks = np.unique(np.asarray(q_tokens, dtype=np.int64))
        assert toks.size == 0 or (toks[0] >= 0 and toks[-1] < T)
        q = np.zeros((T, cfg.hq, cfg.head_dim), dtype=np.uint16 if cfg.dtype == "bf16"
                     else np.float32)
        q[toks] = _draw(rng, (toks.size, cfg.hq, cfg.head_dim), cfg.dtype)
    k = _draw(rng, (T, cfg.hkv, cfg.head_dim), cfg.dtype)
    v = _draw(rng, (T, cfg.hkv, cfg.head_dim), cfg.dtype)
    return {"q": q, "k": k, "v": v, "cu_seqlens": cu_seqlens_of(lens),
            "seq_lens": lens, "dtype": cfg.dtype}


def _seqlens(rng, B, lmin, lmax, seqlens):
    """Cache lengths ~ U{lmin..lmax}, or the given ones (then nothing is drawn
    for them)."""
    if seqlens is None:
        return rng.integers(lmin, lmax, size=B, endpoint=True).astype(np.int32)
    out = np.asarray(seqlens, dtype=np.int32)
    assert out.shape == (B,) and np.all(out >= 0) and np.all(out <= lmax)
    return out


def make_decode(cfg: DecodeConfig, seed: int | None = None, batch=None,
                max_cache_len=None, min_cache_len=None, seqlens=None):
    """Decode inputs: q [B, Hq, D]; k_cache, v_cache [B, Lmax, Hkv, D] with
    NaN rows past each sequence's length; seqlens [B] ~ U{min..max} unless
    given."""
    B = cfg.batch if batch is None else batch
    lmax = cfg.max_cache_len if max_cache_len is None else max_cache_len
    lmin = cfg.min_cache_len if min_cache_len is None else min_cache_len
    rng = np.random.Generator(np.random.PCG64(1000 + cfg.index if seed is None else seed))
    seqlens = _seqlens(rng, B, lmin, lmax, seqlens)
    q = _draw(rng, (B, cfg.hq, cfg.head_dim), cfg.dtype)
    caches = []
    for _ in range(2):
        if cfg.dtype == "bf16":
            c = np.full((B, lmax, cfg.hkv, cfg.head_dim), BF16_NAN_BITS, dtype=np.uint16)
        else:
            c = np.full((B, lmax, cfg.hkv, cfg.head_dim), np.nan, dtype=np.float32)
        for b in range(B):
            c[b, :seqlens[b]] = _draw(rng, (int(seqlens[b]), cfg.hkv, cfg.head_dim), cfg.dtype)
        caches.append(c)
    return {"q": q, "k_cache": caches[0], "v_cache": caches[1],
            "seqlens": seqlens, "dtype": cfg.dtype}


E4M3_NAN_CODE = 0x7F


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 values -> OCP E4M3 byte codes (round to nearest even, by
    torch's float8_e4m3fn conversion); callers keep |x| <= 448."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def make_decode_fp8(cfg: DecodeConfig, seed: int | None = None, batch=None, max_cache_len=None,
                    min_cache_len=None, seqlens=None):
    """FP8-cache decode inputs: the cache lengths, q (bf16) and K/V values
    drawn like make_decode; per-KV-head scales 2^-6 * (1 + h/4) for K and
    2^-6 * (1 + h/8) for V; each cache element stored as the E4M3 code of
    value / scale; rows past a sequence's length hold the NaN code.  The
    cache lengths are drawn as in make_decode unless given."""
    B = cfg.batch if batch is None else batch
    lmax = cfg.max_cache_len if max_cache_len is None else max_cache_len
    lmin = cfg.min_cache_len if min_cache_len is None else min_cache_len
    rng = np.random.Generator(np.random.PCG64(1000 + cfg.index if seed is None else seed))
    seqlens = _seqlens(rng, B, lmin, lmax, seqlens)
    q = _draw(rng, (B, cfg.hq, cfg.head_dim), "bf16")
    h = np.arange(cfg.hkv, dtype=np.float32)
    scales = [(np.float32(2.0 ** -6) * (1.0 + h / 4.0)).astype(np.float32),
              (np.float32(2.0 ** -6) * (1.0 + h / 8.0)).astype(np.float32)]
    caches = []
    for sc in scales:
        c = np.full((B, lmax, cfg.hkv, cfg.head_dim), E4M3_NAN_CODE, dtype=np.uint8)
        for b in range(B):
            L = int(seqlens[b])
            x = _draw(rng, (L, cfg.hkv, cfg.head_dim), "f32")
            c[b, :L] = e4m3_codes(x / sc[None, :, None])
        caches.append(c)
    return {"q": q, "k_cache": caches[0], "v_cache": caches[1], "k_scale": scales[0],
            "v_scale": scales[1], "seqlens": seqlens, "dtype": "bf16"}


def make_chunk(cfg: ChunkConfig, seed: int | None = None, ctx_lens=None, chunk_lens=None,
               max_cache_len=None):
    """Chunked-prefill inputs: q [Tq, Hq, D] for the new tokens (packed);
    k_cache, v_cache [B, Lmax, Hkv, D] whose rows 0 .. ctx_b + n_b - 1 are
    drawn (K taken as already rotated) and the rest NaN.  Draw order: q, then
    the K rows of sequence 0, 1, ..., then the V rows."""
    ctx = tuple(cfg.ctx_lens if ctx_lens is None else ctx_lens)
    lens = tuple(cfg.chunk_lens if chunk_lens is None else chunk_lens)
    lmax = cfg.max_cache_len if max_cache_len is None else max_cache_len
    B = len(lens)
    rng = np.random.Generator(np.random.PCG64(1000 + cfg.index if seed is None else seed))
    Tq = int(sum(lens))
    q = _draw(rng, (Tq, cfg.hq, cfg.head_dim), cfg.dtype)
    caches = []
    for _ in range(2):
        if cfg.dtype == "bf16":
            c = np.full((B, lmax, cfg.hkv, cfg.head_dim), BF16_NAN_BITS, dtype=np.uint16)
        else:
            c = np.full((B, lmax, cfg.hkv, cfg.head_dim), np.nan, dtype=np.float32)
        for b in range(B):
            rows = ctx[b] + lens[b]
            c[b, :rows] = _draw(rng, (rows, cfg.hkv, cfg.head_dim), cfg.dtype)
        caches.append(c)
    return {"q": q, "k_cache": caches[0], "v_cache": caches[1], "cu_seqlens_q": cu_seqlens_of(lens),
            "ctx_lens": np.asarray(ctx, dtype=np.int32), "chunk_lens": lens, "dtype": cfg.dtype,
            "max_cache_len": lmax}


def sample_rows(seq_lens, hq: int, hkv: int, n_random: int = 32, seed: int = 7,
                edge_tiles=(32, 64, 128, 256), edge_span: int = 4):
    """A seeded sample of (token, head) rows of a packed batch for checks at
    sizes where the dense CPU result is too slow: per (sequence, KV group),
    every query head of the group at rows 0-3, every tile edge (and its
    neighbours) in the first ``edge_span`` tiles of each tile size, the last
    three rows, every row of a partial last tile, and ``n_random`` random
    rows."""
    rng = np.random.Generator(np.random.PCG64(seed))
    g = hq // hkv
    out = []
    start = 0
    for n in seq_lens:
        picks = set(range(min(4, n)))
        for tsz in edge_tiles:
            for e in range(1, edge_span + 1):
                for dlt in (-1, 0, 1):
                    r = e * tsz + dlt
                    if 0 <= r < n:
                        picks.add(r)
        picks.update(range(max(0, n - 3), n))
        tail = n % 128
        if tail:
            picks.update(range(n - tail, n))
        for hk in range(hkv):
            rr = set(picks)
            if n > 0:
                rr.update(int(x) for x in rng.integers(0, n, size=n_random))
            for r in sorted(rr):
                for h in range(hk * g, (hk + 1) * g):
                    out.append((start + r, h))
        start += n
    return out


def tile_edge_rows(seq_lens, hq: int, hkv: int, group: int, tile: int = 256):
    """(token, head) rows of one KV group: the first and last row of every
    `tile`-row block of every sequence, for all query heads of the group."""
    g = hq // hkv
    out = []
    start = 0
    for n in seq_lens:
        for r0 in range(0, n, tile):
            for r in sorted({r0, min(n, r0 + tile) - 1}):
                for h in range(group * g, (group + 1) * g):
                    out.append((start + r, h))
        start += n
    return out


# ------------------------------------------------------- algorithmic counts
def prefill_causal_flops(seq_lens, hq: int, head_dim: int) -> int:
    """Algorithmic FLOPs of causal prefill: QK^T and PV (2 FLOP per
    multiply-add each) over every visible (query, key) pair, diagonal
    included: 4 * D * Hq * sum n(n+1)/2."""
    pairs = sum(int(n) * (int(n) + 1) // 2 for n in seq_lens)
    return 4 * int(head_dim) * int(hq) * pairs


def visible_keys(positions, window: int = 0, sinks: int = 0) -> np.ndarray:
    """Number of keys a query at each position attends to: every earlier
    position and itself, or with a window W the min(m+1, W) most recent plus
    the sinks that lie before the window."""
    m = np.asarray(positions, dtype=np.int64)
    if window <= 0:
        return m + 1
    return np.minimum(m + 1, window) + np.minimum(sinks, np.maximum(0, m - window + 1))


def prefill_visible_flops(seq_lens, hq: int, head_dim: int, window: int = 0, sinks: int = 0,
                          ctx_lens=None) -> int:
    """Algorithmic FLOPs (4 * D per visible (query, key) pair per query head)
    of prefill with a window / sinks, or of a chunk after ctx_lens cached
    tokens (positions start there)."""
    pairs = 0
    for b, n in enumerate(seq_lens):
        p0 = 0 if ctx_lens is None else int(ctx_lens[b])
        pairs += int(np.sum(visible_keys(np.arange(p0, p0 + int(n)), window, sinks)))
    return 4 * int(head_dim) * int(hq) * pairs


def decode_visible_bytes(seqlens, hkv: int, head_dim: int, window: int = 0, sinks: int = 0,
                         q_pos=None, elem_bytes: int = 2) -> int:
    """K+V bytes a windowed decode step must read: the cache rows visible
    from the query's position (default: the cache length)."""
    rows = 0
    for b, L in enumerate(seqlens):
        L = int(L)
        m = L if q_pos is None else int(q_pos[b])
        if window <= 0:
            rows += L
        else:
            lo = max(0, m - window + 1)
            rows += max(0, L - lo) + min(sinks, lo, L)
    return 2 * int(hkv) * int(head_dim) * int(elem_bytes) * rows


def dense_attention_flops(seq_len: int, head_dim: int, heads: int = 1) -> int:
    """Non-causal QK^T + PV FLOPs: 4 * T^2 * d per head."""
    return 4 * int(seq_len) ** 2 * int(head_dim) * int(heads)


def decode_kv_bytes(seqlens, hkv: int, head_dim: int, elem_bytes: int = 2) -> int:
    """Bytes of K and V one decode step must read: 2 * Hkv * D * bytes per
    cached token."""
    return 2 * int(hkv) * int(head_dim) * int(elem_bytes) * int(np.sum(np.asarray(seqlens, dtype=np.int64)))


def kv_cache_bytes(n_layers, n_kv_heads, head_dim, seq_len, batch=1, dtype_bytes=2) -> int:
    """Whole-model KV cache size: layers * KV heads * head dim * 2 (K and V)
    * tokens * batch * bytes per element."""
    return (int(n_layers) * int(n_kv_heads) * int(head_dim) * 2 * int(seq_len)
            * int(batch) * int(dtype_bytes))


def score_matrix_bytes(seq_len: int, heads: int, dtype_bytes: int = 2) -> int:
    """Bytes of a materialised T x T score matrix for all heads."""
    return int(seq_len) ** 2 * int(heads) * int(dtype_bytes)


def ceil_div(a: int, b: int) -> int:
    return -(-int(a) // int(b))


def mean_decode_bytes(cfg: DecodeConfig, elem_bytes: int = 2) -> float:
    """Expected K+V bytes of the decode workload for uniform cache lengths."""
    mean_len = (cfg.min_cache_len + cfg.max_cache_len) / 2.0
    return cfg.batch * mean_len * 2 * cfg.hkv * cfg.head_dim * elem_bytes

