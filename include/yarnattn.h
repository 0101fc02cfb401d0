/*
 * yarnattn.h -- C ABI of libyarnattn.so: YaRN-scaled RoPE causal attention
 * for AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every function returns an int status (YR_OK = 0) and never throws or
 *    aborts.  yr_status_string() names a status; yr_last_error() gives the
 *    calling thread's message for its last failing call.
 *  - Arguments are checked on the host before anything is launched; a failed
 *    check launches nothing and writes nothing.
 *  - Device pointers are caller-owned.  The library never allocates, frees or
 *    synchronises: every launch is asynchronous on the caller's stream
 *    (`stream` is a hipStream_t passed as void*; NULL is the null stream).
 *    Scratch memory comes in as `workspace`, sized by the matching
 *    *_workspace_bytes() query; its first 256 bytes are a header the kernels
 *    use for a device-side error word.
 *  - Values that only the device sees (cu_seqlens, seqlens, q_pos) are range
 *    checked by the kernels: out-of-range values are clamped so that no
 *    access leaves its buffer, and a flag is raised in the workspace header;
 *    yr_read_device_error() reads it back.  Nothing is silently truncated
 *    without that flag.
 *  - Layouts are dense row-major with the last dimension contiguous.
 *    Element types: YR_F32 (float) or YR_BF16 (bfloat16 bit patterns).
 *  - Thread safety: the library keeps no global state besides the per-thread
 *    error message, per-device constants it looks up once, and the fixed
 *    scratch of attn_decode_noalloc; concurrent calls are safe when their
 *    outputs and workspaces do not overlap (attn_decode_noalloc: see there).
 *
 * Sources are cited by page title and section ("Arch 03 -- Long Context"
 * slide deck; "Long-context models", blog.ecitis.org; "LLM context window
 * mechanics", randomcommits.com; "Long context (engineering 100k+ tokens)",
 * askaiml academy).
 */
#ifndef YARNATTN_H
#define YARNATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The entry points below are the library's only exported symbols (it is
   built with hidden visibility by default). */
#if defined(__GNUC__)
#pragma GCC visibility push(default)
#endif

/* ---- status codes ------------------------------------------------------ */
#define YR_OK 0
#define YR_ERR_INVALID 1      /* an argument is out of range or inconsistent  */
#define YR_ERR_NULL 2         /* a required pointer is NULL                    */
#define YR_ERR_UNSUPPORTED 3  /* valid, but not provided (head_dim, dtype pair) */
#define YR_ERR_WORKSPACE 4    /* workspace missing or smaller than required    */
#define YR_ERR_HIP 5          /* the HIP runtime reported an error             */
#define YR_ERR_DEVICE_RANGE 6 /* device-side range check failed (see below)    */

/* ---- element types ----------------------------------------------------- */
#define YR_F32 0
#define YR_BF16 1
#define YR_FP8_E4M3 2 /* OCP 8-bit float, 4 exponent / 3 mantissa bits (decode caches only) */

/* ---- frequency rules --------------------------------------------------- */
#define YR_ROPE_PLAIN 0 /* theta_i = base^(-2i/d)                          */
#define YR_ROPE_PI 1    /* theta_i / s                                     */
#define YR_ROPE_NTK 2   /* plain rule over base * s^(d/(d-2))              */
#define YR_ROPE_YARN 3  /* wavelength-ratio ramp between theta/s and theta */

/* ---- device error bits (yr_read_device_error) -------------------------- */
#define YR_DEVERR_CU_SEQLENS 1 /* cu_seqlens not 0 = c0 <= c1 <= ... <= cB = T, or a length > max_seqlen */
#define YR_DEVERR_SEQLENS 2    /* a decode seqlens[b] outside [1, max_cache_len] */
#define YR_DEVERR_QPOS 4       /* a decode q_pos[b] < 0                           */
#define YR_DEVERR_CTX_LENS 8   /* a chunked-prefill ctx_lens[b] < 0 or ctx_lens[b] + n_b > max_cache_len */

/* Bytes at the start of every workspace reserved for the device error word. */
#define YR_WORKSPACE_HEADER_BYTES 256

/*
 * yarn_rope_freqs -- host-only: the rotary frequency table and the logit
 * temperature.
 *
 * "Arch 03 -- Long Context": RoPE slide (theta_i = base^(-2i/d), one per
 * feature pair (2i, 2i+1)), Position Interpolation slide (theta_i / s),
 * NTK-aware slide (base * s^(d/(d-2))), YaRN slide and steps table (wavelength
 * lambda_i = 2 pi / theta_i; alpha = 1, beta = 32; temperature
 * t = 0.1 ln(s) + 1).  For YR_ROPE_YARN with r_i = L / lambda_i
 * (L = original_max_position): r_i >= beta keeps theta_i, r_i <= alpha gives
 * theta_i / s, and in between theta_i/s + gamma (theta_i - theta_i/s) with
 * gamma = (r_i - alpha) / (beta - alpha).  All arithmetic is fp64; the fp32
 * table is the round-to-nearest-even of the fp64 table.
 *
 *   head_dim               even, 2..1024 (rotary dim = head dim); >= 4 for
 *                          YR_ROPE_NTK (d/(d-2) is undefined at d = 2)
 *   base                   > 1
 *   factor                 s >= 1 (ignored by YR_ROPE_PLAIN)
 *   original_max_position  L >= 1 (YR_ROPE_YARN only)
 *   alpha, beta            0 <= alpha < beta (YR_ROPE_YARN only)
 *   inv_freq_f32           host float[head_dim/2] or NULL
 *   inv_freq_f64           host double[head_dim/2] or NULL (the table the
 *                          kernels take, after the caller copies it to the
 *                          device)
 *   attn_factor            host double or NULL: t for YaRN, 1 otherwise
 */
int yarn_rope_freqs(int head_dim, double base, double factor,
                    long long original_max_position, double alpha, double beta,
                    int method, float *inv_freq_f32, double *inv_freq_f64,
                    double *attn_factor);

/*
 * yarn_rope_dynamic_ntk_freqs -- host-only: the Dynamic NTK table for a
 * sequence of seq_len tokens ("Arch 03 -- Long Context", NTK-aware slide:
 * at inference the factor is set to the current sequence length over the
 * training length).  s = max(1, seq_len / original_max_position) (real
 * division), then the YR_ROPE_NTK table for that s (plain RoPE over the base
 * base * s^(d/(d-2))).  At or below the training length s = 1 and the table
 * is the plain one bit for bit.  The logit temperature stays 1 (only YaRN
 * rescales logits).  A caller re-derives the table when the sequence grows.
 *
 *   head_dim               even, 4..1024;  base > 1
 *   seq_len                >= 0, the current sequence length
 *   original_max_position  L_train >= 1
 *   inv_freq_f32, inv_freq_f64   host tables of head_dim/2 entries or NULL
 *   factor                 host double or NULL: receives s
 */
int yarn_rope_dynamic_ntk_freqs(int head_dim, double base, long long seq_len,
                                long long original_max_position, float *inv_freq_f32,
                                double *inv_freq_f64, double *factor);

/*
 * rope_apply -- rotate x in place: pair (2i, 2i+1) of row t turns by
 * positions[t] * theta_i with R = [[cos, -sin], [sin, cos]] ("Arch 03 --
 * Long Context", RoPE slide; "Long-context models", "Position enters
 * attention").  The angle is formed and reduced modulo 2 pi in fp64; the
 * rotation is applied in fp32 and bf16 results are rounded to nearest even.
 *
 *   x             device [T, H, head_dim], dtype YR_F32 or YR_BF16, in place
 *   positions     device int32[T] (any value >= 0)
 *   inv_freq_f64  device double[head_dim/2]
 *   head_dim      even, 2..512
 */
int rope_apply(void *x, int dtype, long long T, int H, int head_dim,
               const int *positions, const double *inv_freq_f64, void *stream);

/*
 * rope_apply_packed -- rotate the rows of a packed ragged batch at their
 * 0-based position inside their own sequence (row t of sequence b sits at
 * t - cu_seqlens[b]), out of place (dst may equal src).  Same rotation as
 * rope_apply.  It is the key pass of prefill, and the way to fill a KV cache
 * with rotated keys.
 *
 *   src, dst      device [T, H, head_dim], dtype YR_F32 or YR_BF16
 *   cu_seqlens    device int32[B+1], checked like attn_prefill_fwd's
 *   dev_error     device int or NULL: receives the YR_DEVERR_CU_SEQLENS bit
 *                 (0 when cu_seqlens is well formed)
 *   head_dim      even, 2..512
 */
int rope_apply_packed(const void *src, void *dst, int dtype, const int *cu_seqlens, int B,
                      int max_seqlen, long long T, int H, int head_dim,
                      const double *inv_freq_f64, int *dev_error, void *stream);

/* attn_prefill_fwd flags */
#define YR_PREFILL_K_ROTATED 1 /* k already holds rotated keys (e.g. from
                                  rope_apply_packed or a rotated cache): no key
                                  pass; queries are still rotated on load when
                                  inv_freq_f64 != NULL */
#define YR_PREFILL_PERMUTED_ORDER 2 /* bf16 path: the workgroups take their work
                                  items (q-tile, sequence, head) in a permuted
                                  order instead of longest first.  Results are
                                  bit-identical (each item is computed alone);
                                  it exists to test that, and is slower. */

/* Workspace bytes attn_prefill_fwd needs for these sizes (with flags = 0). */
size_t attn_prefill_workspace_bytes(long long T, int Hkv, int head_dim, int in_dtype);

/*
 * attn_prefill_fwd -- causal prefill over a packed ragged batch: out and LSE.
 *
 * For each sequence b (rows cu_seqlens[b] .. cu_seqlens[b+1]-1, positions
 * restarting at 0) and query head h with KV head h / (Hq / Hkv): q and k are
 * rotated at their positions, z = softmax_scale * q~ . k~ for keys at or
 * before the query ("Arch 03 -- Long Context", attention slide and the causal
 * rule i - j >= 0 on the ALiBi slide), out = softmax(z) v and
 * lse = ln sum exp(z).  The softmax runs tiled and online ("Long-context
 * models", "Context parallelism distributes exact attention": per-row maxima,
 * sums and output accumulators); no T x T score matrix is ever stored.
 * Pass softmax_scale = t / sqrt(head_dim) for YaRN.
 *
 * Sliding window and sinks: with window = W > 0 a query at position m sees
 * only keys at m-W+1 .. m ("Arch 03 -- Long Context", sliding-window slide:
 * each token attends to the W most recent tokens), plus the first `sinks`
 * positions ("Long context (engineering 100k+ tokens)", attention sinks:
 * keep the first tokens and the last W).  window = 0 is plain causal
 * attention (sinks then change nothing).  Key tiles outside the window and
 * the sinks are skipped, so the work is O(T * (W + sinks)).
 *
 *   q              device [T, Hq, head_dim], unrotated
 *   k, v           device [T, Hkv, head_dim], k unrotated
 *   in_dtype       YR_BF16 (bf16 MFMA path) or YR_F32 (fp32 path)
 *   cu_seqlens     device int32[B+1]: 0, c1, ..., cB = T; lengths <= max_seqlen
 *                  (zero-length sequences are allowed and produce nothing)
 *   inv_freq_f64   device double[head_dim/2], or NULL when q and k are already
 *                  rotated
 *   flags          0 or a combination of YR_PREFILL_K_ROTATED and
 *                  YR_PREFILL_PERMUTED_ORDER
 *   window, sinks  >= 0 (see above)
 *   out            device [T, Hq, head_dim] of out_dtype (YR_F32 or YR_BF16;
 *                  YR_F32 inputs require YR_F32 out)
 *   lse            device float[Hq, T] or NULL
 *   workspace      device, 256-byte aligned, >= attn_prefill_workspace_bytes(T,
 *                  Hkv, head_dim, in_dtype) bytes when the library rotates the
 *                  keys (it holds them), else >= YR_WORKSPACE_HEADER_BYTES;
 *                  its header holds the device error word and the counters of
 *                  the work queues the workgroups take their items from (the
 *                  library clears them on the stream before each launch)
 *   head_dim       64 or 128;  Hq % Hkv == 0
 * With T = 0 (every sequence empty) q, k, v and out may be NULL; cu_seqlens
 * is still checked on the device.
 */
int attn_prefill_fwd(const void *q, const void *k, const void *v, int in_dtype,
                     const int *cu_seqlens, int B, int max_seqlen, long long T,
                     int Hq, int Hkv, int head_dim, const double *inv_freq_f64,
                     int flags, float softmax_scale, int window, int sinks, void *out,
                     int out_dtype, float *lse, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * attn_prefill_chunk -- prefill of new tokens against a per-sequence KV cache
 * (chunked prefill: a long prompt fed in pieces, or new turns after a cached
 * prefix; "Long context (engineering 100k+ tokens)", chunked prefill).
 *
 * Sequence b has ctx_lens[b] tokens cached before this chunk and n_b new ones
 * (q rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1).  The caller has already
 * written the chunk's rotated keys and its values into cache rows
 * ctx_lens[b] .. ctx_lens[b] + n_b - 1 (e.g. rope_apply with those
 * positions).  New token i sits at position ctx_lens[b] + i: q is rotated
 * there and attends to cache rows 0 .. ctx_lens[b] + i (the causal boundary
 * at the bottom-right of the chunk x cache block), with the window / sinks
 * rule of attn_prefill_fwd.  Same kernels as attn_prefill_fwd.
 *
 *   q                device [Tq, Hq, head_dim], unrotated
 *   k_cache,v_cache  device [B, max_cache_len, Hkv, head_dim] (in_dtype),
 *                    keys rotated
 *   cu_seqlens_q     device int32[B+1]: 0, c1, ..., cB = Tq; n_b <= max_seqlen_q
 *   ctx_lens         device int32[B]: 0 <= ctx_lens[b] <= max_cache_len - n_b
 *                    (violations are clamped and reported as
 *                    YR_DEVERR_CTX_LENS)
 *   max_seqlen_q     1 .. max_cache_len
 *   inv_freq_f64     device double[head_dim/2], or NULL when q is rotated
 *   out, lse         as attn_prefill_fwd ([Tq, Hq, head_dim], float[Hq, Tq])
 *   workspace        device, 256-byte aligned, >= YR_WORKSPACE_HEADER_BYTES
 *                    (holds the device error word and work-queue counters, as
 *                    for attn_prefill_fwd)
 * With Tq = 0 q, the caches and out may be NULL; cu_seqlens_q and ctx_lens
 * are still checked on the device.
 */
int attn_prefill_chunk(const void *q, const void *k_cache, const void *v_cache, int in_dtype,
                       const int *cu_seqlens_q, const int *ctx_lens, int B, int max_seqlen_q,
                       long long Tq, int max_cache_len, int Hq, int Hkv, int head_dim,
                       const double *inv_freq_f64, float softmax_scale, int window, int sinks,
                       void *out, int out_dtype, float *lse, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Workspace bytes attn_decode needs for these sizes. */
size_t attn_decode_workspace_bytes(int B, int max_cache_len, int Hq, int head_dim);

/*
 * attn_decode -- one new query per sequence over a contiguous per-sequence KV
 * cache (the cache is read in full every decode step: "Long Context",
 * research hub, "Key math").  The query of sequence b is rotated at q_pos[b]
 * (or at seqlens[b] when q_pos is NULL) and attends, unmasked, to cache rows
 * 0 .. seqlens[b]-1, whose keys are taken as already rotated.  The cache is
 * swept in parallel pieces -- fixed-size key chunks, or for caches of 512K
 * keys or more in all (at most 16384 sequences), equal ranges of 32-key
 * blocks, one per compute unit;
 * each piece yields a partial (out, LSE) and the partials are merged by
 * log-sum-exp ("Long-context models", "Context parallelism distributes exact
 * attention").
 * With window = W > 0 only the cache rows the query's window and sinks make
 * visible are read (rows > m - W, and rows < sinks, m = its position): the
 * rest of the cache costs no bandwidth.  The new token's own row is not in
 * the cache, so a one-token window without sinks would see nothing and is
 * rejected; a query placed (by q_pos) past every visible row gets out = 0
 * and lse = -inf.
 *
 *   q               device [B, Hq, head_dim] (in_dtype), unrotated
 *   k_cache,v_cache device [B, max_cache_len, Hkv, head_dim] (in_dtype)
 *   in_dtype        YR_BF16 or YR_F32
 *   seqlens         device int32[B], each in [1, max_cache_len]
 *   q_pos           device int32[B] or NULL
 *   inv_freq_f64    device double[head_dim/2], or NULL if q is already rotated
 *   out             device [B, Hq, head_dim] of out_dtype (YR_F32 or YR_BF16)
 *   lse             device float[B, Hq] or NULL
 *   workspace       device, >= attn_decode_workspace_bytes(...) bytes,
 *                   256-byte aligned; holds the partials
 *   window, sinks   >= 0; window == 1 needs sinks >= 1
 *   head_dim        64 or 128;  Hq % Hkv == 0;  Hq / Hkv <= 32 for YR_BF16
 *                   inputs, <= 16 for YR_F32 inputs
 * Returns YR_ERR_UNSUPPORTED beyond those limits, YR_ERR_WORKSPACE for a
 * short or misaligned workspace, YR_ERR_INVALID for bad sizes; range errors
 * in seqlens / q_pos are reported through the device error word.
 */
int attn_decode(const void *q, const void *k_cache, const void *v_cache,
                int in_dtype, const int *seqlens, const int *q_pos, int B,
                int max_cache_len, int Hq, int Hkv, int head_dim,
                const double *inv_freq_f64, float softmax_scale, int window, int sinks,
                void *out, int out_dtype, float *lse, void *workspace,
                size_t workspace_bytes, void *stream);

/*
 * attn_decode_fp8 -- attn_decode over an FP8 KV cache.
 *
 * The pages name an 8-bit cache as half the bf16 bytes per token ("Long
 * context (engineering 100k+ tokens)", section 1; "Long-context models",
 * "Memory grows even with efficient attention") but fix no format or scales.
 * Convention here: every cache element is one OCP E4M3 byte (bias 7,
 * subnormals, no infinities, NaN = S.1111.111, largest 448), and the value it
 * stands for is decode(byte) * k_scale[h] (keys) or * v_scale[h] (values) for
 * KV head h.  Keys are already rotated.  Everything else -- q (bf16,
 * unrotated), positions, window / sinks, out, lse, workspace (sized by
 * attn_decode_workspace_bytes) -- is as attn_decode.  The sweep reads the
 * cache bytes once (half the bytes of a bf16 cache); the scales fold into the
 * logit scale and the output.
 *
 *   k_cache, v_cache  device uint8 [B, max_cache_len, Hkv, head_dim], E4M3
 *   k_scale, v_scale  device float[Hkv], finite and > 0
 *   Hq / Hkv <= 32
 */
int attn_decode_fp8(const void *q, const void *k_cache, const void *v_cache,
                    const float *k_scale, const float *v_scale, const int *seqlens,
                    const int *q_pos, int B, int max_cache_len, int Hq, int Hkv, int head_dim,
                    const double *inv_freq_f64, float softmax_scale, int window, int sinks,
                    void *out, int out_dtype, float *lse, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): same arguments and results as attn_decode, without the
 * workspace.  The partials live in a fixed scratch array of the library,
 * 32 MiB per device (one copy on every device the library runs on, held until
 * the process ends); the call allocates nothing.
 *
 *   dev_error   device int or NULL: receives the device error word
 *               (YR_DEVERR_SEQLENS / YR_DEVERR_QPOS bits, 0 when the lengths
 *               are in range), written by the call's first workgroup
 * Returns YR_ERR_WORKSPACE, launching nothing, when the split this call needs
 * (the same one attn_decode picks for these sizes) takes more than the fixed
 * scratch holds; attn_decode has no such limit.
 * Every call on a device shares that device's scratch and leaves its
 * contents behind: calls that may overlap on one device (other streams,
 * other threads) race and must be serialised by the caller.  Calls on one
 * stream are ordered and safe.
 */
int attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                        int in_dtype, const int *seqlens, const int *q_pos, int B,
                        int max_cache_len, int Hq, int Hkv, int head_dim,
                        const double *inv_freq_f64, float softmax_scale, int window,
                        int sinks, void *out, int out_dtype, float *lse, int *dev_error,
                        void *stream);

/*
 * yr_read_device_error -- synchronise `stream`, read the device error word of
 * `workspace` (written by the last prefill/decode call that used it) into
 * *flags (YR_DEVERR_* bits).  Returns YR_ERR_DEVICE_RANGE if any bit is set.
 */
int yr_read_device_error(const void *workspace, void *stream, int *flags);

const char *yr_status_string(int status);
const char *yr_last_error(void);
/* Library version as major*10000 + minor*100 + patch. */
int yr_version(void);

#if defined(__GNUC__)
#pragma GCC visibility pop
#endif

#ifdef __cplusplus
}
#endif

#endif /* YARNATTN_H */
