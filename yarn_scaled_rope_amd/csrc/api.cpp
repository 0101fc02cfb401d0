// C-ABI entry points of libyarnattn.so: host-side validation, workspace
// layout and kernel launches.  Every entry point checks its arguments before
// touching the device, returns a status and never throws.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>

#include "yarnattn.h"
#include "yr_internal.h"

namespace yr {

namespace {
thread_local std::string g_last_error;

constexpr size_t kHeader = YR_WORKSPACE_HEADER_BYTES;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool dims_ok(int head_dim) { return head_dim == 64 || head_dim == 128; }

int *flag_of(void *ws) { return static_cast<int *>(ws); }
// work-queue counters of the queued tail of a large prefill launch: 8 ints at
// byte 128 of the header (a cache line of their own, apart from the error word)
int *queues_of(void *ws) { return reinterpret_cast<int *>(static_cast<char *>(ws) + 128); }
}  // namespace

int fail(int status, const char *msg) {
  g_last_error = msg ? msg : "";
  return status;
}

int fail_hip(hipError_t err, const char *where) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), "%s: HIP error %d (%s)", where, (int)err, hipGetErrorString(err));
  g_last_error = buf;
  return YR_ERR_HIP;
}

namespace {

// attn_decode, attn_decode_fp8 and attn_decode_noalloc: validation, the
// choice of sweep form and split, the workspace layout and the launch.
// cache_dtype is the storage type of the caches (q is YR_F32 with an fp32
// cache, else YR_BF16).  The scratch memory comes either from the caller's
// workspace (checked against attn_decode_workspace_bytes, the bound for any
// split of these sizes) or, when fixed_scratch is set, from the library's
// per-device scratch array, checked against the bytes this call's split
// actually needs.
struct DecodeCall {
  const char *fn;
  const void *q, *k_cache, *v_cache;
  int cache_dtype;
  const float *k_scale, *v_scale;
  const int *seqlens, *q_pos;
  int B, max_cache_len, Hq, Hkv, head_dim;
  const double *inv_freq_f64;
  float softmax_scale;
  int window, sinks;
  void *out;
  int out_dtype;
  float *lse;
  void *workspace;
  size_t workspace_bytes;
  bool fixed_scratch;
  int *dev_error;  // fixed_scratch: where the kernels write the device error word (or NULL)
  void *stream;
};

int decode_impl(const DecodeCall &c) {
  char msg[200];
  auto bad = [&](int st, const char *what) {
    std::snprintf(msg, sizeof msg, "%s: %s", c.fn, what);
    return fail(st, msg);
  };
  const int cache_dtype = c.cache_dtype, B = c.B, Hq = c.Hq, Hkv = c.Hkv;
  const int head_dim = c.head_dim, max_cache_len = c.max_cache_len;
  const int window = c.window, sinks = c.sinks;
  if (cache_dtype != YR_F32 && cache_dtype != YR_BF16 && cache_dtype != YR_FP8_E4M3)
    return bad(YR_ERR_UNSUPPORTED, "in_dtype must be YR_F32 or YR_BF16");
  if (c.out_dtype != YR_F32 && c.out_dtype != YR_BF16)
    return bad(YR_ERR_UNSUPPORTED, "out_dtype must be YR_F32 or YR_BF16");
  if (!dims_ok(head_dim)) return bad(YR_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return bad(YR_ERR_INVALID, "need Hq >= 1, Hkv >= 1, Hq % Hkv == 0");
  if (Hq / Hkv > (cache_dtype == YR_F32 ? 16 : 32))
    return bad(YR_ERR_UNSUPPORTED, "at most 32 (bf16, fp8) or 16 (fp32) query heads per KV head");
  if (B < 1 || max_cache_len < 1) return bad(YR_ERR_INVALID, "need B >= 1, max_cache_len >= 1");
  if ((long long)B * max_cache_len > (1LL << 34)) return bad(YR_ERR_INVALID, "cache too large");
  if (!std::isfinite(c.softmax_scale) || !(c.softmax_scale > 0.f))
    return bad(YR_ERR_INVALID, "softmax_scale must be finite and > 0");
  if (window < 0 || sinks < 0) return bad(YR_ERR_INVALID, "window and sinks must be >= 0");
  if (window == 1 && sinks == 0)
    return bad(YR_ERR_INVALID, "a one-token window without sinks sees no cache row");
  if (!c.q || !c.k_cache || !c.v_cache || !c.seqlens || !c.out)
    return bad(YR_ERR_NULL, "q, caches, seqlens and out are required");
  if (cache_dtype == YR_FP8_E4M3 && (!c.k_scale || !c.v_scale))
    return bad(YR_ERR_NULL, "k_scale and v_scale are required");
  if (!c.fixed_scratch) {
    if (!c.workspace) return bad(YR_ERR_NULL, "workspace is required");
    if ((reinterpret_cast<uintptr_t>(c.workspace) & 255) != 0)
      return bad(YR_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    const size_t need = attn_decode_workspace_bytes(B, max_cache_len, Hq, head_dim);
    if (c.workspace_bytes < need) return bad(YR_ERR_WORKSPACE, "workspace too small");
  }
  hipStream_t stream = (hipStream_t)c.stream;

  // the matrix-core kernel launches one workgroup per group of KV heads, the
  // fp32 one per head: chunk so that either launches enough workgroups
  const bool fp8 = cache_dtype == YR_FP8_E4M3, win = window > 0;
  const bool balanced =
      cache_dtype != YR_F32 && decode_stream_form(B, max_cache_len, Hkv, head_dim, fp8, window, sinks);
  const bool shared = decode_shared_form(fp8, win, balanced);
  const int units = cache_dtype == YR_F32 || shared
                        ? Hkv
                        : Hkv / decode_heads_per_wg(Hkv, head_dim, fp8);
  const int min_chunk =
      cache_dtype == YR_F32 || shared ? kDecodeMinChunk : kDecodeMinChunkMfma;
  int chunk = decode_chunk(B, max_cache_len, units, min_chunk);
  int nsplit = decode_nsplit(max_cache_len, chunk);
  // With a window the matrix-core sweep can split the visible rows alone
  // (normally window - 1 + sinks of them) instead of the whole cache, so that
  // no workgroup starts on rows nobody reads; the workspace is sized for the
  // finer split of the whole cache, so this applies when it needs fewer chunks.
  int vis_split = 0;
  if (window > 0 && cache_dtype != YR_F32) {
    const int span = (int)std::min<long long>(max_cache_len, (long long)window + sinks);
    const int cw = decode_chunk(B, span, units, min_chunk, 1024);
    const int nw = decode_nsplit(span, cw);
    if (nw < nsplit) {
      chunk = cw;
      nsplit = nw;
      vis_split = 1;
    }
  }
  if ((long long)B * Hkv * nsplit > 0x7fffffffLL) return bad(YR_ERR_INVALID, "grid too large");
  size_t rows = (size_t)B * Hq * nsplit;
  // head-per-wave sweep of a large cache, four or eight KV heads per
  // workgroup: split the key blocks evenly over one workgroup per CU instead
  int stream_wg = 0, stream_hpw = 0;
  if (balanced) {
    stream_wg = decode_stream_wgs(stream);
    if (stream_wg <= 0) return bad(YR_ERR_HIP, "cannot query the device's compute units");
    stream_hpw = Hkv / units;
    rows = ((size_t)stream_wg + (size_t)B * units) * (size_t)(Hq / units);
  }
  const size_t o_bytes = align_up(rows * head_dim * 4, 256);
  char *ws = static_cast<char *>(c.workspace);
  int *flag = c.fixed_scratch ? c.dev_error : flag_of(c.workspace);
  if (c.fixed_scratch) {
    const size_t need = kHeader + o_bytes + align_up(rows * 4, 256);
    if (need > kDecodeScratchBytes) {
      std::snprintf(msg, sizeof msg,
                    "%s: this call needs %zu bytes of scratch, more than the fixed %zu", c.fn,
                    need, (size_t)kDecodeScratchBytes);
      return fail(YR_ERR_WORKSPACE, msg);
    }
    void *p = nullptr;
    const hipError_t e = decode_fixed_scratch(stream, &p);
    if (e != hipSuccess) return fail_hip(e, c.fn);
    ws = static_cast<char *>(p);
  }
  DecodeArgs d{};
  d.q = c.q;
  d.k_cache = c.k_cache;
  d.v_cache = c.v_cache;
  d.in_dtype = cache_dtype;
  d.seqlens = c.seqlens;
  d.q_pos = c.q_pos;
  d.B = B;
  d.max_cache_len = max_cache_len;
  d.Hq = Hq;
  d.Hkv = Hkv;
  d.head_dim = head_dim;
  d.theta = c.inv_freq_f64;
  d.softmax_scale = c.softmax_scale;
  d.out = c.out;
  d.out_dtype = c.out_dtype;
  d.lse = c.lse;
  d.part_o = reinterpret_cast<float *>(ws + kHeader);
  d.part_lse = reinterpret_cast<float *>(ws + kHeader + o_bytes);
  d.chunk = chunk;
  d.nsplit = nsplit;
  d.dev_flag = flag;
  d.window = window;
  d.sinks = sinks;
  d.k_scale = c.k_scale;
  d.v_scale = c.v_scale;
  d.vis_split = vis_split;
  d.stream_wg = stream_wg;
  d.stream_hpw = stream_hpw;
  d.shared_form = shared ? 1 : 0;
  const hipError_t e = launch_decode(d, stream);
  if (e != hipSuccess) return fail_hip(e, c.fn);
  return YR_OK;
}

}  // namespace

}  // namespace yr

using namespace yr;

extern "C" {

const char *yr_status_string(int status) {
  switch (status) {
    case YR_OK: return "ok";
    case YR_ERR_INVALID: return "invalid argument";
    case YR_ERR_NULL: return "null pointer";
    case YR_ERR_UNSUPPORTED: return "unsupported configuration";
    case YR_ERR_WORKSPACE: return "workspace too small";
    case YR_ERR_HIP: return "HIP runtime error";
    case YR_ERR_DEVICE_RANGE: return "device-side range check failed";
    default: return "unknown status";
  }
}

const char *yr_last_error(void) { return g_last_error.c_str(); }

int yr_version(void) { return 100; }

int rope_apply(void *x, int dtype, long long T, int H, int head_dim, const int *positions,
               const double *inv_freq_f64, void *stream) {
  if (dtype != YR_F32 && dtype != YR_BF16) return fail(YR_ERR_UNSUPPORTED, "rope_apply: dtype");
  if (T < 0 || H < 1 || head_dim < 2 || head_dim > 512 || (head_dim & 1))
    return fail(YR_ERR_INVALID, "rope_apply: need T >= 0, H >= 1, even head_dim in [2, 512]");
  if (T == 0) return YR_OK;
  if (!x || !positions || !inv_freq_f64) return fail(YR_ERR_NULL, "rope_apply: null pointer");
  if (T * (long long)H * head_dim > (1LL << 46))
    return fail(YR_ERR_INVALID, "rope_apply: tensor too large");
  RopeArgs a{};
  a.src = x;
  a.dst = x;
  a.dtype = dtype;
  a.T = T;
  a.H = H;
  a.head_dim = head_dim;
  a.positions = positions;
  a.theta = inv_freq_f64;
  const hipError_t e = launch_rope(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "rope_apply");
  return YR_OK;
}

int rope_apply_packed(const void *src, void *dst, int dtype, const int *cu_seqlens, int B,
                      int max_seqlen, long long T, int H, int head_dim,
                      const double *inv_freq_f64, int *dev_error, void *stream) {
  if (dtype != YR_F32 && dtype != YR_BF16) return fail(YR_ERR_UNSUPPORTED, "rope_apply_packed: dtype");
  if (T < 0 || H < 1 || head_dim < 2 || head_dim > 512 || (head_dim & 1))
    return fail(YR_ERR_INVALID, "rope_apply_packed: need T >= 0, H >= 1, even head_dim in [2, 512]");
  if (B < 1 || max_seqlen < 1) return fail(YR_ERR_INVALID, "rope_apply_packed: need B >= 1, max_seqlen >= 1");
  if (T * (long long)H * head_dim > (1LL << 46))
    return fail(YR_ERR_INVALID, "rope_apply_packed: tensor too large");
  if (!cu_seqlens || !inv_freq_f64 || ((!src || !dst) && T > 0))
    return fail(YR_ERR_NULL, "rope_apply_packed: null pointer");
  RopeArgs a{};
  a.src = src;
  a.dst = dst;
  a.dtype = dtype;
  a.T = T;
  a.H = H;
  a.head_dim = head_dim;
  a.positions = nullptr;
  a.cu_seqlens = cu_seqlens;
  a.B = B;
  a.max_seqlen = max_seqlen;
  a.theta = inv_freq_f64;
  a.dev_flag = dev_error;
  const hipError_t e = launch_rope(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "rope_apply_packed");
  return YR_OK;
}

size_t attn_prefill_workspace_bytes(long long T, int Hkv, int head_dim, int in_dtype) {
  if (T < 0 || Hkv < 1 || head_dim < 1) return kHeader;
  const size_t elem = in_dtype == YR_F32 ? 4 : 2;
  return kHeader + align_up((size_t)T * (size_t)Hkv * (size_t)head_dim * elem, 256);
}

int attn_prefill_fwd(const void *q, const void *k, const void *v, int in_dtype,
                     const int *cu_seqlens, int B, int max_seqlen, long long T, int Hq, int Hkv,
                     int head_dim, const double *inv_freq_f64, int flags, float softmax_scale,
                     int window, int sinks, void *out, int out_dtype, float *lse, void *workspace,
                     size_t workspace_bytes, void *stream) {
  if (flags & ~(YR_PREFILL_K_ROTATED | YR_PREFILL_PERMUTED_ORDER))
    return fail(YR_ERR_INVALID, "attn_prefill_fwd: unknown flags");
  if (in_dtype != YR_F32 && in_dtype != YR_BF16)
    return fail(YR_ERR_UNSUPPORTED, "attn_prefill_fwd: in_dtype must be YR_F32 or YR_BF16");
  if (out_dtype != YR_F32 && out_dtype != YR_BF16)
    return fail(YR_ERR_UNSUPPORTED, "attn_prefill_fwd: out_dtype must be YR_F32 or YR_BF16");
  if (in_dtype == YR_F32 && out_dtype != YR_F32)
    return fail(YR_ERR_UNSUPPORTED, "attn_prefill_fwd: fp32 inputs need fp32 output");
  if (!dims_ok(head_dim)) return fail(YR_ERR_UNSUPPORTED, "attn_prefill_fwd: head_dim must be 64 or 128");
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(YR_ERR_INVALID, "attn_prefill_fwd: need Hq >= 1, Hkv >= 1, Hq % Hkv == 0");
  if (B < 1 || T < 0 || max_seqlen < 1)
    return fail(YR_ERR_INVALID, "attn_prefill_fwd: need B >= 1, T >= 0, max_seqlen >= 1");
  if (max_seqlen > (1 << 24) || T > (1LL << 31) - 1)
    return fail(YR_ERR_INVALID, "attn_prefill_fwd: max_seqlen or T too large");
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(YR_ERR_INVALID, "attn_prefill_fwd: softmax_scale must be finite and > 0");
  if (window < 0 || sinks < 0) return fail(YR_ERR_INVALID, "attn_prefill_fwd: window and sinks must be >= 0");
  // an empty batch (T = 0) reads and writes no rows: its data pointers may be NULL
  if (!cu_seqlens || !workspace || ((!q || !k || !v || !out) && T > 0))
    return fail(YR_ERR_NULL, "attn_prefill_fwd: q, k, v, cu_seqlens, out and workspace are required");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return fail(YR_ERR_WORKSPACE, "attn_prefill_fwd: workspace must be 256-byte aligned");
  const bool key_pass = inv_freq_f64 != nullptr && !(flags & YR_PREFILL_K_ROTATED);
  const size_t need = key_pass ? attn_prefill_workspace_bytes(T, Hkv, head_dim, in_dtype) : kHeader;
  if (workspace_bytes < need) return fail(YR_ERR_WORKSPACE, "attn_prefill_fwd: workspace too small");
  const long long ntiles = (max_seqlen + 63) / 64;
  if (ntiles * (long long)B * Hq > 0x7fffffffLL)
    return fail(YR_ERR_INVALID, "attn_prefill_fwd: grid too large");

  hipStream_t s = (hipStream_t)stream;
  int *flag = flag_of(workspace);
  PrefillArgs p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.in_dtype = in_dtype;
  p.cu_seqlens = cu_seqlens;
  p.B = B;
  p.max_seqlen = max_seqlen;
  p.T = T;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.head_dim = head_dim;
  p.theta = inv_freq_f64;
  p.softmax_scale = softmax_scale;
  p.out = out;
  p.out_dtype = out_dtype;
  p.lse = lse;
  p.dev_flag = flag;
  p.kv_cache_len = 0;
  p.ctx_lens = nullptr;
  p.window = window;
  p.sinks = sinks;
  p.permuted_order = (flags & YR_PREFILL_PERMUTED_ORDER) ? 1 : 0;
  p.work_queues = queues_of(workspace);

  if (key_pass && T > 0) {
    // rotate every key once into the workspace; the attention kernel rotates
    // queries on load and reads the rotated keys
    void *krot = static_cast<char *>(workspace) + kHeader;
    RopeArgs r{};
    r.src = k;
    r.dst = krot;
    r.dtype = in_dtype;
    r.T = T;
    r.H = Hkv;
    r.head_dim = head_dim;
    r.positions = nullptr;
    r.cu_seqlens = cu_seqlens;
    r.B = B;
    r.max_seqlen = max_seqlen;
    r.theta = inv_freq_f64;
    r.dev_flag = flag;
    hipError_t e = launch_rope(r, s);
    if (e != hipSuccess) return fail_hip(e, "attn_prefill_fwd (key rotation)");
    p.k = krot;
    p.dev_flag = nullptr;  // already validated by the key pass
  }
  const hipError_t e =
      in_dtype == YR_F32 ? launch_prefill_f32(p, s) : launch_prefill_bf16(p, s);
  if (e != hipSuccess) return fail_hip(e, "attn_prefill_fwd");
  return YR_OK;
}

int attn_prefill_chunk(const void *q, const void *k_cache, const void *v_cache, int in_dtype,
                       const int *cu_seqlens_q, const int *ctx_lens, int B, int max_seqlen_q,
                       long long Tq, int max_cache_len, int Hq, int Hkv, int head_dim,
                       const double *inv_freq_f64, float softmax_scale, int window, int sinks,
                       void *out, int out_dtype, float *lse, void *workspace,
                       size_t workspace_bytes, void *stream) {
  if (in_dtype != YR_F32 && in_dtype != YR_BF16)
    return fail(YR_ERR_UNSUPPORTED, "attn_prefill_chunk: in_dtype must be YR_F32 or YR_BF16");
  if (out_dtype != YR_F32 && out_dtype != YR_BF16)
    return fail(YR_ERR_UNSUPPORTED, "attn_prefill_chunk: out_dtype must be YR_F32 or YR_BF16");
  if (in_dtype == YR_F32 && out_dtype != YR_F32)
    return fail(YR_ERR_UNSUPPORTED, "attn_prefill_chunk: fp32 inputs need fp32 output");
  if (!dims_ok(head_dim)) return fail(YR_ERR_UNSUPPORTED, "attn_prefill_chunk: head_dim must be 64 or 128");
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(YR_ERR_INVALID, "attn_prefill_chunk: need Hq >= 1, Hkv >= 1, Hq % Hkv == 0");
  if (B < 1 || Tq < 0 || max_seqlen_q < 1 || max_cache_len < max_seqlen_q)
    return fail(YR_ERR_INVALID,
                "attn_prefill_chunk: need B >= 1, Tq >= 0, 1 <= max_seqlen_q <= max_cache_len");
  if (max_cache_len > (1 << 24) || Tq > (1LL << 31) - 1 ||
      (long long)B * max_cache_len > (1LL << 34))
    return fail(YR_ERR_INVALID, "attn_prefill_chunk: sizes too large");
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(YR_ERR_INVALID, "attn_prefill_chunk: softmax_scale must be finite and > 0");
  if (window < 0 || sinks < 0) return fail(YR_ERR_INVALID, "attn_prefill_chunk: window and sinks must be >= 0");
  // no new token (Tq = 0): nothing is read or written, so q, the caches and out may be NULL
  if (!cu_seqlens_q || !ctx_lens || !workspace ||
      ((!q || !k_cache || !v_cache || !out) && Tq > 0))
    return fail(YR_ERR_NULL, "attn_prefill_chunk: q, caches, cu_seqlens_q, ctx_lens, out and "
                             "workspace are required");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return fail(YR_ERR_WORKSPACE, "attn_prefill_chunk: workspace must be 256-byte aligned");
  if (workspace_bytes < kHeader) return fail(YR_ERR_WORKSPACE, "attn_prefill_chunk: workspace too small");
  const long long ntiles = (max_seqlen_q + 63) / 64;
  if (ntiles * (long long)B * Hq > 0x7fffffffLL)
    return fail(YR_ERR_INVALID, "attn_prefill_chunk: grid too large");
  PrefillArgs p{};
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.in_dtype = in_dtype;
  p.cu_seqlens = cu_seqlens_q;
  p.B = B;
  p.max_seqlen = max_seqlen_q;
  p.T = Tq;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.head_dim = head_dim;
  p.theta = inv_freq_f64;
  p.softmax_scale = softmax_scale;
  p.out = out;
  p.out_dtype = out_dtype;
  p.lse = lse;
  p.dev_flag = flag_of(workspace);
  p.kv_cache_len = max_cache_len;
  p.ctx_lens = ctx_lens;
  p.window = window;
  p.sinks = sinks;
  p.work_queues = queues_of(workspace);
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = in_dtype == YR_F32 ? launch_prefill_f32(p, s) : launch_prefill_bf16(p, s);
  if (e != hipSuccess) return fail_hip(e, "attn_prefill_chunk");
  return YR_OK;
}

size_t attn_decode_workspace_bytes(int B, int max_cache_len, int Hq, int head_dim) {
  if (B < 1 || max_cache_len < 1 || Hq < 1 || head_dim < 1) return kHeader;
  // chunking depends on Hkv only through the split count heuristic; size for
  // the finest chunking any Hkv <= Hq can select
  const int chunk = decode_chunk(B, max_cache_len, 1, kDecodeMinChunk);
  const size_t ns = (size_t)decode_nsplit(max_cache_len, chunk);
  size_t rows = (size_t)B * Hq * ns;
  // the balanced split writes at most (workgroups + segments) partials of
  // Hq / (segments per sequence) query heads each: <= (max workgroups + B) * Hq
  if (decode_stream_eligible(B, max_cache_len))
    rows = std::max(rows, ((size_t)kDecodeStreamMaxWg + B) * Hq);
  return kHeader + align_up(rows * head_dim * 4, 256) + align_up(rows * 4, 256);
}


int attn_decode(const void *q, const void *k_cache, const void *v_cache, int in_dtype,
                const int *seqlens, const int *q_pos, int B, int max_cache_len, int Hq, int Hkv,
                int head_dim, const double *inv_freq_f64, float softmax_scale, int window,
                int sinks, void *out, int out_dtype, float *lse, void *workspace,
                size_t workspace_bytes, void *stream) {
  if (in_dtype != YR_F32 && in_dtype != YR_BF16)
    return fail(YR_ERR_UNSUPPORTED, "attn_decode: in_dtype must be YR_F32 or YR_BF16");
  return decode_impl({"attn_decode", q, k_cache, v_cache, in_dtype, nullptr, nullptr, seqlens,
                      q_pos, B, max_cache_len, Hq, Hkv, head_dim, inv_freq_f64, softmax_scale,
                      window, sinks, out, out_dtype, lse, workspace, workspace_bytes, false,
                      nullptr, stream});
}

int attn_decode_fp8(const void *q, const void *k_cache, const void *v_cache,
                    const float *k_scale, const float *v_scale, const int *seqlens,
                    const int *q_pos, int B, int max_cache_len, int Hq, int Hkv, int head_dim,
                    const double *inv_freq_f64, float softmax_scale, int window, int sinks,
                    void *out, int out_dtype, float *lse, void *workspace,
                    size_t workspace_bytes, void *stream) {
  return decode_impl({"attn_decode_fp8", q, k_cache, v_cache, YR_FP8_E4M3, k_scale, v_scale,
                      seqlens, q_pos, B, max_cache_len, Hq, Hkv, head_dim, inv_freq_f64,
                      softmax_scale, window, sinks, out, out_dtype, lse, workspace,
                      workspace_bytes, false, nullptr, stream});
}

int attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, int in_dtype,
                        const int *seqlens, const int *q_pos, int B, int max_cache_len, int Hq,
                        int Hkv, int head_dim, const double *inv_freq_f64, float softmax_scale,
                        int window, int sinks, void *out, int out_dtype, float *lse,
                        int *dev_error, void *stream) {
  if (in_dtype != YR_F32 && in_dtype != YR_BF16)
    return fail(YR_ERR_UNSUPPORTED, "attn_decode_noalloc: in_dtype must be YR_F32 or YR_BF16");
  return decode_impl({"attn_decode_noalloc", q, k_cache, v_cache, in_dtype, nullptr, nullptr,
                      seqlens, q_pos, B, max_cache_len, Hq, Hkv, head_dim, inv_freq_f64,
                      softmax_scale, window, sinks, out, out_dtype, lse, nullptr, 0, true,
                      dev_error, stream});
}

int yr_read_device_error(const void *workspace, void *stream, int *flags) {
  if (!workspace || !flags) return fail(YR_ERR_NULL, "yr_read_device_error: null pointer");
  int h = 0;
  hipError_t e = hipMemcpyAsync(&h, workspace, sizeof(int), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "yr_read_device_error");
  *flags = h;
  if (h != 0) return fail(YR_ERR_DEVICE_RANGE, "device-side range check failed (see flag bits)");
  return YR_OK;
}

}  // extern "C"
