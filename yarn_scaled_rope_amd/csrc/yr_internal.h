// Internal declarations shared by the C-ABI shim and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "yarnattn.h"

namespace yr {

// Record a message for yr_last_error() and return `status`.
int fail(int status, const char *msg);
int fail_hip(hipError_t err, const char *where);

// ---- launch descriptions (host side; every field already validated) -------
struct RopeArgs {
  const void *src;
  void *dst;             // == src for in-place rotation
  int dtype;             // YR_F32 / YR_BF16
  long long T;
  int H;
  int head_dim;
  const int *positions;  // explicit positions, or NULL to derive from cu_seqlens
  const int *cu_seqlens; // used when positions == NULL
  int B;
  int max_seqlen;
  const double *theta;
  int *dev_flag;         // device error word or NULL (validates cu_seqlens)
};

struct PrefillArgs {
  const void *q;
  const void *k;         // keys as the kernel reads them (already rotated)
  const void *v;
  int in_dtype;
  const int *cu_seqlens;
  int B;
  int max_seqlen;
  long long T;
  int Hq;
  int Hkv;
  int head_dim;
  const double *theta;   // rotate q on load when non-NULL
  float softmax_scale;
  void *out;
  int out_dtype;
  float *lse;
  int *dev_flag;         // non-NULL: this launch validates cu_seqlens (and ctx_lens)
  // key source: kv_cache_len == 0: k/v packed like q ([T, Hkv, D], rows by
  // cu_seqlens); kv_cache_len > 0: k/v are [B, kv_cache_len, Hkv, D] caches
  // and sequence b's queries start at position ctx_lens[b]
  int kv_cache_len;
  const int *ctx_lens;   // NULL = no cached prefix
  int window;            // 0 = plain causal
  int sinks;
};

struct DecodeArgs {
  const void *q;
  const void *k_cache;
  const void *v_cache;
  int in_dtype;
  const int *seqlens;
  const int *q_pos;
  int B;
  int max_cache_len;
  int Hq;
  int Hkv;
  int head_dim;
  const double *theta;
  float softmax_scale;
  void *out;
  int out_dtype;
  float *lse;
  float *part_o;         // [B, Hq, nsplit, D]
  float *part_lse;       // [B, Hq, nsplit]
  int chunk;
  int nsplit;
  int *dev_flag;
  int window;            // 0 = every cache row
  int sinks;
  const float *k_scale;  // YR_FP8_E4M3 caches: per-KV-head scales
  const float *v_scale;
  int vis_split;         // 1: chunks split the visible rows (window), not [0, L)
  // > 0: balanced split of the head-per-wave form over stream_wg workgroups
  // of stream_hpw KV heads (chunk / nsplit unused); partials [stream_wg +
  // B * Hkv / stream_hpw][stream_hpw * Hq / Hkv][D]
  int stream_wg;
  int stream_hpw;
};

hipError_t launch_rope(const RopeArgs &a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs &a, hipStream_t s);
hipError_t launch_prefill_bf16(const PrefillArgs &a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);

// Decode split geometry: keys per chunk and number of chunks for a cache
// length bound, with `units` workgroups per (sequence, chunk).  Pure function
// of its arguments so that workspace sizing and the launch agree.
constexpr int kDecodeMinChunk = 64;       // fp32 kernel (a workgroup per KV head)
constexpr int kDecodeMinChunkMfma = 256;  // head-per-wave decode: >= 8 blocks per wave
int decode_chunk(int B, int max_cache_len, int units, int min_chunk);
// The matrix-core decode has two forms.  Head-per-wave: each wave sweeps a
// whole chunk for one KV head and a workgroup takes 8, 4, 2 or 1 KV heads
// (the largest dividing Hkv whose LDS ring fits the budget).  Shared: four
// waves take alternate blocks of one KV head's chunk and combine in LDS.
constexpr bool decode_shared_form(bool fp8, bool win) { return fp8 || win; }
// Workgroups per (sequence, chunk) of the matrix-core decode, and the least
// chunk length worth a workgroup.
int decode_wg_groups(int Hkv, int head_dim, bool fp8, bool win);
inline int decode_min_chunk_mfma(bool fp8, bool win) {
  return decode_shared_form(fp8, win) ? kDecodeMinChunk : kDecodeMinChunkMfma;
}
// Balanced split: used for the head-per-wave form without a window when the
// caches hold at least kDecodeStreamMinKeys keys in all; at most
// kDecodeStreamMaxWg workgroups (one per CU).
constexpr long long kDecodeStreamMinKeys = 512 * 1024;
constexpr int kDecodeStreamMaxWg = 1024;
inline bool decode_stream_eligible(int B, int max_cache_len) {
  return (long long)B * max_cache_len >= kDecodeStreamMinKeys;
}
// workgroups of the balanced split on the current device (its CU count)
int decode_stream_wgs();
inline int decode_nsplit(int max_cache_len, int chunk) {
  return (max_cache_len + chunk - 1) / chunk;
}

}  // namespace yr
