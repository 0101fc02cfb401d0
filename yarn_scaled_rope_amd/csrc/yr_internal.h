// Internal declarations shared by the C-ABI shim and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
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
  int permuted_order;    // 1: workgroups take the work items in a permuted order
  // 8 ints of device memory (in the workspace header) for the work-queue
  // counters of a large launch's queued tail, or NULL: items by block index
  int *work_queues;
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
  int shared_form;       // matrix-core decode: 1 = shared form, 0 = head per wave
};

hipError_t launch_rope(const RopeArgs &a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs &a, hipStream_t s);
hipError_t launch_prefill_bf16(const PrefillArgs &a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);

// Matrix-core decode geometry shared by the kernels and the host plan.
constexpr int kBlk = 32;                    // keys per block (the MFMA row count)
constexpr int kMfmaStages = 2;              // LDS stages per wave
constexpr int kMfmaLdsBudget = 128 * 1024;  // ring bytes per workgroup
// Ring bytes of a workgroup of W waves (one KV head each).
constexpr int mfma_ring_bytes(int W, int D, int EB) { return W * kMfmaStages * 2 * kBlk * D * EB; }
// KV heads per workgroup of the head-per-wave form: the largest of 8, 4, 2,
// 1 that divides Hkv and keeps the ring within the budget (head_dim 128: 4
// with a bf16 cache, 8 with FP8).
constexpr int heads_per_wg(int Hkv, int D, int EB) {
  return (Hkv % 8 == 0 && mfma_ring_bytes(8, D, EB) <= kMfmaLdsBudget) ? 8
         : (Hkv % 4 == 0 && mfma_ring_bytes(4, D, EB) <= kMfmaLdsBudget) ? 4
         : Hkv % 2 == 0 ? 2 : 1;
}

// Decode split geometry: keys per chunk and number of chunks for a cache
// length bound, with `units` workgroups per (sequence, chunk).  Pure function
// of its arguments so that workspace sizing and the launch agree.
constexpr int kDecodeMinChunk = 64;       // fp32 kernel (a workgroup per KV head)
constexpr int kDecodeMinChunkMfma = 256;  // head-per-wave decode: >= 8 blocks per wave
// target: the least number of workgroups to aim for (2048; the split of a
// window's visible rows aims for 1024: measured 0.052 against 0.055 ms for
// 16 sequences and a 4096-key window, 0.069 ms for 4096)
int decode_chunk(int B, int max_cache_len, int units, int min_chunk, int target = 2048);
// The matrix-core decode has two forms.  Head-per-wave: each wave sweeps a
// whole chunk for one KV head and a workgroup takes 8, 4, 2 or 1 KV heads
// (the largest dividing Hkv whose LDS ring fits the budget).  Shared: four
// waves take alternate blocks of one KV head's chunk and combine in LDS.
// KV heads per workgroup of the head-per-wave form:
int decode_heads_per_wg(int Hkv, int head_dim, bool fp8);
// Balanced split of the head-per-wave form (no window, 4 or 8 KV heads per
// workgroup) when the caches hold at least kDecodeStreamMinKeys keys in all:
// the key blocks are cut evenly over one workgroup per CU (at most
// kDecodeStreamMaxWg).
// Workgroups find their pieces, and merge workgroups the pieces of their
// query head, from sums of the B sequences' block counts spread over their
// threads (O(B / threads) each); kDecodeStreamMaxB bounds the batch (and the
// workspace the split needs, (workgroups + B) partials per head group).
constexpr long long kDecodeStreamMinKeys = 512 * 1024;
constexpr int kDecodeStreamMaxWg = 1024;
constexpr int kDecodeStreamMaxB = 16384;
inline bool decode_stream_eligible(int B, int max_cache_len) {
  return B <= kDecodeStreamMaxB && (long long)B * max_cache_len >= kDecodeStreamMinKeys;
}
// With a window the visible rows decide (window + sinks per sequence at most):
// a short window leaves too few blocks per CU for one workgroup per CU to
// keep enough copies in flight (W 4096 on 16 sequences measured 0.0576 ms
// against 0.0551 ms in shared-form chunks).
inline bool decode_stream_form(int B, int max_cache_len, int Hkv, int head_dim, bool fp8,
                               int window, int sinks) {
  const int hpw = decode_heads_per_wg(Hkv, head_dim, fp8);
  const long long span = window > 0 ? std::min<long long>(max_cache_len, (long long)window + sinks)
                                    : max_cache_len;
  return (hpw == 4 || hpw == 8) && decode_stream_eligible(B, max_cache_len) &&
         (long long)B * span >= kDecodeStreamMinKeys;
}
// Which form without the balanced split: a window takes the shared form (its
// chunks are short), an FP8 cache too (measured: shared 6.0 TB/s,
// head-per-wave in chunks 5.3-5.9, balanced split 6.3); bf16 takes the
// head-per-wave form.
inline bool decode_shared_form(bool fp8, bool win, bool stream) {
  return (win || fp8) && !stream;
}
// workgroups of the balanced split on the device of `stream` (its CU count,
// at most kDecodeStreamMaxWg); 0 if the device cannot be queried
int decode_stream_wgs(hipStream_t stream);
// Fixed scratch of attn_decode_noalloc: a file-scope device array of this
// many bytes (one per device the library runs on, held until the process
// ends).  decode_fixed_scratch() returns its address on the device of
// `stream`, looked up once per device.
constexpr size_t kDecodeScratchBytes = 32u << 20;
hipError_t decode_fixed_scratch(hipStream_t stream, void **ptr);
inline int decode_nsplit(int max_cache_len, int chunk) {
  return (max_cache_len + chunk - 1) / chunk;
}

}  // namespace yr
