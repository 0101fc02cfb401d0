// fp32 causal prefill (gfx950 VALU): the full-precision path for fp32 inputs.
//
// Same semantics as the bf16 MFMA path ("Arch 03 -- Long Context", attention
// slide with the causal rule i - j >= 0; "Long-context models", "Context
// parallelism distributes exact attention" for the running max / sum /
// accumulator update), kept simple: a workgroup owns 64 query rows of one
// query head, two lanes per row each hold half of the head dimension, keys and
// values are staged through LDS 32 rows at a time, and every visible key
// updates the row's online-softmax state in fp32 with accurate expf.  Queries
// are rotated on load (fp64 angle); keys arrive already rotated.
#include "device_common.h"
#include "yr_internal.h"

namespace yr {
namespace {

constexpr int kRows = 64;
constexpr int kKeys = 32;
constexpr int kThreads = 128;

template <int D>
__global__ __launch_bounds__(kThreads) void prefill_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const int *__restrict__ cu, int B, int max_seqlen, long long T, int Hq, int Hkv,
    const double *__restrict__ theta, float scale, float *__restrict__ out,
    float *__restrict__ lse, int ntiles, int *flag, int kv_len, const int *__restrict__ ctx,
    int window, int sinks) {
  constexpr int HD = D / 2;
  __shared__ float ks[kKeys][D];
  __shared__ float vs[kKeys][D];

  if (flag != nullptr && blockIdx.x == 0)
    validate_cu_seqlens(cu, B, T, max_seqlen, flag, kv_len > 0 ? ctx : nullptr, kv_len);

  const long long per = (long long)B * Hq;
  const int tile = ntiles - 1 - (int)(blockIdx.x / per);
  const int rem = (int)(blockIdx.x % per);
  const int b = rem / Hq;
  const int h = rem % Hq;
  const int hk = h / (Hq / Hkv);
  long long s0;
  int n;
  seq_bounds(cu, b, T, max_seqlen, &s0, &n);
  const int q0 = tile * kRows;
  if (q0 >= n) return;
  const int qend = min(n, q0 + kRows);

  // keys packed like q, or a [B, kv_len, Hkv, D] cache whose first P rows
  // precede this chunk (query row i sits at position P + i)
  int P = 0;
  long long krow0 = s0;
  if (kv_len > 0) {
    P = ctx != nullptr ? ctx[b] : 0;
    P = P < 0 ? 0 : (P > kv_len - n ? kv_len - n : P);
    krow0 = (long long)b * kv_len;
  }
  const int nk = P + n;

  const int tid = threadIdx.x;
  const int row = q0 + (tid >> 1);
  const int part = tid & 1;
  const bool valid = row < n;
  const int pos = P + row;

  float qr[HD];
  float acc[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    qr[d] = 0.f;
    acc[d] = 0.f;
  }
  if (valid) {
    const float *qp = q + ((s0 + row) * Hq + h) * (long long)D + part * HD;
#pragma unroll
    for (int d = 0; d < HD; d += 2) {
      float a = qp[d], c2 = qp[d + 1];
      if (theta != nullptr) {
        float c, s;
        rope_cos_sin((double)pos, theta[(part * HD + d) >> 1], &c, &s);
        rotate_pair(a, c2, c, s);
      }
      qr[d] = a;
      qr[d + 1] = c2;
    }
  }
  float m = -INFINITY, l = 0.f;

  for (int kt = 0; kt * kKeys < P + qend; ++kt) {
    // key tiles below the window of the workgroup's first row and past the
    // sinks are invisible to every row
    if (window > 0 && kt * kKeys + kKeys - 1 <= P + q0 - window && kt * kKeys >= sinks) continue;
    __syncthreads();
    for (int e = tid; e < kKeys * D; e += kThreads) {
      const int r = e / D, c = e % D;
      const int key = kt * kKeys + r;
      float kv = 0.f, vv = 0.f;
      if (key < nk) {
        const long long off = ((krow0 + key) * Hkv + hk) * (long long)D + c;
        kv = k[off];
        vv = v[off];
      }
      ks[r][c] = kv;
      vs[r][c] = vv;
    }
    __syncthreads();
    for (int j = 0; j < kKeys; ++j) {
      const int key = kt * kKeys + j;
      float part_dot = 0.f;
#pragma unroll
      for (int d = 0; d < HD; ++d) part_dot += qr[d] * ks[j][part * HD + d];
      const float dot = part_dot + __shfl_xor(part_dot, 1);
      const bool seen = key <= pos && (window == 0 || key > pos - window || key < sinks);
      if (valid && seen) {
        const float z = dot * scale;
        const float mn = fmaxf(m, z);
        const float corr = expf(m - mn);
        const float p = expf(z - mn);
        l = l * corr + p;
#pragma unroll
        for (int d = 0; d < HD; ++d) acc[d] = acc[d] * corr + p * vs[j][part * HD + d];
        m = mn;
      }
    }
  }
  if (!valid) return;
  const float inv = 1.f / l;
  float *op = out + ((s0 + row) * Hq + h) * (long long)D + part * HD;
#pragma unroll
  for (int d = 0; d < HD; ++d) op[d] = acc[d] * inv;
  if (lse != nullptr && part == 0) lse[(long long)h * T + s0 + row] = m + logf(l);
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs &a, hipStream_t s) {
  const int ntiles = (a.max_seqlen + kRows - 1) / kRows;
  const long long blocks = (long long)ntiles * a.B * a.Hq;
  const dim3 grid((unsigned)blocks), block(kThreads);
  if (a.head_dim == 64)
    hipLaunchKernelGGL((prefill_f32_kernel<64>), grid, block, 0, s, (const float *)a.q,
                       (const float *)a.k, (const float *)a.v, a.cu_seqlens, a.B, a.max_seqlen, a.T,
                       a.Hq, a.Hkv, a.theta, a.softmax_scale, (float *)a.out, a.lse, ntiles,
                       a.dev_flag, a.kv_cache_len, a.ctx_lens, a.window, a.sinks);
  else
    hipLaunchKernelGGL((prefill_f32_kernel<128>), grid, block, 0, s, (const float *)a.q,
                       (const float *)a.k, (const float *)a.v, a.cu_seqlens, a.B, a.max_seqlen, a.T,
                       a.Hq, a.Hkv, a.theta, a.softmax_scale, (float *)a.out, a.lse, ntiles,
                       a.dev_flag, a.kv_cache_len, a.ctx_lens, a.window, a.sinks);
  return hipGetLastError();
}

}  // namespace yr
