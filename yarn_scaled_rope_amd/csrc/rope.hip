// rope kernels (gfx950): rotate feature pairs of [T, H, D] rows by
// position * theta_i ("Arch 03 -- Long Context", RoPE slide).
//
// One thread owns one (token, pair) -- or, with 16-byte aligned buffers, a
// run of 2 or 4 pairs: it forms the angles once (fp64 product and
// reduction, fp32 sine/cosine) and applies them in every head, so the
// transcendental work is shared by the H heads of a token.  Lanes of a wave
// cover consecutive pairs of one token, so each head's row is read and written
// as one contiguous segment.  Positions come either from an explicit
// array (rope_apply) or from the row's offset inside its sequence of a packed
// batch (the key pass of prefill, which also writes out of place).
#include <type_traits>

#include "device_common.h"
#include "yr_internal.h"

namespace yr {
namespace {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  __device__ static void load(const float *p, float &a, float &b) {
    const float2 v = *reinterpret_cast<const float2 *>(p);
    a = v.x;
    b = v.y;
  }
  __device__ static void store(float *p, float a, float b) {
    *reinterpret_cast<float2 *>(p) = make_float2(a, b);
  }
};
template <>
struct Elem<uint16_t> {
  __device__ static void load(const uint16_t *p, float &a, float &b) {
    const uint32_t v = *reinterpret_cast<const uint32_t *>(p);
    a = bf16_to_f32(v & 0xffffu);
    b = bf16_to_f32(v >> 16);
  }
  __device__ static void store(uint16_t *p, float a, float b) {
    *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(a, b);
  }
};

// Sequence index of packed row t: the last b with cu[b] <= t.
__device__ __forceinline__ int seq_of_row(const int *__restrict__ cu, int B, long long t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((long long)cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <typename T, bool FROM_CU>
__global__ __launch_bounds__(256) void rope_kernel(const T *src, T *dst,  // may alias (in place)
                                                  long long ntok, int H, int D,
                                                  const int *__restrict__ pos_or_cu, int B,
                                                  int max_seqlen, const double *__restrict__ theta,
                                                  int *flag) {
  if (FROM_CU && flag != nullptr && blockIdx.x == 0)
    validate_cu_seqlens(pos_or_cu, B, ntok, max_seqlen, flag);
  const int half = D >> 1;
  const long long total = ntok * (long long)half;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const long long t = idx / half;
    const int i = (int)(idx - t * half);
    long long pos;
    if (FROM_CU) {
      const int b = seq_of_row(pos_or_cu, B, t);
      long long s0 = pos_or_cu[b];
      s0 = s0 < 0 ? 0 : s0;
      pos = t - s0;
      if (pos < 0) pos = 0;
    } else {
      pos = pos_or_cu[t];
    }
    float c, s;
    rope_cos_sin((double)pos, theta[i], &c, &s);
    const long long row = t * (long long)H * D + 2 * i;
    for (int h = 0; h < H; ++h) {
      float a, b2;
      Elem<T>::load(src + row + (long long)h * D, a, b2);
      rotate_pair(a, b2, c, s);
      Elem<T>::store(dst + row + (long long)h * D, a, b2);
    }
  }
}

// The same rotation with 16-byte accesses (buffers 16-byte aligned): a lane
// owns PPL consecutive pairs of one token (4 in bf16, 2 in fp32), so a wave
// moves 1 KB per access, and the heads are taken up to 32 at a time, all
// loaded before any is stored, so that in-place rotation keeps that many
// loads in flight.  HB (heads per batch) is 32 for 32 heads or more (6.1
// against 5.6 TB/s at 32 heads), else 8: the 32-head batch's registers halve
// the waves a SIMD holds, which costs more than it gives below 32 heads.
template <typename T, bool FROM_CU, int HB>
__global__ __launch_bounds__(256) void rope_vec_kernel(const T *src, T *dst,  // may alias
                                                      long long ntok, int H, int D,
                                                      const int *__restrict__ pos_or_cu, int B,
                                                      int max_seqlen,
                                                      const double *__restrict__ theta, int *flag) {
  constexpr int PPL = 16 / (2 * (int)sizeof(T));  // pairs per lane
  if (FROM_CU && flag != nullptr && blockIdx.x == 0)
    validate_cu_seqlens(pos_or_cu, B, ntok, max_seqlen, flag);
  const int lpr = (D >> 1) / PPL;  // lanes per (token, head) row
  const long long total = ntok * lpr;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const long long t = idx / lpr;
    const int i0 = (int)(idx - t * lpr) * PPL;
    long long pos;
    if (FROM_CU) {
      const int b = seq_of_row(pos_or_cu, B, t);
      long long s0 = pos_or_cu[b];
      s0 = s0 < 0 ? 0 : s0;
      pos = t - s0;
      if (pos < 0) pos = 0;
    } else {
      pos = pos_or_cu[t];
    }
    float c[PPL], sn[PPL];
#pragma unroll
    for (int p = 0; p < PPL; ++p) rope_cos_sin((double)pos, theta[i0 + p], &c[p], &sn[p]);
    const long long row = t * (long long)H * D + 2 * i0;
    auto rot = [&](uint4 v) -> uint4 {
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
          float a = bf16_to_f32(w[p] & 0xffffu), b2 = bf16_to_f32(w[p] >> 16);
          rotate_pair(a, b2, c[p], sn[p]);
          w[p] = pack_bf16x2(a, b2);
        }
      } else {
#pragma unroll
        for (int p = 0; p < PPL; ++p) {
          float a = __uint_as_float(w[2 * p]), b2 = __uint_as_float(w[2 * p + 1]);
          rotate_pair(a, b2, c[p], sn[p]);
          w[2 * p] = __float_as_uint(a);
          w[2 * p + 1] = __float_as_uint(b2);
        }
      }
      return make_uint4(w[0], w[1], w[2], w[3]);
    };
    // heads in batches of HB, then 8, 4, 2, 1: all loads of a batch before
    // its stores
    int h0 = 0;
    auto batch = [&](auto nc) {
      constexpr int N = decltype(nc)::value;
      for (; h0 + N <= H; h0 += N) {
        uint4 v[N];
#pragma unroll
        for (int u = 0; u < N; ++u) v[u] = *reinterpret_cast<const uint4 *>(src + row + (long long)(h0 + u) * D);
#pragma unroll
        for (int u = 0; u < N; ++u) *reinterpret_cast<uint4 *>(dst + row + (long long)(h0 + u) * D) = rot(v[u]);
      }
    };
    batch(std::integral_constant<int, HB>{});
    batch(std::integral_constant<int, 8>{});
    batch(std::integral_constant<int, 4>{});
    batch(std::integral_constant<int, 2>{});
    batch(std::integral_constant<int, 1>{});
  }
}

template <typename T, bool FROM_CU>
void launch_rope_t(const RopeArgs &a, const int *pc, hipStream_t s) {
  // 16-byte accesses need 16-byte aligned buffers and rows that are a whole
  // number of 16-byte chunks (every lane then owns PPL pairs of one row and
  // every row starts aligned); other head dims take the pair-per-thread form
  const bool vec =
      ((reinterpret_cast<uintptr_t>(a.src) | reinterpret_cast<uintptr_t>(a.dst)) & 15) == 0 &&
      ((size_t)a.head_dim * sizeof(T)) % 16 == 0;
  const int per = vec ? (a.head_dim / 2) / (16 / (2 * (int)sizeof(T))) : a.head_dim / 2;
  const long long total = a.T * (long long)per;
  long long blocks = (total + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
  const dim3 grid((unsigned)blocks), block(256);
  if (vec && a.H >= 32)
    hipLaunchKernelGGL((rope_vec_kernel<T, FROM_CU, 32>), grid, block, 0, s, (const T *)a.src,
                       (T *)a.dst, a.T, a.H, a.head_dim, pc, a.B, a.max_seqlen, a.theta,
                       a.dev_flag);
  else if (vec)
    hipLaunchKernelGGL((rope_vec_kernel<T, FROM_CU, 8>), grid, block, 0, s, (const T *)a.src,
                       (T *)a.dst, a.T, a.H, a.head_dim, pc, a.B, a.max_seqlen, a.theta,
                       a.dev_flag);
  else
    hipLaunchKernelGGL((rope_kernel<T, FROM_CU>), grid, block, 0, s, (const T *)a.src, (T *)a.dst,
                       a.T, a.H, a.head_dim, pc, a.B, a.max_seqlen, a.theta, a.dev_flag);
}

}  // namespace

hipError_t launch_rope(const RopeArgs &a, hipStream_t s) {
  const bool from_cu = a.positions == nullptr;
  const int *pc = from_cu ? a.cu_seqlens : a.positions;
  if (a.dtype == YR_F32) {
    if (from_cu) launch_rope_t<float, true>(a, pc, s);
    else launch_rope_t<float, false>(a, pc, s);
  } else {
    if (from_cu) launch_rope_t<uint16_t, true>(a, pc, s);
    else launch_rope_t<uint16_t, false>(a, pc, s);
  }
  return hipGetLastError();
}

}  // namespace yr
