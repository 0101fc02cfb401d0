// Device helpers shared by the gfx950 kernels: bf16 bit conversions, the
// rotary angle (fp64 product and reduction, fp32 sine/cosine) and the
// device-side range checks of cu_seqlens / seqlens.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "yarnattn.h"

namespace yr {

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

typedef __bf16 yr_bf16x2 __attribute__((ext_vector_type(2)));

// float -> bfloat16 bits, round to nearest even (the hardware conversion,
// v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two floats -> packed bf16 pair (lo in bits 0..15), one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const yr_bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// The two halves of a wave combined lane by lane: lane l and lane l ^ 32 both
// get max / sum of their two values.  v_permlane32_swap(x, x) hands lanes
// 0-31 their partner's value in the second result and lanes 32-63 theirs in
// the first (each keeps its own in the other), so one VALU swap replaces the
// LDS-crossbar exchange.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// cos and sin of (pos * theta).  The product and its Cody-Waite reduction by
// pi/2 are done in fp64 (exact to ~1e-11 rad for positions up to 2^20); the
// reduced angle, in [-pi/4, pi/4], goes through the single-precision minimax
// polynomials of the Cephes library (sinf/cosf), and the quadrant picks the
// signs.  Max abs error ~1e-7 (about 1.5 fp32 ulp of 1.0).
__device__ __forceinline__ void rope_cos_sin(double pos, double theta, float *c, float *s) {
#pragma clang fp contract(off)  // the product is rounded before the shift, as rint saw it
  constexpr double kTwoOverPi = 0.63661977236758134308;
  constexpr double kPio2Hi = 1.5707963267948966192;    // nearest double to pi/2
  constexpr double kPio2Lo = 6.123233995736766036e-17;  // pi/2 - kPio2Hi
  // 1.5 * 2^52: adding it rounds a value of magnitude below 2^51 to an
  // integer (to nearest, ties to even, as rint does) held in the low bits of
  // the sum's mantissa, so the quadrant count and its value mod 4 cost one
  // add and one subtract instead of a rint and a 64-bit conversion
  constexpr double kShift = 6755399441055744.0;
  const double x = pos * theta;
  const double t = x * kTwoOverPi + kShift;
  const double kq = t - kShift;
  double r = fma(-kq, kPio2Hi, x);
  r = fma(-kq, kPio2Lo, r);
  const float rf = (float)r, z = rf * rf;
  const float sp = fmaf(rf * z, fmaf(z, fmaf(z, -1.9515295891e-4f, 8.3321608736e-3f), -1.6666654611e-1f), rf);
  const float cp = fmaf(z * z, fmaf(z, fmaf(z, 2.443315711809948e-5f, -1.388731625493765e-3f), 4.166664568298827e-2f),
                        fmaf(-0.5f, z, 1.0f));
  const int quad = (int)(__double_as_longlong(t) & 3);
  float ss = (quad & 1) ? cp : sp;
  float cc = (quad & 1) ? sp : cp;
  if (quad == 1 || quad == 2) cc = -cc;
  if (quad >= 2) ss = -ss;
  *c = cc;
  *s = ss;
}

// Rotate one pair in fp32.  The fused multiply-adds are written out so that
// every kernel that rotates produces the same bits for the same input.
__device__ __forceinline__ void rotate_pair(float &x0, float &x1, float c, float s) {
  const float a = fmaf(x0, c, -(x1 * s));
  const float b = fmaf(x0, s, x1 * c);
  x0 = a;
  x1 = b;
}

// Clamped bounds of sequence b of a packed batch.  Guarantees
// 0 <= start <= start + len <= T and len <= max_seqlen whatever cu holds.
__device__ __forceinline__ void seq_bounds(const int *__restrict__ cu, int b, long long T,
                                           int max_seqlen, long long *start, int *len) {
  long long s0 = cu[b];
  long long s1 = cu[b + 1];
  s0 = s0 < 0 ? 0 : (s0 > T ? T : s0);
  s1 = s1 < s0 ? s0 : (s1 > T ? T : s1);
  long long n = s1 - s0;
  if (n > max_seqlen) n = max_seqlen;
  *start = s0;
  *len = (int)n;
}

// Check cu_seqlens and, for chunked prefill, ctx_lens (one workgroup, all
// threads call it; thread 0 writes the error word).
__device__ inline void validate_cu_seqlens(const int *__restrict__ cu, int B, long long T,
                                           int max_seqlen, int *flag,
                                           const int *__restrict__ ctx = nullptr,
                                           int max_cache_len = 0) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  for (int b = threadIdx.x; b <= B; b += blockDim.x) {
    const long long c = cu[b];
    int e = 0;
    if (b == 0 && c != 0) e = 1;
    if (b == B && c != T) e = 1;
    if (b > 0) {
      const long long p = cu[b - 1];
      if (c < p || c - p > max_seqlen) e = 1;
      if (ctx != nullptr) {
        const long long x = ctx[b - 1];
        if (x < 0 || x + (c - p) > max_cache_len) atomicOr(&bad, YR_DEVERR_CTX_LENS);
      }
    }
    if (e) atomicOr(&bad, YR_DEVERR_CU_SEQLENS);
  }
  __syncthreads();
  if (threadIdx.x == 0) *flag = bad;
}

// Buffer resource word 3 for a raw 32-bit buffer with range checking: a load
// at or past the descriptor's byte count returns zero.
constexpr uint32_t kRsrcWord3 = 0x00020000;

// Buffer descriptor over [base, base + bytes).  Callers pass wave-uniform
// values; readfirstlane puts them in scalar registers, where the descriptor
// must live (otherwise the compiler wraps every load in a waterfall loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void *p = (void *)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           (int)kRsrcWord3);
}

// Check decode seqlens / q_pos (one workgroup, all threads call it; thread 0
// writes the error word).
__device__ inline void validate_decode_lens(const int *__restrict__ seqlens,
                                            const int *__restrict__ qpos, int B, int Lmax,
                                            int *flag) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < B; i += blockDim.x) {
    const int L = seqlens[i];
    if (L < 1 || L > Lmax) atomicOr(&bad, YR_DEVERR_SEQLENS);
    if (qpos != nullptr && qpos[i] < 0) atomicOr(&bad, YR_DEVERR_QPOS);
  }
  __syncthreads();
  if (threadIdx.x == 0) *flag = bad;
}

}  // namespace yr
