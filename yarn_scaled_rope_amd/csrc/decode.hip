// Decode attention on gfx950: one new query per sequence over a contiguous
// per-sequence KV cache, swept split-K, then merged by log-sum-exp.
//
// The cache is read in full on every decode step, so the step is bound by
// HBM bandwidth ("Long Context", research hub, "Key math": the KV cache is
// linear in length but read every decode step; "LLM context window
// mechanics", "The memory wall").  Partial softmax results over disjoint key
// chunks combine exactly through their row max and sum ("Long-context models",
// "Context parallelism distributes exact attention").
//
// Split kernel: a workgroup owns (sequence b, KV head, key chunk).  A key row
// (D elements) is read by D/8 adjacent lanes, 16 bytes each, so one wave load
// covers several whole rows; every byte of K and V is read once and serves all
// query heads of the group.  Each lane group keeps its own online-softmax
// state per query head; the groups of a wave combine through lane exchanges
// and the waves through LDS, and the workgroup writes one normalised partial
// (out, log2-sum-exp) per query head.  Cache loads are non-temporal: the
// sweep reads each byte once.
// Merge kernel: one wave per (sequence, query head) combines the partials.
#include "device_common.h"
#include "yr_internal.h"

namespace yr {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;  // keys per lane group per iteration (loads in flight)
constexpr float kLn2 = 0.69314718055994530942f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 8 consecutive elements of a cache row: loaded raw (non-temporal: the sweep
// reads each byte once), widened to float at use.
template <typename T>
struct Row8;
template <>
struct Row8<uint16_t> {
  struct Raw {
    u32x4 w;
  };
  __device__ static Raw load(const uint16_t *p) {
    return Raw{__builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p))};
  }
  __device__ static Raw zero() { return Raw{u32x4{0u, 0u, 0u, 0u}}; }
  __device__ static void widen(const Raw &r, float *x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_to_f32(r.w[e] & 0xffffu);
      x[2 * e + 1] = bf16_to_f32(r.w[e] >> 16);
    }
  }
  __device__ static float scalar(const uint16_t *p) { return bf16_to_f32(*p); }
};
template <>
struct Row8<float> {
  struct Raw {
    f32x4 a, b;
  };
  __device__ static Raw load(const float *p) {
    return Raw{__builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p)),
               __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + 4))};
  }
  __device__ static Raw zero() { return Raw{f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}}; }
  __device__ static void widen(const Raw &r, float *x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = r.a[e];
      x[4 + e] = r.b[e];
    }
  }
  __device__ static float scalar(const float *p) { return *p; }
};

// Sum over the LPK lanes that share a key row (LPK = 16 or 8 adjacent lanes of
// one DPP row); every lane gets the total.  DPP moves, no LDS round trips.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_move<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_move<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_move<0x141>(x);  // row_half_mirror: quads 0<->1, 2<->3
  if (LPK == 16) x += dpp_move<0x140>(x);  // row_mirror: half rows swap
  return x;
}

// Merge running state (m, l, acc[8]) with another one; -inf maxima mean
// "no key seen yet".
__device__ __forceinline__ void combine_state(float &m, float &l, float *acc, float mo, float lo,
                                              const float *acco) {
  const float mn = fmaxf(m, mo);
  if (mn == -INFINITY) return;
  const float a = __builtin_amdgcn_exp2f(m - mn);
  const float c = __builtin_amdgcn_exp2f(mo - mn);
  l = l * a + lo * c;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = acc[e] * a + acco[e] * c;
  m = mn;
}

template <typename T, int D, int GM>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const T *__restrict__ q, const T *__restrict__ kc, const T *__restrict__ vc,
    const int *__restrict__ seqlens, const int *__restrict__ qpos, int B, int Lmax, int Hq,
    int Hkv, const double *__restrict__ theta, float scale_log2, int chunk, int nsplit,
    float *__restrict__ part_o, float *__restrict__ part_lse, int *flag) {
  constexpr int LPK = D / 8;         // lanes per key row
  constexpr int GPW = 64 / LPK;      // key rows per wave load
  constexpr int KPW = GPW * kUnroll; // keys per wave per iteration
  constexpr int KPI = KPW * kWaves;  // keys per workgroup per iteration

  __shared__ float sm_m[kWaves][GM];
  __shared__ float sm_l[kWaves][GM];
  __shared__ float sm_acc[kWaves][GM][D];

  if (flag != nullptr && blockIdx.x == 0) {
    __shared__ int bad;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < B; i += kThreads) {
      const int L = seqlens[i];
      if (L < 1 || L > Lmax) atomicOr(&bad, YR_DEVERR_SEQLENS);
      if (qpos != nullptr && qpos[i] < 0) atomicOr(&bad, YR_DEVERR_QPOS);
    }
    __syncthreads();
    if (threadIdx.x == 0) *flag = bad;
  }

  const int split = blockIdx.x % nsplit;
  const int rest = blockIdx.x / nsplit;
  const int hk = rest % Hkv;
  const int b = rest / Hkv;
  const int g = Hq / Hkv;
  int L = seqlens[b];
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  const int c0 = split * chunk;
  if (c0 >= L) return;
  const int c1 = min(L, c0 + chunk);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane % LPK;  // which 8-element slice of the row
  const int grp = lane / LPK;  // which key row of the wave load
  const int d0 = sub * 8;

  // query slice, rotated at its position and pre-scaled into log2 units; the
  // angle of a pair is the same for every head of the group
  float qv[GM][8];
  {
    int m = qpos != nullptr ? qpos[b] : L;
    m = m < 0 ? 0 : m;
    float cs[4], sn[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cs[e] = 1.f;
      sn[e] = 0.f;
      if (theta != nullptr) rope_cos_sin((double)m, theta[(d0 >> 1) + e], &cs[e], &sn[e]);
    }
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
      if (gi < g) {
        const T *qp = q + ((long long)b * Hq + hk * g + gi) * D + d0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x0 = Row8<T>::scalar(qp + 2 * e), x1 = Row8<T>::scalar(qp + 2 * e + 1);
          rotate_pair(x0, x1, cs[e], sn[e]);
          qv[gi][2 * e] = x0 * scale_log2;
          qv[gi][2 * e + 1] = x1 * scale_log2;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[gi][e] = 0.f;
      }
    }
  }

  float mrun[GM], lrun[GM], acc[GM][8];
#pragma unroll
  for (int gi = 0; gi < GM; ++gi) {
    mrun[gi] = -INFINITY;
    lrun[gi] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[gi][e] = 0.f;
  }

  const long long rstride = (long long)Hkv * D;
  const T *kb = kc + ((long long)b * Lmax * Hkv + hk) * D + d0;
  const T *vb = vc + ((long long)b * Lmax * Hkv + hk) * D + d0;

  for (int base = c0 + wave * KPW; base < c1; base += KPI) {
    typename Row8<T>::Raw kr[kUnroll], vr[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int key = base + u * GPW + grp;
      ok[u] = key < c1;
      kr[u] = ok[u] ? Row8<T>::load(kb + key * rstride) : Row8<T>::zero();
      vr[u] = ok[u] ? Row8<T>::load(vb + key * rstride) : Row8<T>::zero();
    }
    float sc[GM][kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kx[8];
      Row8<T>::widen(kr[u], kx);
#pragma unroll
      for (int gi = 0; gi < GM; ++gi) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) p = fmaf(qv[gi][e], kx[e], p);
        sc[gi][u] = p;
      }
    }
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float t = group_sum<LPK>(sc[gi][u]);
        sc[gi][u] = ok[u] ? t : -INFINITY;
      }
    }
    float pu[GM][kUnroll];
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
      if (gi >= g) break;
      float mx = sc[gi][0];
#pragma unroll
      for (int u = 1; u < kUnroll; ++u) mx = fmaxf(mx, sc[gi][u]);
      const float mn = fmaxf(mrun[gi], mx);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(mrun[gi] - mu);
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        pu[gi][u] = __builtin_amdgcn_exp2f(sc[gi][u] - mu);
        psum += pu[gi][u];
      }
      lrun[gi] = lrun[gi] * alpha + psum;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[gi][e] *= alpha;
      mrun[gi] = mn;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float vx[8];
      Row8<T>::widen(vr[u], vx);
#pragma unroll
      for (int gi = 0; gi < GM; ++gi) {
        if (gi >= g) break;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[gi][e] = fmaf(pu[gi][u], vx[e], acc[gi][e]);
      }
    }
  }

  // combine the lane groups of the wave (lanes with equal `sub`)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
      const float mo = __shfl_xor(mrun[gi], off);
      const float lo = __shfl_xor(lrun[gi], off);
      float ao[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ao[e] = __shfl_xor(acc[gi][e], off);
      combine_state(mrun[gi], lrun[gi], acc[gi], mo, lo, ao);
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int gi = 0; gi < GM; ++gi) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_acc[wave][gi][d0 + e] = acc[gi][e];
      if (sub == 0) {
        sm_m[wave][gi] = mrun[gi];
        sm_l[wave][gi] = lrun[gi];
      }
    }
  }
  __syncthreads();

  // combine the waves and write the partial of each query head
  for (int idx = tid; idx < g * D; idx += kThreads) {
    const int gi = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][gi]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float s = sm_m[w][gi] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm_m[w][gi] - M);
      num += s * sm_acc[w][gi][d];
      den += s * sm_l[w][gi];
    }
    const long long row = ((long long)b * Hq + hk * g + gi) * nsplit + split;
    part_o[row * D + d] = num / den;
    if (d == 0) part_lse[row] = M + __log2f(den);
  }
}

template <int D, bool OUT_F32>
__global__ __launch_bounds__(64) void decode_merge_kernel(
    const float *__restrict__ part_o, const float *__restrict__ part_lse,
    const int *__restrict__ seqlens, int Hq, int Lmax, int chunk, int nsplit,
    void *__restrict__ out, float *__restrict__ lse) {
  constexpr int PER = D / 64;
  const int b = blockIdx.x / Hq;
  const int h = blockIdx.x % Hq;
  const int lane = threadIdx.x;
  int L = seqlens[b];
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  const int nv = (L + chunk - 1) / chunk;
  const long long row0 = ((long long)b * Hq + h) * nsplit;

  float M = -INFINITY;
  for (int p = lane; p < nv; p += 64) M = fmaxf(M, part_lse[row0 + p]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

  float num[PER], den = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) num[i] = 0.f;
  for (int p = 0; p < nv; ++p) {
    const float w = __builtin_amdgcn_exp2f(part_lse[row0 + p] - M);
    den += w;
#pragma unroll
    for (int i = 0; i < PER; ++i) num[i] += w * part_o[(row0 + p) * D + lane + 64 * i];
  }
  const long long orow = ((long long)b * Hq + h) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const float y = nv > 0 ? num[i] / den : 0.f;
    if (OUT_F32)
      ((float *)out)[orow + lane + 64 * i] = y;
    else
      ((uint16_t *)out)[orow + lane + 64 * i] = (uint16_t)f32_to_bf16(y);
  }
  if (lse != nullptr && lane == 0)
    lse[(long long)b * Hq + h] = nv > 0 ? (M + __log2f(den)) * kLn2 : -INFINITY;
}

template <typename T, int D, int GM>
hipError_t launch_split(const DecodeArgs &a, hipStream_t s) {
  const long long blocks = (long long)a.B * a.Hkv * a.nsplit;
  const float scale_log2 = (float)((double)a.softmax_scale * 1.4426950408889634074);
  hipLaunchKernelGGL((decode_split_kernel<T, D, GM>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     s, (const T *)a.q, (const T *)a.k_cache, (const T *)a.v_cache, a.seqlens,
                     a.q_pos, a.B, a.max_cache_len, a.Hq, a.Hkv, a.theta, scale_log2, a.chunk,
                     a.nsplit, a.part_o, a.part_lse, a.dev_flag);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_split_g(const DecodeArgs &a, hipStream_t s) {
  const int g = a.Hq / a.Hkv;
  if (g <= 1) return launch_split<T, D, 1>(a, s);
  if (g <= 2) return launch_split<T, D, 2>(a, s);
  if (g <= 4) return launch_split<T, D, 4>(a, s);
  if (g <= 8) return launch_split<T, D, 8>(a, s);
  return launch_split<T, D, 16>(a, s);
}

template <int D>
hipError_t launch_merge(const DecodeArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)(a.B * a.Hq)), block(64);
  if (a.out_dtype == YR_F32)
    hipLaunchKernelGGL((decode_merge_kernel<D, true>), grid, block, 0, s, a.part_o, a.part_lse,
                       a.seqlens, a.Hq, a.max_cache_len, a.chunk, a.nsplit, a.out, a.lse);
  else
    hipLaunchKernelGGL((decode_merge_kernel<D, false>), grid, block, 0, s, a.part_o, a.part_lse,
                       a.seqlens, a.Hq, a.max_cache_len, a.chunk, a.nsplit, a.out, a.lse);
  return hipGetLastError();
}

}  // namespace

int decode_chunk(int B, int max_cache_len, int Hkv) {
  // Enough workgroups to fill 256 CUs several times over, with chunks a
  // multiple of the 64 keys a workgroup covers per iteration.
  int chunk = 1024;
  while (chunk > 64 && (long long)B * Hkv * decode_nsplit(max_cache_len, chunk) < 2048) chunk >>= 1;
  return chunk;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  hipError_t e;
  if (a.in_dtype == YR_BF16)
    e = a.head_dim == 64 ? launch_split_g<uint16_t, 64>(a, s) : launch_split_g<uint16_t, 128>(a, s);
  else
    e = a.head_dim == 64 ? launch_split_g<float, 64>(a, s) : launch_split_g<float, 128>(a, s);
  if (e != hipSuccess) return e;
  return a.head_dim == 64 ? launch_merge<64>(a, s) : launch_merge<128>(a, s);
}

}  // namespace yr
