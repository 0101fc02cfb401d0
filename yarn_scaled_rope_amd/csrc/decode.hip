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

#include <atomic>
#include <mutex>
#include <type_traits>

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
    float *__restrict__ part_o, float *__restrict__ part_lse, int *flag, int window, int sinks) {
  constexpr int LPK = D / 8;         // lanes per key row
  constexpr int GPW = 64 / LPK;      // key rows per wave load
  constexpr int KPW = GPW * kUnroll; // keys per wave per iteration
  constexpr int KPI = KPW * kWaves;  // keys per workgroup per iteration

  __shared__ float sm_m[kWaves][GM];
  __shared__ float sm_l[kWaves][GM];
  __shared__ float sm_acc[kWaves][GM][D];

  if (flag != nullptr && blockIdx.x == 0) validate_decode_lens(seqlens, qpos, B, Lmax, flag);

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
  int qm = qpos != nullptr ? qpos[b] : L;  // the query's position
  qm = qm < 0 ? 0 : qm;
  // visible cache rows: the sinks [0, se) and the window [lo, L)
  int lo = 0, se = 0;
  if (window > 0) {
    lo = max(0, qm - window + 1);
    se = min(sinks, lo);
  }
  if (!(c0 < se || max(c0, lo) < c1)) {
    // nothing visible in this chunk: an empty partial (weight 0 in the merge)
    for (int idx = threadIdx.x; idx < g * D; idx += kThreads) {
      const int gi = idx / D, d = idx % D;
      const long long row = ((long long)b * Hq + hk * g + gi) * nsplit + split;
      part_o[row * D + d] = 0.f;
      if (d == 0) part_lse[row] = -INFINITY;
    }
    return;
  }

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
    float cs[4], sn[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cs[e] = 1.f;
      sn[e] = 0.f;
      if (theta != nullptr) rope_cos_sin((double)qm, theta[(d0 >> 1) + e], &cs[e], &sn[e]);
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
      ok[u] = key < c1 && (window == 0 || key >= lo || key < se);
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

// ---- bf16 / FP8 caches: matrix-core split kernel -----------------------------
// Head-per-wave form: a workgroup owns (sequence, key range, group of W KV
// heads), the range being a key chunk or one workgroup's share of a balanced
// split (STREAM below); wave w sweeps the whole range for KV head hg*W + w,
// so the W waves stream the same cache rows side by side and together read
// each row's W heads (W*D elements, contiguous) at about the same time:
// measured 7.1 TB/s for that access pattern against 6.3 TB/s when each
// workgroup owns one head's 256-byte slices of the rows.  Shared form (SH):
// the waves of a workgroup take alternate blocks of one KV head's chunk and
// combine through LDS.  Per 32-key block a wave computes S^T = K Q^T (keys x
// query heads of its KV head, v_mfma_f32_32x32x16_bf16 with those heads as
// the 32 columns) and O^T += V^T P^T, and at the end writes its heads'
// partial (O, log2-sum-exp) itself.  K and V blocks go straight from HBM into a ring of LDS
// stages private to the wave (buffer_load ... lds: no staging registers, no
// workgroup barriers in the sweep); the wave waits on exact vmcnt counts, so
// the next blocks stream in while the current one is computed.
//   K stage: row r holds key r; its 16-byte chunk c sits at slot c ^ (r & (CH-1)),
//     so the A-operand reads (32 rows, one chunk each) hit distinct banks.
//   V stage: row r holds key r; chunk c sits at slot c ^ vswz(r & 3).  The
//     V^T operand comes from ds_read_b64_tr_b16: within 16 lanes, lane t reads
//     4 elements of key row t>>2 and receives column t of 4 consecutive key
//     rows.  Keys 4..7 of a k-step half sit in the other lane half, matching
//     the order in which the score accumulator holds P (slot 4j+i of lane half
//     h is key 8j + 4h + i).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define YR_LDS __attribute__((address_space(3)))


// V chunk swizzle by key row mod 4: bits 1-2 distinct (conflict-free for 16
// lanes on 32 banks) and, with 16 chunks per row, bits 2-3 distinct too
// (conflict-free for 32 lanes on 64 banks).
template <int CH>
__device__ __forceinline__ int vswz(int e) {
  return CH >= 16 ? ((2 * e) ^ (8 * (e & 1))) : 2 * e;
}

// FP8 (E4M3) cache rows: 16-byte slot swizzles that keep the K reads (8
// rows x one 16-byte chunk per pass) and the 8-bit transposing V reads (8 key
// rows 0-3, 8-11 (+4) x one chunk per 16 lanes) on distinct banks.
template <int D>
__device__ __forceinline__ int kswz8(int row) {
  return D >= 128 ? (row & 7) : ((row >> 1) & 3);
}
template <int D>
__device__ __forceinline__ int vswz8(int row) {
  return D >= 128 ? ((row & 3) | (((row >> 3) & 1) << 2)) : (((row >> 1) & 1) | (((row >> 3) & 1) << 1));
}

// Cache element bytes -> bf16 pairs: E4M3 values are exact in bf16.
// HI picks bytes 2-3 of the word instead of 0-1.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return u32x4{fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
               fp8x2_to_bf16x2<true>(w1)};
}

template <int D, int W>
struct MfmaComb {  // the waves' partial states of one KV head, combined at the end
  float o[W][D][33];
  float m[W][32];
  float l[W][32];
};
template <int D, int W, int NB, int EB, bool SH>
struct MfmaSmem {
  union {
    uint8_t ring[W][NB][2][kBlk * D * EB];  // [wave][stage][K|V][row bytes, swizzled chunks]
    std::conditional_t<SH, MfmaComb<D, W>, char> comb;
  } u;
  uint16_t qt[SH ? 32 : 1][D + 8];  // SH: the rotated query heads (bf16), one per row
  float cs[D / 2], sn[D / 2];        // cos / sin of the query position
};


// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
template <int H, int MAXHALVES>
__device__ __forceinline__ void wait_halves(int halves) {
  // halves is wave-uniform: a scalar branch picks the immediate
  if (MAXHALVES >= 7 && halves >= 7) { wait_vm<7 * H>(); return; }
  if (MAXHALVES >= 6 && halves == 6) { wait_vm<6 * H>(); return; }
  if (MAXHALVES >= 5 && halves == 5) { wait_vm<5 * H>(); return; }
  if (MAXHALVES >= 4 && halves == 4) { wait_vm<4 * H>(); return; }
  if (MAXHALVES >= 3 && halves == 3) { wait_vm<3 * H>(); return; }
  if (halves == 2) { wait_vm<2 * H>(); return; }
  if (halves == 1) { wait_vm<H>(); return; }
  wait_vm<0>();
}
// every LDS read issued so far has returned (before a DMA overwrites a stage)
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// LDS byte address of a shared-memory pointer
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const YR_LDS void *)p;
}

// LDS accesses away from the ring, in asm: written as builtins, they would
// make the compiler wait for every LDS DMA of the wave in flight.  The read
// waits for its own result inside the block.
__device__ __forceinline__ void lds_store_f32(uint32_t addr, float v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ f32x4 lds_load_f32x4(uint32_t addr) {
  f32x4 r;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(addr) : "memory");
  return r;
}
// workgroup barrier after this wave's LDS accesses have completed (not its
// global ones, unlike __syncthreads)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The V^T operands of one k-step: for each 32-row block db, two transposing
// reads (key rows +0 and +ROWSTEP bytes).  The reads and the wait for them
// sit in one asm block, so no destination register is live in flight outside
// it.  (Written as a builtin, each such read makes the compiler wait for every
// outstanding LDS DMA of the wave, which would drain the prefetch.)
template <int DBLK, int OFF, int ROWSTEP>
__device__ __forceinline__ void tr_reads(u32x2 (&r)[DBLK][2], const uint32_t (&a)[DBLK]) {
  static_assert(DBLK == 2 || DBLK == 4, "head_dim 64 or 128");
  if constexpr (DBLK == 4) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
        "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
        "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
        "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[1][0]), "=&v"(r[1][1]), "=&v"(r[2][0]),
          "=&v"(r[2][1]), "=&v"(r[3][0]), "=&v"(r[3][1])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF), "i"(OFF + ROWSTEP)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
        "ds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
        "ds_read_b64_tr_b16 %2, %5 offset:%6\n\t"
        "ds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[1][0]), "=&v"(r[1][1])
        : "v"(a[0]), "v"(a[1]), "i"(OFF), "i"(OFF + ROWSTEP)
        : "memory");
  }
}

// The 8-bit V^T operands of one k-step: one transposing read per 32-row block
// db (within 16 lanes, lane t receives byte t & 7 of the 8 bytes addressed by
// lane 2e + (t >> 3) as element e: 8 keys of one column), reads and wait in one
// asm block as above.
template <int DBLK, int OFF>
__device__ __forceinline__ void tr8_reads(u32x2 (&r)[DBLK], const uint32_t (&a)[DBLK]) {
  static_assert(DBLK == 2 || DBLK == 4, "head_dim 64 or 128");
  if constexpr (DBLK == 4) {
    asm volatile(
        "ds_read_b64_tr_b8 %0, %4 offset:%8\n\t"
        "ds_read_b64_tr_b8 %1, %5 offset:%8\n\t"
        "ds_read_b64_tr_b8 %2, %6 offset:%8\n\t"
        "ds_read_b64_tr_b8 %3, %7 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b8 %0, %2 offset:%4\n\t"
        "ds_read_b64_tr_b8 %1, %3 offset:%4\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1])
        : "v"(a[0]), "v"(a[1]), "i"(OFF)
        : "memory");
  }
}

// WIN: sliding window / sinks (compiled out without it).  SH: the W waves
// share one KV head and take alternate blocks of the chunk, then combine
// through LDS (the FP8 form: its blocks are half the bytes and twice the
// conversion work, and measured faster this way, 6.2 against 5.9 TB/s).
// Cache rows of sequence bb that its query sees: all of [0, L), or with a
// window the sinks [0, se) and the window [lo, L) (the query at q_pos or L).
__device__ __forceinline__ int decode_visible_rows(int bb, const int *seqlens, const int *qpos,
                                                   int Lmax, int window, int sinks) {
  int L = seqlens[bb];
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  if (window <= 0) return L;
  int qm = qpos != nullptr ? qpos[bb] : L;
  qm = qm < 0 ? 0 : qm;
  const int lo = max(0, qm - window + 1);
  const int se = min(sinks, lo);
  return se + max(0, L - lo);
}

// STREAM (head-per-wave form): instead of one chunk per
// workgroup, the flattened space of (sequence, head group, 32-key block) is
// cut into gridDim.x equal ranges, one per workgroup (one per CU); a
// workgroup sweeps the pieces of the segments its range meets and writes one
// partial per piece, at index (workgroup + segment).  Every CU then streams
// the same number of blocks, and no CU waits for a last round of chunks.
template <int D, int W, int NB, bool FP8, bool WIN, bool SH, bool STREAM>
__global__ __launch_bounds__(W * 64) void decode_mfma_kernel(
    const uint16_t *__restrict__ q, const void *__restrict__ kc,
    const void *__restrict__ vc, const int *__restrict__ seqlens,
    const int *__restrict__ qpos, int B, int Lmax, int Hq, int Hkv,
    const double *__restrict__ theta, float scale_log2, int chunk, int nsplit,
    float *__restrict__ part_o, float *__restrict__ part_lse, int *flag, int window, int sinks,
    const float *__restrict__ k_scale, const float *__restrict__ v_scale, int vis_split) {
  if constexpr (!WIN) {
    window = 0;
    sinks = 0;
    vis_split = 0;
  }
  constexpr int EB = FP8 ? 1 : 2;  // bytes per cached element
  constexpr int ROWB = D * EB;     // bytes per cached key row
  constexpr int CH = ROWB / 16;    // 16-byte chunks per row
  constexpr int H = kBlk * ROWB / 1024;  // DMA instructions per K or V block (1 KB each)
  constexpr int RPI = 64 / CH;     // rows per DMA instruction
  constexpr int KSTEPS = D / 16;   // score k-steps over the head dim
  constexpr int DBLK = D / 32;     // 32-row blocks of O^T
  constexpr int NT = W * 64;
  static_assert((2 * NB - 1) * H < 64, "vmcnt range");

  __shared__ __align__(16) MfmaSmem<D, W, NB, EB, SH> sm;
  constexpr int HW = SH ? 1 : W;  // KV heads of the workgroup

  if (flag != nullptr && blockIdx.x == 0) validate_decode_lens(seqlens, qpos, B, Lmax, flag);
  static_assert(!STREAM || !SH, "the balanced split is for the head-per-wave form");

  // STREAM: this workgroup's range [r, r1) of the flattened block space;
  // a sequence contributes the 32-key blocks of its visible rows (all of
  // [0, L), or with a window the sinks and then the window, counted in order)
  auto nblocks_of = [&](int bb) {
    return (decode_visible_rows(bb, seqlens, qpos, Lmax, window, sinks) + kBlk - 1) / kBlk;
  };
  const int ngr = Hkv / HW;
  // STREAM: [r, r1) is this workgroup's range; (bcur, basecur) the sequence
  // that holds block r and the index of that sequence's first block.  Each
  // thread sums the blocks of a contiguous chunk of sequences, a scan over
  // the chunks (LDS) gives the total and each chunk's first block, and the
  // thread whose chunk holds block r walks it to the sequence: O(B / threads)
  // per workgroup, whatever the batch size.
  long long r = 0, r1 = 0, basecur = 0;
  int bcur = 0;
  if constexpr (STREAM) {
    __shared__ int scan[NT];
    __shared__ int first_b;
    __shared__ long long first_base;
    const int t = threadIdx.x;
    const int cpt = (B + NT - 1) / NT;
    const int bb0 = min(B, t * cpt), bb1 = min(B, bb0 + cpt);
    int loc = 0;
    for (int bb = bb0; bb < bb1; ++bb) loc += nblocks_of(bb);
    scan[t] = loc;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
      const int v = t >= off ? scan[t - off] : 0;
      __syncthreads();
      scan[t] += v;
      __syncthreads();
    }
    const long long tb = (long long)ngr * scan[NT - 1];
    const long long per = tb > 0 ? (tb + gridDim.x - 1) / gridDim.x : 1;
    const long long rs = (long long)blockIdx.x * per;
    if (rs >= tb) return;  // uniform: every thread read the same total
    const long long before = (long long)ngr * (t > 0 ? scan[t - 1] : 0);
    const long long after = (long long)ngr * scan[t];
    if (rs >= before && rs < after) {
      long long base = before;
      int bb = bb0;
      for (;; ++bb) {
        const long long nb = (long long)ngr * nblocks_of(bb);
        if (rs < base + nb) break;
        base += nb;
      }
      first_b = bb;
      first_base = base;
    }
    __syncthreads();
    bcur = first_b;
    basecur = first_base;
    r = rs;
    r1 = min(tb, rs + per);
  }
  for (;;) {  // STREAM: one pass per piece; otherwise a single pass
  int hg, split, b, c0, cnt = 0;
  if constexpr (STREAM) {
    // the segment (sequence b, head group hg) holding block r, and the piece
    // of it in this range; split = index of this piece's partial.  Later
    // pieces lie in later segments: step forward from the previous one.
    int nbk = nblocks_of(bcur);
    while (r >= basecur + (long long)ngr * nbk) {
      basecur += (long long)ngr * nbk;
      nbk = nblocks_of(++bcur);
    }
    b = bcur;
    hg = (int)((r - basecur) / nbk);
    const int blk0 = (int)((r - basecur) % nbk);
    cnt = (int)min((long long)(nbk - blk0), r1 - r);
    c0 = blk0 * kBlk;
    split = (int)blockIdx.x + b * ngr + hg;
  } else if constexpr (SH) {
    // Shared: chunk fastest (measured faster for that form)
    split = blockIdx.x % nsplit;
    const int rest = blockIdx.x / nsplit;
    hg = rest % Hkv;
    b = rest / Hkv;
    c0 = split * chunk;
  } else {
    // Head-per-wave: head group fastest, so that the workgroups that read the
    // other heads of the same cache rows are launched next to this one
    hg = blockIdx.x % ngr;
    const int rest = blockIdx.x / ngr;
    split = rest % nsplit;
    b = rest / nsplit;
    c0 = split * chunk;
  }
  const int g = Hq / Hkv;
  int L = seqlens[b];
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  if (!STREAM && vis_split == 0 && c0 >= L) return;
  int qm = qpos != nullptr ? qpos[b] : L;  // the query's position
  qm = qm < 0 ? 0 : qm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hk = SH ? hg : hg * W + wave;  // this wave's KV head
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int gc = min(g, 32);

  // Visible cache rows: the sinks [0, se) and the window [lo, L) (no window:
  // all of [0, L)).  This chunk sweeps its share of each as 32-key blocks:
  // blocks 0 .. nba-1 cover [c0, c0 + na), the rest cover [b0, b0 + nb).
  // Chunks split the cache rows [0, L), or (vis_split) the visible rows
  // alone, counted in order: the sinks, then the window; the last chunk then
  // takes every visible row from its start on, so any query position is
  // covered.
  int lo = 0, se = 0;
  if (window > 0) {
    lo = max(0, qm - window + 1);
    se = min(sinks, lo);
  }
  int na, b0, nb;
  if (vis_split != 0 || (STREAM && WIN)) {
    const int nvis = se + max(0, L - lo);
    const int v1 = STREAM ? min(nvis, c0 + cnt * kBlk)
                          : (split == nsplit - 1 ? nvis : min(nvis, c0 + chunk));
    na = max(0, min(v1, se) - c0);
    b0 = lo + max(c0, se) - se;
    nb = max(0, v1 - max(c0, se));
  } else {
    const int c1 = STREAM ? min(L, c0 + cnt * kBlk) : min(L, c0 + chunk);
    na = max(0, min(c1, se) - c0);
    b0 = max(c0, lo);
    nb = max(0, c1 - b0);
  }
  const int nba = (na + kBlk - 1) / kBlk;
  const int nblk = nba + (nb + kBlk - 1) / kBlk;
  if (nblk == 0) {
    // nothing visible here: empty partials (weight 0 in the merge) for every
    // query head of the workgroup's KV heads
    for (int idx = tid; idx < HW * gc * D; idx += NT) {
      const int w = idx / (gc * D), gi = (idx / D) % gc, d = idx % D;
      const long long row = ((long long)b * Hq + (hg * HW + w) * g + gi) * nsplit + split;
      part_o[row * D + d] = 0.f;
      if (d == 0) part_lse[row] = -INFINITY;
    }
    return;
  }
  auto blk_start = [&](int gb) { return gb < nba ? c0 + gb * kBlk : b0 + (gb - nba) * kBlk; };
  auto blk_rows = [&](int gb) {
    return gb < nba ? min(kBlk, na - gb * kBlk) : min(kBlk, nb - (gb - nba) * kBlk);
  };

  const long long rstride = (long long)Hkv * ROWB;  // bytes between keys
  const uint8_t *kbase = (const uint8_t *)kc + ((long long)b * Lmax * Hkv + hk) * ROWB;
  const uint8_t *vbase = (const uint8_t *)vc + ((long long)b * Lmax * Hkv + hk) * ROWB;
  // blocks of this wave: every block of the chunk, or (SH) every W-th
  const int nmine = SH ? (nblk > wave ? (nblk - wave + W - 1) / W : 0) : nblk;
  auto gblk = [&](int t) { return SH ? wave + t * W : t; };
  // FP8: the per-head scales fold into the logit scale and the output
  float sl = scale_log2, vsc = 1.f;
  if constexpr (FP8) {
    sl = scale_log2 * k_scale[hk];
    vsc = v_scale[hk];
  }

  // DMA lane mapping: instruction p of a block fills LDS bytes [1024p, 1024p+1024)
  // in lane order; lane l lands on row p*RPI + l/CH, slot l%CH, so it fetches
  // the source chunk that belongs in that slot.
  const int drow = lane / CH, dslot = lane % CH;
  uint32_t voff_k[H], voff_v[H];
#pragma unroll
  for (int p = 0; p < H; ++p) {
    const int r = p * RPI + drow;
    const int kx = FP8 ? kswz8<D>(r) : (r & (CH - 1));
    const int vx = FP8 ? vswz8<D>(r) : vswz<CH>(r & 3);
    voff_k[p] = (uint32_t)(r * rstride + 16 * (dslot ^ kx));
    voff_v[p] = (uint32_t)(r * rstride + 16 * (dslot ^ vx));
  }

  // t-th block of this wave -> stage; rows past the block's share read 0,
  // and so does the whole stage when the wave has no t-th block (the first
  // stages are always issued, so that every path has the same loads in flight
  // and the compiler's waits for the query loads stay partial)
  auto issue = [&](int t, int stage, int which) {
    const bool ok = t < nmine;
    const int key0 = ok ? blk_start(gblk(t)) : 0;
    const int rows = ok ? blk_rows(gblk(t)) : 0;
    const uint32_t bytes = ok ? (uint32_t)((rows - 1) * rstride + ROWB) : 0u;
    const uint8_t *src = (which == 0 ? kbase : vbase) + key0 * rstride;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, bytes);
    uint8_t *dst = sm.u.ring[wave][stage][which];
#pragma unroll
    for (int p = 0; p < H; ++p) {
      const uint32_t vo = which == 0 ? voff_k[p] : voff_v[p];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (YR_LDS void *)(dst + p * 1024), 16, (int)vo, 0,
                                               0, 2 /* non-temporal */);
    }
  };

  // ---- query heads of the wave's KV head (one per MFMA column l32; columns
  // past the group are zero), rotated at the new token's position and rounded
  // to bf16.  k-step kk, lane half hh covers head dims qd(kk) .. +7:
  // 16 kk + 8 hh, or with an FP8 cache, where one 16-byte read of a K row
  // serves two k-steps, 16 (2 (kk / 2) + hh) + 8 (kk % 2).
  auto qd = [&](int kk) { return FP8 ? 16 * (2 * (kk / 2) + hh) + 8 * (kk % 2) : 16 * kk + 8 * hh; };
  static_assert(D / 2 <= NT, "one frequency per thread");
  // Head-per-wave: each lane loads its query row ahead of the first blocks,
  // so that the wait for it does not take in theirs, and the LDS round trip
  // of cos / sin goes through asm for the same reason.
  u32x4 qraw[KSTEPS];
  double th = 0.0;
  if constexpr (!SH) {
    const uint16_t *qrow = q + ((long long)b * Hq + hk * g + min(l32, gc - 1)) * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qraw[kk] = *reinterpret_cast<const u32x4 *>(qrow + qd(kk));
    if (theta != nullptr) th = theta[tid & (D / 2 - 1)];
  }

#pragma unroll
  for (int s = 0; s < NB; ++s) {
    issue(s, s, 0);
    issue(s, s, 1);
  }

  bf16x8 qf[KSTEPS];
  if constexpr (SH) {
    // Shared: the waves stage the one group's heads through LDS; the
    // barriers here also wait for the first blocks, so the waves start the
    // sweep together (measured faster for this form than letting each start
    // as soon as its query is in, 6.0 against 5.7 TB/s with FP8)
    if (tid < D / 2) {
      float c = 1.f, s = 0.f;
      if (theta != nullptr) rope_cos_sin((double)qm, theta[tid], &c, &s);
      sm.cs[tid] = c;
      sm.sn[tid] = s;
    }
    __syncthreads();
    for (int idx = tid; idx < 32 * (D / 2); idx += NT) {
      const int col = idx / (D / 2), pr = idx % (D / 2);
      float x0 = 0.f, x1 = 0.f;
      if (col < gc) {
        const uint16_t *qp = q + ((long long)b * Hq + hk * g + col) * D + 2 * pr;
        x0 = bf16_to_f32(qp[0]);
        x1 = bf16_to_f32(qp[1]);
        rotate_pair(x0, x1, sm.cs[pr], sm.sn[pr]);
      }
      *reinterpret_cast<uint32_t *>(&sm.qt[col][2 * pr]) = pack_bf16x2(x0, x1);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&sm.qt[l32][qd(kk)]));
  } else {
    const uint32_t cs_addr = lds_addr(sm.cs), sn_addr = lds_addr(sm.sn);
    if (tid < D / 2) {
      float c = 1.f, s = 0.f;
      if (theta != nullptr) rope_cos_sin((double)qm, th, &c, &s);
      lds_store_f32(cs_addr + 4 * tid, c);
      lds_store_f32(sn_addr + 4 * tid, s);
    }
    lds_barrier();
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const int d0 = qd(kk);  // pairs d0 / 2 .. +3: one aligned 16-byte read each
      const f32x4 c4 = lds_load_f32x4(cs_addr + 2 * d0), s4 = lds_load_f32x4(sn_addr + 2 * d0);
      u32x4 w = qraw[kk];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x0 = bf16_to_f32(w[e] & 0xffffu), x1 = bf16_to_f32(w[e] >> 16);
        rotate_pair(x0, x1, c4[e], s4[e]);
        w[e] = l32 < gc ? pack_bf16x2(x0, x1) : 0u;
      }
      qf[kk] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x16 o[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float mrun = -INFINITY;  // running max of the column, log2 units
  float lsum = 0.f;        // this lane's share of the column's sum

  // LDS read offsets within a stage: K row l32, 16-byte chunk slot c ^ kx
  const int kx = FP8 ? kswz8<D>(l32) : (l32 & (CH - 1));
  // V^T operand addresses (LDS bytes, stage 0 of this wave; the stage, k-step
  // and row-half offsets are immediates).
  //   bf16: lane t of a 16-lane group points at 4 elements of key row
  //     4*hh + (t >> 2) (+16 ks + 8 r), column block 4*db + its chunk within the
  //     16 columns of the group.
  //   FP8: lane t points at the 8 bytes of key row 8 (e >> 2) + 4 hh + (e & 3),
  //     e = t >> 1 (+16 ks), columns 32 db + 16 (group parity) + 8 (t & 1).
  constexpr int kStageBytes = 2 * kBlk * ROWB;
  uint32_t vaddr[DBLK];
  {
    const int t16 = lane & 15;
    const uint32_t ring0 = lds_addr(sm.u.ring[wave][0][0]);
    if constexpr (FP8) {
      const int e = t16 >> 1;
      const int vrow = 8 * (e >> 2) + 4 * hh + (e & 3);
      const int vx = vswz8<D>(vrow);
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
        vaddr[db] = ring0 + (uint32_t)(vrow * ROWB + 16 * ((2 * db + ((lane >> 4) & 1)) ^ vx) +
                                       8 * (t16 & 1));
    } else {
      const int vrow = 4 * hh + (t16 >> 2);
      const int vx = vswz<CH>(t16 >> 2);
      const int vcol = 2 * ((lane >> 4) & 1) + ((t16 & 3) >> 1);
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
        vaddr[db] = ring0 + (uint32_t)((vrow * D + 8 * ((4 * db + vcol) ^ vx) + 4 * (t16 & 1)) * 2);
    }
  }

  auto block = [&](int t, auto stage_c) {
    constexpr int S = decltype(stage_c)::value;
    const int rows = blk_rows(gblk(t));
    const int ahead = min(NB - 1, nmine - 1 - t);  // later blocks already issued
    const bool refill = t + NB < nmine;

    wait_halves<H, 2 * NB - 1>(1 + 2 * ahead);  // K of block t has landed
    const uint8_t *ks_ = sm.u.ring[wave][S][0];
    f32x16 sc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[e] = 0.f;
    if constexpr (FP8) {
#pragma unroll
      for (int kp = 0; kp < KSTEPS / 2; ++kp) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(ks_ + l32 * ROWB + 16 * ((2 * kp + hh) ^ kx));
        const u32x4 a0 = fp8x8_to_bf16x8(w[0], w[1]);
        const u32x4 a1 = fp8x8_to_bf16x8(w[2], w[3]);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a0), qf[2 * kp], sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a1), qf[2 * kp + 1], sc, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(ks_ + l32 * ROWB + 16 * ((2 * kk + hh) ^ kx));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[kk], sc, 0, 0, 0);
      }
    }
    if (refill) {
      wait_lds();
      issue(t + NB, S, 0);
    }

    // online softmax of the column (query head) l32 over this block
    if (rows < kBlk) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 8 * (e >> 2) + 4 * hh + (e & 3);
        sc[e] = r < rows ? sc[e] : -INFINITY;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sc[e]);
    mx = half_max(mx);
    const float mnew = fmaxf(mrun, mx * sl);
    // lazy rescale: keep the reference max until some column's max has grown
    // by more than 2^8 (p stays <= 256, exact in fp32 sums, fine in bf16)
    if (__builtin_amdgcn_ballot_w64(mnew > mrun + 8.f) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      mrun = mnew;
    }
    float p[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = __builtin_amdgcn_exp2f(fmaf(sc[e], sl, -mrun));
      lsum += p[e];
    }
    bf16x8 pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(p[8 * ks + 2 * e], p[8 * ks + 2 * e + 1]);
      pf[ks] = __builtin_bit_cast(bf16x8, w);
    }

    wait_halves<H, 2 * NB - 1>(2 * ahead + (refill ? 1 : 0));  // V of block t has landed
    auto pv_step = [&](auto ks_c) {
      constexpr int KS = decltype(ks_c)::value;
      if constexpr (FP8) {
        u32x2 b8[DBLK];
        tr8_reads<DBLK, S * kStageBytes + kBlk * ROWB + KS * 16 * ROWB>(b8, vaddr);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          const u32x4 a = fp8x8_to_bf16x8(b8[db][0], b8[db][1]);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pf[KS],
                                                          o[db], 0, 0, 0);
        }
      } else {
        u32x2 h2[DBLK][2];
        tr_reads<DBLK, S * kStageBytes + kBlk * ROWB + KS * 16 * ROWB, 8 * ROWB>(h2, vaddr);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          const u32x4 a = {h2[db][0][0], h2[db][0][1], h2[db][1][0], h2[db][1][1]};
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pf[KS],
                                                          o[db], 0, 0, 0);
        }
      }
    };
    pv_step(std::integral_constant<int, 0>{});
    pv_step(std::integral_constant<int, 1>{});
    if (refill) {
      wait_lds();
      issue(t + NB, S, 1);
    }
  };

  for (int t = 0; t < nmine; t += NB) {
    block(t, std::integral_constant<int, 0>{});
    if (NB > 1 && t + 1 < nmine) block(t + 1, std::integral_constant<int, (NB > 1 ? 1 : 0)>{});
    if (NB > 2 && t + 2 < nmine) block(t + 2, std::integral_constant<int, (NB > 2 ? 2 : 0)>{});
    if (NB > 3 && t + 3 < nmine) block(t + 3, std::integral_constant<int, (NB > 3 ? 3 : 0)>{});
  }

  // ---- the two lane halves of a column hold disjoint keys of the same
  // query head
  lsum = half_sum(lsum);
  if constexpr (!SH) {
    // the wave saw the whole chunk for its KV head: it writes the partials
    // (STREAM: partial `split` holds the W*g query heads of the group)
    if (l32 < gc) {
      const long long row = STREAM ? (long long)split * (W * g) + wave * g + l32
                                   : ((long long)b * Hq + hk * g + l32) * nsplit + split;
      const float inv = vsc / lsum;
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<float4 *>(part_o + row * D + 32 * db + 8 * j + 4 * hh) =
              make_float4(o[db][4 * j] * inv, o[db][4 * j + 1] * inv, o[db][4 * j + 2] * inv,
                          o[db][4 * j + 3] * inv);
      if (hh == 0) part_lse[row] = mrun + __log2f(lsum);
    }
  } else {
    // the waves saw alternate blocks: combine them through LDS (the ring is
    // free once every wave is here); a wave without blocks has m = -inf
    __syncthreads();
    if (l32 < gc) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          sm.u.comb.o[wave][32 * db + 8 * (e >> 2) + 4 * hh + (e & 3)][l32] = o[db][e];
      if (hh == 0) {
        sm.u.comb.m[wave][l32] = mrun;
        sm.u.comb.l[wave][l32] = lsum;
      }
    }
    __syncthreads();
    for (int idx = tid; idx < gc * D; idx += NT) {
      const int gi = idx / D, d = idx % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < W; ++w) M = fmaxf(M, sm.u.comb.m[w][gi]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float mw = sm.u.comb.m[w][gi];
        const float sc_ = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        num += sc_ * sm.u.comb.o[w][d][gi];
        den += sc_ * sm.u.comb.l[w][gi];
      }
      const long long row = ((long long)b * Hq + hk * g + gi) * nsplit + split;
      part_o[row * D + d] = num / den * vsc;
      if (d == 0) part_lse[row] = M + __log2f(den);
    }
  }
  if constexpr (!STREAM) {
    break;
  } else {
    r += cnt;
    if (r >= r1) break;
    lds_barrier();  // every wave is past its reads of cos / sin
  }
  }  // piece loop
}

// nwg > 0: the partials of a balanced split (decode_mfma_kernel<..., STREAM>)
// over nwg workgroups of hpw KV heads each; the pieces of this query head's
// segment are found from seqlens the same way the split found them.
// PERWAVE: a workgroup takes 4 query heads of one sequence, one per wave (for
// few partials per head: the sequence's place in the batch is found once for
// the 4 heads, and no wave waits on the others); otherwise its 4 waves share
// the partials of one head.
template <int D, bool OUT_F32, bool PERWAVE>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float *__restrict__ part_o, const float *__restrict__ part_lse,
    const int *__restrict__ seqlens, int Hq, int Lmax, int chunk, int nsplit, int vis_split,
    void *__restrict__ out, float *__restrict__ lse, int B, int Hkv, int nwg, int hpw,
    const int *__restrict__ qpos, int window, int sinks) {
  constexpr int PER = D / 64;  // output elements per lane
  constexpr int NW = 4;        // waves of the workgroup
  // waves sharing one head: wave w takes partials w, w + MW, ...
  constexpr int MW = PERWAVE ? 1 : NW;
  constexpr int U = 4;         // partials per wave in flight
  __shared__ float sm_num[MW][D];
  __shared__ float sm_den[MW];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hpb = PERWAVE ? Hq / NW : Hq;  // workgroups per sequence
  const int b = blockIdx.x / hpb;
  const int h = PERWAVE ? (blockIdx.x % hpb) * NW + wave : blockIdx.x % hpb;
  const int wv = PERWAVE ? 0 : wave;  // this wave's first partial
  int L = seqlens[b];
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  // partials written: every chunk of the visible rows, or the chunks of
  // [0, L) (those starting past L exit without one); partial p is row
  // row0 + p * stride
  int nv;
  long long row0, stride = 1;
  if (nwg > 0) {
    const int g = Hq / Hkv, ngr = Hkv / hpw;
    const int hk = h / g, hg = hk / hpw;
    auto nblocks_of = [&](int bb) {
      return (decode_visible_rows(bb, seqlens, qpos, Lmax, window, sinks) + kBlk - 1) / kBlk;
    };
    // blocks of the whole batch and of the sequences before b: strided
    // sums over the threads, then the waves' sums through LDS
    int all = 0, lt = 0;
    for (int bb = threadIdx.x; bb < B; bb += 256) {
      const int n = nblocks_of(bb);
      all += n;
      if (bb < b) lt += n;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      all += __shfl_xor(all, off);
      lt += __shfl_xor(lt, off);
    }
    __shared__ int red[2][NW];
    if (lane == 0) {
      red[0][wave] = all;
      red[1][wave] = lt;
    }
    __syncthreads();
    all = lt = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      all += red[0][w];
      lt += red[1][w];
    }
    const long long tb = (long long)ngr * all, base = (long long)ngr * lt;
    const long long per = tb > 0 ? (tb + nwg - 1) / nwg : 1;
    const int nbk = nblocks_of(b);
    const long long s0 = base + (long long)hg * nbk;  // first block of the segment
    const long long w0 = s0 / per;
    nv = nbk > 0 ? (int)((s0 + nbk - 1) / per - w0 + 1) : 0;
    stride = (long long)hpw * g;
    row0 = (w0 + (long long)b * ngr + hg) * stride + (hk % hpw) * g + h % g;
  } else {
    nv = vis_split != 0 ? nsplit : (L + chunk - 1) / chunk;
    row0 = ((long long)b * Hq + h) * nsplit;
  }

  // The wave's first U partials are loaded before the reference below is
  // known, so that both loads are in flight together.
  float w0[U], x0[U][PER];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int pu = wv + u * MW;
    w0[u] = -INFINITY;
#pragma unroll
    for (int i = 0; i < PER; ++i) x0[u][i] = 0.f;
    if (pu < nv) {
      const long long rw = row0 + pu * stride;
      w0[u] = part_lse[rw];
#pragma unroll
      for (int i = 0; i < PER; ++i) x0[u][i] = part_o[rw * D + lane + 64 * i];
    }
  }
  // common reference: the largest partial log2-sum-exp (every wave computes it)
  float M = -INFINITY;
  for (int p = lane; p < nv; p += 64) M = fmaxf(M, part_lse[row0 + p * stride]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  // no visible key in any chunk (a query placed past its window): empty result
  const bool none = nv == 0 || M == -INFINITY;
  if (none) M = 0.f;

  float num[PER], den = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) num[i] = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // partials past nv (w0 = -inf) and empty ones weigh 0
    const float e = w0[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(w0[u] - M);
    den += e;
#pragma unroll
    for (int i = 0; i < PER; ++i) num[i] = fmaf(e, x0[u][i], num[i]);
  }
  int p = wv + U * MW;
  for (; p + (U - 1) * MW < nv; p += U * MW) {
    float w[U], x[U][PER];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long rw = row0 + (p + u * MW) * stride;
      w[u] = part_lse[rw];
#pragma unroll
      for (int i = 0; i < PER; ++i) x[u][i] = part_o[rw * D + lane + 64 * i];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float e = __builtin_amdgcn_exp2f(w[u] - M);
      den += e;
#pragma unroll
      for (int i = 0; i < PER; ++i) num[i] = fmaf(e, x[u][i], num[i]);
    }
  }
  for (; p < nv; p += MW) {
    const long long rw = row0 + p * stride;
    const float e = __builtin_amdgcn_exp2f(part_lse[rw] - M);
    den += e;
#pragma unroll
    for (int i = 0; i < PER; ++i) num[i] = fmaf(e, part_o[rw * D + lane + 64 * i], num[i]);
  }
  if constexpr (!PERWAVE) {
#pragma unroll
    for (int i = 0; i < PER; ++i) sm_num[wave][lane + 64 * i] = num[i];
    if (lane == 0) sm_den[wave] = den;
    __syncthreads();
    if (wave != 0) return;
    den = 0.f;
#pragma unroll
    for (int w = 0; w < MW; ++w) den += sm_den[w];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < MW; ++w) t += sm_num[w][lane + 64 * i];
      num[i] = t;
    }
  }
  const long long orow = ((long long)b * Hq + h) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const float y = none ? 0.f : num[i] / den;
    if (OUT_F32)
      ((float *)out)[orow + lane + 64 * i] = y;
    else
      ((uint16_t *)out)[orow + lane + 64 * i] = (uint16_t)f32_to_bf16(y);
  }
  if (lse != nullptr && lane == 0)
    lse[(long long)b * Hq + h] = none ? -INFINITY : (M + __log2f(den)) * kLn2;
}

template <typename T, int D, int GM>
hipError_t launch_split(const DecodeArgs &a, hipStream_t s) {
  const long long blocks = (long long)a.B * a.Hkv * a.nsplit;
  const float scale_log2 = (float)((double)a.softmax_scale * 1.4426950408889634074);
  hipLaunchKernelGGL((decode_split_kernel<T, D, GM>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     s, (const T *)a.q, (const T *)a.k_cache, (const T *)a.v_cache, a.seqlens,
                     a.q_pos, a.B, a.max_cache_len, a.Hq, a.Hkv, a.theta, scale_log2, a.chunk,
                     a.nsplit, a.part_o, a.part_lse, a.dev_flag, a.window, a.sinks);
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

template <int D, bool FP8, bool WIN, int W, bool SH = false, bool STREAM = false>
hipError_t launch_mfma_w(const DecodeArgs &a, hipStream_t s) {
  constexpr int NB = SH ? 1 : kMfmaStages;
  const long long blocks =
      STREAM ? a.stream_wg : (long long)a.B * (SH ? a.Hkv : a.Hkv / W) * a.nsplit;
  const float scale_log2 = (float)((double)a.softmax_scale * 1.4426950408889634074);
  hipLaunchKernelGGL((decode_mfma_kernel<D, W, NB, FP8, WIN, SH, STREAM>), dim3((unsigned)blocks), dim3(W * 64), 0,
                     s, (const uint16_t *)a.q, a.k_cache, a.v_cache, a.seqlens, a.q_pos, a.B,
                     a.max_cache_len, a.Hq, a.Hkv, a.theta, scale_log2, a.chunk, a.nsplit,
                     a.part_o, a.part_lse, a.dev_flag, a.window, a.sinks, a.k_scale, a.v_scale,
                     a.vis_split);
  return hipGetLastError();
}

template <int D, bool FP8, bool WIN>
hipError_t launch_mfma(const DecodeArgs &a, hipStream_t s) {
  constexpr int EB = FP8 ? 1 : 2;
  if (a.shared_form) {
    return launch_mfma_w<D, FP8, WIN, 4, true>(a, s);
  } else {
    switch (heads_per_wg(a.Hkv, D, EB)) {
      case 8:
        if constexpr (mfma_ring_bytes(8, D, EB) <= kMfmaLdsBudget) {
          if (a.stream_wg > 0) return launch_mfma_w<D, FP8, WIN, 8, false, true>(a, s);
          return launch_mfma_w<D, FP8, WIN, 8>(a, s);
        }
        return hipErrorInvalidValue;
      case 4:
        if (a.stream_wg > 0) return launch_mfma_w<D, FP8, WIN, 4, false, true>(a, s);
        return launch_mfma_w<D, FP8, WIN, 4>(a, s);
      case 2: return launch_mfma_w<D, FP8, WIN, 2>(a, s);
      default: return launch_mfma_w<D, FP8, WIN, 1>(a, s);
    }
  }
}

template <int D, bool OUT_F32, bool PERWAVE>
hipError_t launch_merge_k(const DecodeArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)(PERWAVE ? a.B * (a.Hq / 4) : a.B * a.Hq)), block(256);
  hipLaunchKernelGGL((decode_merge_kernel<D, OUT_F32, PERWAVE>), grid, block, 0, s, a.part_o,
                     a.part_lse, a.seqlens, a.Hq, a.max_cache_len, a.chunk, a.nsplit,
                     a.vis_split, a.out, a.lse, a.B, a.Hkv, a.stream_wg, a.stream_hpw, a.q_pos,
                     a.window, a.sinks);
  return hipGetLastError();
}

// One wave per query head when a head has few partials: a balanced split
// with at least as many (sequence, head group) segments as workgroups (a
// segment then spans about two pieces), or at most 8 chunks per head.
template <int D>
hipError_t launch_merge(const DecodeArgs &a, hipStream_t s) {
  const bool few = a.stream_wg > 0
                       ? (long long)a.B * (a.Hkv / a.stream_hpw) >= a.stream_wg
                       : a.nsplit <= 8;
  const bool perwave = a.Hq % 4 == 0 && few;
  if (a.out_dtype == YR_F32)
    return perwave ? launch_merge_k<D, true, true>(a, s) : launch_merge_k<D, true, false>(a, s);
  return perwave ? launch_merge_k<D, false, true>(a, s) : launch_merge_k<D, false, false>(a, s);
}

}  // namespace

namespace {
constexpr int kMaxDevices = 64;

// Device that owns `stream` (the current device for the null stream).
hipError_t stream_device(hipStream_t stream, int *dev) {
  hipDevice_t d = 0;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &d) : hipGetDevice(&d);
  if (e != hipSuccess) return e;
  if (d < 0 || d >= kMaxDevices) return hipErrorInvalidDevice;
  *dev = (int)d;
  return hipSuccess;
}

// Fixed scratch of attn_decode_noalloc (partials of the split sweep and the
// merge).  The name is a host-side stand-in: host code uses the device
// address that hipGetSymbolAddress returns for each device, never the name.
__device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];
}  // namespace

int decode_stream_wgs(hipStream_t stream) {
  // one workgroup per CU (the head-per-wave ring takes most of a CU's LDS);
  // the CU count is read once per device (a racing first call on two threads
  // reads it twice and stores the same value)
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (stream_device(stream, &dev) != hipSuccess) return 0;
  const int c = cached[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 0;
  n = n < kDecodeStreamMaxWg ? n : kDecodeStreamMaxWg;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t decode_fixed_scratch(hipStream_t stream, void **ptr) {
  // looked up once per device, with that device current (each device holds
  // its own copy of the array at its own address)
  static std::atomic<void *> addr[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  hipError_t e = stream_device(stream, &dev);
  if (e != hipSuccess) return e;
  void *p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
      int cur = 0;
      e = hipGetDevice(&cur);
      if (e != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
      if (e != hipSuccess) return e;
      if (e2 != hipSuccess) return e2;
      if (p == nullptr) return hipErrorInvalidSymbol;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  hipError_t e;
  const bool win = a.window > 0;
  if (a.in_dtype == YR_FP8_E4M3)
    e = a.head_dim == 64 ? (win ? launch_mfma<64, true, true>(a, s) : launch_mfma<64, true, false>(a, s))
                         : (win ? launch_mfma<128, true, true>(a, s) : launch_mfma<128, true, false>(a, s));
  else if (a.in_dtype == YR_BF16)
    e = a.head_dim == 64 ? (win ? launch_mfma<64, false, true>(a, s) : launch_mfma<64, false, false>(a, s))
                         : (win ? launch_mfma<128, false, true>(a, s) : launch_mfma<128, false, false>(a, s));
  else
    e = a.head_dim == 64 ? launch_split_g<float, 64>(a, s) : launch_split_g<float, 128>(a, s);
  if (e != hipSuccess) return e;
  return a.head_dim == 64 ? launch_merge<64>(a, s) : launch_merge<128>(a, s);
}

}  // namespace yr
