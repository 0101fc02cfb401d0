// bf16 causal prefill on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Method: scaled dot-product attention with the causal rule ("Arch 03 --
// Long Context", attention slide; ALiBi slide for i - j >= 0), tiled with an
// online softmax so that no score matrix is stored ("Long-context models",
// "Context parallelism distributes exact attention": running row maxima,
// sums and output accumulators; "LLM context window mechanics": tiles kept on
// chip).  Queries are rotated on load with fp64 angles; keys arrive rotated.
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one head):
//   * Every wave owns 32 consecutive query rows.  Scores are formed
//     transposed, S^T = K * Q^T, so the 32x32 accumulator of a lane holds ONE
//     query (lane % 32) against 16 keys; the row max and row sum need only the
//     lane's own registers plus one exchange with lane ^ 32.
//   * The output is also formed transposed, O^T = V^T * P^T, so the lane that
//     owns a query owns its output column and its rescale factor: the online
//     rescale is a per-lane multiply.
//   * P^T is fed straight from the score accumulator into the B operand: the
//     8 consecutive accumulator registers 8*(ks%2)..+7 of key block ks/2 are
//     exactly one 16-key k-step, with the key order permuted identically in
//     the V^T operand.
//   * K tiles are staged row-major in LDS, V tiles transposed (V^T[d][key]),
//     both double-buffered: one barrier per 64-key tile, and the global loads
//     of tile j+1 are in flight while tile j is computed.
//   * Tiles wholly above a wave's diagonal are skipped by that wave; masking
//     runs only on tiles that cross the diagonal or the sequence end.
//   * Workgroups are issued longest-first: the q-tile index runs from the last
//     tile down, and consecutive workgroups are consecutive heads, so heads
//     that share a KV head run together and share its tiles in L2.
#include "device_common.h"
#include "yr_internal.h"

namespace yr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kBQ = 128;   // query rows per workgroup
constexpr int kBC = 64;    // keys per tile
constexpr int kKPad = 8;   // bf16 elements of padding per K row  (row = 68 dwords)
constexpr int kVPad = 4;   // bf16 elements of padding per V^T row (row = 34 dwords)
constexpr float kLn2 = 0.69314718055994530942f;

template <int D>
struct Smem {
  uint16_t k[2][kBC][D + kKPad];
  uint16_t vt[2][D][kBC + kVPad];
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ uint32_t sel16(uint32_t w, int hi) { return hi ? (w >> 16) : (w & 0xffffu); }

template <int D, bool OUT_F32, bool ROTATE_Q>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const int *__restrict__ cu, int B, int max_seqlen,
    long long T, int Hq, int Hkv, const double *__restrict__ theta, float scale_log2,
    void *__restrict__ out, float *__restrict__ lse, int ntiles, int *flag) {
  constexpr int KSTEPS = D / 16;        // MFMA k-steps over the head dim
  constexpr int DBLK = D / 32;          // 32-row blocks of O^T
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int KROWS = kThreads / CH;  // K rows per load pass
  constexpr int KPASS = kBC / KROWS;
  constexpr int VUNITS = CH * (kBC / 4);  // (chunk, 4-key group) units of a V tile
  static_assert(VUNITS <= kThreads, "V tile mapping");

  __shared__ __align__(16) Smem<D> sm;

  if (flag != nullptr && blockIdx.x == 0) validate_cu_seqlens(cu, B, T, max_seqlen, flag);

  const long long per = (long long)B * Hq;
  const int tile = ntiles - 1 - (int)(blockIdx.x / per);
  const int rem = (int)(blockIdx.x % per);
  const int b = rem / Hq;
  const int h = rem % Hq;
  const int hk = h / (Hq / Hkv);
  long long s0;
  int n;
  seq_bounds(cu, b, T, max_seqlen, &s0, &n);
  const int q0 = tile * kBQ;
  if (q0 >= n) return;
  const int qend = min(n, q0 + kBQ);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int tw0 = q0 + wave * 32;  // first query row of this wave
  const int tq = tw0 + l32;        // this lane's query row
  const bool qvalid = tq < n;

  // ---- Q fragment (B operand of S^T = K Q^T), rotated on load ------------
  bf16x8 qf[KSTEPS];
  {
    const uint16_t *qp = q + ((s0 + (qvalid ? tq : 0)) * Hq + h) * (long long)D + hh * 8;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qvalid) {
        w = *reinterpret_cast<const u32x4 *>(qp + kk * 16);
        if (ROTATE_Q) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x0 = bf16_to_f32(w[e] & 0xffffu), x1 = bf16_to_f32(w[e] >> 16);
            float c, s;
            rope_cos_sin((double)tq, theta[kk * 8 + hh * 4 + e], &c, &s);
            rotate_pair(x0, x1, c, s);
            w[e] = pack_bf16x2(x0, x1);
          }
        }
      }
      qf[kk] = as_bf16x8(w);
    }
  }

  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) o[i] = f32x16{};
  float m_run = -INFINITY;
  float l_part = 0.f;

  // ---- staging maps ------------------------------------------------------
  const int krow0 = tid / CH, kch = tid % CH;       // K: row krow0 + KROWS*p, chunk kch
  const int vch = tid % CH, vkey = (tid / CH) * 4;  // V: chunk vch, keys vkey..vkey+3
  const bool vact = tid < VUNITS;
  const uint16_t *kbase_ptr = k + (s0 * Hkv + hk) * (long long)D;
  const uint16_t *vbase_ptr = v + (s0 * Hkv + hk) * (long long)D;
  const long long rstride = (long long)Hkv * D;

  u32x4 kreg[KPASS];
  u32x4 vreg[4];
  auto gload = [&](int j) {
    const int key0 = j * kBC;
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      const int key = key0 + krow0 + p * KROWS;
      kreg[p] = key < n ? *reinterpret_cast<const u32x4 *>(kbase_ptr + key * rstride + kch * 8)
                        : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + vkey + r;
      vreg[r] = (vact && key < n)
                    ? *reinterpret_cast<const u32x4 *>(vbase_ptr + key * rstride + vch * 8)
                    : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int p = 0; p < KPASS; ++p)
      *reinterpret_cast<u32x4 *>(&sm.k[buf][krow0 + p * KROWS][kch * 8]) = kreg[p];
    if (vact) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wsel = e >> 1, hi = e & 1;
        u32x2 pk;
        pk[0] = sel16(vreg[0][wsel], hi) | (sel16(vreg[1][wsel], hi) << 16);
        pk[1] = sel16(vreg[2][wsel], hi) | (sel16(vreg[3][wsel], hi) << 16);
        *reinterpret_cast<u32x2 *>(&sm.vt[buf][vch * 8 + e][vkey]) = pk;
      }
    }
  };

  const int last_tile = (qend - 1) / kBC;
  gload(0);
  for (int j = 0; j <= last_tile; ++j) {
    const int buf = j & 1;
    swrite(buf);
    __syncthreads();
    if (j < last_tile) gload(j + 1);

    const int key0 = j * kBC;
    if (key0 > tw0 + 31 || tw0 >= n) continue;  // tile wholly above this wave's diagonal

    // ---- S^T = K Q^T : two 32-key blocks --------------------------------
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x16{};
      const uint16_t *kr = &sm.k[buf][kb * 32 + l32][hh * 8];
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4 *>(kr + kk * 16));
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sc[kb], 0, 0, 0);
      }
    }

    // ---- mask, row max (on raw scores: the scale is positive) ----------
    const bool need_mask = (key0 + kBC - 1 > tw0) || (key0 + kBC > n);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
          if (key > tq || key >= n) sc[kb][r] = -INFINITY;
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;

    // ---- lazy rescale: the reference max moves only when the row max
    // exceeds it by more than 2^8, so exp2 stays <= 256 and the O rescale
    // (64 multiplies) is skipped on most tiles; softmax does not depend on
    // the reference, so the result is unchanged up to rounding.
    const bool grow = mx > m_run + 8.0f;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
      m_run = m_new;
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < DBLK; ++i) o[i] *= alpha;
    }
    const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;

    // ---- P^T in bf16, 4 k-steps of 16 keys ------------------------------
    bf16x8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[ks >> 1][(ks & 1) * 8 + 2 * e], scale_log2, neg_m));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[ks >> 1][(ks & 1) * 8 + 2 * e + 1], scale_log2, neg_m));
        l_part += p0 + p1;
        w[e] = pack_bf16x2(p0, p1);
      }
      pf[ks] = as_bf16x8(w);
    }

    // ---- O^T += V^T P^T ---------------------------------------------------
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const uint16_t *vr = &sm.vt[buf][db * 32 + l32][hh * 4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x2 lo = *reinterpret_cast<const u32x2 *>(vr + ks * 16);
        const u32x2 hi = *reinterpret_cast<const u32x2 *>(vr + ks * 16 + 8);
        const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(w), pf[ks], o[db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l) -------------------
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  if (!qvalid) return;
  const float inv = 1.f / l_tot;
  const long long orow = ((s0 + tq) * Hq + h) * (long long)D;
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d0 = db * 32 + jj * 8 + hh * 4;
      const float y0 = o[db][jj * 4 + 0] * inv, y1 = o[db][jj * 4 + 1] * inv;
      const float y2 = o[db][jj * 4 + 2] * inv, y3 = o[db][jj * 4 + 3] * inv;
      if (OUT_F32) {
        *reinterpret_cast<float4 *>((float *)out + orow + d0) = make_float4(y0, y1, y2, y3);
      } else {
        u32x2 pk;
        pk[0] = pack_bf16x2(y0, y1);
        pk[1] = pack_bf16x2(y2, y3);
        *reinterpret_cast<u32x2 *>((uint16_t *)out + orow + d0) = pk;
      }
    }
  }
  if (lse != nullptr && hh == 0) lse[(long long)h * T + s0 + tq] = (m_run + __log2f(l_tot)) * kLn2;
}

template <int D, bool OUT_F32, bool ROT>
hipError_t launch_one(const PrefillArgs &a, hipStream_t s) {
  const int ntiles = (a.max_seqlen + kBQ - 1) / kBQ;
  const long long blocks = (long long)ntiles * a.B * a.Hq;
  const float scale_log2 = (float)((double)a.softmax_scale * 1.4426950408889634074);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, OUT_F32, ROT>), dim3((unsigned)blocks),
                     dim3(kThreads), 0, s, (const uint16_t *)a.q, (const uint16_t *)a.k,
                     (const uint16_t *)a.v, a.cu_seqlens, a.B, a.max_seqlen, a.T, a.Hq, a.Hkv,
                     a.theta, scale_log2, a.out, a.lse, ntiles, a.dev_flag);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs &a, hipStream_t s) {
  const bool f32 = a.out_dtype == YR_F32;
  const bool rot = a.theta != nullptr;
  if (f32) return rot ? launch_one<D, true, true>(a, s) : launch_one<D, true, false>(a, s);
  return rot ? launch_one<D, false, true>(a, s) : launch_one<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs &a, hipStream_t s) {
  return a.head_dim == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace yr
