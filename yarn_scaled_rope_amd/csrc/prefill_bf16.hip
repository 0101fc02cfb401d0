// bf16 causal prefill on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Method: scaled dot-product attention with the causal rule ("Arch 03 --
// Long Context", attention slide; ALiBi slide for i - j >= 0), tiled with an
// online softmax so that no score matrix is stored ("Long-context models",
// "Context parallelism distributes exact attention": running row maxima,
// sums and output accumulators; "LLM context window mechanics": tiles kept on
// chip).  Queries are rotated on load with fp64 angles; keys arrive rotated.
//
// Work decomposition (one workgroup = 8 waves = 256 query rows of one head):
//   * Every wave owns 32 consecutive query rows.  Scores are formed
//     transposed, S^T = K * Q^T, so the 32x32 accumulator of a lane holds ONE
//     query (lane % 32) against 16 keys; the row max and row sum need only
//     the lane's own registers plus one exchange with lane ^ 32.
//   * The output is also formed transposed, O^T = V^T * P^T, so the lane that
//     owns a query owns its output column and its rescale factor.
//   * P^T goes straight from the score accumulator into the B operand: the
//     8 accumulator registers 8*(ks%2)..+7 of key block ks/2 are one 16-key
//     k-step.  The V^T operand comes from transposing LDS reads
//     (ds_read_b64_tr_b16) whose key order matches that register order.
//   * K and V tiles (64 keys) are copied from HBM straight into LDS
//     (buffer_load ... lds): no staging registers, no VALU, no LDS writes.
//     Each lane fetches the source chunk that belongs in its LDS slot, which
//     realises the XOR swizzles that keep the operand reads free of bank
//     conflicts.  Loads are buffer loads whose range ends at the sequence
//     end, so rows past it read as 0.
//   * Software pipeline inside each wave: step j copies the tiles two steps
//     ahead, then issues the score MFMAs of tile j+1 and, independent of
//     them, the softmax of tile j (VALU and transcendental work), then the PV
//     MFMAs of tile j.  One barrier per step.
//   * The running max is lazy: it moves only when a row max exceeds it by
//     more than 2^8, so the O rescale is skipped on most tiles.
//   * Tiles wholly above a wave's diagonal are skipped by that wave; masking
//     runs only on tiles that cross the diagonal or the sequence end.
//   * Workgroups run longest-first (q-tile index from the last tile down) and
//     are spread over the 8 XCDs so that the query heads of one KV head land
//     on one XCD and share its L2.
#include "device_common.h"
#include "yr_internal.h"

#include <type_traits>

namespace yr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
#define YR_LDS __attribute__((address_space(3)))
#define YR_INLINE __attribute__((always_inline))

constexpr int kThreads = 512;
constexpr int kBQ = kThreads / 2;  // query rows per workgroup (32 per wave)
constexpr int kBC = 64;            // keys per tile
constexpr int KB = kBC / 32;       // 32-key blocks of a tile (score accumulators)
constexpr int KS = kBC / 16;       // 16-key k-steps of a tile (P fragments)
constexpr int kXcds = 8;
constexpr int kMaxRankedSeqs = 64;  // chunked prefill orders up to this many sequences
constexpr float kLn2 = 0.69314718055994530942f;

// V chunk swizzle by key row mod 4: for 16 lanes of a transposing read (4 key
// rows x 2 chunks) the 8 slots are distinct mod 8 (32 banks) and, with 16
// chunks per row, the 32 lanes of both 16-column halves are distinct mod 16
// (64 banks).
template <int CH>
__device__ __forceinline__ int vswz(int e) {
  return CH >= 16 ? ((2 * e) ^ (8 * (e & 1))) : 2 * e;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// s_waitcnt vmcnt(N) only (gfx9 encoding): at most N of this wave's tile
// copies into LDS are still in flight
template <int N>
__device__ __forceinline__ void wait_dma() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// EXT: keys from a cache with a prefix (chunked prefill) and / or a sliding
// window with sinks; without it those are compiled out (plain causal).
template <int D, bool OUT_F32, bool ROTATE_Q, bool EXT>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const int *__restrict__ cu, int B, int max_seqlen,
    long long T, int Hq, int Hkv, const double *__restrict__ theta, float scale_log2,
    void *__restrict__ out, float *__restrict__ lse, int ntiles, int *flag, int kv_len,
    const int *__restrict__ ctx, int window, int sinks) {
  constexpr int KSTEPS = D / 16;     // MFMA k-steps over the head dim
  constexpr int DBLK = D / 32;       // 32-row blocks of O^T
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int RPI = 64 / CH;       // rows per 1 KB tile copy instruction
  constexpr int DPW = kBC / RPI / (kThreads / 64);  // copy instructions per wave per tile
  constexpr int TILE = kBC * D;      // elements of a K or V tile

  if constexpr (!EXT) {
    kv_len = 0;
    ctx = nullptr;
    window = 0;
    sinks = 0;
  }
  // Two LDS stages of K and of V (a third measured no faster, and spills).
  // One array per stage: the compiler then tells a stage being read from the
  // copies in flight into the other stage, and adds no wait for them.
  constexpr int NS = 2;
  __shared__ __align__(16) uint16_t sk0[TILE], sk1[TILE];
  __shared__ __align__(16) uint16_t sv0[TILE], sv1[TILE];

  if (flag != nullptr && blockIdx.x == 0)
    validate_cu_seqlens(cu, B, T, max_seqlen, flag, kv_len > 0 ? ctx : nullptr, kv_len);

  // ---- block -> (q-tile, sequence, head): longest first, XCD-grouped heads
  // Packed prefill: q-tiles from the last (the work of a tile grows with its
  // index), every sequence and head at each tile index.  Chunked prefill:
  // a tile's work is dominated by its sequence's cached prefix, so the
  // sequences go longest first (by prefix + chunk keys), each with all its
  // q-tiles and heads; consecutive blocks spread a tile's heads over the XCDs
  // so that the heads of one KV head share an L2.
  int tile, b, h;
  if (kv_len > 0 && B <= kMaxRankedSeqs) {
    __shared__ int ranked_b;
    const int per = ntiles * Hq;
    const int rank = (int)(blockIdx.x / per);
    const int rem = (int)(blockIdx.x % per);
    tile = ntiles - 1 - rem / Hq;
    int hr = rem % Hq;
    if (Hq % kXcds == 0) hr = (hr % kXcds) * (Hq / kXcds) + hr / kXcds;
    h = hr;
    if (threadIdx.x == 0) ranked_b = B;  // rank past the last sequence: no work
    __syncthreads();
    for (int i = threadIdx.x; i < B; i += blockDim.x) {
      auto keys = [&](int j) {
        const int c = ctx != nullptr ? ctx[j] : 0;
        return (long long)(c < 0 ? 0 : c) + (cu[j + 1] - cu[j]);
      };
      const long long ki = keys(i);
      int rk = 0;
      for (int j = 0; j < B; ++j) {
        const long long kj = keys(j);
        rk += (kj > ki) || (kj == ki && j < i);
      }
      if (rk == rank) ranked_b = i;
    }
    __syncthreads();
    b = ranked_b;
    if (b >= B) return;
  } else {
    const int per = B * Hq;
    tile = ntiles - 1 - (int)(blockIdx.x / per);
    int r = (int)(blockIdx.x % per);
    if (per % kXcds == 0) r = (r % kXcds) * (per / kXcds) + r / kXcds;
    b = r / Hq;
    h = r % Hq;
  }
  const int hk = h / (Hq / Hkv);
  long long s0;
  int n;
  seq_bounds(cu, b, T, max_seqlen, &s0, &n);
  // uniform across the workgroup: keep them in scalar registers so the
  // per-tile buffer descriptors need no per-lane fix-up
  n = __builtin_amdgcn_readfirstlane(n);
  s0 = ((long long)__builtin_amdgcn_readfirstlane((int)(s0 >> 32)) << 32) |
       (unsigned)__builtin_amdgcn_readfirstlane((int)(s0 & 0xffffffff));
  const int q0 = tile * kBQ;
  if (q0 >= n) return;
  const int qend = min(n, q0 + kBQ);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int tw0 = q0 + wave * 32;  // first query row of this wave
  const int tq = tw0 + l32;        // this lane's query row

  // Keys: packed like q (kv_len == 0), or a [B, kv_len, Hkv, D] cache whose
  // first P rows precede this chunk: query row i then sits at position P + i
  // and sees cache rows up to P + i.  Positions below are cache rows.
  const long long rstride = (long long)Hkv * D;  // elements between key rows
  int P = 0;
  long long krow0 = s0;
  if (kv_len > 0) {
    P = ctx != nullptr ? ctx[b] : 0;
    P = P < 0 ? 0 : (P > kv_len - n ? kv_len - n : P);
    P = __builtin_amdgcn_readfirstlane(P);
    krow0 = (long long)b * kv_len;
  }
  const int nk = P + n;  // key rows of the sequence

  // ---- tile copies HBM -> LDS (buffer_load ... lds, no registers) ---------
  // Copy instruction p of a tile fills LDS bytes [1024p, 1024p + 1024) in lane
  // order: lane l lands on row p*RPI + l/CH, slot l%CH, so it fetches the
  // source chunk that belongs in that slot.  K: slot = chunk ^ (row % CH);
  // V: slot = chunk ^ vswz(row % 4).  Rows past the sequence end read 0.
  const uint16_t *kseq = k + (krow0 * Hkv + hk) * (long long)D;
  const uint16_t *vseq = v + (krow0 * Hkv + hk) * (long long)D;
  const uint32_t rbytes = (uint32_t)(rstride * 2);
  const int drow = lane / CH, dslot = lane % CH;
  uint32_t koff[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int row = (wave * DPW + i) * RPI + drow;
    koff[i] = drow * rbytes + 16 * (dslot ^ (row & (CH - 1)));
  }
  const uint32_t voff = drow * rbytes + 16 * (dslot ^ vswz<CH>(drow & 3));
  auto copy_tile = [&](uint16_t *dst, const uint16_t *seq, int t, bool is_v) YR_INLINE {
    const int key0 = t * kBC;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(seq + key0 * rstride, (uint32_t)min(kBC, nk - key0) * rbytes);
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int p = wave * DPW + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (YR_LDS void *)(dst + p * 512), 16,
                                               (int)(is_v ? voff : koff[i]),
                                               (int)(p * RPI * rbytes), 0, 0);
    }
  };
  // tile t lives in stage t % NS; `par` below is that stage index
  auto kst = [&](auto par) YR_INLINE -> uint16_t * {
    constexpr int P = decltype(par)::value;
    if constexpr (P == 0) return sk0; else return sk1;
  };
  auto vst = [&](auto par) YR_INLINE -> uint16_t * {
    constexpr int P = decltype(par)::value;
    if constexpr (P == 0) return sv0; else return sv1;
  };
  // Key tiles the workgroup visits, as a list: the sink tiles [0, js), then
  // the tiles [jw, last] from the window start of its first row to the
  // diagonal of its last row (without a window: every tile 0..last).
  const int last = (P + qend - 1) / kBC;
  int js = 0, jw = 0;
  if (window > 0) {
    const int lo = max(0, P + q0 - window + 1);
    jw = lo / kBC;
    js = min((min(sinks, lo) + kBC - 1) / kBC, jw);
  }
  const int count = js + (last - jw + 1);
  auto tile_of = [&](int i) YR_INLINE { return i < js ? i : jw + (i - js); };
  // prologue copies (K of tiles 0..NS-1, V of tiles 0..NS-2 of the list) go
  // out before the query work so that they are in flight meanwhile
  static_for<0, NS>([&](auto ic) YR_INLINE {
    constexpr int I = decltype(ic)::value;
    if (I < count) copy_tile(kst(ic), kseq, tile_of(I), false);
    if (I + 1 < NS && I < count) copy_tile(vst(ic), vseq, tile_of(I), true);
  });

  // ---- Q fragments (B operand of S^T = K Q^T), rotated on load -----------
  bf16x8 qf[KSTEPS];
  {
    const bool qvalid = tq < n;
    const uint16_t *qp = q + ((s0 + (qvalid ? tq : 0)) * Hq + h) * (long long)D + hh * 8;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qvalid) {
        w = *reinterpret_cast<const u32x4 *>(qp + kk * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // the logit scale (log2 units) folded into the query before its one
          // rounding to bf16, so that the scores come out of the matrix cores
          // ready for exp2
          float x0 = bf16_to_f32(w[e] & 0xffffu), x1 = bf16_to_f32(w[e] >> 16);
          if (ROTATE_Q) {
            float c, s;
            rope_cos_sin((double)(P + tq), theta[kk * 8 + hh * 4 + e], &c, &s);
            rotate_pair(x0, x1, c, s);
          }
          w[e] = pack_bf16x2(x0 * scale_log2, x1 * scale_log2);
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
  // -m_run (0 while m_run = -inf) in every slot: the accumulator the score
  // MFMAs start from, so that they return s * scale - m directly
  f32x16 negm = f32x16{};

  // LDS operand addresses (elements).  K: row kb*32 + l32, chunk 2kk + hh.
  // V^T (transposing reads): lane t of a 16-lane group reads 4 elements of key
  // row 4*hh + (t >> 2) (+32 kb + 16 ks' + 8 r) at columns 32*db + 16*group
  // parity + 4*(t & 3), and receives column t of 4 consecutive key rows.
  const int kx = l32 & (CH - 1);
  int vbase[DBLK];
  {
    const int t16 = lane & 15;
    const int vrow = 4 * hh + (t16 >> 2);
    const int vx = vswz<CH>(t16 >> 2);
    const int vcol = 2 * ((lane >> 4) & 1) + ((t16 & 3) >> 1);
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
      vbase[db] = vrow * D + 8 * ((4 * db + vcol) ^ vx) + 4 * (t16 & 1);
  }

  // ---- per-tile work -------------------------------------------------------
  // Tile j has keys j*64 .. j*64+63.  The wave (rows tw0 .. tw0+31, positions
  // P + row) skips it when it lies wholly above the wave's diagonal, or, with
  // a window, wholly below the window of the wave's first row and past the
  // sinks.
  auto active = [&](int j) YR_INLINE {
    if (tw0 >= n || j * kBC > P + tw0 + 31) return false;
    return window == 0 || j * kBC + kBC - 1 > P + tw0 - window || j * kBC < sinks;
  };

  // S^T = K Q^T for one tile (two 32-key blocks); accumulator slot rr of block
  // kb (lane half hh) holds key 32 kb + 8 (rr >> 2) + 4 hh + (rr & 3)
  auto scores = [&](auto par, f32x16 (&s)[KB]) YR_INLINE {
    const uint16_t *ks = kst(par);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const bf16x8 a = as_bf16x8(
            *reinterpret_cast<const u32x4 *>(ks + (kb * 32 + l32) * D + 8 * ((2 * kk + hh) ^ kx)));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], kk == 0 ? negm : s[kb], 0, 0, 0);
      }
    }
  };

  // softmax front half of tile j: mask (diagonal/tail tiles only), row max,
  // lazy rescale of the running state; returns -m for the exp2 argument
  // nx: the scores of the next tile, already issued against the old -m_run,
  // which move to the new reference with this tile's
  auto softmax_front = [&](int j, f32x16 (&s)[KB], f32x16 (&nx)[KB], bool may_mask) YR_INLINE -> float {
    const int key0 = j * kBC;
    const bool wmask = window > 0 && key0 <= P + tw0 + 31 - window && key0 + kBC > sinks;
    if (may_mask && ((key0 + kBC - 1 > P + tw0) || (key0 + kBC > nk) || wmask)) {
      const int pos = P + tq;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = key0 + kb * 32 + (rr >> 2) * 8 + hh * 4 + (rr & 3);
          const bool hide = key > pos || key >= nk ||
                            (window > 0 && key <= pos - window && key >= sinks);
          if (hide) s[kb][rr] = -INFINITY;
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[kb][rr]);
    }
    // the tile's row max less m_run (the scores carry -m_run already)
    mx = half_max(mx);
    const bool first = m_run == -INFINITY;
    const bool grow = first ? mx > -INFINITY : mx > 8.0f;  // lazy running max
    if (__any(grow)) {
      const float m_new = grow ? (first ? mx : m_run + mx) : m_run;
      // 0 when m_run = -inf; 1 for a row that has seen no visible key yet
      // (with a window a row can meet tiles it does not see at all)
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      // move this tile's scores to the new reference
      const float shift = (first ? 0.f : m_run) - (m_new == -INFINITY ? 0.f : m_new);
      m_run = m_new;
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < DBLK; ++i) o[i] *= alpha;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          s[kb][rr] += shift;
          nx[kb][rr] += shift;
        }
      const float nm = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) negm[rr] = nm;
    }
    return 0.f;
  };

  // softmax back half: P = exp2(s*scale - m) in bf16, row sum.  The 8
  // accumulator slots 8 (ks & 1) .. +7 of block ks >> 1 form k-step ks.
  auto softmax_back = [&](f32x16 (&s)[KB], float neg_m, bf16x8 (&pf)[KS]) YR_INLINE {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(s[ks >> 1][(ks & 1) * 8 + 2 * e]);
        const float p1 = __builtin_amdgcn_exp2f(s[ks >> 1][(ks & 1) * 8 + 2 * e + 1]);
        l_part += p0 + p1;
        w[e] = pack_bf16x2(p0, p1);
      }
      pf[ks] = as_bf16x8(w);
    }
  };

  // O^T += V^T P^T (k-step major: the MFMAs of k-step ks need only pf[ks]).
  // Element e of the operands is key 16 ks + 4 hh + 8 (e >> 2) + (e & 3), the
  // order in which the score accumulator holds P.
  auto pv = [&](auto par, bf16x8 (&pf)[KS]) YR_INLINE {
    const uint16_t *vs = vst(par);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const uint16_t *ap = vs + vbase[db] + 16 * ks * D;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YR_LDS i16x4 *)(ap));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YR_LDS i16x4 *)(ap + 8 * D));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 w = {l2[0], l2[1], h2[0], h2[1]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(w), pf[ks], o[db], 0, 0, 0);
      }
    }
  };

  // One pipeline step i over the tile list (stage par = i % 2; tile(i) is
  // the list's i-th tile): after the barrier the K stage of tile(i) (read by
  // the scores of step i-1) and the V stage of tile(i-1) are free; copy
  // K(tile(i+2)) and V(tile(i+1)) into them, then run the score MFMAs of
  // tile(i+1) alongside the softmax of tile(i), then the PV MFMAs of tile(i).
  // Before the barrier each wave waits for its own copies of K(tile(i+1)) and
  // V(tile(i)), issued by the previous step.
  auto nextp = [](auto par) YR_INLINE { return std::integral_constant<int, (decltype(par)::value + 1) % NS>{}; };
  auto prevp = [](auto par) YR_INLINE { return std::integral_constant<int, (decltype(par)::value + NS - 1) % NS>{}; };
  auto stage = [&](auto par, int i) YR_INLINE {
    wait_dma<0>();
    __syncthreads();
    if (i + NS < count) copy_tile(kst(par), kseq, tile_of(i + NS), false);
    if (i + NS - 1 < count) copy_tile(vst(prevp(par)), vseq, tile_of(i + NS - 1), true);
  };
  // General step (diagonal, window-edge and tail tiles, the last step): every
  // check.
  auto step = [&](auto par, int i, f32x16 (&cur)[KB], f32x16 (&nxt)[KB]) YR_INLINE {
    stage(par, i);
    if (i + 1 < count && active(tile_of(i + 1))) scores(nextp(par), nxt);
    if (active(tile_of(i))) {
      const float neg_m = softmax_front(tile_of(i), cur, nxt, true);
      bf16x8 pf[KS];
      softmax_back(cur, neg_m, pf);
      pv(par, pf);
    }
  };
  // Clear step: tiles i and i+1 of the list need no mask for any row (below
  // the diagonal of the workgroup's first row, inside the window of its last
  // row) and every wave works on both, so the score MFMAs of tile i+1 go out
  // first, right after the barrier, and the row max, exp / convert work of
  // tile i and its PV MFMAs follow (measured 1-1.5% faster than issuing the
  // scores after the row max).
  auto step_clear = [&](auto par, int i, f32x16 (&cur)[KB], f32x16 (&nxt)[KB]) YR_INLINE {
    stage(par, i);
    scores(nextp(par), nxt);
    const float neg_m = softmax_front(tile_of(i), cur, nxt, false);
    bf16x8 pf[KS];
    softmax_back(cur, neg_m, pf);
    pv(par, pf);
  };

  // prologue: every prologue copy landed; S(tile(0))
  wait_dma<0>();
  __syncthreads();
  f32x16 sa[KB], sb[KB];
  if (active(tile_of(0))) scores(std::integral_constant<int, 0>{}, sa);
  // Steps are unrolled over the stage index (i % NS) and the score buffer
  // (i % 2), so every LDS array and register array is picked at compile time.
  constexpr int BL = 2;
  auto sbuf = [&](auto ic) YR_INLINE -> f32x16(&)[KB] {
    if constexpr (decltype(ic)::value % 2 == 0) return sa; else return sb;
  };
  auto obuf = [&](auto ic) YR_INLINE -> f32x16(&)[KB] {
    if constexpr (decltype(ic)::value % 2 == 0) return sb; else return sa;
  };
  // The tiles that need no mask for any row form one run of the list: from
  // the first tile at or past the window start of the workgroup's last row to
  // the last tile below the diagonal of its first row (list positions
  // [c0, c1)).  Steps before it and after it take the general body; a clear
  // step i needs tiles i and i+1 in the run.  Separate loops keep each body's
  // registers to itself.
  int c0 = count, c1 = count;
  {
    const int jd = (P + q0 + 1) / kBC - 1;  // last tile wholly below the first row's diagonal
    const int jc = window > 0 ? max(jw, (P + qend - window + kBC - 1) / kBC) : 0;
    if (jd >= jc) {
      c0 = js + (jc - jw);
      c1 = js + (jd - jw) + 1;
    }
  }
  auto general_block = [&](int i) YR_INLINE {
    static_for<0, BL>([&](auto ic) YR_INLINE {
      constexpr int I = decltype(ic)::value;
      if (i + I < count) step(std::integral_constant<int, I % NS>{}, i + I, sbuf(ic), obuf(ic));
    });
  };
  int i = 0;
  for (; i < c0; i += BL) general_block(i);
  // the unmasked run in blocks of 4 steps (two stage / buffer cycles; +0.5-1%
  // over blocks of 2), its remainder in blocks of 2
  constexpr int BLC = 4;
  for (; i + BLC < c1; i += BLC) {
    static_for<0, BLC>([&](auto ic) YR_INLINE {
      constexpr int I = decltype(ic)::value;
      step_clear(std::integral_constant<int, I % NS>{}, i + I, sbuf(ic), obuf(ic));
    });
  }
  for (; i + BL < c1; i += BL) {
    static_for<0, BL>([&](auto ic) YR_INLINE {
      constexpr int I = decltype(ic)::value;
      step_clear(std::integral_constant<int, I % NS>{}, i + I, sbuf(ic), obuf(ic));
    });
  }
  for (; i < count; i += BL) general_block(i);

  // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l) ---------------------
  const float l_tot = half_sum(l_part);
  if (tq >= n) return;
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

template <int D, bool OUT_F32, bool ROT, bool EXT>
hipError_t launch_one(const PrefillArgs &a, hipStream_t s) {
  const int ntiles = (a.max_seqlen + kBQ - 1) / kBQ;
  const long long blocks = (long long)ntiles * a.B * a.Hq;
  const float scale_log2 = (float)((double)a.softmax_scale * 1.4426950408889634074);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, OUT_F32, ROT, EXT>), dim3((unsigned)blocks), dim3(kThreads),
                     0, s, (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                     a.cu_seqlens, a.B, a.max_seqlen, a.T, a.Hq, a.Hkv, a.theta, scale_log2, a.out,
                     a.lse, ntiles, a.dev_flag, a.kv_cache_len, a.ctx_lens, a.window, a.sinks);
  return hipGetLastError();
}

template <int D, bool EXT>
hipError_t launch_d(const PrefillArgs &a, hipStream_t s) {
  const bool f32 = a.out_dtype == YR_F32;
  const bool rot = a.theta != nullptr;
  if (f32) return rot ? launch_one<D, true, true, EXT>(a, s) : launch_one<D, true, false, EXT>(a, s);
  return rot ? launch_one<D, false, true, EXT>(a, s) : launch_one<D, false, false, EXT>(a, s);
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs &a, hipStream_t s) {
  if (a.kv_cache_len > 0 || a.window > 0)
    return a.head_dim == 64 ? launch_d<64, true>(a, s) : launch_d<128, true>(a, s);
  return a.head_dim == 64 ? launch_d<64, false>(a, s) : launch_d<128, false>(a, s);
}

}  // namespace yr
