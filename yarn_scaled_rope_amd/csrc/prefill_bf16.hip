// bf16 causal prefill on gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Method: scaled dot-product attention with the causal rule ("Arch 03 --
// Long Context", attention slide; ALiBi slide for i - j >= 0), tiled with an
// online softmax so that no score matrix is stored ("Long-context models",
// "Context parallelism distributes exact attention": running row maxima,
// sums and output accumulators; "LLM context window mechanics": tiles kept on
// chip).  Queries are rotated on load with fp64 angles; keys arrive rotated.
//
// Work decomposition (one workgroup = 8 waves = 256 query rows of one head):
//   * Every wave owns 32 consecutive query rows, as two 16-row blocks.
//     Scores are formed transposed, S^T = K * Q^T, in 16x16 blocks: lane l
//     holds rows l % 16 of both row blocks against 4 keys of each 16-key
//     block, so a row's keys lie in the four lanes l % 16 + 16 g, which
//     exchange values only for the row max of the slow path and the row sum
//     at the end.  Each K fragment feeds the MFMAs of both row blocks.
//   * The output is also formed transposed, O^T = V^T * P^T, so the lanes
//     that own a row own its output columns and its rescale factor.
//   * P^T goes straight from the score accumulators into the B operand: the
//     4 + 4 accumulator values of key blocks 2p and 2p+1 are one 32-key
//     k-step (k-position 8 g + e stands for key 16 (2p + e/4) + 4 g + e%4).
//     The V^T operand comes from two transposing LDS reads
//     (ds_read_b64_tr_b16) per k-step whose key order matches.
//   * The 16x16x32 shape rather than 32x32x16: with random operands the part
//     runs this kernel at its power limit, and the smaller shape moves fewer
//     accumulator bits per FLOP (a probe of back-to-back MFMAs with N(0,1)
//     bf16 operands: 2.09 against 1.85 PFLOP/s).
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
//   * The running max is lazy: every exponent stays at most 2^8 against it,
//     so the O rescale is skipped on most tiles.  Every tile is exponentiated
//     against the current reference straight away; a lane's tile sum bounds
//     each of its P, so only a sum above 2^8 (rare) or a row without a
//     reference yet sends the wave through the row max and a second pass.
//   * Tiles wholly above a wave's diagonal (or before its window) are
//     skipped by that wave; masking runs only on tiles that cross the
//     diagonal, a window edge, the sinks or the sequence end.
//   * Workgroups run longest-first (q-tile index from the last tile down) and
//     are spread over the 8 XCDs so that the query heads of one KV head land
//     on one XCD and share its L2; with a window, each sweeps its window
//     rotated so that neighbouring q-tiles read the same tile together.
//     Large launches hand out the last third of their items through per-XCD
//     work queues, so that XCDs at a higher clock take up the tail of the
//     slower ones.
#include "device_common.h"
#include "yr_internal.h"

#include <type_traits>

namespace yr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
#define YR_LDS __attribute__((address_space(3)))
#define YR_INLINE __attribute__((always_inline))

constexpr int kThreads = 512;
constexpr int kBQ = kThreads / 2;  // query rows per workgroup (32 per wave)
constexpr int kBC = 64;            // keys per tile
constexpr int NKB = kBC / 16;      // 16-key blocks of a tile (score accumulators)
constexpr int NPS = kBC / 32;      // 32-key k-steps of the PV product
constexpr int RB = 2;              // 16-row blocks of a wave's 32 query rows
constexpr int kXcds = 8;
constexpr int kMaxRankedSeqs = 64;  // chunked prefill orders up to this many sequences
constexpr float kLn2 = 0.69314718055994530942f;

// V chunk swizzle by key row mod 8.  Half a wave of transposing reads takes
// 8 consecutive key rows x the 2 chunks of 16 head dims; slot = chunk ^ vswz
// puts those 16 (row, chunk) pairs on 16 distinct 4-bank groups of the 64
// banks: with 16 chunks per row (256 bytes) vswz = 2 (row % 8), with 8 chunks
// (two 128-byte rows per bank line) vswz = row % 8 rounded down to even, for
// the 4 rows of each parity.
template <int CH>
__device__ __forceinline__ int vswz(int r8) {
  return CH >= 16 ? 2 * r8 : (r8 & 6);
}

// The four lanes l16 + 16 g4 (one query row) combined: each gets their max /
// sum.
__device__ __forceinline__ float quarter_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float quarter_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
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

// Work item `item` of a packed ragged batch: (q-tile, sequence, query head).
// In causal prefill the work of q-tile t grows with t in every sequence, so
// the items run longest first: tile index from the top down, and at each
// index every sequence that has a tile there and every query head.  Only
// existing tiles are numbered (a short sequence leaves no idle workgroups
// behind when a long one still has tiles), and the items of one tile index
// are spread over the 8 XCDs (consecutive workgroups go to consecutive XCDs)
// as runs of consecutive heads, so that the query heads of a KV head share
// one L2.  Every wave of the workgroup computes the same answer: a binary
// search over the tile index on S(t) = sum_b max(0, tiles_b - t), the number
// of q-tiles at index t or above, with the sequences spread over the lanes.
// Up to 256 sequences, each lane reads the bounds of its sequences once and
// the search runs on registers (reading cu_seqlens again for every probe put
// a chain of dependent loads in front of every workgroup's first tile).
// Returns false for workgroups past the last item; else the item and the
// bounds of its sequence (as seq_bounds gives them).
__device__ __forceinline__ bool packed_item(const int *__restrict__ cu, int B, long long T,
                                            int max_seqlen, int Hq, int ntiles, int item,
                                            int *tile, int *bo, int *ho, long long *so,
                                            int *no) {
  constexpr int NC = 4;  // sequences per lane held in registers
  const int lane = threadIdx.x & 63;
  auto tiles_of_n = [](int n) { return (n + kBQ - 1) / kBQ; };
  // Up to kScalarSeqs sequences the whole search is uniform: every value is
  // read with a uniform address into scalar registers, and the probes need
  // no cross-lane reduction (a probe's chain of six dependent lane shuffles
  // was most of the search time).
  constexpr int kScalarSeqs = 16;
  if (B <= kScalarSeqs) {
    int tn[kScalarSeqs];
#pragma unroll
    for (int bb = 0; bb < kScalarSeqs; ++bb) {
      tn[bb] = 0;
      if (bb < B) {
        long long s0b;
        int nb;
        seq_bounds(cu, bb, T, max_seqlen, &s0b, &nb);
        tn[bb] = __builtin_amdgcn_readfirstlane(tiles_of_n(nb));
      }
    }
    auto count_u = [&](int t) {
      int acc = 0;
#pragma unroll
      for (int bb = 0; bb < kScalarSeqs; ++bb) acc += max(0, tn[bb] - t);
      return acc;
    };
    if ((long long)Hq * count_u(0) <= item) return false;
    int lo = 0, hi = ntiles - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((long long)Hq * count_u(mid) > item) lo = mid; else hi = mid - 1;
    }
    const int above = count_u(lo + 1);
    const int cnt = count_u(lo) - above;
    const long long first = (long long)Hq * above;
    const int nt = cnt * Hq;
    int j = (int)(item - first);
    if (first % kXcds == 0 && nt % kXcds == 0) j = (j % kXcds) * (nt / kXcds) + j / kXcds;
    int k = j / Hq;
    *ho = j % Hq;
    *tile = lo;
    int bsel = 0;
#pragma unroll
    for (int bb = 0; bb < kScalarSeqs; ++bb) {
      if (tn[bb] > lo) {
        if (k == 0) bsel = bb;
        --k;
      }
    }
    *bo = bsel;
    seq_bounds(cu, bsel, T, max_seqlen, so, no);
    return true;
  }
  auto tiles_of = [&](int bb) {
    long long s0;
    int n;
    seq_bounds(cu, bb, T, max_seqlen, &s0, &n);
    return tiles_of_n(n);
  };
  const bool cached = B <= 64 * NC;
  long long cs[NC];
  int cn[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    cs[c] = 0;
    cn[c] = 0;
    const int bb = lane + 64 * c;
    if (cached && bb < B) seq_bounds(cu, bb, T, max_seqlen, &cs[c], &cn[c]);
  }
  auto count_from = [&](int t) {
    int acc = 0;
    if (cached) {
#pragma unroll
      for (int c = 0; c < NC; ++c) acc += max(0, tiles_of_n(cn[c]) - t);
    } else {
      for (int bb = lane; bb < B; bb += 64) acc += max(0, tiles_of(bb) - t);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    return __builtin_amdgcn_readfirstlane(acc);
  };
  if ((long long)Hq * count_from(0) <= item) return false;
  int lo = 0, hi = ntiles - 1;  // Hq * S(lo) > item throughout
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((long long)Hq * count_from(mid) > item) lo = mid; else hi = mid - 1;
  }
  const int above = count_from(lo + 1);
  const int cnt = count_from(lo) - above;           // sequences with a tile at index lo
  const long long first = (long long)Hq * above;    // items at higher tile indices
  const int nt = cnt * Hq;
  int j = (int)(item - first);
  if (first % kXcds == 0 && nt % kXcds == 0) j = (j % kXcds) * (nt / kXcds) + j / kXcds;
  int k = j / Hq;
  *ho = j % Hq;
  *tile = lo;
  // the k-th sequence (in batch order) that has a tile at index lo
  for (int base = 0; base < B; base += 64) {
    const int bb = base + lane;
    int n_l = 0;
    long long s_l = 0;
    if (cached) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        if (base == 64 * c) {
          n_l = cn[c];
          s_l = cs[c];
        }
    } else if (bb < B) {
      seq_bounds(cu, bb, T, max_seqlen, &s_l, &n_l);
    }
    const bool has = bb < B && tiles_of_n(n_l) > lo;
    const unsigned long long m = __ballot(has);
    const int c = __popcll(m);
    if (k < c) {
      const unsigned long long below = m & ((1ull << lane) - 1ull);
      const unsigned long long w = __ballot(has && __popcll(below) == k);
      const int src = __ffsll((long long)w) - 1;
      *bo = base + src;
      *no = __shfl(n_l, src);
      *so = ((long long)__shfl((int)(s_l >> 32), src) << 32) |
            (unsigned)__shfl((int)(s_l & 0xffffffff), src);
      return true;
    }
    k -= c;
  }
  return false;  // not reached: cnt > k
}

// Number of q-tiles of a packed batch, sum_b ceil(n_b / kBQ) (uniform over
// the wave; the sequences spread over the lanes).
__device__ __forceinline__ int packed_tiles(const int *__restrict__ cu, int B, long long T,
                                            int max_seqlen) {
  int acc = 0;
  for (int bb = (int)(threadIdx.x & 63); bb < B; bb += 64) {
    long long s0;
    int nb;
    seq_bounds(cu, bb, T, max_seqlen, &s0, &nb);
    acc += (nb + kBQ - 1) / kBQ;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  return __builtin_amdgcn_readfirstlane(acc);
}

// Work queues for the tail of a large packed launch.  The XCDs run at
// different clocks (a spread of ~6% on one part), and each runs the
// workgroups of its share of block indices at its own pace, so with a static
// map the fastest idles at the end while the slowest finishes.  Items below
// `static_items` (a multiple of 8) go by block index; counter x hands out the
// items above it that are congruent to x modulo 8, in increasing order (its
// k-th take returns static_items + x + 8k), the items the block-index map
// would give XCD x.  A workgroup past the static part takes from the queue of
// its XCD and, once that is empty, from the others in turn; with a few more
// workgroups than items an XCD that runs ahead takes tail items a slower one
// has not reached.  Counters only grow; a take past the end is harmless.
// Only thread 0 calls this.
__device__ __forceinline__ int queue_take(int *queues, int x) {
  return x + kXcds * atomicAdd(queues + x, 1);
}

// EXT: keys from a cache with a prefix (chunked prefill) and / or a sliding
// window with sinks; without it those are compiled out (plain causal).
template <int D, bool OUT_F32, bool ROTATE_Q, bool EXT>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const int *__restrict__ cu, int B, int max_seqlen,
    long long T, int Hq, int Hkv, const double *__restrict__ theta, float scale_log2,
    void *__restrict__ out, float *__restrict__ lse, int ntiles, int *flag, int kv_len,
    const int *__restrict__ ctx, int window, int sinks, int permuted, int *__restrict__ queues,
    int static_items) {
  constexpr int KQ = D / 32;         // score MFMA k-steps over the head dim
  constexpr int DB = D / 16;         // 16-row blocks of O^T (head dims)
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
  long long s0;
  int n;
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
    seq_bounds(cu, b, T, max_seqlen, &s0, &n);
  } else {
    int item = (int)blockIdx.x;
    int total = -1;  // items of the packed map, formed when needed
    if (queues != nullptr && item >= static_items) {
      // the first take goes out before the item count is formed, so that the
      // atomic's round trip overlaps the count's loads
      __shared__ int item_slot;
      const int x0 = (int)(blockIdx.x % kXcds);
      int it = 0;
      if (threadIdx.x == 0) it = static_items + queue_take(queues, x0);
      total = Hq * packed_tiles(cu, B, T, max_seqlen);
      if (threadIdx.x == 0) {
        for (int d = 1; it >= total && d < kXcds; ++d)
          it = static_items + queue_take(queues, (x0 + d) % kXcds);
        item_slot = it < total ? it : -1;
      }
      __syncthreads();
      item = item_slot;
      if (item < 0) return;
    }
    if (permuted) {  // any bijection of the items (order-independence test)
      if (total < 0) total = Hq * packed_tiles(cu, B, T, max_seqlen);
      if (item >= total) return;
      item = (int)(((long long)(total - 1 - item) + total / 3) % total);
    }
    if (!packed_item(cu, B, T, max_seqlen, Hq, ntiles, item, &tile, &b, &h, &s0, &n)) return;
  }
  const int hk = h / (Hq / Hkv);
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
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int tw0 = q0 + wave * 32;  // first query row of this wave

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
  // V: slot = chunk ^ vswz(row % 8).  Rows past the sequence end read 0.
  const uint16_t *kseq = k + (krow0 * Hkv + hk) * (long long)D;
  const uint16_t *vseq = v + (krow0 * Hkv + hk) * (long long)D;
  const uint32_t rbytes = (uint32_t)(rstride * 2);
  const int drow = lane / CH, dslot = lane % CH;
  uint32_t koff[DPW], voff[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int row = (wave * DPW + i) * RPI + drow;
    koff[i] = drow * rbytes + 16 * (dslot ^ (row & (CH - 1)));
    voff[i] = drow * rbytes + 16 * (dslot ^ vswz<CH>(row & 7));
  }
  auto copy_tile = [&](uint16_t *dst, const uint16_t *seq, int t, bool is_v) YR_INLINE {
    const int key0 = t * kBC;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(seq + key0 * rstride, (uint32_t)min(kBC, nk - key0) * rbytes);
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int p = wave * DPW + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (YR_LDS void *)(dst + p * 512), 16,
                                               (int)(is_v ? voff[i] : koff[i]),
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
  // With a window the workgroup sweeps its window tiles rotated: list
  // position js + s holds the window tile congruent to s modulo the window's
  // length in tiles.  Workgroups of neighbouring q-tiles (windows a few tiles
  // apart, launched together) then read the same tile at the same step, so
  // L2 serves them; swept from its start, each would read a tile a few steps
  // after the other, about an L2's worth of traffic later.
  const int nw = last - jw + 1;
  const int r0 = window > 0 ? (nw - jw % nw) % nw : 0;
  auto tile_of = [&](int i) YR_INLINE {
    if constexpr (!EXT) {
      return i;
    } else {
      if (i < js) return i;
      int p = i - js + r0;
      p = p >= nw ? p - nw : p;
      return jw + p;
    }
  };
  // prologue copies (K of tiles 0..NS-1, V of tiles 0..NS-2 of the list) go
  // out before the query work so that they are in flight meanwhile
  static_for<0, NS>([&](auto ic) YR_INLINE {
    constexpr int I = decltype(ic)::value;
    if (I < count) copy_tile(kst(ic), kseq, tile_of(I), false);
    if (I + 1 < NS && I < count) copy_tile(vst(ic), vseq, tile_of(I), true);
  });

  // ---- Q fragments (B operand of S^T = K Q^T), rotated on load -----------
  // Lane l holds query rows tq[rb] = tw0 + 16 rb + l16 (rb = 0, 1) and, for
  // k-step ks, head dims 32 ks + 8 g4 .. +7.  Every load goes out before any
  // arithmetic: written per fragment, the compiler waited for each
  // fragment's loads in turn (and the first wait also for the tile copies
  // issued above), 8 round trips in a row before the first tile.  A row past
  // the sequence end reads row 0 and is zeroed.
  bf16x8 qf[RB][KQ];
  int tq[RB];
  u32x4 qw[RB][KQ];
  double thq[KQ][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    tq[rb] = tw0 + 16 * rb + l16;
    const uint16_t *qp = q + ((s0 + (tq[rb] < n ? tq[rb] : 0)) * Hq + h) * (long long)D + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < KQ; ++ks) qw[rb][ks] = *reinterpret_cast<const u32x4 *>(qp + ks * 32);
  }
  if (ROTATE_Q) {
#pragma unroll
    for (int ks = 0; ks < KQ; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) thq[ks][e] = theta[ks * 16 + g4 * 4 + e];
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const bool qvalid = tq[rb] < n;
#pragma unroll
    for (int ks = 0; ks < KQ; ++ks) {
      u32x4 w = qw[rb][ks];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // the logit scale (log2 units) folded into the query before its one
        // rounding to bf16, so that the scores come out of the matrix cores
        // ready for exp2
        float x0 = bf16_to_f32(w[e] & 0xffffu), x1 = bf16_to_f32(w[e] >> 16);
        if (ROTATE_Q) {
          float c, sn;
          rope_cos_sin((double)(P + tq[rb]), thq[ks][e], &c, &sn);
          rotate_pair(x0, x1, c, sn);
        }
        w[e] = qvalid ? pack_bf16x2(x0 * scale_log2, x1 * scale_log2) : 0u;
      }
      qf[rb][ks] = as_bf16x8(w);
    }
  }

  f32x4 o[DB][RB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) o[i][rb] = f32x4{};
  float m_run[RB], l_part[RB];
  // -m_run (0 while m_run = -inf) in every slot: the accumulators the score
  // MFMAs start from, so that they return s * scale - m directly
  f32x4 negm[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_part[rb] = 0.f;
    negm[rb] = f32x4{};
  }

  // LDS operand addresses (elements).  K: row 16 kb + l16, chunk 4 ks + g4.
  // V^T (transposing reads): lane t = l16 of group g4 reads 4 elements of key
  // row 4 g4 + (t >> 2) (+16 kb) at head dims 16 db + 4 (t & 3) and receives
  // head dim 16 db + t of 4 consecutive key rows.
  const int kx = l16 & (CH - 1);
  const int vrow = 4 * g4 + (l16 >> 2);
  // element offset of the lane's V^T read for head-dim block db:
  // vrow * D + 8 * ((2 db + (l16 & 3) / 2) ^ vswz(vrow % 8)) + 4 (l16 & 1).
  // With 16 chunks a row, vswz = 2 (vrow % 8) only flips the bits of 2 db, so
  // the offset is vbase ^ (16 db): one base register for every block.
  const int vbase = vrow * D + 8 * ((((l16 & 3) >> 1)) ^ vswz<CH>(vrow & 7)) + 4 * (l16 & 1);
  auto voffs = [&](int vb, int db) YR_INLINE {
    if constexpr (CH >= 16) {
      return vb ^ (16 * db);
    } else {
      return vrow * D + 8 * ((2 * db + ((l16 & 3) >> 1)) ^ vswz<CH>(vrow & 7)) + 4 * (l16 & 1);
    }
  };

  // ---- per-tile work -------------------------------------------------------
  // Tile j has keys j*64 .. j*64+63.  The wave (rows tw0 .. tw0+31, positions
  // P + row) skips it when it lies wholly above the wave's diagonal, or, with
  // a window, wholly below the window of the wave's first row and past the
  // sinks.
  auto active = [&](int j) YR_INLINE {
    if (tw0 >= n || j * kBC > P + tw0 + 31) return false;
    return window == 0 || j * kBC + kBC - 1 > P + tw0 - window || j * kBC < sinks;
  };

  // S^T = K Q^T for one tile (four 16-key blocks by two 16-row blocks); slot
  // r of accumulator [kb][rb] holds key 16 kb + 4 g4 + r of row tq[rb].  Each
  // K fragment feeds the MFMAs of both row blocks.
  auto scores = [&](auto par, f32x4 (&s)[NKB][RB]) YR_INLINE {
    const uint16_t *ks_ = kst(par);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int ks = 0; ks < KQ; ++ks) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4 *>(
            ks_ + (kb * 16 + l16) * D + 8 * ((4 * ks + g4) ^ kx)));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          s[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[rb][ks],
                                                              ks == 0 ? negm[rb] : s[kb][rb], 0, 0,
                                                              0);
      }
    }
  };

  // Slow path of the softmax (a tile sum above 2^8, or a row without a
  // reference yet): move each row's reference to its running maximum, so that
  // the tile's P are at most 1 afterwards.  The tile's scores and the
  // already issued scores of the next tile (nx, computed against the old
  // reference) shift with it, and O and the row sum are rescaled.  A row that
  // has seen no visible key keeps -inf (alpha 1).  A row's 64 keys lie in the
  // four lanes l16 + 16 g4, which exchange their maxima.
  auto move_reference = [&](f32x4 (&s)[NKB][RB], f32x4 (&nx)[NKB][RB]) YR_INLINE {
    float mx[RB];
    bool grow[RB], first[RB];
    bool any = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float x = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) x = fmaxf(x, s[kb][rb][r]);
      // the tile's row max less m_run (the scores carry -m_run already)
      mx[rb] = quarter_max(x);
      first[rb] = m_run[rb] == -INFINITY;
      grow[rb] = first[rb] ? mx[rb] > -INFINITY : mx[rb] > 0.f;
      any = any || grow[rb];
    }
    if (__any(any)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float m_new = grow[rb] ? (first[rb] ? mx[rb] : m_run[rb] + mx[rb]) : m_run[rb];
        // 0 when m_run = -inf; 1 for a row that has seen no visible key yet
        // (with a window a row can meet tiles it does not see at all)
        const float alpha =
            m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
        // move this tile's scores to the new reference
        const float shift = (first[rb] ? 0.f : m_run[rb]) - (m_new == -INFINITY ? 0.f : m_new);
        m_run[rb] = m_new;
        l_part[rb] *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) o[i][rb] *= alpha;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            s[kb][rb][r] += shift;
            nx[kb][rb][r] += shift;
          }
        const float nm = m_run[rb] == -INFINITY ? 0.f : -m_run[rb];
#pragma unroll
        for (int r = 0; r < 4; ++r) negm[rb][r] = nm;
      }
    }
  };

  // O^T += V^T P^T over two 32-key k-steps.  In k-step ps, k-position
  // 8 g4 + e stands for key 16 (2 ps + e / 4) + 4 g4 + e % 4: the B operand is
  // the lane's own P of key blocks 2 ps and 2 ps + 1, and the A operand is two
  // transposing reads of those key rows.  Each V^T fragment feeds the MFMAs
  // of both row blocks.
  auto pv = [&](auto par, bf16x8 (&pf)[NPS][RB]) YR_INLINE {
    const uint16_t *vs = vst(par);
    // an opaque copy of the base, so that the eight offsets are formed here
    // (one XOR each) rather than held in registers across the loop
    int vb = vbase;
    asm volatile("" : "+v"(vb));
#pragma unroll
    for (int ps = 0; ps < NPS; ++ps) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t *ap = vs + 32 * ps * D + voffs(vb, db);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YR_LDS i16x4 *)(ap));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YR_LDS i16x4 *)(ap + 16 * D));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const bf16x8 a = as_bf16x8(u32x4{l2[0], l2[1], h2[0], h2[1]});
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          o[db][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[ps][rb], o[db][rb], 0, 0, 0);
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
  // P = exp2(s - m) of a whole tile into bf16 fragments, in the B-operand
  // order of pv; ts[rb] gets the lane's sum of row tq[rb]'s 16 P of the tile
  auto exp_tile = [&](f32x4 (&s)[NKB][RB], bf16x8 (&pf)[NPS][RB], float (&ts)[RB]) YR_INLINE {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float t = 0.f;
#pragma unroll
      for (int ps = 0; ps < NPS; ++ps) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x4 &x = s[2 * ps + (e >> 1)][rb];
          const float p0 = __builtin_amdgcn_exp2f(x[2 * (e & 1)]);
          const float p1 = __builtin_amdgcn_exp2f(x[2 * (e & 1) + 1]);
          t += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pf[ps][rb] = as_bf16x8(w);
      }
      ts[rb] = t;
    }
  };
  // Mask of a diagonal, window-edge, sink or tail tile: the keys of the tile
  // row tq[rb] sees, as offsets c from the tile's first key, are c <= hi
  // (causal, and inside the sequence) and c >= lo (inside the window), or
  // c < se (a sink).  Slot r of block kb holds offset 16 kb + 4 g4 + r; the
  // lane's 4 g4 goes into the bounds, so each slot compares a constant.
  auto apply_mask = [&](int j, f32x4 (&s)[NKB][RB]) YR_INLINE {
    const int key0 = j * kBC;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int pos = P + tq[rb];
      const int hi = min(pos, nk - 1) - key0 - 4 * g4;
      if (window > 0) {
        const int lo = pos - window + 1 - key0 - 4 * g4;
        const int se = sinks - key0 - 4 * g4;
        const unsigned span = (unsigned)(hi - lo);
        if (key0 < sinks) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int c = kb * 16 + r;
              const bool vis = c <= hi && (c >= lo || c < se);
              s[kb][rb][r] = vis ? s[kb][rb][r] : -INFINITY;
            }
        } else {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int c = kb * 16 + r;
              // lo <= c <= hi as one unsigned compare (empty when hi < lo)
              const bool vis = hi >= lo && (unsigned)(c - lo) <= span;
              s[kb][rb][r] = vis ? s[kb][rb][r] : -INFINITY;
            }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int c = kb * 16 + r;
            s[kb][rb][r] = c <= hi ? s[kb][rb][r] : -INFINITY;
          }
      }
    }
  };
  // Optimistic softmax: exponentiate against the current reference first.
  // Every P of the tile is at most 2^8 when the lane's tile sum is (P >= 0),
  // which is the lazy-max bound; only when a sum exceeds it (or is not a
  // number, or a row has no reference yet) does the wave take the row max,
  // move the reference to it and exponentiate again.
  auto softmax_pv = [&](auto par, f32x4 (&cur)[NKB][RB], f32x4 (&nxt)[NKB][RB]) YR_INLINE {
    bf16x8 pf[NPS][RB];
    float ts[RB];
    exp_tile(cur, pf, ts);
    bool slow = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) slow = slow || !(ts[rb] <= 256.f) || m_run[rb] == -INFINITY;
    if (__any(slow)) {
      move_reference(cur, nxt);
      exp_tile(cur, pf, ts);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) l_part[rb] += ts[rb];
    pv(par, pf);
  };
  // General step (diagonal, window-edge and tail tiles, the last step): every
  // check.  The mask goes first; then the same optimistic softmax as the
  // clear steps (a row that has seen no key yet takes the row max path).
  auto step = [&](auto par, int i, f32x4 (&cur)[NKB][RB], f32x4 (&nxt)[NKB][RB]) YR_INLINE {
    stage(par, i);
    if (i + 1 < count && active(tile_of(i + 1))) scores(nextp(par), nxt);
    if (active(tile_of(i))) {
      const int j = tile_of(i);
      const int key0 = j * kBC;
      const bool wmask = window > 0 && key0 <= P + tw0 + 31 - window && key0 + kBC > sinks;
      if ((key0 + kBC - 1 > P + tw0) || (key0 + kBC > nk) || wmask) apply_mask(j, cur);
      softmax_pv(par, cur, nxt);
    }
  };
  // Clear step: tiles i and i+1 of the list need no mask for any row (below
  // the diagonal of the workgroup's first row, inside the window of its last
  // row) and every wave works on both, so the score MFMAs of tile i+1 go out
  // first, right after the barrier, and the exp / convert work of tile i and
  // its PV MFMAs follow.
  auto step_clear = [&](auto par, int i, f32x4 (&cur)[NKB][RB], f32x4 (&nxt)[NKB][RB]) YR_INLINE {
    stage(par, i);
    scores(nextp(par), nxt);
    softmax_pv(par, cur, nxt);
  };

  // prologue: every prologue copy landed; S(tile(0))
  wait_dma<0>();
  __syncthreads();
  f32x4 sa[NKB][RB], sb[NKB][RB];
  if (active(tile_of(0))) scores(std::integral_constant<int, 0>{}, sa);
  // Steps are unrolled over the stage index (i % NS) and the score buffer
  // (i % 2), so every LDS array and register array is picked at compile time.
  constexpr int BL = 2;
  auto sbuf = [&](auto ic) YR_INLINE -> f32x4(&)[NKB][RB] {
    if constexpr (decltype(ic)::value % 2 == 0) return sa; else return sb;
  };
  auto obuf = [&](auto ic) YR_INLINE -> f32x4(&)[NKB][RB] {
    if constexpr (decltype(ic)::value % 2 == 0) return sb; else return sa;
  };
  // The tiles that need no mask for any row form one run of the list: from
  // the first tile at or past the window start of the workgroup's last row to
  // the last tile below the diagonal of its first row (list positions
  // [c0, c1)).  Steps before it and after it take the general body; a clear
  // step i needs tiles i and i+1 in the run.  Separate loops keep each body's
  // registers to itself.
  // In list positions the clear tiles [jc, jd] form one run, or two when the
  // rotation wraps them: [c0, c1) and [c2, c3), c1 <= c2.
  int c0 = count, c1 = count, c2 = count, c3 = count;
  {
    const int jd = (P + q0 + 1) / kBC - 1;  // last tile wholly below the first row's diagonal
    const int jc = window > 0 ? max(jw, (P + qend - window + kBC - 1) / kBC) : 0;
    if (jd >= jc) {
      if constexpr (!EXT) {
        c0 = jc;
        c1 = jd + 1;
      } else {
        int a = jc - jw - r0;
        a = a < 0 ? a + nw : a;
        const int len = jd - jc + 1;
        if (a + len <= nw) {
          c0 = js + a;
          c1 = c0 + len;
        } else {
          c0 = js;
          c1 = js + (a + len - nw);
          c2 = js + a;
          c3 = count;
        }
      }
    }
  }
  auto general_block = [&](int i) YR_INLINE {
    static_for<0, BL>([&](auto ic) YR_INLINE {
      constexpr int I = decltype(ic)::value;
      if (i + I < count) step(std::integral_constant<int, I % NS>{}, i + I, sbuf(ic), obuf(ic));
    });
  };
  // the unmasked run in blocks of 4 steps (two stage / buffer cycles; +0.5-1%
  // over blocks of 2), its remainder in blocks of 2
  constexpr int BLC = 4;
  int i = 0;
  for (; i < c0; i += BL) general_block(i);
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
  if constexpr (EXT) {  // the second run, where the rotation wraps the first
    for (; i < c2; i += BL) general_block(i);
    for (; i + BLC < c3; i += BLC) {
      static_for<0, BLC>([&](auto ic) YR_INLINE {
        constexpr int I = decltype(ic)::value;
        step_clear(std::integral_constant<int, I % NS>{}, i + I, sbuf(ic), obuf(ic));
      });
    }
    for (; i + BL < c3; i += BL) {
      static_for<0, BL>([&](auto ic) YR_INLINE {
        constexpr int I = decltype(ic)::value;
        step_clear(std::integral_constant<int, I % NS>{}, i + I, sbuf(ic), obuf(ic));
      });
    }
  }
  for (; i < count; i += BL) general_block(i);

  // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l) ---------------------
  // lane l holds head dims 16 db + 4 g4 .. +3 of row tq[rb]
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = quarter_sum(l_part[rb]);
    if (tq[rb] >= n) continue;
    const float inv = 1.f / l_tot;
    const long long orow = ((s0 + tq[rb]) * Hq + h) * (long long)D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d0 = db * 16 + 4 * g4;
      const f32x4 y = o[db][rb] * inv;
      if (OUT_F32) {
        *reinterpret_cast<float4 *>((float *)out + orow + d0) = make_float4(y[0], y[1], y[2], y[3]);
      } else {
        u32x2 pk;
        pk[0] = pack_bf16x2(y[0], y[1]);
        pk[1] = pack_bf16x2(y[2], y[3]);
        *reinterpret_cast<u32x2 *>((uint16_t *)out + orow + d0) = pk;
      }
    }
    if (lse != nullptr && g4 == 0)
      lse[(long long)h * T + s0 + tq[rb]] = (m_run[rb] + __log2f(l_tot)) * kLn2;
  }
}

// Zeroes the work-queue counters (a kernel rather than a memset, so that a
// captured graph replays it correctly).
__global__ void prefill_queue_reset(int *queues) {
  if (threadIdx.x < kXcds) queues[threadIdx.x] = 0;
}

// Packed launches of at least this many work items (32 per CU on 256 CUs)
// hand out the last third of their items through the work queues; shorter
// ones gain less from it than the atomics cost (16K MHA: -2% with every item
// queued, the 128K GQA and ragged 70B launches +1.2 to +1.6%).
constexpr long long kQueueMinItems = 8192;

template <int D, bool OUT_F32, bool ROT, bool EXT>
hipError_t launch_one(const PrefillArgs &a, hipStream_t s) {
  const int ntiles = (a.max_seqlen + kBQ - 1) / kBQ;
  const float scale_log2 = (float)((double)a.softmax_scale * 1.4426950408889634074);
  // The ranked map of chunked prefill takes one block per (rank, q-tile,
  // head).  The packed map has at most Hq * min(ntiles * B, ceil(T / kBQ) +
  // B) items (sum_b ceil(n_b / kBQ) is at most both); large launches add 1/16
  // spare workgroups for the queued tail.
  const bool ranked = a.kv_cache_len > 0 && a.B <= kMaxRankedSeqs;
  long long blocks = (long long)ntiles * a.B * a.Hq;
  int *queues = nullptr;
  int static_items = 0;
  if (!ranked) {
    const long long tiles = std::min<long long>((long long)ntiles * a.B, (a.T + kBQ - 1) / kBQ + a.B);
    const long long items = tiles * a.Hq;
    blocks = items;
    if (a.work_queues != nullptr && items >= kQueueMinItems) {
      static_items = (int)(items * 2 / 3) & ~(kXcds - 1);
      blocks = items + items / 16 + kXcds;
      queues = a.work_queues;
      hipLaunchKernelGGL(prefill_queue_reset, dim3(1), dim3(64), 0, s, queues);
    }
  }
  if (blocks < 1) blocks = 1;  // validates cu_seqlens even when nothing is computed
  hipLaunchKernelGGL((prefill_bf16_kernel<D, OUT_F32, ROT, EXT>), dim3((unsigned)blocks), dim3(kThreads),
                     0, s, (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                     a.cu_seqlens, a.B, a.max_seqlen, a.T, a.Hq, a.Hkv, a.theta, scale_log2, a.out,
                     a.lse, ntiles, a.dev_flag, a.kv_cache_len, a.ctx_lens, a.window, a.sinks,
                     a.permuted_order, queues, static_items);
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
