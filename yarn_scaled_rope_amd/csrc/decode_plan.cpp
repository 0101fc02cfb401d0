// Host side of the decode split: chunk size and KV heads per workgroup.
// Pure functions of the sizes, shared by the workspace query and the launch
// (host code only, no device code).
#include "yr_internal.h"

namespace yr {

int decode_heads_per_wg(int Hkv, int head_dim, bool fp8) {
  return heads_per_wg(Hkv, head_dim, fp8 ? 1 : 2);
}

int decode_chunk(int B, int max_cache_len, int units, int min_chunk, int target) {
  // At least `target` workgroups (several per CU); chunks are powers of two,
  // at most 2048 keys so that a workgroup's start-up and combine stay small
  // next to its sweep, and at least min_chunk.
  int chunk = 2048;
  while (chunk > min_chunk && (long long)B * units * decode_nsplit(max_cache_len, chunk) < target)
    chunk >>= 1;
  return chunk;
}

}  // namespace yr
