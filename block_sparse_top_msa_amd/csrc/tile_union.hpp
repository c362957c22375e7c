// Per-tile block union built in LDS (msa_sparse_attention page, summary: the
// union metadata is built internally from q2k_indices).
//
// The tile's selected block ids are OR-ed into an LDS bitmap indexed by block
// id; a prefix popcount over the bitmap words turns it into an ascending
// list, and a second pass records, per list entry, the mask of tile tokens
// that selected it.  Cost is O(ntok * topk + words) with words =
// ceil(n_blocks / 32), independent of how the selections are spread.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace msa {

struct UnionLds {
  uint32_t bitmap[kMaxBitmapWords];
  int32_t prefix[kMaxBitmapWords];
  int32_t list[kMaxUnion];
  unsigned long long mask[kMaxUnion];
  int32_t count;
};

// All threads of the workgroup must call this.  `rows` points at the
// q2k row of the tile's first token for this KV head; rows are `topk` apart.
// With `use_pre` (ntok * topk <= NT), thread e already holds entry e in
// `pre` and the entries are not read again.  Returns the union size (also
// in u.count).  Ends with a barrier.
template <int NT>
__device__ int build_tile_union(UnionLds& u, const int32_t* __restrict__ rows, int ntok,
                                int topk, int n_blocks, int pre = -1, bool use_pre = false) {
  const int tid = threadIdx.x;
  const int words = (n_blocks + 31) >> 5;
  for (int w = tid; w < words; w += NT) u.bitmap[w] = 0u;
  __syncthreads();

  const int n = ntok * topk;
  for (int e = tid; e < n; e += NT) {
    int id = use_pre ? pre : rows[e];
    if (id >= 0 && id < n_blocks) atomicOr(&u.bitmap[id >> 5], 1u << (id & 31));
  }
  __syncthreads();

  // exclusive prefix of per-word popcounts, by the first wave
  if (tid < kWave) {
    const int per = (words + kWave - 1) / kWave;
    const int w0 = tid * per;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      int w = w0 + i;
      if (w < words) local += __popc(u.bitmap[w]);
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      int o = __shfl_up(incl, off, kWave);
      if (tid >= off) incl += o;
    }
    int run = incl - local;
    for (int i = 0; i < per; ++i) {
      int w = w0 + i;
      if (w < words) {
        u.prefix[w] = run;
        run += __popc(u.bitmap[w]);
      }
    }
    if (tid == kWave - 1) u.count = incl;
  }
  __syncthreads();

  const int cnt = u.count;
  for (int w = tid; w < words; w += NT) {
    uint32_t bits = u.bitmap[w];
    int pos = u.prefix[w];
    while (bits) {
      int b = __ffs(bits) - 1;
      u.list[pos++] = (w << 5) + b;
      bits &= bits - 1u;
    }
  }
  for (int i = tid; i < cnt; i += NT) u.mask[i] = 0ull;
  __syncthreads();

  for (int e = tid; e < n; e += NT) {
    int id = use_pre ? pre : rows[e];
    if (id >= 0 && id < n_blocks) {
      int w = id >> 5;
      int pos = u.prefix[w] + __popc(u.bitmap[w] & ((1u << (id & 31)) - 1u));
      atomicOr(&u.mask[pos], 1ull << (e / topk));
    }
  }
  __syncthreads();
  return cnt;
}

}  // namespace msa
