// Exact top-K of a wave's candidates (the block select of the MSA hot path,
// msa_sparse_attention page, Parameters: q2k_indices), shared by the top-K
// kernels and the proxy kernel's per-chunk selection.
#pragma once

#include "common.hpp"

namespace msa {

__device__ __forceinline__ int popc64(unsigned long long x) { return __popcll(x); }

// The `topk` largest of a wave's candidates (key[c] of lane l is candidate
// l + 64 c, valid[c] false for padding), equal keys going to the lower
// candidate number: chosen[c] marks them.
template <int C>
__device__ __forceinline__ void select_topk(const uint32_t (&key)[C], const bool (&valid)[C],
                                            int topk, int lane, bool (&chosen)[C]) {
  int nvalid = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) nvalid += popc64(__ballot(valid[c]));

  if (nvalid <= topk) {
#pragma unroll
    for (int c = 0; c < C; ++c) chosen[c] = valid[c];
  } else {
    // largest x with #{key >= x} >= topk: the topk-th largest key
    uint32_t x = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = x | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int c = 0; c < C; ++c) cnt += popc64(__ballot(valid[c] && key[c] >= cand));
      if (cnt >= topk) x = cand;
    }
    int ngt = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) ngt += popc64(__ballot(valid[c] && key[c] > x));
    const int need = topk - ngt;  // ties at x to take, lowest block ids first
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    int run = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bool eq = valid[c] && key[c] == x;
      const unsigned long long m = __ballot(eq);
      const int rank = run + popc64(m & below);
      chosen[c] = (valid[c] && key[c] > x) || (eq && rank < need);
      run += popc64(m);
    }
  }
}

}  // namespace msa
