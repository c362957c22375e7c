// Exact top-K of a wave's candidates (the block select of the MSA hot path,
// msa_sparse_attention page, Parameters: q2k_indices), shared by the top-K
// kernels and the proxy kernel's per-chunk selection.
#pragma once

#include "common.hpp"

namespace msa {

__device__ __forceinline__ int popc64(unsigned long long x) { return __popcll(x); }

// OR / AND of v over the wave: DPP shifts within each 16-lane row, then the
// row broadcasts (lane 15 to the next row, lane 31 to rows 2 and 3); lane 63
// ends with the whole wave's value.  Lanes a step does not reach keep the
// identity.
template <bool AND>
__device__ __forceinline__ uint32_t wave_bits(uint32_t v) {
  constexpr int id = AND ? -1 : 0;
  auto op = [](uint32_t a, uint32_t b) { return AND ? (a & b) : (a | b); };
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x111, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x112, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x114, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x118, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xa, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

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
    // largest x with #{key >= x} >= topk: the topk-th largest key, found
    // bit by bit below the prefix every valid key shares (all keys are at
    // least the prefix, none reaches the next prefix value).  Once exactly
    // topk keys are >= x, they are the selection: no tie crosses x.
    uint32_t kor = 0u, kand = ~0u;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      kor |= valid[c] ? key[c] : 0u;
      kand &= valid[c] ? key[c] : ~0u;
    }
    kor = wave_bits<false>(kor);
    kand = wave_bits<true>(kand);
    const int top = kor == kand ? -1 : 31 - __builtin_clz(kor ^ kand);
    uint32_t x = top < 0 ? kand : kand & ~((2u << top) - 1u);
    for (int bit = top; bit >= 0; --bit) {
      const uint32_t cand = x | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int c = 0; c < C; ++c) cnt += popc64(__ballot(valid[c] && key[c] >= cand));
      if (cnt >= topk) {
        x = cand;
        if (cnt == topk) {
#pragma unroll
          for (int c = 0; c < C; ++c) chosen[c] = valid[c] && key[c] >= x;
          return;
        }
      }
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
