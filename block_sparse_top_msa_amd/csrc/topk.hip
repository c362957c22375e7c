// Top-K block select on gfx950: q2k[g, i, :] = the `topk` blocks with the
// largest finite max_score, equal scores going to the lower block id, written
// ascending and -1 padded (msa_sparse_attention page, Parameters: q2k_indices;
// msa_proxy_score page, summary: the scores feed the top-K select).
//
// One wave per selection row.  Lane l holds the candidates t = l + 64 c.
// Scores are compared through an order-preserving uint32 map (-0 == +0), the
// topk-th largest value is found by a 32-step bitwise search with ballot
// counts, and ties at that value are resolved by ascending block id using
// ballot prefix counts.  The result is exact and independent of scheduling.
#include "common.hpp"
#include "internal.hpp"

namespace msa {

__device__ __forceinline__ int popc64(unsigned long long x) { return __popcll(x); }

template <int C>
__global__ __launch_bounds__(256) void msa_topk_kernel(const float* __restrict__ scores,
                                                      int hs, int T, int total_q, int topk,
                                                      int hkv, int mode, int sel_rows,
                                                      int32_t* __restrict__ q2k) {
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (wave >= sel_rows * total_q) return;
  const int i = wave % total_q;
  const int gs = wave / total_q;  // selection head

  // score heads feeding this selection
  int h_lo, h_hi;
  if (mode == 1) {          // all heads, one shared selection
    h_lo = 0; h_hi = hs;
  } else if (mode == 2) {   // group of heads per KV head
    const int gsz = hs / hkv;
    h_lo = gs * gsz; h_hi = h_lo + gsz;
  } else {
    h_lo = gs; h_hi = gs + 1;
  }

  uint32_t key[C];
  bool valid[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int t = lane + kWave * c;
    float s = -INFINITY;
    if (t < T) {
      s = scores[((int64_t)h_lo * T + t) * total_q + i];
      for (int h = h_lo + 1; h < h_hi; ++h)
        s = fmaxf(s, scores[((int64_t)h * T + t) * total_q + i]);
    }
    // finite only: -inf, +inf and NaN are never selected
    valid[c] = (t < T) && (__float_as_uint(s) & 0x7F800000u) != 0x7F800000u;
    key[c] = valid[c] ? ordered_f32(s) : 0u;
  }

  int nvalid = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) nvalid += popc64(__ballot(valid[c]));

  bool chosen[C];
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

  // write ascending (t = lane + 64 c is ascending in (c, lane) order)
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int g_lo = (mode == 1) ? 0 : gs;
  const int g_hi = (mode == 1) ? hkv : gs + 1;
  int base = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const unsigned long long m = __ballot(chosen[c]);
    if (chosen[c]) {
      const int pos = base + popc64(m & below);
      for (int g = g_lo; g < g_hi; ++g)
        q2k[((int64_t)g * total_q + i) * topk + pos] = lane + kWave * c;
    }
    base += popc64(m);
  }
  for (int pos = base + lane; pos < topk; pos += kWave)
    for (int g = g_lo; g < g_hi; ++g) q2k[((int64_t)g * total_q + i) * topk + pos] = -1;
}

template <int C>
static hipError_t launch_topk_c(const float* scores, int hs, int T, int total_q, int topk,
                                int hkv, int mode, int32_t* q2k, hipStream_t stream) {
  const int sel_rows = (mode == 1) ? 1 : hkv;
  const int64_t waves = (int64_t)sel_rows * total_q;
  if (waves <= 0) return hipSuccess;
  const int grid = (int)((waves + 3) / 4);
  hipLaunchKernelGGL((msa_topk_kernel<C>), dim3(grid), dim3(256), 0, stream, scores, hs, T,
                     total_q, topk, hkv, mode, sel_rows, q2k);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int score_heads, int T, int total_q, int topk,
                       int hkv, int mode, int32_t* q2k, hipStream_t stream) {
  const int c = (T + kWave - 1) / kWave;
  if (c <= 1) return launch_topk_c<1>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
  if (c <= 2) return launch_topk_c<2>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
  if (c <= 4) return launch_topk_c<4>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
  if (c <= 8) return launch_topk_c<8>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
  if (c <= 16) return launch_topk_c<16>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
  if (c <= 32) return launch_topk_c<32>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
  return launch_topk_c<64>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
}

}  // namespace msa
