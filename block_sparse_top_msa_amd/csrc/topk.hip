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
#include "topk.hpp"

namespace msa {

// Workgroups reach the XCDs round-robin: the remap gives each XCD a run of
// consecutive rows, whose scores share cache lines (query index fastest).
template <int C>
__global__ __launch_bounds__(256) void msa_topk_kernel(const float* __restrict__ scores,
                                                      int hs, int T, int total_q, int topk,
                                                      int hkv, int mode, int sel_rows,
                                                      int n_wg, int32_t* __restrict__ q2k) {
  const int wg = xcd_remap(blockIdx.x, n_wg);
  if (wg < 0) return;
  const int wave = wg * 4 + threadIdx.x / kWave;
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

  bool chosen[C];
  select_topk<C>(key, valid, topk, lane, chosen);

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

// Long rows (more than 256 candidates): one workgroup of 16 waves per row.
// Wave w takes candidates [64 C1 w, 64 C1 (w + 1)) and keeps its own top-K
// (same order: larger score, then lower block id); the row's top-K lies in
// the union of those, which one wave then selects from.  The survivors are
// laid out by wave and then ascending id, so candidate order is block order
// and the second selection breaks ties by block id too.
constexpr int kWideWaves = 16;

struct WideLds {
  uint32_t ckey[kWideWaves * kMaxTopk];
  int32_t cblk[kWideWaves * kMaxTopk];
  int32_t ccount[kWideWaves];
};

// The two-stage selection of one row over blocks t < T whose keys key_of(t)
// returns (0: not a candidate), written to q2k rows g_lo .. g_hi - 1 of
// query i.  All 16 waves call it.
template <int C1, int C2, class KeyOf>
__device__ __forceinline__ void wide_select(WideLds& w, KeyOf key_of, int T, int total_q,
                                            int topk, int i, int g_lo, int g_hi,
                                            int32_t* __restrict__ q2k) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  // stage 1: this wave's candidates
  const int t0 = 64 * C1 * wave;
  uint32_t key[C1];
  bool valid[C1];
#pragma unroll
  for (int c = 0; c < C1; ++c) {
    const int t = t0 + lane + kWave * c;
    key[c] = t < T ? key_of(t) : 0u;
    valid[c] = key[c] != 0u;
  }
  bool chosen[C1];
  select_topk<C1>(key, valid, topk, lane, chosen);
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int base = 0;
#pragma unroll
  for (int c = 0; c < C1; ++c) {
    const unsigned long long m = __ballot(chosen[c]);
    if (chosen[c]) {
      const int pos = wave * topk + base + popc64(m & below);
      w.ckey[pos] = key[c];
      w.cblk[pos] = t0 + lane + kWave * c;
    }
    base += popc64(m);
  }
  if (lane == 0) w.ccount[wave] = base;
  __syncthreads();
  if (wave != 0) return;

  // stage 2: the survivors, candidate e = lane + 64 c (wave e / topk, rank e % topk)
  uint32_t key2[C2];
  bool valid2[C2];
  int blk2[C2];
#pragma unroll
  for (int c = 0; c < C2; ++c) {
    const int e = lane + kWave * c;
    const int ww = e / topk, r = e % topk;
    valid2[c] = ww < kWideWaves && r < w.ccount[ww];
    key2[c] = valid2[c] ? w.ckey[e] : 0u;
    blk2[c] = valid2[c] ? w.cblk[e] : -1;
  }
  bool chosen2[C2];
  select_topk<C2>(key2, valid2, topk, lane, chosen2);
  base = 0;
#pragma unroll
  for (int c = 0; c < C2; ++c) {
    const unsigned long long m = __ballot(chosen2[c]);
    if (chosen2[c]) {
      const int pos = base + popc64(m & below);
      for (int g = g_lo; g < g_hi; ++g) q2k[((int64_t)g * total_q + i) * topk + pos] = blk2[c];
    }
    base += popc64(m);
  }
  for (int pos = base + lane; pos < topk; pos += kWave)
    for (int g = g_lo; g < g_hi; ++g) q2k[((int64_t)g * total_q + i) * topk + pos] = -1;
}

// finite scores only: -inf, +inf and NaN are never selected
__device__ __forceinline__ uint32_t select_key(float s) {
  return (__float_as_uint(s) & 0x7F800000u) != 0x7F800000u ? ordered_f32(s) : 0u;
}

template <int C1, int C2>
__global__ __launch_bounds__(kWideWaves * 64) void msa_topk_wide_kernel(
    const float* __restrict__ scores, int hs, int T, int total_q, int topk, int hkv, int mode,
    int sel_rows, int n_wg, int32_t* __restrict__ q2k) {
  __shared__ WideLds w;
  const int row = xcd_remap(blockIdx.x, n_wg);
  if (row < 0 || row >= sel_rows * total_q) return;
  const int i = row % total_q;
  const int gs = row / total_q;
  int h_lo, h_hi;
  if (mode == 1) {
    h_lo = 0; h_hi = hs;
  } else if (mode == 2) {
    const int gsz = hs / hkv;
    h_lo = gs * gsz; h_hi = h_lo + gsz;
  } else {
    h_lo = gs; h_hi = gs + 1;
  }
  // finite scores only (ordered keys of finite values are never 0)
  auto key_of = [&](int t) {
    float s = scores[((int64_t)h_lo * T + t) * total_q + i];
    for (int h = h_lo + 1; h < h_hi; ++h) s = fmaxf(s, scores[((int64_t)h * T + t) * total_q + i]);
    return select_key(s);
  };
  wide_select<C1, C2>(w, key_of, T, total_q, topk, i, mode == 1 ? 0 : gs,
                      mode == 1 ? hkv : gs + 1, q2k);
}

// Merge of per-chunk candidates (the proxy's running top-K): for one
// selection row and query, the (score, id) candidates of every chunk (and,
// for a selection shared by all KV heads, of every KV head's head-group
// maximum) are folded into a dense LDS row by id, keeping each id's largest
// score, and the row's top-K is selected from it.  Exact: a block of the
// true top-K is in the chunk top-K of the KV head that attains its maximum,
// with that maximum as its score; any other id's folded score is at most
// its true score, which cannot move it ahead of a true member.
template <int C1, int C2>
__global__ __launch_bounds__(kWideWaves * 64) void msa_topk_merge_kernel(
    const float* __restrict__ cand_s, const int32_t* __restrict__ cand_id, int n_cand, int T,
    int total_q, int topk, int hkv, int shared, int sel_rows, int n_wg,
    int32_t* __restrict__ q2k) {
  extern __shared__ uint32_t dense[];   // T keys
  __shared__ WideLds w;
  const int row = xcd_remap(blockIdx.x, n_wg);
  if (row < 0 || row >= sel_rows * total_q) return;
  const int i = row % total_q;
  const int gs = row / total_q;
  for (int t = threadIdx.x; t < T; t += kWideWaves * 64) dense[t] = 0u;
  __syncthreads();
  const int64_t base = (int64_t)row * n_cand;
  for (int e = threadIdx.x; e < n_cand; e += kWideWaves * 64) {
    const int id = cand_id[base + e];
    const uint32_t k = select_key(cand_s[base + e]);
    if (id >= 0 && id < T && k != 0u) atomicMax(&dense[id], k);
  }
  __syncthreads();
  auto key_of = [&](int t) { return dense[t]; };
  wide_select<C1, C2>(w, key_of, T, total_q, topk, i, shared ? 0 : gs, shared ? hkv : gs + 1,
                      q2k);
}

template <int C>
static hipError_t launch_topk_c(const float* scores, int hs, int T, int total_q, int topk,
                                int hkv, int mode, int32_t* q2k, hipStream_t stream) {
  const int sel_rows = (mode == 1) ? 1 : hkv;
  const int64_t waves = (int64_t)sel_rows * total_q;
  if (waves <= 0) return hipSuccess;
  const int n_wg = (int)((waves + 3) / 4);
  hipLaunchKernelGGL((msa_topk_kernel<C>), dim3(8 * ((n_wg + 7) / 8)), dim3(256), 0, stream,
                     scores, hs, T, total_q, topk, hkv, mode, sel_rows, n_wg, q2k);
  return hipGetLastError();
}

template <int C1, int C2>
static hipError_t launch_topk_wide(const float* scores, int hs, int T, int total_q, int topk,
                                   int hkv, int mode, int32_t* q2k, hipStream_t stream) {
  const int sel_rows = (mode == 1) ? 1 : hkv;
  const int n = sel_rows * total_q;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL((msa_topk_wide_kernel<C1, C2>), dim3(8 * ((n + 7) / 8)),
                     dim3(kWideWaves * 64), 0, stream, scores, hs, T, total_q, topk, hkv, mode,
                     sel_rows, n, q2k);
  return hipGetLastError();
}

template <int C1>
static hipError_t launch_topk_wide_c2(const float* scores, int hs, int T, int total_q, int topk,
                                      int hkv, int mode, int32_t* q2k, hipStream_t stream) {
  // survivors: kWideWaves * topk candidates, 64 per lane column
  if (topk <= 16) return launch_topk_wide<C1, 4>(scores, hs, T, total_q, topk, hkv, mode, q2k, stream);
  if (topk <= 32) return launch_topk_wide<C1, 8>(scores, hs, T, total_q, topk, hkv, mode, q2k, stream);
  return launch_topk_wide<C1, 16>(scores, hs, T, total_q, topk, hkv, mode, q2k, stream);
}

template <int C1, int C2>
static hipError_t launch_merge_t(const float* cs, const int32_t* ci, int n_cand, int T,
                                 int total_q, int topk, int hkv, int shared, int32_t* q2k,
                                 hipStream_t stream) {
  const int sel_rows = shared ? 1 : hkv;
  const int n = sel_rows * total_q;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL((msa_topk_merge_kernel<C1, C2>), dim3(8 * ((n + 7) / 8)),
                     dim3(kWideWaves * 64), (size_t)T * 4, stream, cs, ci, n_cand, T, total_q,
                     topk, hkv, shared, sel_rows, n, q2k);
  return hipGetLastError();
}

template <int C1>
static hipError_t launch_merge_c2(const float* cs, const int32_t* ci, int n_cand, int T,
                                  int total_q, int topk, int hkv, int shared, int32_t* q2k,
                                  hipStream_t stream) {
  if (topk <= 16) return launch_merge_t<C1, 4>(cs, ci, n_cand, T, total_q, topk, hkv, shared, q2k, stream);
  if (topk <= 32) return launch_merge_t<C1, 8>(cs, ci, n_cand, T, total_q, topk, hkv, shared, q2k, stream);
  return launch_merge_t<C1, 16>(cs, ci, n_cand, T, total_q, topk, hkv, shared, q2k, stream);
}

hipError_t launch_topk_merge(const float* cand_s, const int32_t* cand_id, int n_cand, int T,
                             int total_q, int topk, int hkv, int shared, int32_t* q2k,
                             hipStream_t stream) {
  const int c1 = (T + 64 * kWideWaves - 1) / (64 * kWideWaves);
  if (c1 <= 1) return launch_merge_c2<1>(cand_s, cand_id, n_cand, T, total_q, topk, hkv, shared, q2k, stream);
  if (c1 <= 2) return launch_merge_c2<2>(cand_s, cand_id, n_cand, T, total_q, topk, hkv, shared, q2k, stream);
  if (c1 <= 4) return launch_merge_c2<4>(cand_s, cand_id, n_cand, T, total_q, topk, hkv, shared, q2k, stream);
  if (c1 <= 8) return launch_merge_c2<8>(cand_s, cand_id, n_cand, T, total_q, topk, hkv, shared, q2k, stream);
  return launch_merge_c2<16>(cand_s, cand_id, n_cand, T, total_q, topk, hkv, shared, q2k, stream);
}

hipError_t launch_topk(const float* scores, int score_heads, int T, int total_q, int topk,
                       int hkv, int mode, int32_t* q2k, hipStream_t stream) {
  const int c = (T + kWave - 1) / kWave;
  if (c > 4) {
    // per wave: ceil(T / 1024) candidates per lane
    const int c1 = (T + 64 * kWideWaves - 1) / (64 * kWideWaves);
    if (c1 <= 1) return launch_topk_wide_c2<1>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
    if (c1 <= 2) return launch_topk_wide_c2<2>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
    if (c1 <= 4) return launch_topk_wide_c2<4>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
    if (c1 <= 8) return launch_topk_wide_c2<8>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
    if (c1 <= 16) return launch_topk_wide_c2<16>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
  }
  if (c <= 1) return launch_topk_c<1>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
  if (c <= 2) return launch_topk_c<2>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
  if (c <= 4) return launch_topk_c<4>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
  if (c <= 8) return launch_topk_c<8>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
  if (c <= 16) return launch_topk_c<16>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
  if (c <= 32) return launch_topk_c<32>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
  return launch_topk_c<64>(scores, score_heads, T, total_q, topk, hkv, mode, q2k, stream);
}

}  // namespace msa
