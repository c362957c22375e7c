// Export of the per-tile block union (msa_sparse_attention page, summary:
// the union metadata is built internally from q2k_indices), built by the same
// LDS builder the attention kernels use, for inspection and tests.
#include "common.hpp"
#include "internal.hpp"
#include "tile_union.hpp"

namespace msa {

// ---------------------------------------------------------------------------
// Tile union export (same builder as the attention kernel).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void msa_tile_union_kernel(
    const int32_t* __restrict__ q2k, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ len_k, int total_q, int hkv, int topk, int tiles_per_req,
    int max_k_tiles, int tile_tokens, int max_union, int32_t* __restrict__ ublocks,
    unsigned long long* __restrict__ umasks, int32_t* __restrict__ ucount) {
  __shared__ UnionLds un;
  const int tile = blockIdx.x % tiles_per_req;
  const int g = (blockIdx.x / tiles_per_req) % hkv;
  const int b = blockIdx.x / (tiles_per_req * hkv);
  const int q0 = cu_q[b];
  const int lq = cu_q[b + 1] - q0;
  const int i0 = tile * tile_tokens;
  const int64_t out_idx = ((int64_t)g * (gridDim.x / hkv) + (int64_t)b * tiles_per_req + tile);
  int32_t* ob = ublocks + out_idx * max_union;
  unsigned long long* om = umasks + out_idx * max_union;
  int cnt = 0;
  if (i0 < lq) {
    const int ntok = min(tile_tokens, lq - i0);
    const int nblk = max(0, min((len_k[b] + kBlock - 1) / kBlock, max_k_tiles));
    cnt = build_tile_union<256>(un, q2k + ((int64_t)g * total_q + q0 + i0) * topk, ntok, topk, nblk);
    for (int i = threadIdx.x; i < cnt; i += 256) {
      ob[i] = un.list[i];
      om[i] = un.mask[i];
    }
  }
  for (int i = cnt + threadIdx.x; i < max_union; i += 256) {
    ob[i] = -1;
    om[i] = 0ull;
  }
  if (threadIdx.x == 0) ucount[out_idx] = cnt;
}

hipError_t launch_tile_union(const int32_t* q2k, const int32_t* cu_q, const int32_t* len_k,
                             int batch, int total_q, int hkv, int topk, int max_seqlen_q,
                             int max_k_tiles, int tile_tokens, int max_union,
                             int32_t* ublocks, uint64_t* umasks, int32_t* ucount,
                             hipStream_t stream) {
  const int tiles = (max_seqlen_q + tile_tokens - 1) / tile_tokens;
  const int n = batch * hkv * tiles;
  if (n <= 0) return hipSuccess;
  // the kernel indexes outputs as [g][b][tile]; gridDim.x / hkv == batch * tiles
  hipLaunchKernelGGL(msa_tile_union_kernel, dim3(n), dim3(256), 0, stream, q2k, cu_q, len_k,
                     total_q, hkv, topk, tiles, max_k_tiles, tile_tokens, max_union, ublocks,
                     reinterpret_cast<unsigned long long*>(umasks), ucount);
  return hipGetLastError();
}

}  // namespace msa
