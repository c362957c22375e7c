// Device-side check of the caller contracts of the sparse attention call
// (msa_sparse_attention page, Parameters: cu_seqlens_q, cu_seqlens_k,
// q2k_indices, page_table, seqused_k).  Debug path only: the timed path never
// runs it.  Every violation found is folded into one 64-bit word by an
// atomic minimum of (kind << 48 | position), so the report names the first
// kind and, within it, the first position, whatever the thread order.
#include <algorithm>
#include <mutex>

#include "validate.hpp"

namespace msa {

namespace {

__device__ unsigned long long g_violation;

__global__ void msa_validate_reset_kernel() { g_violation = ~0ull; }

__device__ __forceinline__ void report(int kind, int64_t pos) {
  atomicMin(&g_violation, ((unsigned long long)kind << 48) | (unsigned long long)pos);
}

__global__ __launch_bounds__(256) void msa_validate_kernel(ValidateParams p) {
  const int64_t n_cu = (int64_t)p.batch + 1;
  const int64_t n_pt = p.paged ? (int64_t)p.batch * p.pt_width : 0;
  const int64_t n_rows = (int64_t)p.hkv * p.total_q;
  const int64_t n = n_cu + n_pt + n_rows;
  const int64_t kv_cap = 128 * (int64_t)(p.paged ? min(p.max_k_tiles, p.pt_width) : p.max_k_tiles);
  for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < n;
       x += (int64_t)gridDim.x * blockDim.x) {
    if (x < n_cu) {
      const int b = (int)x;
      if (b == 0 && p.cu_q[0] != 0) report(kValCuQ, b);
      if (b == p.batch && p.cu_q[b] != p.total_q) report(kValCuQ, b);
      if (b < p.batch) {
        const int lq = p.cu_q[b + 1] - p.cu_q[b];
        if (lq < 0 || lq > p.max_seqlen_q) report(kValCuQ, b);
        if (!p.paged && p.cu_k[b + 1] < p.cu_k[b]) report(kValCuK, b);
        const int64_t lk = p.paged ? p.seqused[b] : (int64_t)p.cu_k[b + 1] - p.cu_k[b];
        if (lk < 0 || lk > kv_cap) report(kValKvLen, b);
      }
    } else if (x < n_cu + n_pt) {
      const int64_t y = x - n_cu;
      const int b = (int)(y / p.pt_width);
      const int t = (int)(y % p.pt_width);
      const int64_t lk = p.seqused[b];
      if (lk >= 0 && lk <= 128 * (int64_t)p.pt_width && t < (lk + 127) / 128 &&
          p.page_table[y] < 0)
        report(kValPage, y);
    } else {
      const int64_t r = x - n_cu - n_pt;
      const int32_t* row = p.q2k + r * p.topk;
      int prev = -1;
      bool padded = false;
      for (int e = 0; e < p.topk; ++e) {
        const int v = row[e];
        if (v < 0) {
          padded = true;
          continue;
        }
        if (padded) { report(kValQ2kPad, r * p.topk + e); break; }
        if (v <= prev) { report(kValQ2kOrder, r * p.topk + e); break; }
        prev = v;
      }
    }
  }
}

}  // namespace

// The result word is one per process and device: checks are serialised
// (each holds the lock from the reset to the copy back and waits for its
// stream), so concurrent callers on different threads or streams do not
// interleave their reset, minimum and read.
std::mutex g_validate_mu;

hipError_t run_validate(const ValidateParams& p, hipStream_t stream, unsigned long long* word) {
  std::lock_guard<std::mutex> lock(g_validate_mu);
  void* dev = nullptr;
  hipError_t e = hipGetSymbolAddress(&dev, HIP_SYMBOL(g_violation));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(msa_validate_reset_kernel, dim3(1), dim3(1), 0, stream);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t n = (int64_t)p.batch + 1 + (p.paged ? (int64_t)p.batch * p.pt_width : 0) +
                    (int64_t)p.hkv * p.total_q;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(msa_validate_kernel, dim3(blocks), dim3(256), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = hipMemcpyAsync(word, dev, sizeof(*word), hipMemcpyDeviceToHost, stream)) != hipSuccess)
    return e;
  return hipStreamSynchronize(stream);
}

}  // namespace msa
