// bf16 staging of fp8 / E2M1 K/V for the prefill route (see stage16.hpp).
// Whole mode: one workgroup per (request, block) converts every KV head's 128
// rows of K and V of a visible block (rows past the sequence become zeros)
// and records the identity page id; blocks past the sequence only get the
// page id, so every id the attention kernel could look up is a valid page.
// Selected mode (short queries): one workgroup per (request, slot) finds the
// slot-th block that some query of the request selected (any KV head) and
// converts only that block into the request's slot page; the page table maps
// each selected block to its slot, and blocks no query selected are never
// looked up by the attention kernel.
#include "common.hpp"
#include "stage16.hpp"
#include "tile_union.hpp"

#include <algorithm>

namespace msa {

namespace {

constexpr int64_t kPageRow = 128 * 2;   // bytes of one bf16 row (head dim 128)

struct Stage16Params {
  AttnParams src;
  int fmt;
  uint8_t* kdst;
  uint8_t* vdst;
  int32_t* pt;       // [batch, max_k_tiles]
  int32_t* lens;     // [batch]
  int slots;         // pages per request in the pool (selected mode), else 0
};

__device__ __forceinline__ void put16(uint8_t* dst, const float (&x)[16]) {
  u32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    b[e] = pack_bf16x2(x[8 + 2 * e], x[9 + 2 * e]);
  }
  *reinterpret_cast<u32x4*>(dst) = a;
  *reinterpret_cast<u32x4*>(dst + 16) = b;
}

struct SelectLds {
  uint32_t bitmap[kMaxBitmapWords];
  int32_t prefix[kMaxBitmapWords];
  int32_t count;
  int32_t block;
};

__global__ __launch_bounds__(256) void msa_stage16_kernel(Stage16Params s) {
  const AttnParams& p = s.src;
  const int M = p.max_k_tiles;
  const int per = s.slots ? s.slots : M;
  const int b = blockIdx.x / per;
  if (b >= p.batch) return;
  const int lk = p.paged ? p.seqused_k[b] : (p.cu_k[b + 1] - p.cu_k[b]);
  const int nblk = min(max(0, (lk + kBlock - 1) / kBlock), M);
  int t;
  int64_t page;
  if (!s.slots) {
    t = blockIdx.x % M;
    page = (int64_t)b * M + t;
    if (threadIdx.x == 0) {
      s.pt[page] = (int32_t)page;
      if (t == 0) s.lens[b] = lk;
    }
    if (t >= nblk) return;
  } else {
    // the request's selected blocks (every KV head, every query) as a
    // bitmap, its word prefix counts, and this slot's block
    __shared__ SelectLds sl;
    const int slot = blockIdx.x % per;
    const int tid = threadIdx.x;
    const int words = (nblk + 31) >> 5;
    for (int w = tid; w < words; w += 256) sl.bitmap[w] = 0u;
    if (tid == 0) sl.block = -1;
    __syncthreads();
    const int q0 = p.cu_q[b], lq = p.cu_q[b + 1] - q0;
    const int per_head = lq * p.topk;
    for (int e = tid; e < p.hkv * per_head; e += 256) {
      const int g = e / per_head, r = e % per_head;
      const int id = p.q2k[((int64_t)g * p.total_q + q0) * p.topk + r];
      if (id >= 0 && id < nblk) atomicOr(&sl.bitmap[id >> 5], 1u << (id & 31));
    }
    __syncthreads();
    if (tid < kWave) {
      const int pw = (words + kWave - 1) / kWave;
      int local = 0;
      for (int i = 0; i < pw; ++i)
        if (tid * pw + i < words) local += __popc(sl.bitmap[tid * pw + i]);
      int incl = local;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off, kWave);
        if (tid >= off) incl += o;
      }
      int run = incl - local;
      for (int i = 0; i < pw; ++i) {
        const int w = tid * pw + i;
        if (w < words) {
          sl.prefix[w] = run;
          run += __popc(sl.bitmap[w]);
        }
      }
      if (tid == kWave - 1) sl.count = incl;
    }
    __syncthreads();
    for (int w = tid; w < words; w += 256) {
      uint32_t bits = sl.bitmap[w];
      const int k = slot - sl.prefix[w];
      if (k >= 0 && k < __popc(bits)) {
        for (int i = 0; i < k; ++i) bits &= bits - 1u;
        sl.block = (w << 5) + __ffs(bits) - 1;
      }
    }
    __syncthreads();
    if (slot == 0 && tid == 0) s.lens[b] = lk;
    t = sl.block;
    if (t < 0) return;                       // fewer selected blocks than slots
    page = (int64_t)b * per + slot;
    if (tid == 0) s.pt[(int64_t)b * M + t] = (int32_t)page;
  }
  const int nvalid = min(kBlock, lk - kBlock * t);
  // source block: page of the caller's table, or 128 rows of the flat tensor
  int64_t ko, vo, kso = 0, vso = 0;
  if (p.paged) {
    const int64_t sp = p.page_table[(int64_t)b * p.pt_width + t];
    ko = sp * p.k_st.page;
    vo = sp * p.v_st.page;
    kso = sp * p.ks_st.page;
    vso = sp * p.vs_st.page;
  } else {
    const int64_t r0 = (int64_t)p.cu_k[b] + kBlock * t;
    ko = r0 * p.k_st.token;
    vo = r0 * p.v_st.token;
    kso = r0 * p.ks_st.token;
    vso = r0 * p.vs_st.token;
  }
  // items: (side, head, row, 16-value piece)
  const int per_side = p.hkv * kBlock * 8;
  for (int it = threadIdx.x; it < 2 * per_side; it += 256) {
    const bool isv = it >= per_side;
    const int w = isv ? it - per_side : it;
    const int j = w & 7;
    const int r = (w >> 3) & (kBlock - 1);
    const int g = w >> 10;
    uint8_t* dst = (isv ? s.vdst : s.kdst) + ((page * p.hkv + g) * kBlock + r) * kPageRow + 32 * j;
    float x[16];
    if (r >= nvalid) {
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = 0.f;
    } else if (s.fmt == kFmtFp8) {
      // E4M3 -> bf16 with the hardware conversion (scale 1: exact)
      const uint8_t* src = (isv ? p.v + vo + g * p.v_st.head + r * p.v_st.token
                                : p.k + ko + g * p.k_st.head + r * p.k_st.token) + 16 * j;
      const u32x4 q = *reinterpret_cast<const u32x4*>(src);
      u32x4 a, c;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        a[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[h], 1.0f, false));
        a[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[h], 1.0f, true));
        c[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[2 + h], 1.0f, false));
        c[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[2 + h], 1.0f, true));
      }
      *reinterpret_cast<u32x4*>(dst) = a;
      *reinterpret_cast<u32x4*>(dst + 16) = c;
      continue;
    } else {
      const uint8_t* src = (isv ? p.v + vo + g * p.v_st.head + r * p.v_st.token
                                : p.k + ko + g * p.k_st.head + r * p.k_st.token) + 8 * j;
      const uint8_t* sc = isv ? p.vs + vso + g * p.vs_st.head + r * p.vs_st.token
                              : p.ks + kso + g * p.ks_st.head + r * p.ks_st.token;
      const u32x2 q = *reinterpret_cast<const u32x2*>(src);
      const float f = e4m3_to_f32(sc[j]);
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = e2m1_to_f32((q[e >> 3] >> (4 * (e & 7))) & 0xFu) * f;
    }
    put16(dst, x);
  }
}

}  // namespace

int stage16_slots(int max_seqlen_q, int hkv, int topk, int max_k_tiles) {
  const int64_t sel = (int64_t)std::max(1, max_seqlen_q) * hkv * topk;
  return sel <= kStageSelectMax ? (int)std::min<int64_t>(sel, max_k_tiles) : 0;
}

size_t stage16_bytes(int batch, int max_k_tiles, int hkv, int slots) {
  const size_t pages = (size_t)batch * (slots ? slots : max_k_tiles);
  const size_t pool = pages * hkv * kBlock * kPageRow;
  const size_t table = (size_t)batch * max_k_tiles;
  return 2 * pool + ((table * 4 + 255) / 256) * 256 + (size_t)batch * 4;
}

hipError_t launch_stage16(const AttnParams& p, int fmt, int slots, void* ws, AttnParams* pq,
                          hipStream_t stream) {
  const size_t pages = (size_t)p.batch * (slots ? slots : p.max_k_tiles);
  const size_t pool = pages * p.hkv * kBlock * kPageRow;
  const size_t table = (size_t)p.batch * p.max_k_tiles;
  Stage16Params s;
  s.src = p;
  s.fmt = fmt;
  s.slots = slots;
  s.kdst = static_cast<uint8_t*>(ws);
  s.vdst = s.kdst + pool;
  s.pt = reinterpret_cast<int32_t*>(s.vdst + pool);
  s.lens = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(s.pt) + ((table * 4 + 255) / 256) * 256);
  if (pages > 0) {
    hipLaunchKernelGGL(msa_stage16_kernel, dim3((unsigned)pages), dim3(256), 0, stream, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  *pq = p;
  pq->k = s.kdst;
  pq->v = s.vdst;
  pq->ks = pq->vs = nullptr;
  pq->k_st = Strides{(int64_t)p.hkv * kBlock * kPageRow, kBlock * kPageRow, kPageRow};
  pq->v_st = pq->k_st;
  pq->paged = 1;
  pq->page_table = s.pt;
  pq->pt_width = p.max_k_tiles;
  pq->seqused_k = s.lens;
  pq->cu_k = nullptr;
  return hipSuccess;
}

}  // namespace msa
