// Packed query sparse attention over caller-listed tokens (qsa page: the
// indexed and bitmap APIs; outputs BF16 and FP32 [T, Hq, 256] and the natural-log LSE
// [Hq, T]; an empty selection gives zero output and -inf LSE).
//
// gfx950 design, one wave per (query token, KV head):
//  * The token's G <= 16 query heads of the KV head fill one 16-row tile of
//    v_mfma_f32_16x16x32_bf16.  Its index row is consumed 32 entries at a
//    time (eight 4-token groups); entries < 0 are padding and are masked.
//  * K is gathered straight into MFMA operand registers: k-step s of
//    S^T = K Q^T gives lane (key l % 16, quarter q = l / 16) head dims
//    32 s + 8 q .. + 7 of its key row, so the four lanes of a key read 64
//    contiguous bytes per load (16 cache-line segments per wave load, not
//    64); the query fragments use the same permutation of the head
//    dimension, so the dot products are unchanged.
//  * V rows are gathered into LDS with global_load_lds (no register
//    staging) and read back transposed with ds_read_b64_tr_b16, which hands
//    O^T += V^T P^T its A operand; P comes from the S^T registers in the key
//    order they hold (keys 4 q .. 4 q + 3 and 16 + 4 q .. 16 + 4 q + 3).
//  * Online softmax in log2 units with a per-chunk row max; the row's 32
//    scores of a chunk sit in four lanes (l % 16 + 16 q).
// Every (token, head) is computed by one wave in index order: the result is
// bitwise repeatable.
#include "async_lds.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace msa {

namespace {

constexpr int kQsaDim = 256;
constexpr int kQsaRowBytes = kQsaDim * 2;   // one bf16 K or V row of one head
constexpr float kQsaLn2 = 0.69314718055994530942f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 lds_tr16(uint32_t a) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (__attribute__((address_space(3))) s16x4*)(uintptr_t)a));
}

__device__ __forceinline__ float xmax_16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, kWave));
  return fmaxf(x, __shfl_xor(x, 32, kWave));
}
__device__ __forceinline__ float xsum_16_32(float x) {
  x += __shfl_xor(x, 16, kWave);
  return x + __shfl_xor(x, 32, kWave);
}

struct QsaLds {
  uint8_t v[32 * kQsaRowBytes];   // V rows of the chunk (16 KiB)
  int32_t ids[32];                // the chunk's index entries (-1: padding)
  int32_t blk[8];                 // bitmap source: the chunk's selected blocks
};

}  // namespace

// BITMAP: the keys come from a uint8 [T, num_blocks] block bitmap instead of
// index rows; each chunk takes the next eight selected blocks (32 tokens),
// found with a ballot over 64 bitmap bytes at a time, so no [T, NB] index
// scratch is ever written (qsa page: the bitmap API and its compact-index
// scratch).
template <bool BITMAP>
__global__ __launch_bounds__(64, 2) void msa_qsa_kernel(QsaParams p) {
  __shared__ __attribute__((aligned(16))) QsaLds lds;
  // last tokens first: causal selections grow with the position, so the
  // longest waves start earliest and the short ones fill the tail
  const int tok = p.total_q - 1 - (int)(blockIdx.x / p.hkv);
  const int g = blockIdx.x % p.hkv;
  if (tok < 0) return;
  const int lane = threadIdx.x;
  const int l16 = lane & 15;
  const int q = lane >> 4;
  const int G = p.group;
  const int hrow = g * G + l16;              // this lane's query head (row l16)
  const bool live = l16 < G;

  // query fragments: row l16, head dims 32 s + 8 q .. + 7 for k-step s
  bf16x8 qf[8];
  {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) +
                        ((int64_t)tok * p.hq + (live ? hrow : g * G)) * kQsaRowBytes + 16 * q;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(qp + 64 * s);
      qf[s] = as_bf16x8(live ? w : u32x4{0, 0, 0, 0});
    }
  }

  const int32_t* irow = BITMAP ? nullptr : p.indices + (int64_t)tok * p.width;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k) + (int64_t)g * p.k_head_stride;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v) + (int64_t)g * p.v_head_stride;
  const uint32_t vlds = __builtin_amdgcn_readfirstlane(lds_addr(lds.v));
  const float C = p.scale_log2;

  float m = -INFINITY, l = 0.f;
  f32x4 o[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = BITMAP ? 0 : (p.width + 31) / 32;
  const uint8_t* brow = BITMAP ? p.bitmap + (int64_t)tok * p.num_blocks : nullptr;
  int cursor = 0;   // bitmap: the next block to scan (wave-uniform)
  for (int c = 0;; ++c) {
    if (!BITMAP && c >= nchunks) break;
    // every LDS read of the previous chunk has completed before its
    // buffers are refilled
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if constexpr (BITMAP) {
      int have = 0;
      while (have < 8 && cursor < p.num_blocks) {
        const int b = cursor + lane;
        const bool sel = b < p.num_blocks && brow[b] != 0;
        const unsigned long long sm = __ballot(sel);
        const int cnt = __popcll(sm);
        const int take = min(8 - have, cnt);
        const int rank = __popcll(sm & ((1ull << lane) - 1ull));
        if (sel && rank < take) lds.blk[have + rank] = b;
        if (take < cnt) {
          unsigned long long rest = sm;
          for (int k = 0; k < take; ++k) rest &= rest - 1ull;
          cursor += __builtin_ctzll(rest);   // the first selected block not taken
        } else {
          cursor += 64;
        }
        have += take;
      }
      if (have == 0) break;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (lane < 32) {
        int id = -1;
        if ((lane >> 2) < have) {
          const int t = 4 * lds.blk[lane >> 2] + (lane & 3);
          id = t < p.num_kv_tokens ? t : -1;
        }
        lds.ids[lane] = id;
      }
    } else {
      if (lane < 32) {
        const int e = 32 * c + lane;
        lds.ids[lane] = e < p.width ? irow[e] : -1;
      }
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

    // V rows 2 n and 2 n + 1 per load: lane l fills 16 bytes of row
    // 2 n + l / 32 (padding entries read row 0: finite, and their P is 0)
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const int id = lds.ids[2 * n + (lane >> 5)];
      const uint8_t* src = vbase + (int64_t)(id >= 0 ? id : 0) * p.v_row_stride + 16 * (lane & 31);
      g2lds16(src, vlds + 1024 * n);
    }

    // K operand fragments of the two 16-key tiles
    u32x4 kw[2][8];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int id = lds.ids[16 * kt + l16];
      const uint8_t* kp = kbase + (int64_t)(id >= 0 ? id : 0) * p.k_row_stride + 16 * q;
#pragma unroll
      for (int s = 0; s < 8; ++s) kw[kt][s] = *reinterpret_cast<const u32x4*>(kp + 64 * s);
    }
    // validity of the eight keys whose scores this lane holds
    const int4 va = *reinterpret_cast<const int4*>(&lds.ids[4 * q]);
    const int4 vb = *reinterpret_cast<const int4*>(&lds.ids[16 + 4 * q]);

    f32x4 acc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 8; ++s) acc[kt] = mfma16(as_bf16x8(kw[kt][s]), qf[s], acc[kt]);
    }
    const int vid[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
    float sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = acc[j >> 2][j & 3] * C;
      sc[j] = vid[j] >= 0 ? x : -INFINITY;
    }
    float cm = sc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) cm = fmaxf(cm, sc[j]);
    cm = xmax_16_32(cm);
    const float mn = fmaxf(m, cm);
    const float mu = mn == -INFINITY ? 0.f : mn;   // no visible key yet: p = 0 below
    const float alpha = __builtin_amdgcn_exp2f(m - mu);
    float e[8], ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      e[j] = __builtin_amdgcn_exp2f(sc[j] - mu);
      ps += e[j];
    }
    l = l * alpha + ps;
    m = mn;
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) o[dt] *= alpha;
    const bf16x8 pf = as_bf16x8(u32x4{cvt_pk_bf16(e[0], e[1]), cvt_pk_bf16(e[2], e[3]),
                                      cvt_pk_bf16(e[4], e[5]), cvt_pk_bf16(e[6], e[7])});

    // V^T fragments: head dims 16 dt + l % 16; lane 4 e + a of a 16-lane
    // group addresses row 4 q + e (and + 16), columns 4 a .. 4 a + 3
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const int vrow = 4 * q + (l16 >> 2);
    const uint32_t va0 = vlds + vrow * kQsaRowBytes + 8 * (l16 & 3);
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      const u32x2 lo = lds_tr16(va0 + 32 * dt);
      const u32x2 hi = lds_tr16(va0 + 32 * dt + 16 * kQsaRowBytes);
      o[dt] = mfma16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pf, o[dt]);
    }
  }

  // epilogue: lane (row l16, quarter q) holds O^T[16 dt + 4 q + i][row]
  const float lsum = xsum_16_32(l);
  if (!live) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const int64_t orow = ((int64_t)tok * p.hq + hrow) * kQsaDim + 4 * q;
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) {
    const f32x4 r = o[dt] * inv;
    *reinterpret_cast<u32x2*>(p.out + orow + 16 * dt) =
        u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
    if (p.out_f32) *reinterpret_cast<f32x4*>(p.out_f32 + orow + 16 * dt) = r;
  }
  if (p.lse && q == 0)
    p.lse[(int64_t)hrow * p.total_q + tok] = lsum > 0.f ? (m + __log2f(lsum)) * kQsaLn2 : -INFINITY;
}

hipError_t launch_qsa(const QsaParams& p, hipStream_t stream) {
  const int64_t n = (int64_t)p.total_q * p.hkv;
  if (n <= 0) return hipSuccess;
  if (p.bitmap)
    hipLaunchKernelGGL(msa_qsa_kernel<true>, dim3((unsigned)n), dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL(msa_qsa_kernel<false>, dim3((unsigned)n), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace msa
