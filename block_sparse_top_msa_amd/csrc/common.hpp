// Device helpers shared by the MSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kBlock = 128;     // KV block / page size in tokens
constexpr int kHeadDim = 128;   // head dimension
constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// MFMA wrappers.
//
// 16x16x32 bf16: A is 16 x 32 (M x K), B is 32 x 16 (K x N).  Lane l holds
// A row (l % 16) and B column (l % 16), each with 8 consecutive K values
// chosen by the lane group (l / 16).  The D tile is 16 x 16 fp32: lane l
// holds column (l % 16), rows 4 * (l / 16) + r for r = 0..3.  Any permutation
// of K applied identically to A and B leaves D unchanged; the kernels use
// that to feed softmax probabilities straight from D registers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16: lane l holds A row (l % 32) / B column (l % 32) with 8 K
// values chosen by (l / 32).  D: lane l holds column (l % 32), rows
// 8 * (r / 4) + 4 * (l / 32) + (r % 4) for r = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp16 operands of the same shapes (bf16x8 is used as a 16-byte container).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma16_f16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Round-to-nearest-even fp32 pair -> two fp16 (low half first).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// bf16 helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------------------
// In-register dequantisation.
//
// E4M3FN byte s.eeee.mmm has value 2^(e-7) * 1.mmm (normal) or
// 2^-6 * 0.mmm (e = 0).  Placing the 7 magnitude bits at bits 26..20 of an
// fp32 word gives 2^(e-127) * 1.mmm (or the fp32 subnormal 2^-126 * 0.mmm),
// i.e. exactly the value times 2^-120, so one multiply by 2^120 restores it
// with no rounding.  The NaN codes s.1111.111 decode to NaN, as the
// hardware conversion does.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  uint32_t bits = ((byte & 0x80u) << 24) | ((byte & 0x7Fu) << 20);
  return (byte & 0x7Fu) == 0x7Fu ? __uint_as_float(0x7FC00000u) : __uint_as_float(bits) * 0x1p120f;
}

// E2M1 nibble s.ee.m -> value: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
// The 3 magnitude bits placed at fp32 bits 24..22 give 2^(e-127) * 1.m for
// e >= 1, so multiplying by 2^126 yields 2^(e-1) * 1.m; e = 0 gives the fp32
// subnormal 2^-126 * 0.m -> 0.m/1 * 2^0 ... times 2^126 = 0.5 * m.  Exact.
__device__ __forceinline__ float e2m1_to_f32(uint32_t nib) {
  uint32_t bits = ((nib & 0x8u) << 28) | ((nib & 0x7u) << 22);
  return __uint_as_float(bits) * 0x1p126f;
}

// ---------------------------------------------------------------------------
// Wave reductions (within groups of lanes sharing a query column).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, kWave));
}
__device__ __forceinline__ float xor_sum(float v, int mask) {
  return v + __shfl_xor(v, mask, kWave);
}

// Order-preserving map of fp32 to uint32 (-0 canonicalised to +0), so that
// unsigned comparison matches IEEE comparison on non-NaN values.
__device__ __forceinline__ uint32_t ordered_f32(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exact atomic max of fp32 values in global memory (order-independent).
__device__ __forceinline__ void atomic_max_f32(float* addr, float v) {
  if (__float_as_uint(v) == 0x80000000u) v = 0.0f;
  if (!(v < 0.0f)) {
    atomicMax(reinterpret_cast<int*>(addr), __float_as_int(v));
  } else {
    atomicMin(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
  }
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// KV position of local query iq (query row i) of a request with lq queries
// and lk keys, for the causal mask: right-aligned (mode 0), base + iq (1),
// or the caller's per-row position (2).
__device__ __forceinline__ int query_pos(const int32_t* rows, int mode, int base, int i, int iq,
                                         int lq, int lk) {
  return mode == 2 ? rows[i] : (mode == 1 ? base + iq : lk - lq + iq);
}

// Workgroups are handed to the 8 XCDs round-robin by id.  Remapping so that
// consecutive logical ids share an XCD keeps a (request, KV head)'s K/V in
// one L2.  `n` logical ids; returns -1 for the padding ids of the last round.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  constexpr int kXcd = 8;
  int per = (n + kXcd - 1) / kXcd;
  int l = (bid % kXcd) * per + bid / kXcd;
  return l < n ? l : -1;
}

}  // namespace msa
