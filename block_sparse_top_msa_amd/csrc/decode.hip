// MSA sparse attention, decode shape: few query rows per (request, KV head)
// (seqlen_q x G <= 64), K/V read from a paged (or flat) cache, bf16, fp8
// E4M3 or packed E2M1 with E4M3 block scales (prepare_msa_nvfp4_sparse_decode
// page, summary and Parameters: q, k, v, k_scale, v_scale, page_table,
// seqused_k; msa_sparse_attention page, Parameters: k, k_scale,
// k_global_scale, v_global_scale).
//
// gfx950 design (HBM-bound: every selected page is read once):
//  * One workgroup of 4 waves per (request, KV head, split).  The union of
//    the request's tokens' selected pages is built in LDS; a split takes a
//    contiguous share of it.  Page ids for the share are looked up once.
//  * Pages stream global -> LDS with global_load_lds (16 B per lane, no
//    register staging) through a ring of NST stages, raw bytes as stored.
//    Every wave issues the same number of 1 KiB loads per page, so waiting
//    for a page is one vmcnt immediate.  Rows past the sequence end are
//    filled from the page's row 0 (finite; those keys are masked).
//  * Wave w owns keys 32w..32w+31 of every page.  K fragments are read from
//    LDS and dequantised in registers (fp8: cvt_scalef32_pk_bf16_fp8; E2M1:
//    nibbles -> f32 -> x block scale -> bf16); V^T fragments come from the
//    transposing LDS reads (ds_read_b64_tr_b16 / _b8 / _b4) on row-major V,
//    E2M1 codes scaled per key.  S^T = K Q^T and O^T += V^T P^T on
//    v_mfma_f32_16x16x32_bf16, 16-row tiles (one tile per token at G = 16).
//  * The four waves' softmax states are merged through LDS at the end.  With
//    one split the output is written directly; otherwise each split writes
//    an fp32 partial (O / l and its LSE) and counts its arrival on the unit's
//    counter; the last split to arrive merges them by LSE and resets the
//    counter (prepare_msa_nvfp4_sparse_decode page, Parameters:
//    workspace_buffer).  The partials are written and read only as
//    device-scope atomic accesses, which stay coherent across the XCDs' L2s
//    without an L2 writeback or invalidate, and every writer waits for its
//    stores to complete before it counts; a device-scope fence instead (an
//    L2 writeback and invalidate on this chip) measured slower than the
//    separate merge launch it replaces.
#include "async_lds.hpp"
#include "common.hpp"
#include "internal.hpp"
#include "tile_union.hpp"

namespace msa {

// Lazy softmax rescale (log2 units): the reference max of a row moves only
// when a score passes it by more than 64; a lane's 8 exponentials of a page
// then stay below 8 * 2^64.
constexpr float kDecRescaleSlack = 64.0f;
constexpr float kDecSumLimit = 0x1p67f;

// fp16 P holds at most 65504: the slack drops to 15, and a lane's eight
// exponentials must sum to at most 2^15, so that no single p can pass 2^15
// unnoticed (for bf16 any p below the 2^67 sum limit is representable).
template <int FMT>
struct DecSoft {
  static constexpr float kSlack = FMT == kFmtF16 ? 15.0f : kDecRescaleSlack;
  static constexpr float kLimit = FMT == kFmtF16 ? 0x1p15f : kDecSumLimit;
};

template <int FMT>
__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
  if constexpr (FMT == kFmtF16) return mfma16_f16(a, b, c);
  else return mfma16(a, b, c);
}
template <int FMT>
__device__ __forceinline__ uint32_t pk_p(float lo, float hi) {
  if constexpr (FMT == kFmtF16) return pack_f16x2(lo, hi);
  else return cvt_pk_bf16(lo, hi);
}
template <int FMT>
__device__ __forceinline__ uint32_t pk_out(float lo, float hi) {
  if constexpr (FMT == kFmtF16) return pack_f16x2(lo, hi);
  else return pack_bf16x2(lo, hi);
}

namespace {

constexpr float kLn2d = 0.69314718055994530942f;

// Device-scope relaxed float store / load (the split partials): coherent
// across the XCDs' L2s without a fence.
typedef float f32x2_dev __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_dev(float* a, float v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* a) {
  return __hip_atomic_load(const_cast<float*>(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// four floats at a 16-byte aligned address, stored with the device-scope
// coherence bit (sc1) that the 32- and 64-bit device-scope atomic stores
// carry, as one 16-byte write
__device__ __forceinline__ void st_dev4(float* a, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ f32x2_dev ld_dev2(const float* a) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(a)),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return f32x2_dev{__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32))};
}
constexpr int kPtCache = 1024;   // page-table entries read ahead into LDS

// Per-wave staging geometry: wave w stages (and alone reads) key rows
// 32w..32w+31 of K and V of every page, so waves pipeline independently.
template <int FMT>
struct DecGeom;

template <>
struct DecGeom<kFmtBf16> {
  static constexpr int kRow = 256;                 // bytes per K / V row
  static constexpr int kSide = 32 * kRow;          // 8 KiB per wave and side
  static constexpr int kStage = 2 * kSide;         // K | V
  static constexpr int kStages = 2;                // pages in flight per wave
  static constexpr int kLoads = kStage / 1024;     // 1 KiB loads per wave per page
};

template <>
struct DecGeom<kFmtF16> : DecGeom<kFmtBf16> {};   // 16-bit rows, same staging

template <>
struct DecGeom<kFmtFp8> {
  static constexpr int kRow = 128;
  static constexpr int kSide = 32 * kRow;          // 4 KiB
  static constexpr int kStage = 2 * kSide;
  static constexpr int kStages = 3;
  static constexpr int kLoads = kStage / 1024;
};

template <>
struct DecGeom<kFmtE2m1> {
  static constexpr int kRow = 64;                  // 128 nibbles
  static constexpr int kSide = 32 * kRow;          // 2 KiB
  static constexpr int kScale = 32 * 8;            // 256 B of E4M3 scales per side
  // K | V | K scales | V scales | 512 B target of the scale load's idle lanes
  static constexpr int kStage = 2 * kSide + 2 * kScale + 512;
  static constexpr int kStages = 3;
  static constexpr int kLoads = kStage / 1024;     // 5
};

template <int FMT, int NWV>
struct DecodeLds {
  static constexpr int kRing = NWV * DecGeom<FMT>::kStages * DecGeom<FMT>::kStage;
  uint8_t ring[kRing];       // [wave][stage][K | V | (scales)]
  UnionLds un;
  int32_t page[kMaxUnion];   // page id (paged) or first row (flat) of each entry of the share
  int32_t ptrow[kPtCache];   // the request's page-table row, when it is this short
};

// Rows padded by 16 bytes: the 16 rows one wave writes at the same column
// then fall on distinct banks.
constexpr int kMergePitch = kHeadDim + 4;

template <int NWV>
struct MergeLds {
  float o[NWV][16][kMergePitch];
  float m[NWV][16];
  float l[NWV][16];
  float lt[NWV][16];   // temperature sums
};

__device__ __forceinline__ float xsum16_32(float x) {
  x += __shfl_xor(x, 16, kWave);
  return x + __shfl_xor(x, 32, kWave);
}
__device__ __forceinline__ float xmax16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, kWave));
  return fmaxf(x, __shfl_xor(x, 32, kWave));
}

// ---- LDS fragment reads (asm, so that in-flight LDS-DMA writes of other
// stages do not make the compiler wait for every outstanding load).
__device__ __forceinline__ void lds_b128x4(u32x4 (&k)[4], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}

__device__ __forceinline__ void lds_b128x2_u16x2(u32x4 (&k)[2], uint32_t (&s)[2],
                                                 const uint32_t (&a)[2], const uint32_t (&as)[2]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_u16 %2, %6\n\t"
      "ds_read_u16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(s[0]), "=&v"(s[1])
      : "v"(a[0]), "v"(a[1]), "v"(as[0]), "v"(as[1]));
}

// bf16 V^T: for head-dim tile dt, reads at a[dt] (keys 4q..4q+3) and
// a[dt] + 4096 (keys 16 + 4q..): lane j of a 16-lane group receives element
// j % 4 of the 8 bytes at lane 4e + j / 4's address for e = 0..3.
__device__ __forceinline__ void vtr16_issue(u32x2 (&v)[16], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %2, %17\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:4096\n\t"
      "ds_read_b64_tr_b16 %4, %18\n\t"
      "ds_read_b64_tr_b16 %5, %18 offset:4096\n\t"
      "ds_read_b64_tr_b16 %6, %19\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:4096\n\t"
      "ds_read_b64_tr_b16 %8, %20\n\t"
      "ds_read_b64_tr_b16 %9, %20 offset:4096\n\t"
      "ds_read_b64_tr_b16 %10, %21\n\t"
      "ds_read_b64_tr_b16 %11, %21 offset:4096\n\t"
      "ds_read_b64_tr_b16 %12, %22\n\t"
      "ds_read_b64_tr_b16 %13, %22 offset:4096\n\t"
      "ds_read_b64_tr_b16 %14, %23\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:4096"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
        "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]),
        "=&v"(v[13]), "=&v"(v[14]), "=&v"(v[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
}
__device__ __forceinline__ void wait16(u32x2 (&v)[16]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                 "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]),
                 "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15]));
}

// fp8 V^T (ds_read_b64_tr_b8): lane j of a 16-lane group receives byte
// j % 8 of the 8 bytes at lane 2e + j / 8's address for e = 0..7.
// E2M1 V^T (ds_read_b64_tr_b4): lane j receives nibble j of the 8 bytes at
// lane e's address, for e = 0..15 (nibble e of the result).
template <bool B4>
__device__ __forceinline__ void vtr8_issue(u32x2 (&v)[8], const uint32_t (&a)[8]) {
  if constexpr (B4) {
    asm volatile(
        "ds_read_b64_tr_b4 %0, %8\n\t"
        "ds_read_b64_tr_b4 %1, %9\n\t"
        "ds_read_b64_tr_b4 %2, %10\n\t"
        "ds_read_b64_tr_b4 %3, %11\n\t"
        "ds_read_b64_tr_b4 %4, %12\n\t"
        "ds_read_b64_tr_b4 %5, %13\n\t"
        "ds_read_b64_tr_b4 %6, %14\n\t"
        "ds_read_b64_tr_b4 %7, %15"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
          "=&v"(v[6]), "=&v"(v[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
  } else {
    asm volatile(
        "ds_read_b64_tr_b8 %0, %8\n\t"
        "ds_read_b64_tr_b8 %1, %9\n\t"
        "ds_read_b64_tr_b8 %2, %10\n\t"
        "ds_read_b64_tr_b8 %3, %11\n\t"
        "ds_read_b64_tr_b8 %4, %12\n\t"
        "ds_read_b64_tr_b8 %5, %13\n\t"
        "ds_read_b64_tr_b8 %6, %14\n\t"
        "ds_read_b64_tr_b8 %7, %15"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
          "=&v"(v[6]), "=&v"(v[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
  }
}
__device__ __forceinline__ void wait8(u32x2 (&v)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                 "+v"(v[6]), "+v"(v[7]));
}

// The eight E4M3 V-scale rows (8 bytes each) of this lane's keys.
__device__ __forceinline__ void lds_b64x8(u32x2 (&v)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64 %0, %8\n\t"
      "ds_read_b64 %1, %9\n\t"
      "ds_read_b64 %2, %10\n\t"
      "ds_read_b64 %3, %11\n\t"
      "ds_read_b64 %4, %12\n\t"
      "ds_read_b64 %5, %13\n\t"
      "ds_read_b64 %6, %14\n\t"
      "ds_read_b64 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
}

// ---- in-register dequantisation (exact: E4M3 and E2M1 values and their
// products with E4M3 scales fit bf16 / fp32 without rounding, except a
// product of two E4M3-range numbers, rounded once to bf16)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// 8 fp8 E4M3 bytes (two dwords) -> 8 bf16
__device__ __forceinline__ u32x4 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  return u32x4{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))};
}

// 8 E2M1 nibbles (one dword, low nibble = even element) x scale -> 8 bf16
__device__ __forceinline__ u32x4 e2m1x8_scaled(uint32_t w, float s) {
  u32x4 r;
  f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  r[0] = cvt_pk_bf16(a[0] * s, a[1] * s);
  a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  r[1] = cvt_pk_bf16(a[0] * s, a[1] * s);
  a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  r[2] = cvt_pk_bf16(a[0] * s, a[1] * s);
  a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  r[3] = cvt_pk_bf16(a[0] * s, a[1] * s);
  return r;
}

// 8 E2M1 nibbles of 8 different keys x each key's scale -> 8 bf16
__device__ __forceinline__ u32x4 e2m1x8_keyscaled(uint32_t w, const float (&s)[8]) {
  u32x4 r;
  f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  r[0] = cvt_pk_bf16(a[0] * s[0], a[1] * s[1]);
  a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  r[1] = cvt_pk_bf16(a[0] * s[2], a[1] * s[3]);
  a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  r[2] = cvt_pk_bf16(a[0] * s[4], a[1] * s[5]);
  a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  r[3] = cvt_pk_bf16(a[0] * s[6], a[1] * s[7]);
  return r;
}

// byte `sel` (0..3) of each of four dwords packed into one dword
__device__ __forceinline__ uint32_t gather_byte(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                                int sel) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u + 0x0101u * (uint32_t)sel);
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x04000c0cu + 0x01010000u * (uint32_t)sel);
  return ab | cd;
}

}  // namespace

// TEMP: also accumulate the temperature LSE, sum 2^(tau (x - m)) beside the
// row sum against the same reference max, whose slack shrinks to 64 / tau
// for tau > 1 so that no term passes 2^64.
template <int FMT, int RT, int NWV, bool TEMP>
__global__ __launch_bounds__(NWV * 64) void msa_decode_kernel(AttnParams p) {
  using Geo = DecGeom<FMT>;
  constexpr int NST = Geo::kStages;
  constexpr int LOADS = Geo::kLoads;
  constexpr int NT = NWV * 64;
  static_assert(NWV == 4 || NWV == 8, "4 waves, or 8 taking alternate pages");
  static_assert(sizeof(MergeLds<NWV>) <= DecodeLds<FMT, NWV>::kRing, "merge buffer inside the ring");
  __shared__ __attribute__((aligned(16))) DecodeLds<FMT, NWV> lds;
  __shared__ int s_last;   // this workgroup merges the unit's splits

  // Consecutive logical workgroups (the splits and token tiles of one
  // request and KV head) run on one XCD, so the pages their selections share
  // are fetched into that XCD's L2 once.
  const int lid = xcd_remap(blockIdx.x, p.batch * p.hkv * p.tiles_per_req * p.splits);
  if (lid < 0) return;
  const int split = lid % p.splits;
  const int unit = lid / p.splits;           // (request, KV head, token tile)
  const int jt = unit % p.tiles_per_req;
  const int g = (unit / p.tiles_per_req) % p.hkv;
  const int b = unit / p.tiles_per_req / p.hkv;
  if (b >= p.batch) return;
  const int G = p.group;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int l16 = lane & 15;
  const int q = lane >> 4;

  // ---- prologue.  Every global read it needs starts at once, so that the
  // pages' loads wait on one memory round trip: the query rows and the q2k
  // entries are read where request b starts if every request has the same
  // length (b * tiles_per_req * tok_per_tile, the decode layout), the
  // page-table row up to its width, and the lengths beside them.  A tile
  // elsewhere or shorter reads its rows again once its start is known.
  const int ntok_s = p.tok_per_tile;
  const int q0s = (b * p.tiles_per_req + jt) * ntok_s;
  // Per row tile: lane l holds query row 16 rt + l % 16 (token r / G, head r % G).
  bf16x8 qf[RT][4];
  auto load_q = [&](int qs, int rows_n) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int r = 16 * rt + l16;
      const int tk = r / G;
      if (r < rows_n && qs + tk < p.total_q) {
        const uint8_t* qp = reinterpret_cast<const uint8_t*>(
            p.q + ((int64_t)(qs + tk) * p.hq + g * G + r % G) * kHeadDim) + 64 * q;
#pragma unroll
        for (int ds = 0; ds < 4; ++ds)
          qf[rt][ds] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * ds));
      } else {
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) qf[rt][ds] = as_bf16x8(u32x4{0, 0, 0, 0});
      }
    }
  };
  load_q(q0s, ntok_s * G);
  // q2k entry `tid` of the speculated rows
  const int nsel_s = ntok_s * p.topk;
  const bool pre_fits = nsel_s <= NT;
  int pre_id = -1;
  if (pre_fits && tid < nsel_s && q0s + tid / p.topk < p.total_q)
    pre_id = p.q2k[((int64_t)g * p.total_q + q0s) * p.topk + tid];
  const int ptw = p.paged ? min(p.pt_width, kPtCache) : 0;
  int32_t ptr_[kPtCache / NT];
  {
    const int32_t* prow = p.page_table + (int64_t)b * p.pt_width;
#pragma unroll
    for (int k = 0; k < kPtCache / NT; ++k) {
      const int t = tid + NT * k;
      ptr_[k] = t < ptw ? prow[t] : 0;
    }
  }

  // the lengths are read after the rows above (scalar reads return out of
  // order: waiting for one waits for all, so they go last)
  const int qb = p.cu_q[b];
  const int lq = p.cu_q[b + 1] - qb;          // the request's query tokens
  const int lk = p.paged ? p.seqused_k[b] : (p.cu_k[b + 1] - p.cu_k[b]);
  const int j0 = jt * p.tok_per_tile;         // the tile's first token in the request
  if (lq - j0 <= 0) return;
  const int q0 = qb + j0;
  const int ntok = min(lq - j0, p.tok_per_tile);
  const int R = ntok * G;
  const int nblk = max(0, min((lk + kBlock - 1) / kBlock, p.max_k_tiles));
  const bool spec = q0 == q0s && ntok == ntok_s;   // workgroup-uniform
  if (!spec) load_q(q0, R);

  int tk_[RT], pos_[RT];
  unsigned long long tokmask[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = 16 * rt + l16;
    const int tk = r < R ? r / G : 64;
    tk_[rt] = tk;
    pos_[rt] = tk < ntok ? query_pos(p.qpos.rows, p.qpos.mode, p.qpos.base, q0 + tk, j0 + tk,
                                     lq, lk)
                         : 0;
    const int tfirst = (16 * rt) / G;
    const int tlast = min((16 * rt + 15) / G, ntok - 1);
    unsigned long long m = 0;
    for (int t = tfirst; t <= tlast && t < 64; ++t) m |= 1ull << t;
    tokmask[rt] = uniform64((16 * rt < R) ? m : 0ull);
  }
  const bool ptc = p.paged && nblk <= ptw;

  const int32_t* rows = p.q2k + ((int64_t)g * p.total_q + q0) * p.topk;
  const bool use_pre = spec && pre_fits;
  int ucount;
  if (ntok == 1) {
    // one token: its row is the union when ascending without repeats (the
    // q2k contract); checked, with the general builder as the fallback
    int id = use_pre ? pre_id : -1;
    if (!use_pre && tid < p.topk) id = rows[tid];
    const bool in = tid < p.topk && id >= 0 && id < nblk;
    int bad = 0;
    if (wave == 0) {
      const unsigned long long bal = __ballot(in);
      const unsigned long long below = bal & ((1ull << lane) - 1ull);
      const int pos = __popcll(below);
      // each in-range id must exceed the previous in-range id
      const int pl = below ? 63 - __clzll(below) : lane;
      const int pid = __shfl(id, pl, kWave);
      bad = __ballot(in && below != 0ull && pid >= id) != 0ull;
      if (in) {
        lds.un.list[pos] = id;
        lds.un.mask[pos] = 1ull;
      }
      if (lane == 0) lds.un.count = bad ? -1 : (int)__popcll(bal);
    }
    __syncthreads();
    ucount = lds.un.count;
    if (ucount < 0) ucount = build_tile_union<NT>(lds.un, rows, ntok, p.topk, nblk, pre_id, use_pre);
  } else {
    ucount = build_tile_union<NT>(lds.un, rows, ntok, p.topk, nblk, pre_id, use_pre);
  }
  ucount = __builtin_amdgcn_readfirstlane(ucount);
  const int u0 = (int)(((int64_t)ucount * split) / p.splits);
  const int u1 = (int)(((int64_t)ucount * (split + 1)) / p.splits);
  const int n = u1 - u0;
  if (ptc) {
#pragma unroll
    for (int k = 0; k < kPtCache / NT; ++k) {
      const int t = tid + NT * k;
      if (t < nblk) lds.ptrow[t] = ptr_[k];
    }
    __syncthreads();
  }
  for (int i = tid; i < n; i += NT) {
    const int t = lds.un.list[u0 + i];
    lds.page[i] = ptc ? lds.ptrow[t]
                      : (p.paged ? p.page_table[(int64_t)b * p.pt_width + t] : p.cu_k[b] + kBlock * t);
  }

  // settle the Q loads before the loop (see the prefill kernel)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      u32x4 w = __builtin_bit_cast(u32x4, qf[rt][ds]);
      asm volatile("" : "+v"(w));
      qf[rt][ds] = as_bf16x8(w);
    }

  float m_[RT], l_[RT], lt_[RT];
  f32x4 o_[RT][8];
  const float slack = TEMP ? p.tslack : DecSoft<FMT>::kSlack;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_[rt] = -INFINITY;
    l_[rt] = 0.f;
    lt_[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o_[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();  // page ids visible

  // ---- staging: wave w's load nn (< LOADS) of a page fills bytes
  // [1024 nn, 1024 nn + 1024) of its stage; lane l writes 16 bytes at 16 l.
  // Rows are the wave's local key rows 0..31 (key 32 w + row).
  // With 8 waves, waves 4..7 take the odd entries of the share and 0..3
  // the even ones: two independent page streams per SIMD.
  const uint32_t wring = __builtin_amdgcn_readfirstlane(lds_addr(lds.ring)) +
                         wave * NST * Geo::kStage;
  const int64_t kst = p.k_st.token, vst = p.v_st.token;
  const int kw0 = 32 * (wave & 3);  // this wave's first key of every page
  constexpr int PSTRIDE = NWV / 4;
  const int par = wave >> 2;        // page parity (8 waves)
  const int nj = n > par ? (n - par + PSTRIDE - 1) / PSTRIDE : 0;   // this wave's pages
  auto issue = [&](int j, int stage) {
    const int i = par + PSTRIDE * j;
    const int t = __builtin_amdgcn_readfirstlane(lds.un.list[u0 + i]);
    const int pg = __builtin_amdgcn_readfirstlane(lds.page[i]);
    const int nvalid = min(kBlock, lk - kBlock * t) - kw0;  // valid local rows
    const uint8_t* kb;
    const uint8_t* vb;
    if (p.paged) {
      kb = p.k + (int64_t)pg * p.k_st.page + g * p.k_st.head;
      vb = p.v + (int64_t)pg * p.v_st.page + g * p.v_st.head;
    } else {
      kb = p.k + (int64_t)pg * kst + g * p.k_st.head;
      vb = p.v + (int64_t)pg * vst + g * p.v_st.head;
    }
    kb += kw0 * kst;
    vb += kw0 * vst;
    const uint32_t dst = wring + stage * Geo::kStage;
#pragma unroll
    for (int nn = 0; nn < LOADS; ++nn) {
      const uint8_t* src;
      if constexpr (FMT == kFmtBf16 || FMT == kFmtF16) {
        // rows of 256 B: 4 rows per load
        constexpr int kHalf = LOADS / 2;
        const bool isv = nn >= kHalf;
        const int row = 4 * (isv ? nn - kHalf : nn) + (lane >> 4);
        const int rr = row < nvalid ? row : -kw0;   // past the end: the page's row 0
        const int c = isv ? ((lane & 15) ^ ((row & 3) << 1)) : ((lane & 15) ^ (row & 15));
        src = (isv ? vb + rr * vst : kb + rr * kst) + 16 * c;
      } else if constexpr (FMT == kFmtFp8) {
        // rows of 128 B: 8 rows per load
        constexpr int kHalf = LOADS / 2;
        const bool isv = nn >= kHalf;
        const int row = 8 * (isv ? nn - kHalf : nn) + (lane >> 3);
        const int rr = row < nvalid ? row : -kw0;
        const int gv = (row & 3) | (((row >> 4) & 1) << 2);
        const int c = isv ? ((lane & 7) ^ gv) : ((lane & 7) ^ (row & 7));
        src = (isv ? vb + rr * vst : kb + rr * kst) + 16 * c;
      } else {
        if (nn < 4) {
          // data rows of 64 B: 16 rows per load (K: loads 0-1, V: 2-3)
          const bool isv = nn >= 2;
          const int row = 16 * (nn & 1) + (lane >> 2);
          const int rr = row < nvalid ? row : -kw0;
          const int gv = ((row >> 1) & 1) | (((row >> 4) & 1) << 1);
          const int c = isv ? ((lane & 3) ^ gv) : ((lane & 3) ^ ((row >> 1) & 3));
          src = (isv ? vb + rr * vst : kb + rr * kst) + 16 * c;
        } else {
          // scale rows of 8 B, two per lane: lanes 0-15 K scales, 16-31 V
          // scales; lanes 32-63 repeat the K scales into the spare bytes
          const bool isv = lane >= 16 && lane < 32;
          const int row = 2 * (lane & 15);
          const int rr = kw0 + (row < nvalid ? row : -kw0);
          const uint8_t* sb = isv ? p.vs + (int64_t)pg * p.vs_st.page + g * p.vs_st.head
                                  : p.ks + (int64_t)pg * p.ks_st.page + g * p.ks_st.head;
          src = sb + rr * 8;
        }
      }
      g2lds16(src, dst + 1024 * nn);
    }
  };

#pragma unroll
  for (int s = 0; s < NST; ++s)
    if (s < nj) issue(s, s);

  const float C = p.scale_log2;

  for (int j = 0; j < nj; ++j) {
    const int i = par + PSTRIDE * j;
    const int stage = j % NST;
    // wait for this page's loads; the wave's later pages (up to NST - 1)
    // stay in flight
    const int later = min(NST - 1, nj - 1 - j);
    if (later >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * LOADS) : "memory");
    else if (later == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LOADS) : "memory");
    else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    const int u = u0 + i;
    const int t = __builtin_amdgcn_readfirstlane(lds.un.list[u]);
    const unsigned long long umask = uniform64(lds.un.mask[u]);
    const int nvalid = min(kBlock, lk - kBlock * t);
    bool any = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) any |= (umask & tokmask[rt]) != 0ull;
    const uint32_t sb = wring + stage * Geo::kStage;
    if (any) {
    // ---- K fragments (A operand of S^T): key kw0 + 16 kt + l % 16,
    // head dims 32 q + 8 ds .. + 7 for k-step ds
    bf16x8 kf[2][4];
    if constexpr (FMT == kFmtBf16 || FMT == kFmtF16) {
      u32x4 kw[8];
      uint32_t a[8];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int row = 16 * kt + l16;   // local row
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) a[4 * kt + ds] = sb + row * 256 + 16 * ((4 * q + ds) ^ (row & 15));
      }
      kfrag_load(kw, a);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) kf[kt][ds] = as_bf16x8(kw[4 * kt + ds]);
    } else if constexpr (FMT == kFmtFp8) {
      u32x4 kw[4];
      uint32_t a[4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int row = 16 * kt + l16;   // local row
#pragma unroll
        for (int j = 0; j < 2; ++j) a[2 * kt + j] = sb + row * 128 + 16 * ((2 * q + j) ^ (row & 7));
      }
      lds_b128x4(kw, a);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x4 w = kw[2 * kt + j];
          kf[kt][2 * j] = as_bf16x8(fp8x8_to_bf16(w[0], w[1]));
          kf[kt][2 * j + 1] = as_bf16x8(fp8x8_to_bf16(w[2], w[3]));
        }
    } else {
      u32x4 kw[2];
      uint32_t ks[2];
      uint32_t a[2], as[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int row = 16 * kt + l16;   // local row
        a[kt] = sb + row * 64 + 16 * (q ^ ((row >> 1) & 3));
        as[kt] = sb + 2 * Geo::kSide + row * 8 + 2 * q;
      }
      lds_b128x2_u16x2(kw, ks, a, as);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const f32x2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ks[kt], 1.0f, false);
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) kf[kt][ds] = as_bf16x8(e2m1x8_scaled(kw[kt][ds], ds < 2 ? sc[0] : sc[1]));
      }
    }

    // ---- V^T fragments (A operand of O^T): head dim 16 dt + l % 16, keys
    // kw0 + {4q..4q+3, 16+4q..16+4q+3} (the order of P in the S^T registers)
    bf16x8 vf[8];
    if constexpr (FMT == kFmtBf16 || FMT == kFmtF16) {
      u32x2 vv[16];
      uint32_t a[8];
      const int e = l16 >> 2, aa = lane & 3;
      const int row = 4 * q + e;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) a[dt] = sb + Geo::kSide + row * 256 + 32 * (dt ^ e) + 8 * aa;
      vtr16_issue(vv, a);
      wait16(vv);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        vf[dt] = as_bf16x8(u32x4{vv[2 * dt][0], vv[2 * dt][1], vv[2 * dt + 1][0], vv[2 * dt + 1][1]});
    } else if constexpr (FMT == kFmtFp8) {
      u32x2 vv[8];
      uint32_t a[8];
      const int e = l16 >> 1, aa = lane & 1;
      const int row = e < 4 ? 4 * q + e : 16 + 4 * q + e - 4;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) a[dt] = sb + Geo::kSide + row * 128 + 16 * (dt ^ e) + 8 * aa;
      vtr8_issue<false>(vv, a);
      wait8(vv);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        vf[dt] = as_bf16x8(fp8x8_to_bf16(vv[dt][0], vv[dt][1]));
      }
    } else {
      u32x2 vv[8], vsr[8];
      uint32_t a[8], asr[8];
      const int e = l16 & 7;
      const int row = e < 4 ? 4 * q + e : 16 + 4 * q + e - 4;
      const int gv = ((row >> 1) & 1) | (((row >> 4) & 1) << 1);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        a[dt] = sb + Geo::kSide + row * 64 + 16 * ((dt >> 1) ^ gv) + 8 * (dt & 1);
      vtr8_issue<true>(vv, a);
      // scale rows of this lane's eight keys
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int rk = k < 4 ? 4 * q + k : 16 + 4 * q + k - 4;
        asr[k] = sb + 2 * Geo::kSide + Geo::kScale + rk * 8;
      }
      lds_b64x8(vsr, asr);
      wait8(vv);   // orders the uses of the transposed reads after their wait
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int rk = kw0 + (k < 4 ? 4 * q + k : 16 + 4 * q + k - 4);
        if (rk >= nvalid) vsr[k] = u32x2{0u, 0u};   // no scale of a key past the end
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int w = dt >> 2, sel = dt & 3;
        const uint32_t s03 = gather_byte(vsr[0][w], vsr[1][w], vsr[2][w], vsr[3][w], sel);
        const uint32_t s47 = gather_byte(vsr[4][w], vsr[5][w], vsr[6][w], vsr[7][w], sel);
        float s[8];
        f32x2_t x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s03, 1.0f, false);
        s[0] = x[0]; s[1] = x[1];
        x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s03, 1.0f, true);
        s[2] = x[0]; s[3] = x[1];
        x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s47, 1.0f, false);
        s[4] = x[0]; s[5] = x[1];
        x = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s47, 1.0f, true);
        s[6] = x[0]; s[7] = x[1];
        vf[dt] = as_bf16x8(e2m1x8_keyscaled(vv[dt][0], s));
      }
    }

#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if ((umask & tokmask[rt]) == 0ull) continue;
      f32x4 acc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) acc[kt] = mma16<FMT>(kf[kt][ds], qf[rt][ds], acc[kt]);
      }
      const bool sel = (tk_[rt] < ntok) && ((umask >> tk_[rt]) & 1ull);
      int lim = nvalid - 1;
      if (p.causal) lim = min(lim, pos_[rt] - kBlock * t);
      lim = sel ? lim : -1;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kw0 + 16 * kt + 4 * q + r;
          acc[kt][r] = key <= lim ? acc[kt][r] * C : -INFINITY;
        }
      // Exponentials against the row's reference max m as it stands (no
      // per-page max): a score more than the slack above m makes some p pass
      // 2^64 and the lane's 8-term sum pass 2^67, which sends the rows (with
      // rows that have no reference yet) down the rare path, where the page's
      // row max moves m and O and l are rescaled.  Otherwise p <= 2^67.
      const float mu = m_[rt] > -INFINITY ? m_[rt] : INFINITY;
      float e[8];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) e[4 * kt + r] = __builtin_amdgcn_exp2f(acc[kt][r] - mu);
      float lp = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      float ltp = 0.f;
      if constexpr (TEMP) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) ltp += __builtin_amdgcn_exp2f(p.tau * (acc[kt][r] - mu));
      }
      if (__ballot(sel && (m_[rt] == -INFINITY || !(lp <= DecSoft<FMT>::kLimit) ||
                           (TEMP && !(ltp <= DecSoft<FMT>::kLimit)))) != 0ull) {
        float mx = fmaxf(fmaxf(fmaxf(acc[0][0], acc[0][1]), fmaxf(acc[0][2], acc[0][3])),
                         fmaxf(fmaxf(acc[1][0], acc[1][1]), fmaxf(acc[1][2], acc[1][3])));
        mx = xmax16_32(mx);   // the row's keys are spread over four lanes
        const bool up = mx > m_[rt] + slack;
        if (__ballot(up && m_[rt] > -INFINITY) != 0ull) {
          const float alpha = up ? __builtin_amdgcn_exp2f(m_[rt] - mx) : 1.0f;
          l_[rt] *= alpha;
          if constexpr (TEMP) lt_[rt] *= up ? __builtin_amdgcn_exp2f(p.tau * (m_[rt] - mx)) : 1.0f;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o_[rt][dt] *= alpha;
        }
        m_[rt] = up ? mx : m_[rt];
        const float mu2 = m_[rt] > -INFINITY ? m_[rt] : INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) e[4 * kt + r] = __builtin_amdgcn_exp2f(acc[kt][r] - mu2);
        lp = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
        if constexpr (TEMP) {
          ltp = 0.f;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) ltp += __builtin_amdgcn_exp2f(p.tau * (acc[kt][r] - mu2));
        }
      }
      l_[rt] += lp;
      if constexpr (TEMP) lt_[rt] += ltp;
      const bf16x8 pf = as_bf16x8(u32x4{pk_p<FMT>(e[0], e[1]), pk_p<FMT>(e[2], e[3]),
                                        pk_p<FMT>(e[4], e[5]), pk_p<FMT>(e[6], e[7])});
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o_[rt][dt] = mma16<FMT>(vf[dt], pf, o_[rt][dt]);
    }
    }  // any
    // the stage's reads completed (every fragment read above waited for
    // its data), so it takes the page NST ahead
    if (j + NST < nj) issue(j + NST, stage);
  }

  // ---- merge the waves' states row tile by row tile through LDS.  The
  // barriers only order LDS accesses (the ring is reused), so they wait on
  // LDS counters alone and leave the output stores in flight.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  block_barrier();
  MergeLds<NWV>& mg = *reinterpret_cast<MergeLds<NWV>*>(lds.ring);
  const int unit_split = unit * p.splits + split;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    if (16 * rt >= R) break;
    const float lsum = xsum16_32(l_[rt]);
    const float ltsum = TEMP ? xsum16_32(lt_[rt]) : 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<f32x4*>(&mg.o[wave][l16][16 * dt + 4 * q]) = o_[rt][dt];
    if (q == 0) {
      mg.m[wave][l16] = m_[rt];
      mg.l[wave][l16] = lsum;
      if constexpr (TEMP) mg.lt[wave][l16] = ltsum;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    block_barrier();
    const int rr = (tid >> 4) & 15;   // row within the tile (threads 0..255)
    const int d0 = 8 * (tid & 15);
    const int row = 16 * rt + rr;
    if (tid < 256 && row < R) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NWV; ++w) M = fmaxf(M, mg.m[w][rr]);
      const float Mu = M == -INFINITY ? 0.f : M;
      float wk[NWV], L = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        wk[w] = __builtin_amdgcn_exp2f(mg.m[w][rr] - Mu);
        L += mg.l[w][rr] * wk[w];
      }
      const float invL = L > 0.f ? 1.f / L : 0.f;
      float acc8[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) x += mg.o[w][rr][d0 + k] * wk[w];
        acc8[k] = x * invL;
      }
      const float lse_nat = L > 0.f ? (M + __log2f(L)) * kLn2d : -INFINITY;
      float lset_nat = -INFINITY;
      if constexpr (TEMP) {
        float Lt = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w)
          Lt += mg.lt[w][rr] * __builtin_amdgcn_exp2f(p.tau * (mg.m[w][rr] - Mu));
        lset_nat = (L > 0.f && Lt > 0.f) ? (p.tau * M + __log2f(Lt)) * kLn2d : -INFINITY;
      }
      if (p.splits == 1) {
        const int64_t orow = (int64_t)(q0 + row / G) * p.hq + g * G + row % G;
        u32x4 w4;
#pragma unroll
        for (int k = 0; k < 4; ++k) w4[k] = pk_out<FMT>(acc8[2 * k] * p.v_gs, acc8[2 * k + 1] * p.v_gs);
        *reinterpret_cast<u32x4*>(p.out + orow * kHeadDim + d0) = w4;
        if (p.lse && d0 == 0) p.lse[orow] = lse_nat;
        if (TEMP && d0 == 0) p.lse_t[orow] = lset_nat;
      } else {
        float* po = p.ws_o + ((int64_t)unit_split * p.ws_rows + row) * kHeadDim + d0;
        st_dev4(po, f32x4{acc8[0], acc8[1], acc8[2], acc8[3]});
        st_dev4(po + 4, f32x4{acc8[4], acc8[5], acc8[6], acc8[7]});
        if (d0 == 0) st_dev(p.ws_lse + (int64_t)unit_split * p.ws_lse_rows + row, lse_nat);
        if (TEMP && d0 == 0)
          st_dev(p.ws_lse_t + (int64_t)unit_split * p.ws_lse_rows + row, lset_nat);
      }
    }
    if (rt + 1 < RT && 16 * (rt + 1) < R) {   // the next tile rewrites the merge buffer
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      block_barrier();
    }
  }
  if (p.splits == 1) return;
  // ---- split arrival: the partial stores of every thread have completed
  // (device scope) before the unit's counter counts this split
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(p.ws_count + unit, 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(p.splits - 1);
  __syncthreads();
  if (!s_last) return;
  // the last split merges: lse = ln sum_s exp(lse_s), out = v_gs * sum_s
  // exp(lse_s - lse) O_s, then resets the counter for the next launch
  const int nsp = p.splits;
  for (int task = tid; task < R * 16; task += NT) {
    const int row = task >> 4, d0 = 8 * (task & 15);
    const float* lsep = p.ws_lse + (int64_t)unit * nsp * p.ws_lse_rows + row;
    float M = -INFINITY;
    for (int s = 0; s < nsp; ++s) M = fmaxf(M, ld_dev(lsep + (int64_t)s * p.ws_lse_rows));
    const float Mu = M == -INFINITY ? 0.f : M;
    float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float W = 0.f;
    for (int s = 0; s < nsp; ++s) {
      const float w = __builtin_amdgcn_exp2f((ld_dev(lsep + (int64_t)s * p.ws_lse_rows) - Mu) *
                                             1.4426950408889634f);
      W += w;
      const float* po = p.ws_o + (((int64_t)unit * nsp + s) * p.ws_rows + row) * kHeadDim + d0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x2_dev x = ld_dev2(po + 2 * k);
        acc8[2 * k] += w * x[0];
        acc8[2 * k + 1] += w * x[1];
      }
    }
    const float sc = W > 0.f ? p.v_gs / W : 0.f;
    const int64_t orow = (int64_t)(q0 + row / G) * p.hq + g * G + row % G;
    u32x4 w4;
#pragma unroll
    for (int k = 0; k < 4; ++k) w4[k] = pk_out<FMT>(acc8[2 * k] * sc, acc8[2 * k + 1] * sc);
    *reinterpret_cast<u32x4*>(p.out + orow * kHeadDim + d0) = w4;
    if (p.lse && d0 == 0) p.lse[orow] = W > 0.f ? M + __logf(W) : -INFINITY;
    if (TEMP && d0 == 0) {
      const float* ltp = p.ws_lse_t + (int64_t)unit * nsp * p.ws_lse_rows + row;
      float Mt = -INFINITY;
      for (int s = 0; s < nsp; ++s) Mt = fmaxf(Mt, ld_dev(ltp + (int64_t)s * p.ws_lse_rows));
      float St = 0.f;
      if (Mt > -INFINITY)
        for (int s = 0; s < nsp; ++s) St += __expf(ld_dev(ltp + (int64_t)s * p.ws_lse_rows) - Mt);
      p.lse_t[orow] = St > 0.f ? Mt + __logf(St) : -INFINITY;
    }
  }
  if (tid == 0) __hip_atomic_store(p.ws_count + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

}

template <int FMT, int RT, int NWV = 4>
static hipError_t launch_decode_t(const AttnParams& p, hipStream_t stream) {
  const int n = p.batch * p.hkv * p.tiles_per_req * p.splits;
  if (n <= 0) return hipSuccess;
  const dim3 grid(8 * ((n + 7) / 8));
  if (p.lse_t)
    hipLaunchKernelGGL((msa_decode_kernel<FMT, RT, NWV, true>), grid, dim3(NWV * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((msa_decode_kernel<FMT, RT, NWV, false>), grid, dim3(NWV * 64), 0, stream, p);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_decode_fmt(const AttnParams& p, hipStream_t stream) {
  const int rows = p.tok_per_tile * p.group;
  // E2M1 stages are small enough for 8 waves (two page streams per SIMD)
  if (rows <= 16) return launch_decode_t<FMT, 1, FMT == kFmtE2m1 ? 8 : 4>(p, stream);
  if (rows <= 32) return launch_decode_t<FMT, 2>(p, stream);
  if (rows <= 48) return launch_decode_t<FMT, 3>(p, stream);
  return launch_decode_t<FMT, 4>(p, stream);
}

hipError_t launch_decode(const AttnParams& p, int fmt, hipStream_t stream) {
  switch (fmt) {
    case kFmtBf16: return launch_decode_fmt<kFmtBf16>(p, stream);
    case kFmtFp8: return launch_decode_fmt<kFmtFp8>(p, stream);
    case kFmtF16: return launch_decode_fmt<kFmtF16>(p, stream);
    default: return launch_decode_fmt<kFmtE2m1>(p, stream);
  }
}

int decode_workgroups_per_cu(int fmt, int rows) {
  // more than one row tile takes over half the register file
  if (rows > 16) return 1;
  auto per = [](int bytes) { return (160 * 1024) / bytes; };
  switch (fmt) {
    case kFmtBf16:
    case kFmtF16: return per(sizeof(DecodeLds<kFmtBf16, 4>));
    case kFmtFp8: return per(sizeof(DecodeLds<kFmtFp8, 4>));
    default: return per(sizeof(DecodeLds<kFmtE2m1, 8>));
  }
}

}  // namespace msa
