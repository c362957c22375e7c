// Packed query sparse attention over caller-listed tokens (qsa page: the
// indexed and bitmap APIs; outputs BF16 and FP32 [T, Hq, 256] and the natural-log LSE
// [Hq, T]; an empty selection gives zero output and -inf LSE).
//
// gfx950 design: one workgroup of eight waves per (tile of TT consecutive
// packed query tokens, KV head), TT = min(16, 128 / G).  The tile's TT x G
// query rows (token-major) are cut into 16-row slots, one per wave, on
// v_mfma_f32_16x16x32_bf16.
//  * Shared keys.  The tile's selections are folded into one 32-bit word per
//    key in LDS (bit j: token j of the tile lists the key), one window of
//    16384 keys of the tile's key range at a time, then compacted, in
//    ascending key order, into (key offset, token mask) words.  The keys are consumed 32 at a time: every chunk's K
//    and V rows (512 bytes each) are staged global -> LDS with
//    global_load_lds by all eight waves into a ring of 2-4 chunk buffers
//    (one barrier per chunk), so a key listed by several tokens of the tile
//    is read once per tile rather than once per token.  Every slot computes
//    the whole chunk and masks the keys its row's token did not list.
//  * S^T = K Q^T (keys on M, query rows on N), K fragments from LDS (ring
//    rows XOR-swizzled in 16-byte units so that operand reads are
//    conflict-free); online softmax in log2 units against a per-row
//    reference max that moves (rescaling O and l) only when the row meets
//    its first listed key or a chunk's partial sum reveals a score past it
//    by more than 64; O^T += V^T P^T
//    with V^T from ds_read_b64_tr_b16 and P straight from the S^T registers
//    (keys 4 q .. 4 q + 3 and 16 + 4 q .. 16 + 4 q + 3 of lane group q).
//    The softmax state carries over from window to window.
//  * Per-token keys.  When the tile's keys span more than 64 windows, or
//    the union is large against what its tokens listed (masking would then
//    compute far more scores than gathering each token's own keys), the
//    eight waves take the tile's tokens one at a time instead: one wave per
//    (token, KV head) gathers the token's keys 32 at a time in index order
//    (K straight into MFMA operand registers, four lanes reading 64
//    contiguous bytes of a key; V through the wave's own LDS buffer).
// Both routes are deterministic: results are bitwise repeatable.
#include "async_lds.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace msa {

namespace {

constexpr int kQsaDim = 256;
constexpr int kQsaRowBytes = kQsaDim * 2;   // one bf16 K or V row of one head
constexpr float kQsaLn2 = 0.69314718055994530942f;
constexpr int kQsaWaves = 8;
constexpr int kQsaThreads = kQsaWaves * kWave;
constexpr int kQsaTileRows = 16 * kQsaWaves;      // query rows of a tile
constexpr int kQsaMaxTokens = 16;                 // token bits of a key's mask word
constexpr int kQsaWin = 16384;                    // keys of one window of a tile's key range
constexpr int kQsaMaxWin = 64;                    // windows the shared route takes (1 Mi keys)
// Shared route when kTileCost * union * (slot rounds) <= kTokenCost * listed
// entries: per union key a round of four 16-row slots costs about 5/8 of one
// per-token key gather (1 KiB per key and token, measured rates).
constexpr int kTileCost = 5;
constexpr int kTokenCost = 8;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 lds_tr16(uint32_t a) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (__attribute__((address_space(3))) s16x4*)(uintptr_t)a));
}
__device__ __forceinline__ u32x4 lds_b128(uint32_t a) {
  return *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)a;
}

__device__ __forceinline__ float xmax_16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, kWave));
  return fmaxf(x, __shfl_xor(x, 32, kWave));
}
__device__ __forceinline__ float xsum_16_32(float x) {
  x += __shfl_xor(x, 16, kWave);
  return x + __shfl_xor(x, 32, kWave);
}

// One wave's LDS on the per-token route.
struct QsaTokLds {
  uint8_t v[32 * kQsaRowBytes];   // V rows of the chunk (16 KiB)
  int32_t ids[32];                // the chunk's index entries (-1: padding)
  int32_t blk[8];                 // bitmap source: the chunk's selected blocks
};

// Workgroup LDS (bytes), all 160 KiB.  Shared route: the key-mask words of
// the tile's key range from offset 0 (at most 64 KiB), compacted in place
// into the union list; then a ring of [K | V] chunk buffers right after the
// list (four when the union has at most 8192 keys, else three), and a few
// words of reduction scratch at the top (read only before the ring is
// filled).  Per-token route: one QsaTokLds per wave from offset 0.
constexpr int kQsaLds = 160 * 1024;
constexpr int kMiscOff = kQsaLds - 256;
// Ring rows are unpadded (512 bytes) and XOR-swizzled in 16-byte units:
// unit u of K row r sits at u ^ (r % 16), of V row r at u ^ 2 (r % 8), so the
// 16 keys one K operand read touches and the rows one transposing V read
// touches fall on distinct banks.  (Rows padded to 528 / 544 bytes instead,
// with per-row loads, measured 16x the bank-conflict cycles and 12 % more
// time.)
constexpr int kKPitch = kQsaRowBytes;
constexpr int kVPitch = kQsaRowBytes;
constexpr int kKChunk = 32 * kKPitch;
constexpr int kPairBytes = kKChunk + 32 * kVPitch;   // one ring buffer: K and V of a chunk
constexpr int kQsaMaxBuf = 4;
// A lane's eight exponentials of a chunk sum to at most 8 * 2^64 while every
// score is within 64 (log2 units) of the row's reference max.
constexpr float kQsaSumLimit = 0x1p68f;
static_assert(sizeof(QsaTokLds) % 16 == 0, "per-wave regions stay 16-byte aligned");
static_assert(kQsaWaves * (int)sizeof(QsaTokLds) <= kMiscOff, "per-wave regions fit below the scratch");
static_assert(4 * kQsaWin + 2 * kPairBytes <= kQsaLds, "two ring buffers fit after the widest list");

// Per-token route: one wave computes query token `tok` against KV head g,
// its G <= 16 query heads as the 16 rows of the MFMA tile, the token's keys
// in index order (BITMAP: the tokens of its selected blocks, ascending).
template <bool BITMAP>
__device__ __forceinline__ void qsa_token(const QsaParams& p, int tok, int g, QsaTokLds& lds) {
  const int lane = threadIdx.x & (kWave - 1);
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

// Index entries e0 + tid + 512 i (i < NI) of the tile's rows j < 16, all
// loads in flight together; rows past the tile re-read its last row and
// entries past the row its last entry (the caller skips both).
template <int NI>
__device__ __forceinline__ void index_batch(const QsaParams& p, int t0, int nt, int e0,
                                            int (&id)[kQsaMaxTokens][NI]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kQsaMaxTokens; ++j) {
    const int32_t* row = p.indices + (int64_t)(t0 + min(j, nt - 1)) * p.width;
#pragma unroll
    for (int i = 0; i < NI; ++i) id[j][i] = row[min(e0 + tid + kQsaThreads * i, p.width - 1)];
  }
}

// Token bits of blocks b0 + tid + 512 i (i < 4): bit j set when the tile's
// token j selects the block (bitmap byte non-zero); blocks past the map read
// its last block (the caller skips them).
__device__ __forceinline__ void block_masks(const QsaParams& p, int t0, int nt, int b0,
                                            uint32_t (&mk)[4]) {
  const int tid = threadIdx.x;
  uint8_t v[kQsaMaxTokens][4];
#pragma unroll
  for (int j = 0; j < kQsaMaxTokens; ++j) {
    const uint8_t* row = p.bitmap + (int64_t)(t0 + min(j, nt - 1)) * p.num_blocks;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[j][i] = row[min(b0 + tid + kQsaThreads * i, p.num_blocks - 1)];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < kQsaMaxTokens; ++j) m |= (j < nt && v[j][i] != 0 ? 1u : 0u) << j;
    mk[i] = m;
  }
}

}  // namespace

// BITMAP: the keys come from a uint8 [T, num_blocks] block bitmap instead of
// index rows (a non-zero byte b selects tokens 4 b .. 4 b + 3 below Tk), so no
// [T, NB] index scratch is ever written (qsa page: the bitmap API and its
// compact-index scratch).
template <bool BITMAP>
__global__ __launch_bounds__(kQsaThreads, 1) void msa_qsa_kernel(QsaParams p, int TT) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kQsaLds];
  const int tiles = (p.total_q + TT - 1) / TT;
  // last tiles first: causal selections grow with the position, so the
  // longest tiles start earliest and the short ones fill the tail
  const int tile = tiles - 1 - (int)(blockIdx.x / p.hkv);
  const int g = blockIdx.x % p.hkv;
  if (tile < 0) return;
  const int t0 = tile * TT;
  const int nt = min(TT, p.total_q - t0);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.group;
  uint32_t* M = reinterpret_cast<uint32_t*>(smem);
  int* misc = reinterpret_cast<int*>(smem + kMiscOff);

  // ---- pass 1: listed entries (saturated: only compared with the union
  // below) and the lowest and highest listed key of the tile.  Loads go out
  // 16 rows x 4 entries per thread at a time (rows past the tile re-read its
  // last row, entries past the row its last entry; neither is counted).  A
  // bitmap over at most 16384 keys also writes every key's token bits here,
  // at key offset 0 (base 0). ----
  const bool direct = BITMAP && p.num_kv_tokens <= kQsaWin;
  int cnt = 0, lo = INT32_MAX, hi = -1;
  if constexpr (BITMAP) {
    const int nb = p.num_blocks;
    for (int b0 = 0; b0 < nb; b0 += 4 * kQsaThreads) {
      uint32_t mk[4];
      block_masks(p, t0, nt, b0, mk);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = b0 + tid + kQsaThreads * i;
        if (b >= nb) continue;
        const int last = min(4 * b + 3, p.num_kv_tokens - 1);
        if (mk[i]) {
          cnt += __popc(mk[i]) * (last - 4 * b + 1);
          lo = min(lo, 4 * b);
          hi = max(hi, last);
        }
        if (direct) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * b + e <= last) M[4 * b + e] = mk[i];
        }
      }
    }
  } else {
    for (int e0 = 0; e0 < p.width; e0 += 4 * kQsaThreads) {
      int id[kQsaMaxTokens][4];
      index_batch<4>(p, t0, nt, e0, id);
#pragma unroll
      for (int j = 0; j < kQsaMaxTokens; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (j < nt && e0 + tid + kQsaThreads * i < p.width && id[j][i] >= 0) {
            ++cnt;
            lo = min(lo, id[j][i]);
            hi = max(hi, id[j][i]);
          }
    }
  }
  cnt = min(cnt, 1 << 20);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    cnt += __shfl_xor(cnt, d, kWave);
    lo = min(lo, __shfl_xor(lo, d, kWave));
    hi = max(hi, __shfl_xor(hi, d, kWave));
  }
  if (lane == 0) {
    misc[w] = cnt;
    misc[8 + w] = lo;
    misc[16 + w] = hi;
  }
  __syncthreads();
  int listed = 0;
  lo = INT32_MAX;
  hi = -1;
#pragma unroll
  for (int i = 0; i < kQsaWaves; ++i) {
    listed += misc[i];
    lo = min(lo, misc[8 + i]);
    hi = max(hi, misc[16 + i]);
  }

  const int live_waves = (nt * G + 15) >> 4;
  // The tile's key range [base, hi] in windows of kQsaWin keys; the key
  // union is built, compacted and consumed one window at a time.
  const int base = hi < 0 || direct ? 0 : lo;
  const int nwin = hi < 0 ? 0 : (hi - base) / kQsaWin + 1;

  // Token bits of the keys in [wb, wb + kQsaWin) (and <= hi) in M, compacted
  // ascending into (key offset from wb << 16 | token mask) entries, the last
  // chunk padded with the window's lowest listed key (no token); returns the
  // window's union size (uniform).  Every thread calls it.
  auto build = [&](int wb) -> int {
    const int whi = hi - wb < kQsaWin ? hi : wb + kQsaWin - 1;
    const int range = whi - wb + 1;
    if constexpr (BITMAP) {
      if (!direct) {
        // every block of the window written, selected or not (wb and the
        // window length are multiples of 4)
        for (int b0 = wb >> 2; b0 <= (whi >> 2); b0 += 4 * kQsaThreads) {
          uint32_t mk[4];
          block_masks(p, t0, nt, b0, mk);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int b = b0 + tid + kQsaThreads * i;
            if (b > (whi >> 2)) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (4 * b + e <= whi) M[4 * b + e - wb] = mk[i];
          }
        }
      }
    } else {
      if (32 * tid < range) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          *reinterpret_cast<u32x4*>(M + 32 * tid + 4 * i) = u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
      // two entries per row in flight (the softmax state may be live here)
      for (int e0 = 0; e0 < p.width; e0 += 2 * kQsaThreads) {
        int id[kQsaMaxTokens][2];
        index_batch<2>(p, t0, nt, e0, id);
#pragma unroll
        for (int j = 0; j < kQsaMaxTokens; ++j)
#pragma unroll
          for (int i = 0; i < 2; ++i)
            if (j < nt && e0 + tid + kQsaThreads * i < p.width && id[j][i] >= wb &&
                id[j][i] <= whi)
              atomicOr(M + (id[j][i] - wb), 1u << j);
      }
    }
    __syncthreads();
    // compaction, ascending
    uint32_t vals[32];
    int c = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 x = 32 * tid < range ? *reinterpret_cast<const u32x4*>(M + 32 * tid + 4 * i)
                                       : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // words past the range were never written
        vals[4 * i + k] = 32 * tid + 4 * i + k < range ? x[k] : 0u;
        c += vals[4 * i + k] != 0u;
      }
    }
    int x = c;   // inclusive scan over the wave
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int y = __shfl_up(x, d, kWave);
      if (lane >= d) x += y;
    }
    if (lane == kWave - 1) misc[32 + w] = x;
    __syncthreads();
    int before = 0, u = 0;
#pragma unroll
    for (int i = 0; i < kQsaWaves; ++i) {
      const int sw = misc[32 + i];
      before += i < w ? sw : 0;
      u += sw;
    }
    int rank = before + x - c;
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (vals[i]) M[rank++] = (uint32_t)(32 * tid + i) << 16 | vals[i];
    __syncthreads();
    // the last chunk's padding: no token, the window's lowest listed key
    // (entry 0); every thread has read the scan words before a later call
    // writes them again
    if (u > 0 && u + tid < ((u + 31) & ~31)) M[u + tid] = M[0] & 0xffff0000u;
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(u);
  };

  // The whole union first (every window built and counted), for the route;
  // with one window its list stays in M for the shared route.  Nothing
  // listed: the shared route writes 0 / -inf.
  int U = 0;
  const int ncount = nwin <= kQsaMaxWin ? nwin : 0;
  for (int wi = 0; wi < ncount; ++wi) U += build(base + wi * kQsaWin);
  const bool shared = nwin <= kQsaMaxWin && (int64_t)kTileCost * U * ((live_waves + 3) >> 2) <=
                                                (int64_t)kTokenCost * listed;

  if (!shared) {
    // every thread has read the scratch words the per-wave regions cover
    __syncthreads();
    QsaTokLds& mine = *reinterpret_cast<QsaTokLds*>(smem + w * (int)sizeof(QsaTokLds));
    for (int j = w; j < nt; j += kQsaWaves) qsa_token<BITMAP>(p, t0 + j, g, mine);
    return;
  }

  // ---- shared route ----
  const int l16 = lane & 15;
  const int q = lane >> 4;
  const int row = 16 * w + l16;            // tile row: token row / G, head row % G
  const bool live = row < nt * G;
  const int tl = live ? row / G : 0;
  const int hh = live ? row - tl * G : 0;
  const bool wave_live = w < live_waves;

  const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) +
                      ((int64_t)(t0 + tl) * p.hq + g * G + hh) * kQsaRowBytes + 16 * q;

  const uint8_t* kg = reinterpret_cast<const uint8_t*>(p.k) + (int64_t)g * p.k_head_stride;
  const uint8_t* vg = reinterpret_cast<const uint8_t*>(p.v) + (int64_t)g * p.v_head_stride;
  const float C = p.scale_log2;
  const uint32_t mlds = __builtin_amdgcn_readfirstlane(lds_addr(M));

  // reference max m (log2 units; -inf until the row's first listed key) and
  // the row sum: p = 2^(s - m), m moved (rescaling O and l) only when a
  // lane's chunk sum reveals a score past it by the slack, or the row meets
  // its first listed key
  float m = -INFINITY, l = 0.f;
  f32x4 o[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t bit = live ? 1u << tl : 0u;   // the row's token bit in a key's mask
  // K fragment (key 16 kt + l % 16, k-step s): unit 4 s + q of the key's row;
  // V^T fragment (head dims 16 dt + l % 16): lane 4 e + a of a 16-lane group
  // reads 8 bytes (head dims 16 dt + 4 a ..) of rows 4 q + e and
  // 16 + 4 q + e, each at its swizzled unit
  const int vrow = 4 * q + (l16 >> 2);
  const int vsw = (vrow & 7) << 1;
  const uint32_t vofs = kKChunk + vrow * kVPitch + 8 * (l16 & 1);

  // one window: its Uw union keys (listed from M, offsets from wb) in
  // 32-key chunks; the softmax state carries over from window to window
  auto run = [&](int Uw, int wb) {
    // query fragments (re-read per window, so that they are not held while
    // a window's union is built)
    bf16x8 qf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qp + 64 * s);
      qf[s] = as_bf16x8(live ? v : u32x4{0, 0, 0, 0});
    }
    const int nch = (Uw + 31) >> 5;
    const uint32_t ring = mlds + 128 * nch;   // right after the union list
    const int nbuf = min(kQsaMaxBuf, (kQsaLds - 128 * nch) / kPairBytes);

    // chunk K and V rows into ring buffer b: wave w stages keys 4 w .. 4 w + 3,
    // whose union entries `ent` it has read beforehand, two rows per load
    // (lane l: row 4 w + 2 i + l / 32, 16-byte unit l % 32, read from its
    // swizzled source unit); four loads per wave
    auto entries = [&](int c) { return lds_b128(mlds + 128 * c + 16 * w); };
    auto stage = [&](int b, u32x4 ent) {
      const uint32_t kb = ring + b * kPairBytes;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 4 * w + 2 * i + (lane >> 5);
        const uint32_t e = (lane >> 5) ? ent[2 * i + 1] : ent[2 * i];
        const int64_t id = wb + (int)(e >> 16);
        const int u = lane & 31;
        const uint32_t dst = kb + (4 * w + 2 * i) * kQsaRowBytes;
        g2lds16(kg + id * p.k_row_stride + 16 * (u ^ (r & 15)), dst);
        g2lds16(vg + id * p.v_row_stride + 16 * (u ^ ((r & 7) << 1)), dst + kKChunk);
      }
    };

    // chunks 0 .. nbuf - 2 in flight before the first one is computed
    for (int c = 0; c < min(nbuf - 1, nch); ++c) stage(c, entries(c));
    int bc = 0;   // ring buffer of chunk c
    for (int c = 0; c < nch; ++c) {
      const int cn = c + nbuf - 1;   // the chunk staged in this step
      const u32x4 ent = entries(cn < nch ? cn : c);
      // chunk c has landed for every wave (the later chunks staged so far may
      // still be in flight: four loads each), and every wave is done with
      // chunk c - 1, whose buffer chunk cn now refills
      const int ahead = min(nbuf - 2, nch - 1 - c);
      if (ahead >= 2)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else if (ahead == 1)
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      block_barrier();
      if (cn < nch) stage(bc == 0 ? nbuf - 1 : bc - 1, ent);
      const int b = bc;
      bc = bc + 1 == nbuf ? 0 : bc + 1;
      if (!wave_live) continue;
      const uint32_t kb = ring + b * kPairBytes;

      // every K fragment and the token masks of the lane's eight keys in
      // flight at once, then S^T = K Q^T
      u32x4 kf[2][8];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int s = 0; s < 8; ++s)
          kf[kt][s] = lds_b128(kb + (16 * kt + l16) * kKPitch + 16 * ((4 * s + q) ^ l16));
      const uint32_t mrow = mlds + 128 * c;
      const u32x4 ma = lds_b128(mrow + 16 * q);
      const u32x4 mb = lds_b128(mrow + 64 + 16 * q);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) acc[kt] = mfma16(as_bf16x8(kf[kt][s]), qf[s], acc[kt]);
      __builtin_amdgcn_sched_barrier(0);
      // V^T fragments, read while the softmax below runs
      u32x4 vt[16];
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        const uint32_t a = kb + vofs + 16 * ((2 * dt + ((l16 & 3) >> 1)) ^ vsw);
        const u32x2 lo2 = lds_tr16(a);
        const u32x2 hi2 = lds_tr16(a + 16 * kVPitch);
        vt[dt] = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
      }
      __builtin_amdgcn_sched_barrier(0);

      const uint32_t mk[8] = {ma[0], ma[1], ma[2], ma[3], mb[0], mb[1], mb[2], mb[3]};
      bool vis[8];
      float e[8], ps = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        vis[j] = (mk[j] & bit) != 0u;
        const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[j >> 2][j & 3], C, -m));
        e[j] = vis[j] ? x : 0.f;
        ps += e[j];
      }
      if (__ballot(!(ps <= kQsaSumLimit))) {
        // rows whose chunk passed the reference (or met their first listed
        // key) move it to their max; other rows keep theirs (alpha 1, the
        // same exponentials), so a row's result does not depend on its mates
        const float trig = xmax_16_32(!(ps <= kQsaSumLimit) ? 1.f : 0.f);
        float cm = -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j) cm = fmaxf(cm, vis[j] ? acc[j >> 2][j & 3] * C : -INFINITY);
        cm = xmax_16_32(cm);
        const float mn = trig > 0.f ? fmaxf(m, cm) : m;
        const float alpha = mn == m ? 1.f : __builtin_amdgcn_exp2f(m - mn);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < 16; ++dt) o[dt] *= alpha;
        ps = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[j >> 2][j & 3], C, -m));
          e[j] = vis[j] ? x : 0.f;
          ps += e[j];
        }
      }
      l += ps;
      const bf16x8 pf = as_bf16x8(u32x4{cvt_pk_bf16(e[0], e[1]), cvt_pk_bf16(e[2], e[3]),
                                        cvt_pk_bf16(e[4], e[5]), cvt_pk_bf16(e[6], e[7])});
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) o[dt] = mfma16(as_bf16x8(vt[dt]), pf, o[dt]);
    }

  };
  for (int wi = 0; wi < nwin; ++wi) {
    const int wb = base + wi * kQsaWin;
    // one window: still listed from the route decision; several: rebuilt
    run(nwin == 1 ? U : build(wb), wb);
    // every wave is done with this window's list and ring before the next
    // window is built over them (no load is in flight: the last chunk
    // waited for every one)
    if (nwin > 1) __syncthreads();
  }

  if (!wave_live) return;
  // epilogue: lane (row l16, quarter q) holds O^T[16 dt + 4 q + i][row]
  const float lsum = xsum_16_32(l);
  if (!live) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const int tok = t0 + tl;
  const int head = g * G + hh;
  const int64_t orow = ((int64_t)tok * p.hq + head) * kQsaDim + 4 * q;
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) {
    const f32x4 r = o[dt] * inv;
    *reinterpret_cast<u32x2*>(p.out + orow + 16 * dt) =
        u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
    if (p.out_f32) *reinterpret_cast<f32x4*>(p.out_f32 + orow + 16 * dt) = r;
  }
  if (p.lse && q == 0)
    p.lse[(int64_t)head * p.total_q + tok] = lsum > 0.f ? (m + __log2f(lsum)) * kQsaLn2 : -INFINITY;
}

hipError_t launch_qsa(const QsaParams& p, hipStream_t stream) {
  if (p.total_q <= 0) return hipSuccess;
  // G <= 16 (checked by the caller): 8 to 16 tokens per tile
  const int tt = min(kQsaMaxTokens, kQsaTileRows / p.group);
  const int64_t n = (int64_t)((p.total_q + tt - 1) / tt) * p.hkv;
  if (p.bitmap)
    hipLaunchKernelGGL(msa_qsa_kernel<true>, dim3((unsigned)n), dim3(kQsaThreads), 0, stream, p, tt);
  else
    hipLaunchKernelGGL(msa_qsa_kernel<false>, dim3((unsigned)n), dim3(kQsaThreads), 0, stream, p, tt);
  return hipGetLastError();
}

}  // namespace msa
