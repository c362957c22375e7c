// Packed query sparse attention over caller-listed tokens (qsa page: the
// indexed and bitmap APIs; outputs BF16 and FP32 [T, Hq, 256] and the natural-log LSE
// [Hq, T]; an empty selection gives zero output and -inf LSE).
//
// gfx950 design: one workgroup of eight waves per (tile of TT consecutive
// packed query tokens, KV head), TT = min(16, 128 / G).  The tile's TT x G
// query rows (token-major) are cut into 16-row slots, one per wave, on
// v_mfma_f32_16x16x32_bf16.
//  * Shared keys.  The tile's selections are folded into one 32-bit word per
//    key of the tile's key range in LDS (bit j: token j of the tile lists
//    the key), then compacted, in ascending key order, into (key offset,
//    token mask) words.  The keys are consumed 32 at a time: every chunk's K
//    and V rows (512 bytes each) are staged global -> LDS with
//    global_load_lds by all eight waves, double buffered with one barrier
//    per chunk, so a key listed by several tokens of the tile is read once
//    per tile rather than once per token.  Every slot computes the whole
//    chunk and masks the keys its row's token did not list.
//  * S^T = K Q^T (keys on M, query rows on N), K fragments from LDS with the
//    rows XOR-swizzled in 16-byte units (conflict-free operand reads at a
//    512-byte pitch); online softmax in log2 units against a per-row
//    reference max that moves (rescaling O and l) only when a chunk's max
//    passes it by more than 64; O^T += V^T P^T with V^T from
//    ds_read_b64_tr_b16 and P straight from the S^T registers (keys 4 q ..
//    4 q + 3 and 16 + 4 q .. 16 + 4 q + 3 of lane group q).
//  * Per-token keys.  When the tile's keys span more than 16384 tokens, or
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
constexpr int kQsaChunkBytes = 32 * kQsaRowBytes; // 32 K (or V) rows: 16 KiB
constexpr int kQsaWin = 16384;                    // key range the shared route covers
constexpr float kQsaSlack = 64.0f;                // p = 2^(s - m) <= 2^64 between rescales
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

// Workgroup LDS (bytes).  Shared route: [2 buffers][K | V] chunk ring, the
// key-mask words of the tile's key range (then the compacted union), and a
// few words of reduction scratch.  Per-token route: one QsaTokLds per wave
// over the same bytes.
constexpr int kRingBytes = 2 * 2 * kQsaChunkBytes;
constexpr int kMaskOff = kRingBytes;
constexpr int kMiscOff = kMaskOff + 4 * kQsaWin;
constexpr int kSharedLds = kMiscOff + 256;
constexpr int kTokenLds = kQsaWaves * (int)sizeof(QsaTokLds);
constexpr int kQsaLds = kSharedLds > kTokenLds ? kSharedLds : kTokenLds;
static_assert(sizeof(QsaTokLds) % 16 == 0, "per-wave regions stay 16-byte aligned");

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
  uint32_t* M = reinterpret_cast<uint32_t*>(smem + kMaskOff);
  int* misc = reinterpret_cast<int*>(smem + kMiscOff);

  // ---- pass 1: listed entries (saturated: only compared with the union
  // below) and the lowest and highest listed key of the tile ----
  int cnt = 0, lo = INT32_MAX, hi = -1;
  if constexpr (BITMAP) {
    for (int j = 0; j < nt; ++j) {
      const uint8_t* row = p.bitmap + (int64_t)(t0 + j) * p.num_blocks;
      for (int b = tid; b < p.num_blocks; b += kQsaThreads) {
        if (row[b]) {
          const int last = min(4 * b + 3, p.num_kv_tokens - 1);
          cnt += last - 4 * b + 1;
          lo = min(lo, 4 * b);
          hi = max(hi, last);
        }
      }
    }
  } else {
    for (int j = 0; j < nt; ++j) {
      const int32_t* row = p.indices + (int64_t)(t0 + j) * p.width;
      for (int e = tid; e < p.width; e += kQsaThreads) {
        const int id = row[e];
        if (id >= 0) {
          ++cnt;
          lo = min(lo, id);
          hi = max(hi, id);
        }
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
  bool shared = true;   // nothing listed: the shared route writes 0 / -inf
  int U = 0;            // union size
  const int base = hi >= 0 ? lo : 0;
  if (hi >= 0 && hi - lo >= kQsaWin) {
    shared = false;
  } else if (hi >= 0) {
    const int range = hi - lo + 1;
    // ---- pass 2: token bits of every key in [lo, hi] ----
    if (32 * tid < range) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4*>(M + 32 * tid + 4 * i) = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    if constexpr (BITMAP) {
      for (int b = (lo >> 2) + tid; b <= (hi >> 2); b += kQsaThreads) {
        uint32_t mk = 0;
        for (int j = 0; j < nt; ++j)
          mk |= (p.bitmap[(int64_t)(t0 + j) * p.num_blocks + b] != 0 ? 1u : 0u) << j;
        if (mk) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * b + e <= hi) M[4 * b + e - base] = mk;
        }
      }
    } else {
      for (int j = 0; j < nt; ++j) {
        const int32_t* row = p.indices + (int64_t)(t0 + j) * p.width;
        for (int e = tid; e < p.width; e += kQsaThreads) {
          const int id = row[e];
          if (id >= 0) atomicOr(M + (id - base), 1u << j);
        }
      }
    }
    __syncthreads();
    // ---- compaction, ascending: (key offset << 16 | token mask) ----
    uint32_t vals[32];
    int c = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 x = 32 * tid < range ? *reinterpret_cast<const u32x4*>(M + 32 * tid + 4 * i)
                                       : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        vals[4 * i + k] = x[k];
        c += x[k] != 0u;
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
    int before = 0;
#pragma unroll
    for (int i = 0; i < kQsaWaves; ++i) {
      const int s = misc[32 + i];
      before += i < w ? s : 0;
      U += s;
    }
    int rank = before + x - c;
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (vals[i]) M[rank++] = (uint32_t)(32 * tid + i) << 16 | vals[i];
    // the last chunk's padding: no token, key offset 0 (a listed key)
    if (U + tid < ((U + 31) & ~31)) M[U + tid] = 0u;
    __syncthreads();
    shared = (int64_t)kTileCost * U * ((live_waves + 3) >> 2) <= (int64_t)kTokenCost * listed;
  }

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

  bf16x8 qf[8];
  {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) +
                        ((int64_t)(t0 + tl) * p.hq + g * G + hh) * kQsaRowBytes + 16 * q;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qp + 64 * s);
      qf[s] = as_bf16x8(live ? v : u32x4{0, 0, 0, 0});
    }
  }

  const uint8_t* kg = reinterpret_cast<const uint8_t*>(p.k) + (int64_t)g * p.k_head_stride;
  const uint8_t* vg = reinterpret_cast<const uint8_t*>(p.v) + (int64_t)g * p.v_head_stride;
  const uint32_t ring = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const uint32_t mlds = __builtin_amdgcn_readfirstlane(lds_addr(M));
  const float C = p.scale_log2;
  const int nch = (U + 31) >> 5;

  // chunk c's K and V rows into buffer c & 1: wave w stages keys 4 w .. 4 w + 3,
  // two rows per load (lane l: row 4 w + 2 i + l / 32, 16-byte unit l % 32,
  // read from its swizzled source unit)
  auto stage = [&](int c) {
    const uint32_t kb = ring + (c & 1) * 2 * kQsaChunkBytes;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 4 * w + 2 * i + (lane >> 5);
      const uint32_t ent = M[32 * c + r];
      const int64_t id = base + (int)(ent >> 16);
      const int u = lane & 31;
      const uint32_t dst = kb + (4 * w + 2 * i) * kQsaRowBytes;
      g2lds16(kg + id * p.k_row_stride + 16 * (u ^ (r & 15)), dst);
      g2lds16(vg + id * p.v_row_stride + 16 * (u ^ ((r & 7) << 1)), dst + kQsaChunkBytes);
    }
  };

  float m = -INFINITY, l = 0.f;
  f32x4 o[16];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nch > 0) stage(0);
  for (int c = 0; c < nch; ++c) {
    // chunk c has landed for every wave, and every wave is done with chunk
    // c - 1, whose buffer chunk c + 1 now refills
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    block_barrier();
    if (c + 1 < nch) stage(c + 1);
    if (!wave_live) continue;
    const uint32_t kb = ring + (c & 1) * 2 * kQsaChunkBytes;
    const uint32_t vb = kb + kQsaChunkBytes;

    f32x4 acc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint32_t ka = kb + (16 * kt + l16) * kQsaRowBytes;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        acc[kt] = mfma16(as_bf16x8(lds_b128(ka + 16 * ((4 * s + q) ^ l16))), qf[s], acc[kt]);
    }
    // token masks of the eight keys whose scores this lane holds
    const u32x4 ma = lds_b128(mlds + 128 * c + 16 * q);
    const u32x4 mb = lds_b128(mlds + 128 * c + 64 + 16 * q);
    const uint32_t mk[8] = {ma[0], ma[1], ma[2], ma[3], mb[0], mb[1], mb[2], mb[3]};
    float sc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float s = acc[j >> 2][j & 3] * C;
      sc[j] = live && ((mk[j] >> tl) & 1u) ? s : -INFINITY;
    }
    float cm = sc[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) cm = fmaxf(cm, sc[j]);
    cm = xmax_16_32(cm);
    // move the reference max only when a score passes it by the slack (or
    // the row sees its first listed key)
    const bool move = cm > m + kQsaSlack;
    if (__ballot(move)) {
      const float alpha = move ? __builtin_amdgcn_exp2f(m - cm) : 1.f;
      m = move ? cm : m;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) o[dt] *= alpha;
    }
    const float mu = m == -INFINITY ? 0.f : m;   // no listed key yet: p = 0
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      e[j] = __builtin_amdgcn_exp2f(sc[j] - mu);
      l += e[j];
    }
    const bf16x8 pf = as_bf16x8(u32x4{cvt_pk_bf16(e[0], e[1]), cvt_pk_bf16(e[2], e[3]),
                                      cvt_pk_bf16(e[4], e[5]), cvt_pk_bf16(e[6], e[7])});

    // V^T fragments: head dims 16 dt + l % 16; lane 4 e + a of a 16-lane
    // group reads 8 bytes (head dims 16 dt + 4 a ..) of rows 4 q + e and
    // 16 + 4 q + e, found at their swizzled 16-byte units
    const int vrow = 4 * q + (l16 >> 2);
    const int vsw = (vrow & 7) << 1;
    const uint32_t va0 = vb + vrow * kQsaRowBytes + 8 * (l16 & 1);
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      const uint32_t a = va0 + 16 * ((2 * dt + ((l16 & 3) >> 1)) ^ vsw);
      const u32x2 lo2 = lds_tr16(a);
      const u32x2 hi2 = lds_tr16(a + 16 * kQsaRowBytes);
      o[dt] = mfma16(as_bf16x8(u32x4{lo2[0], lo2[1], hi2[0], hi2[1]}), pf, o[dt]);
    }
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
