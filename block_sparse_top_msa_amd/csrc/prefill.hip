// MSA sparse attention, prefill shape, bf16 K/V (msa_sparse_attention page,
// summary: query tiles, each running one online softmax over the union of
// the blocks its tokens selected, writing the output directly).
//
// gfx950 design:
//  * Tile = TOK query tokens of one request x the G query heads of one KV
//    head, as token-major rows cut into 32-row slots; each of NW waves owns
//    SPW slots.  32-row slots because v_mfma_f32_32x32x16_bf16 reads half
//    the LDS operand bytes per FLOP of the 16x16x32 shape and runs ~10%
//    faster per FLOP on this chip (measured: 32 vs ~17.5 cycles per
//    instruction for twice the work).
//  * The tile's block union is built in LDS (tile_union.hpp).  Each union
//    block (128 keys of K and V, 64 KiB) is staged global -> LDS with
//    global_load_lds (16 B per lane, no VGPR staging), double buffered: block
//    u+1 streams in while block u is computed.  Rows are XOR-swizzled in
//    16-byte chunks so every operand read is bank-conflict free with an
//    unpadded 256-byte row pitch.
//  * Per 32-key chunk: S^T = K Q^T (keys on the MFMA M axis, query rows on
//    N), the softmax, and O^T += V^T P^T with P taken straight from the S^T
//    registers; V^T comes from row-major V through the transposing
//    ds_read_b64_tr_b16.  The chunks are software pipelined per wave (the
//    softmax of chunk c runs beside the MFMAs of S^T(c + 1) and of
//    O^T += V^T P^T for chunk c - 1), written as groups of one MFMA, its LDS
//    reads and a few vector instructions so that one wave keeps the matrix
//    core and the vector ALU busy together; O^T += V^T P^T of a block's last
//    chunk runs in the next block.
//  * Softmax: p = exp2(s * c - m) is one FMA + one exp per score against a
//    per-row reference max m, taken from the row's first scores and moved
//    (rescaling O and l) only when a score passes it by more than 64 in log2
//    units, which an overflowing partial row sum reveals without a per-chunk
//    max; row sums stay per lane until the end.  A slot none of whose tokens
//    chose a block skips it (one scalar branch per slot and block).
#include "async_lds.hpp"
#include "common.hpp"
#include "internal.hpp"
#include "tile_union.hpp"

namespace msa {

namespace {

constexpr int kTileBytes = kBlock * kHeadDim * 2;   // 32 KiB of bf16 per side
constexpr float kLn2f = 0.69314718055994530942f;
// log2 units: p = 2^(s - m) <= 2^64.  Safe in bf16 (P operand) and in the
// fp32 O / l accumulators (sums stay far below 2^128), and precision does not
// depend on magnitude, so O is rescaled only if a row's max jumps by more
// than 64 (in log2 units) after its first block.
constexpr float kRescaleSlack = 64.0f;
// A lane's 16 exponentials of a chunk sum to at most 16 * 2^64 while every
// score is within the slack of the reference max.
constexpr float kSumLimit = 0x1p68f;

// fp16 Q/K/V (and P): P holds at most 65504, so the slack drops to 15 and a
// lane's 16 exponentials must sum to at most 2^15 (no single p can pass
// 2^15 unnoticed); bf16 P represents anything below the 2^68 sum limit.
template <bool F16>
struct Soft {
  static constexpr float kSlack = F16 ? 15.0f : kRescaleSlack;
  static constexpr float kLimit = F16 ? 0x1p15f : kSumLimit;
};

template <bool F16>
__device__ __forceinline__ f32x16 mm32(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (F16) return mfma32_f16(a, b, c);
  else return mfma32(a, b, c);
}
template <bool F16>
__device__ __forceinline__ uint32_t pk_p(float lo, float hi) {
  if constexpr (F16) return pack_f16x2(lo, hi);
  else return cvt_pk_bf16(lo, hi);
}

struct PrefillLds {
  uint8_t kv[2][2 * kTileBytes];   // [buffer][K | V]
  UnionLds un;
  int64_t kbase[kMaxUnion];        // byte offset of each union block's row 0 in K
  int64_t vbase[kMaxUnion];        // ... and in V
};

// 16-byte chunk swizzles (chunk index 0..15 within a 256-byte row).  K: the
// 16 consecutive rows one MFMA operand fetch reads per pass land on distinct
// chunks.  V: the four rows a 16-lane transposed read touches land on
// distinct chunk quads.
__device__ __forceinline__ int swz_k(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int swz_v(int r, int c) { return c ^ ((r & 3) << 2); }

typedef short s16x4 __attribute__((ext_vector_type(4)));

// LDS reads through the compiler's builtins: it tracks their completion (LDS
// reads return in order, so it waits with exact lgkmcnt values) and may place
// them among the MFMAs of a scheduling region.
__device__ __forceinline__ u32x4 lds_b128(uint32_t a) {
  return *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)a;
}
// ds_read_b64_tr_b16: in each group of 16 lanes, lane j receives element
// j % 4 of the 8 bytes at lane 4e + j / 4's address, for e = 0..3.
__device__ __forceinline__ u32x2 lds_tr16(uint32_t a) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (__attribute__((address_space(3))) s16x4*)(uintptr_t)a));
}

__device__ __forceinline__ float swap32_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float swap32_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}


// Per-lane LDS addresses of the current block's operands (the buffer's base
// included, moved with it from block to block, so that the chunk and row
// offsets below are instruction immediates).  K fragment ks of 32-key chunk
// c: k[ks] + 8192 c.  V^T fragments of chunk c for head-dim tile dt:
// v[dt] + 8192 c + 2048 e, e = 0..3 (rows r, r + 8, r + 16, r + 24).
struct ChunkAddr {
  uint32_t k[8];
  uint32_t v[4];
};

__device__ __forceinline__ void load_k(u32x4 (&kw)[8], const ChunkAddr& a, int c) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kw[ks] = lds_b128(a.k[ks] + 8192 * c);
}

// O^T += V^T P^T for one chunk (two 16-key k-steps per head-dim tile).
template <bool F16>
__device__ __forceinline__ void pv(f32x16 (&o)[4], const u32x2 (&vv)[16], u32x4 p0, u32x4 p1) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const u32x4 w0 = {vv[4 * dt][0], vv[4 * dt][1], vv[4 * dt + 1][0], vv[4 * dt + 1][1]};
    const u32x4 w1 = {vv[4 * dt + 2][0], vv[4 * dt + 2][1], vv[4 * dt + 3][0], vv[4 * dt + 3][1]};
    o[dt] = mm32<F16>(as_bf16x8(w0), as_bf16x8(p0), o[dt]);
    o[dt] = mm32<F16>(as_bf16x8(w1), as_bf16x8(p1), o[dt]);
  }
}

__device__ __forceinline__ float max16(const f32x16& a) {
  const float x = fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])),
                        fmaxf(fmaxf(a[4], a[5]), fmaxf(a[6], a[7])));
  return fmaxf(x, fmaxf(fmaxf(fmaxf(a[8], a[9]), fmaxf(a[10], a[11])),
                        fmaxf(fmaxf(a[12], a[13]), fmaxf(a[14], a[15]))));
}

// Per-wave pipeline state of one 32-row slot.  It persists across blocks:
// O^T += V^T P^T of a block's last chunk runs in the wave's next active
// block (or after the last one).
struct SlotPipe {
  f32x16 s;        // S^T of the chunk whose softmax comes next
  u32x4 kw[8];     // K fragments of the chunk after that
  u32x2 vv[16];    // V^T fragments of the chunk awaiting O^T += V^T P^T
  u32x4 p0, p1;    // P^T of that chunk
};

// One MFMA of O^T += V^T P^T: head-dim tile g / 2, k-step g % 2 (its V^T
// fragments are vv[2 g] and vv[2 g + 1]).
template <bool F16>
__device__ __forceinline__ void pv_step(f32x16 (&o)[4], const u32x2 (&vv)[16], u32x4 p0, u32x4 p1,
                                        int g) {
  const u32x4 w = {vv[2 * g][0], vv[2 * g][1], vv[2 * g + 1][0], vv[2 * g + 1][1]};
  o[g >> 1] = mm32<F16>(as_bf16x8(w), as_bf16x8((g & 1) ? p1 : p0), o[g >> 1]);
}

// The two V^T fragments vv[2 g], vv[2 g + 1] of chunk c.
__device__ __forceinline__ void load_v2(u32x2 (&vv)[16], const ChunkAddr& a, int c, int g) {
  const uint32_t base = a.v[g >> 1] + 8192 * c + 4096 * (g & 1);
  vv[2 * g] = lds_tr16(base);
  vv[2 * g + 1] = lds_tr16(base + 2048);
}

// MFMA k-step g of S^T (keys x query rows over head dims 16 g .. 16 g + 15).
template <bool F16>
__device__ __forceinline__ f32x16 score_step(f32x16 s, const u32x4 (&kw)[8], const bf16x8 (&qf)[8],
                                             int g) {
  if (g == 0) {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return mm32<F16>(as_bf16x8(kw[0]), qf[0], z);
  }
  return mm32<F16>(as_bf16x8(kw[g]), qf[g], s);
}

// p = 2^(s c - mu) of scores r and r + 1, packed to one bf16 pair of P^T;
// returns their sum.
template <bool F16>
__device__ __forceinline__ float exp_pair(const f32x16& acc, int r, float cs, float mu, uint32_t& pw) {
  const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[r], cs, -mu));
  const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[r + 1], cs, -mu));
  pw = pk_p<F16>(e0, e1);
  return e0 + e1;
}

// The chunk's 16 exponentials, their row sum and P^T, without scheduling
// constraints (rare path).  The sum runs in the common path's order (pair
// sums added one after another), so a row whose reference max did not move
// gets bitwise the same sum whether or not another row of its wave took the
// rare path: a row's result does not depend on the other tokens of its slot.
template <bool F16>
__device__ __forceinline__ float exp_all(const f32x16& acc, float cs, float mu, u32x4& q0, u32x4& q1) {
  float ps[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t w;
    ps[i] = exp_pair<F16>(acc, 2 * i, cs, mu, w);
    if (i < 4) q0[i] = w;
    else q1[i - 4] = w;
  }
  float l = ps[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) l += ps[i];
  return l;
}

// One 32-key chunk C of a block, software pipelined as groups of one MFMA,
// its share of the LDS reads and a few vector-ALU instructions, each group
// closed by a scheduling barrier so that a single wave keeps the matrix core
// busy while it computes the softmax.  The softmax of chunk C reads S^T(C),
// finished half a chunk earlier, and is spread over both halves:
//  * first half: S^T of chunk C + 1 (K(C + 1) was read one chunk earlier)
//    and the reads of V^T(C - 1);
//  * second half: O^T += V^T P^T of chunk C - 1 (for chunk 0: the previous
//    active block's last chunk, or zero), then the reads of K(C + 2) into the
//    registers S^T(C + 1) released, or for chunk 3 the reads of V^T(3) into
//    the registers each MFMA releases.
//
// The exponentials take the row's current reference max m as it stands, with
// no max of the chunk in the common path: a score more than the slack above
// m makes some p exceed 2^64 and the lane's 16-term sum exceed 2^68, which
// sends the row (with rows that have no reference yet) down the rare path.
// There the chunk's row max moves m, O^T (holding chunk C - 1 by then) and l
// are rescaled, and the exponentials are redone.  Without the rare path every
// p stays at most 2^68: exact in bf16 and fp32 range, like the sums.
//
// TEMP: the temperature sum lt += 2^(tau (x - m)) of the same exponents x
// (one multiply, exp and add per score beside e), whose own overflow check
// joins the rare path's; there the reference max moves past `slack`
// (64 / tau for tau > 1), so no temperature term passes 2^64.
template <int C, bool F16, bool TEMP>
__device__ __forceinline__ void prefill_chunk(SlotPipe& sp, f32x16 (&o)[4], float& m, float& l,
                                              float& lt, const bf16x8 (&qf)[8],
                                              const ChunkAddr& ad, bool rowsel, int lim, int hf,
                                              float cs, float tau, float slack) {
  f32x16 acc = sp.s;
  // mask (diagonal / partial block only)
  if (__ballot(rowsel && lim < 32 * C + 31) != 0ull) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * C + 8 * (r >> 2) + 4 * hf + (r & 3);
      acc[r] = key <= lim ? acc[r] : -INFINITY;
    }
  }
  // +inf for rows that take no keys here (p = 0) or have no reference yet
  const float mu = (rowsel && m > -INFINITY) ? m : INFINITY;
  // The softmax work of score r (fma, exp, then pack and sum with r - 1) is
  // skewed over three groups, so that no instruction waits on a result of
  // its own group: group G computes the fma of score G + 2, the exp of
  // score G + 1 and packs the pair ending at G.
  float x[16], e[16], ps[8];
  uint32_t pw[8];
  float lp = 0.f, ltp = 0.f;
  f32x16 sn = sp.s;
  x[0] = __builtin_fmaf(acc[0], cs, -mu);
  x[1] = __builtin_fmaf(acc[1], cs, -mu);
  e[0] = __builtin_amdgcn_exp2f(x[0]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int G = 0; G < 16; ++G) {
    const int g = G & 7;
    if (G < 8) {
      if constexpr (C < 3) sn = score_step<F16>(sn, sp.kw, qf, g);
      if constexpr (C > 0) load_v2(sp.vv, ad, C - 1, g);
    } else {
      pv_step<F16>(o, sp.vv, sp.p0, sp.p1, g);
      if constexpr (C < 2) sp.kw[g] = lds_b128(ad.k[g] + 8192 * (C + 2));
      if constexpr (C == 3) load_v2(sp.vv, ad, 3, g);
    }
    if (G + 2 < 16) x[G + 2] = __builtin_fmaf(acc[G + 2], cs, -mu);
    if (G + 1 < 16) e[G + 1] = __builtin_amdgcn_exp2f(x[G + 1]);
    if constexpr (TEMP) ltp += __builtin_amdgcn_exp2f(tau * x[G]);
    if (G & 1) {
      pw[G >> 1] = pk_p<F16>(e[G - 1], e[G]);
      ps[G >> 1] = e[G - 1] + e[G];
    } else if (G >= 2) {
      lp += ps[(G >> 1) - 1];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (C < 3) sp.s = sn;
  lp += ps[7];
  u32x4 q0 = {pw[0], pw[1], pw[2], pw[3]}, q1 = {pw[4], pw[5], pw[6], pw[7]};
  if (__ballot(rowsel && (m == -INFINITY || !(lp <= Soft<F16>::kLimit) ||
                          (TEMP && !(ltp <= Soft<F16>::kLimit)))) != 0ull) {
    float mx = max16(acc);
    mx = rowsel ? mx * cs : -INFINITY;
    const float mr = swap32_max(mx);   // the row's other 16 keys sit in lane l ^ 32
    // first scores of a row: the max becomes the reference (O and l are
    // still zero); afterwards m moves only when the max passed the slack
    const bool up = mr > m + (TEMP ? slack : Soft<F16>::kSlack);
    if (__ballot(up && m > -INFINITY) != 0ull) {
      const float alpha = up ? __builtin_amdgcn_exp2f(m - mr) : 1.0f;
      l *= alpha;
      if constexpr (TEMP) lt *= up ? __builtin_amdgcn_exp2f(tau * (m - mr)) : 1.0f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    }
    m = up ? mr : m;
    const float mu2 = (rowsel && m > -INFINITY) ? m : INFINITY;
    lp = exp_all<F16>(acc, cs, mu2, q0, q1);
    if constexpr (TEMP) {
      ltp = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) ltp += __builtin_amdgcn_exp2f(tau * __builtin_fmaf(acc[r], cs, -mu2));
    }
  }
  l += lp;
  if constexpr (TEMP) lt += ltp;
  sp.p0 = q0;
  sp.p1 = q1;
}

}  // namespace

template <int NW, int SPW, bool F16, bool TEMP>
__global__ __launch_bounds__(NW * kWave) void msa_prefill_kernel(AttnParams p) {
  constexpr int NT = NW * kWave;
  constexpr int LOADS = 64 / NW;   // 1 KiB load instructions per wave per block
  constexpr int KLOADS = LOADS / 2;
  static_assert(64 % NW == 0 && LOADS <= 63, "64 KiB per block split evenly over waves");
  static_assert((4 * NW) % 16 == 0, "a lane's staged rows keep one swizzle phase");
  __shared__ PrefillLds lds;

  // Workgroup -> (request, KV head, tile).  Workgroups reach the 8 XCDs
  // round-robin by id.  Each (request, KV head) unit keeps to its own XCDs so
  // its K/V stays in their L2, and its tiles are dealt to those XCDs
  // alternately, later (heavier) tiles first, so every XCD gets the same mix.
  const int units = p.batch * p.hkv;
  int unit, jr;
  if (units <= 8 && 8 % units == 0) {
    const int xpu = 8 / units;
    const int x = blockIdx.x % 8, k = blockIdx.x / 8;
    unit = x / xpu;
    jr = k * xpu + x % xpu;
    if (jr >= p.tiles_per_req) return;
  } else {
    const int lid = xcd_remap(blockIdx.x, units * p.tiles_per_req);
    if (lid < 0) return;
    unit = lid / p.tiles_per_req;
    jr = lid % p.tiles_per_req;
  }
  const int g = unit % p.hkv;
  const int b = unit / p.hkv;
  const int j = p.tiles_per_req - 1 - jr;  // later tiles (more visible blocks) first
  const int q0 = p.cu_q[b];
  const int lq = p.cu_q[b + 1] - q0;
  const int i0 = j * p.tok_per_tile;
  if (i0 >= lq) return;
  const int ntok = min(p.tok_per_tile, lq - i0);
  const int lk = p.paged ? p.seqused_k[b] : (p.cu_k[b + 1] - p.cu_k[b]);
  const int nblk = max(0, min((lk + kBlock - 1) / kBlock, p.max_k_tiles));

  const int tid = threadIdx.x;
  // wave-uniform values live in scalar registers, so per-slot decisions are
  // scalar branches rather than exec-masked selects
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int G = p.group;

  const int32_t* rows = p.q2k + ((int64_t)g * p.total_q + q0 + i0) * p.topk;
  const int ucount = __builtin_amdgcn_readfirstlane(
      build_tile_union<NT>(lds.un, rows, ntok, p.topk, nblk));

  const int64_t kst = p.k_st.token, vst = p.v_st.token;
  for (int u = tid; u < ucount; u += NT) {  // page lookups, once per block
    const int t = lds.un.list[u];
    if (p.paged) {
      const int64_t page = p.page_table[(int64_t)b * p.pt_width + t];
      lds.kbase[u] = page * p.k_st.page + g * p.k_st.head;
      lds.vbase[u] = page * p.v_st.page + g * p.v_st.head;
    } else {
      const int64_t row0 = (int64_t)p.cu_k[b] + kBlock * t;
      lds.kbase[u] = row0 * kst + g * p.k_st.head;
      lds.vbase[u] = row0 * vst + g * p.v_st.head;
    }
  }

  // ---- per-slot lane data: lane l owns query row 32 * slot + l % 32
  bf16x8 qf[SPW][8];
  int tk_[SPW], pos_[SPW];
  unsigned long long tokmask[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int slot = wave * SPW + s;
    const int r = 32 * slot + l32;
    const int tk = r / G;
    const int hh = r % G;
    tk_[s] = tk;
    pos_[s] = tk < ntok ? query_pos(p.qpos.rows, p.qpos.mode, p.qpos.base, q0 + i0 + tk, i0 + tk,
                                    lq, lk)
                        : 0;
    const int tfirst = (32 * slot) / G;
    const int tlast = min((32 * slot + 31) / G, ntok - 1);
    unsigned long long m = 0;
    for (int t = tfirst; t <= tlast && t < 64; ++t) m |= 1ull << t;
    tokmask[s] = uniform64((tfirst < ntok) ? m : 0ull);
    if (tk < ntok) {
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(
          p.q + ((int64_t)(q0 + i0 + tk) * p.hq + g * G + hh) * kHeadDim);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        qf[s][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 2 * (16 * ks + 8 * hf)));
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[s][ks] = as_bf16x8(u32x4{0, 0, 0, 0});
    }
  }

  // Settle the Q fragments once: the empty asm takes them as in/out operands,
  // so the loads are waited for here and the loop does not see them as
  // pending (it would otherwise wait on vmcnt inside the loop, where the
  // counter also holds the prefetch of the next block).
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 w = __builtin_bit_cast(u32x4, qf[s][ks]);
      asm volatile("" : "+v"(w));
      qf[s][ks] = as_bf16x8(w);
    }

  float m_[SPW], l_[SPW], lt_[SPW];
  f32x16 o_[SPW][4];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    m_[s] = -INFINITY;
    l_[s] = 0.f;
    lt_[s] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o_[s][dt][r] = 0.f;
  }
  __syncthreads();  // kbase / vbase visible; q loads done

  // Staging: lane l of wave w loads the 16-byte chunk (row r_i, logical
  // chunk c) for physical position (r_i, l % 16), r_i = 4 w + l / 16 + 16 i.
  // Addresses are a scalar base (block start + 16 i rows) plus the lane's
  // 32-bit offset within the row group (token strides are at most 16 MiB).
  const int lr0 = 4 * wave + (lane >> 4);
  const uint32_t koff0 = (uint32_t)(lr0 * kst) + 16 * swz_k(lr0, lane & 15);
  const uint32_t voff0 = (uint32_t)(lr0 * vst) + 16 * swz_v(lr0, lane & 15);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds.kv[0])) + wave * 1024;

  auto issue = [&](int u, int buf) {
    const int t = __builtin_amdgcn_readfirstlane(lds.un.list[u]);
    const int nvalid = min(kBlock, lk - kBlock * t);
    const uint8_t* kb = p.k + (int64_t)uniform64((unsigned long long)lds.kbase[u]);
    const uint8_t* vb = p.v + (int64_t)uniform64((unsigned long long)lds.vbase[u]);
    const uint32_t dst = lds0 + buf * (2 * kTileBytes);
    // recomputed per block from an opaque copy of the lane's row: hoisted out
    // of the loop, the per-row offsets would hold registers through the
    // attention math
    int lr = lr0;
    asm volatile("" : "+v"(lr));
    if (nvalid == kBlock) {
#pragma unroll
      for (int i = 0; i < KLOADS; ++i)
        g2lds16_sv(kb + (int64_t)(4 * NW * i) * kst, koff0, dst + i * NW * 1024);
#pragma unroll
      for (int i = 0; i < KLOADS; ++i)
        g2lds16_sv(vb + (int64_t)(4 * NW * i) * vst, voff0, dst + kTileBytes + i * NW * 1024);
    } else {
      // partial last block: rows past Lk read the block's row 0 instead
      // (finite values; those keys are masked and their P is 0)
#pragma unroll
      for (int i = 0; i < KLOADS; ++i) {
        const int row = lr + 4 * NW * i;
        g2lds16_sv(kb, (uint32_t)((row < nvalid ? row : 0) * kst) + 16 * swz_k(lr, lane & 15),
                   dst + i * NW * 1024);
      }
#pragma unroll
      for (int i = 0; i < KLOADS; ++i) {
        const int row = lr + 4 * NW * i;
        g2lds16_sv(vb, (uint32_t)((row < nvalid ? row : 0) * vst) + 16 * swz_v(lr, lane & 15),
                   dst + kTileBytes + i * NW * 1024);
      }
    }
  };

  const float C = p.scale_log2;
  if (ucount > 0) issue(0, 0);

  // per-lane constant parts of the operand reads.  K: lane l reads row
  // l % 32, logical chunk 2 ks + l / 32.  V^T: 16-lane group q16 covers key
  // half q16 / 2 and head-dim columns 16 * (q16 % 2) + 0..15 of a 32-column
  // tile; its lane 4e + q reads row 4 * half + e, columns 4q..4q+3.
  ChunkAddr ad;
  const uint32_t kv0 = lds_addr(lds.kv[0]);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) ad.k[ks] = kv0 + l32 * 256 + 16 * swz_k(l32, 2 * ks + hf);
  {
    const int q16 = lane >> 4;
    const int vrow = 4 * (q16 >> 1) + ((lane & 15) >> 2);
    const int vchunk = 2 * (q16 & 1) + ((lane & 3) >> 1);
    // the V swizzle depends on the row only through row % 4, the same for
    // rows vrow + 8 i
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      ad.v[dt] = kv0 + kTileBytes + vrow * 256 + 16 * swz_v(vrow, 4 * dt + vchunk) + 8 * (lane & 1);
  }

  static_assert(SPW == 1, "the software-pipelined loop runs one slot per wave");
  const unsigned long long tokmask0 = tokmask[0];
  const int tk0 = tk_[0];
  const int pos0 = pos_[0];

  // the first active block's O^T += V^T P^T of "the previous block" adds
  // zero
  SlotPipe sp;
#pragma unroll
  for (int i = 0; i < 16; ++i) sp.vv[i] = u32x2{0, 0};
  sp.p0 = u32x4{0, 0, 0, 0};
  sp.p1 = u32x4{0, 0, 0, 0};
  for (int u = 0; u < ucount; ++u) {
    const int buf = u & 1;
    const int t = __builtin_amdgcn_readfirstlane(lds.un.list[u]);
    const unsigned long long umask = uniform64(lds.un.mask[u]);
    const int nvalid = min(kBlock, lk - kBlock * t);
    // One barrier per block: past it, every wave's loads of block u have
    // landed and every wave has finished reading block u - 1, whose buffer
    // the prefetch of block u + 1 then refills.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    block_barrier();
    if (u + 1 < ucount) issue(u + 1, buf ^ 1);

    const bool rowsel = (tk0 < ntok) && ((umask >> tk0) & 1ull);
    int lim = nvalid - 1;
    if (p.causal) lim = min(lim, pos0 - kBlock * t);

    if ((umask & tokmask0) != 0ull) {
      // prologue: S^T of chunk 0; K(1) reads refill K(0)'s registers as the
      // MFMAs release them
      load_k(sp.kw, ad, 0);
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        sp.s = score_step<F16>(sp.s, sp.kw, qf[0], g);
        sp.kw[g] = lds_b128(ad.k[g] + 8192);
        __builtin_amdgcn_sched_barrier(0);
      }
      prefill_chunk<0, F16, TEMP>(sp, o_[0], m_[0], l_[0], lt_[0], qf[0], ad, rowsel, lim, hf, C,
                                  p.tau, p.tslack);
      prefill_chunk<1, F16, TEMP>(sp, o_[0], m_[0], l_[0], lt_[0], qf[0], ad, rowsel, lim, hf, C,
                                  p.tau, p.tslack);
      prefill_chunk<2, F16, TEMP>(sp, o_[0], m_[0], l_[0], lt_[0], qf[0], ad, rowsel, lim, hf, C,
                                  p.tau, p.tslack);
      prefill_chunk<3, F16, TEMP>(sp, o_[0], m_[0], l_[0], lt_[0], qf[0], ad, rowsel, lim, hf, C,
                                  p.tau, p.tslack);
    }
    // the operand addresses move to the other buffer
    const uint32_t step = buf ? (uint32_t)(-2 * kTileBytes) : (uint32_t)(2 * kTileBytes);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ad.k[ks] += step;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) ad.v[dt] += step;
  }
  // O^T += V^T P^T of the last active block's last chunk
  pv<F16>(o_[0], sp.vv, sp.p0, sp.p1);

  // ---- epilogue: out = O / l * v_gs (bf16), lse = (m + log2 l) * ln 2.
  // Lane quantities are recomputed from an opaque copy of the thread id:
  // carried over from the prologue they would hold registers through the
  // loop.
  int etid = threadIdx.x;
  asm volatile("" : "+v"(etid));
  const int el32 = etid & 31, ehf = (etid >> 5) & 1;
  const int out_row0 = q0 + i0;
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const float lsum = swap32_sum(l_[s]);
    const int slot = wave * SPW + s;
    const int r = 32 * slot + el32;
    const int tk = r / G;
    if (tk >= ntok) continue;
    const int hh = r % G;
    const int64_t row = (int64_t)(out_row0 + tk) * p.hq + g * G + hh;
    const float inv = lsum > 0.f ? p.v_gs / lsum : 0.f;
    uint16_t* op = p.out + row * kHeadDim + 4 * ehf;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x2*>(op + 32 * dt + 8 * q) =
            F16 ? u32x2{pack_f16x2(o_[s][dt][4 * q] * inv, o_[s][dt][4 * q + 1] * inv),
                        pack_f16x2(o_[s][dt][4 * q + 2] * inv, o_[s][dt][4 * q + 3] * inv)}
                : u32x2{pack_bf16x2(o_[s][dt][4 * q] * inv, o_[s][dt][4 * q + 1] * inv),
                        pack_bf16x2(o_[s][dt][4 * q + 2] * inv, o_[s][dt][4 * q + 3] * inv)};
    if (p.lse && ehf == 0)
      p.lse[row] = lsum > 0.f ? (m_[s] + __log2f(lsum)) * kLn2f : -INFINITY;
    if constexpr (TEMP) {
      const float ltsum = swap32_sum(lt_[s]);
      if (ehf == 0)
        p.lse_t[row] = (lsum > 0.f && ltsum > 0.f) ? (p.tau * m_[s] + __log2f(ltsum)) * kLn2f
                                                   : -INFINITY;
    }
  }
}

template <int NW, int SPW, bool F16, bool TEMP>
static hipError_t launch_prefill_t(const AttnParams& p, hipStream_t stream) {
  const int units = p.batch * p.hkv;
  if (units <= 0 || p.tiles_per_req <= 0) return hipSuccess;
  int grid;
  if (units <= 8 && 8 % units == 0) {
    const int xpu = 8 / units;
    grid = 8 * ((p.tiles_per_req + xpu - 1) / xpu);
  } else {
    const int n = units * p.tiles_per_req;
    grid = 8 * ((n + 7) / 8);
  }
  hipLaunchKernelGGL((msa_prefill_kernel<NW, SPW, F16, TEMP>), dim3(grid), dim3(NW * kWave), 0,
                     stream, p);
  return hipGetLastError();
}

// Tiles of 256 rows: 8 waves x one 32-row slot.
hipError_t launch_prefill_bf16(const AttnParams& p, hipStream_t stream) {
  if (p.lse_t)
    return p.out_f16 ? launch_prefill_t<8, 1, true, true>(p, stream)
                     : launch_prefill_t<8, 1, false, true>(p, stream);
  return p.out_f16 ? launch_prefill_t<8, 1, true, false>(p, stream)
                   : launch_prefill_t<8, 1, false, false>(p, stream);
}

}  // namespace msa
