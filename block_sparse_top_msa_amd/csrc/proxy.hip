// MSA stage 1 on gfx950: max_score[h, t, i] = max over the keys of block t of
// the unscaled, causally masked q[i, h] . k[j, h / G] (msa_proxy_score page,
// summary).  -inf where the block is past the sequence or wholly above the
// causal limit.  No softmax and no V.
//
// A workgroup owns a tile of query rows (token x head of one KV head, token
// major) and a chunk of KV blocks.  Each block is staged once into LDS as bf16
// (fp8 K upconverted in-kernel, msa_proxy_score page, Parameters: k) and read
// by every wave.  S^T = K Q^T on 32x32x16 bf16 MFMA puts keys on the M axis,
// so a query's block max is a max over its own registers plus one cross-half
// step.  With reduce_heads (all heads, or the G heads of each KV head) the
// max over query heads happens in-kernel: within
// a wave across the G heads of a token, then across KV heads with an exact
// order-independent atomic max into an output pre-filled with -inf.
#include <climits>
#include <type_traits>

#include "async_lds.hpp"
#include "common.hpp"
#include "internal.hpp"
#include "topk.hpp"

namespace msa {

// ---------------------------------------------------------------------------
// Decode-shaped proxy (at most 64 query rows per request and KV head, e.g.
// a few MTP tokens x G heads): HBM-bound, every K page is read once.  Each
// wave scores whole blocks (t_beg + wave, + 4, ...) on its own, without
// barriers: the blocks stream global -> LDS (global_load_lds, raw bytes)
// through a per-wave stage of one block, refilled 32 keys at a time: as soon
// as a 32-key chunk has been read into registers the same chunk of the
// wave's next block is requested, so close to a block's worth of loads stays
// in flight through the scoring.  Lane (key l % 32, half l / 32) then reads its key row's bytes for
// head dims 64 half .. 64 half + 63; with the same permutation of the head
// dimension on Q that is exactly the A operand of S^T = K Q^T on 32x32x16
// MFMA (k-step s covers dims 64 half + 8 s ..).  fp8 K is converted in
// registers.  Page ids of the workgroup's blocks are looked up once, into LDS.
// ---------------------------------------------------------------------------
template <int FMT>
struct RowsGeom;
template <>
struct RowsGeom<kFmtFp8> {
  static constexpr int kRow = 128;
  static constexpr int kStage = kBlock * kRow;   // 16 KiB
  static constexpr int kLoads = kStage / 1024;
  static constexpr int kLaneBytes = 64;          // per lane and 32-key chunk
};
template <>
struct RowsGeom<kFmtBf16> {
  static constexpr int kRow = 256;
  static constexpr int kStage = kBlock * kRow;   // 32 KiB
  static constexpr int kLoads = kStage / 1024;
  static constexpr int kLaneBytes = 128;
};

constexpr int kRowsMaxBpw = 32;   // blocks per workgroup on this path

template <>
struct RowsGeom<kFmtF16> : RowsGeom<kFmtBf16> {};   // fp16 rows: same bytes as bf16

template <int FMT>
struct RowsLds {
  uint8_t ring[4 * RowsGeom<FMT>::kStage];   // [wave]: one block
  int32_t page[kRowsMaxBpw];
  // block maxima per wave, block and row: written out after the block loop,
  // so that no global store or atomic (counted by vmcnt like the staging
  // loads) is issued between a page's loads and the wait for them
  float res[4][kRowsMaxBpw / 4][64];
};

__device__ __forceinline__ bf16x8 fp8x8_bf16(uint32_t w0, uint32_t w1) {
  return as_bf16x8(u32x4{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))});
}

// fp16 proxy Q and K run on the fp16 MFMA; bf16 and fp8 K on the bf16 one.
template <int FMT>
__device__ __forceinline__ f32x16 mm32(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (FMT == kFmtF16) return mfma32_f16(a, b, c);
  else return mfma32(a, b, c);
}

__device__ __forceinline__ float max16(const f32x16& a) {
  return fmaxf(fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])),
                     fmaxf(fmaxf(a[4], a[5]), fmaxf(a[6], a[7]))),
               fmaxf(fmaxf(fmaxf(a[8], a[9]), fmaxf(a[10], a[11])),
                     fmaxf(fmaxf(a[12], a[13]), fmaxf(a[14], a[15]))));
}

// Four 16-byte LDS reads, waited for (outputs early-clobber).
__device__ __forceinline__ void lds_rd4(u32x4 (&k)[4], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}

// Four 16-byte LDS reads, not waited for (outputs early-clobber); pair with
// lds_wait4 on the same registers before their use.
__device__ __forceinline__ void lds_rd4_issue(u32x4 (&k)[4], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}
// Same, at a[j] + OFF (the instruction's immediate offset).
template <int OFF>
__device__ __forceinline__ void lds_rd4_issue_at(u32x4 (&k)[4], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%8\n\t"
      "ds_read_b128 %1, %5 offset:%8\n\t"
      "ds_read_b128 %2, %6 offset:%8\n\t"
      "ds_read_b128 %3, %7 offset:%8"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "n"(OFF));
}
__device__ __forceinline__ void lds_wait4(u32x4 (&k)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]));
}

__device__ __forceinline__ uint32_t lds_addr32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// fp8 stages fit two workgroups per CU (256 VGPRs per wave); bf16 stages
// take the LDS of one, whose waves may then use the whole register file.
//
// FUSE (running top-K, msa_proxy_score page, Parameters: reduce_heads: the
// reduction and the selection folded into the kernel): no score is written;
// per query, the workgroup takes the maximum over its KV head's query heads
// of each of its chunk's blocks and writes that chunk's top-K (score, block
// id) candidates, ascending, -1 padded; the merge kernel then selects the
// row's top-K from every chunk's (and, for a selection shared by all heads,
// every KV head's) candidates.
template <int NT, int FMT, bool REDUCE, bool FUSE = false>
__global__ __launch_bounds__(256, FMT == kFmtFp8 ? 2 : 1) void msa_proxy_rows_kernel(ProxyParams p) {
  using Geo = RowsGeom<FMT>;
  constexpr int LOADS = Geo::kLoads;
  constexpr int QL = LOADS / 4;   // loads per 32-key chunk
  __shared__ __attribute__((aligned(16))) RowsLds<FMT> lds;

  const int chunk = blockIdx.x % p.block_chunks;
  const int rest = blockIdx.x / p.block_chunks;
  const int g = rest % p.hkv;
  const int b = rest / p.hkv;
  if (b >= p.batch) return;

  const int G = p.group;
  // reduced output row block: all heads -> row 0, group of KV head g -> row g
  const int64_t rbase = p.reduce == 2 ? (int64_t)g * p.max_k_tiles : 0;
  const int q0 = p.cu_q[b];
  const int lq = p.cu_q[b + 1] - q0;
  const int nrows = lq * G;
  if (nrows <= 0) return;
  const int lk = p.paged ? p.seqused_k[b] : (p.cu_k[b + 1] - p.cu_k[b]);
  const int nblk = max(0, (lk + kBlock - 1) / kBlock);
  const int t_beg = chunk * p.blocks_per_wg;
  const int t_end = min(t_beg + p.blocks_per_wg, p.max_k_tiles);
  if (t_beg >= t_end) return;
  // causal positions of the first and last token (bounds of the block
  // range and of fully visible blocks); per-row positions have no order,
  // so they bound nothing
  const bool rowpos = p.qpos.mode == 2;
  const int pos0 = query_pos(p.qpos.rows, p.qpos.mode, p.qpos.base, q0, 0, lq, lk);
  const int pos_min = rowpos ? INT_MIN : pos0;
  const int pos_max = rowpos ? INT_MAX : pos0 + (nrows - 1) / G;
  int t_act = min(t_end, nblk);
  if (p.paged) t_act = min(t_act, p.pt_width);
  if (p.causal) t_act = min(t_act, pos_max < 0 ? 0 : pos_max / kBlock + 1);
  t_act = max(t_act, t_beg);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid & (kWave - 1);
  const int col = lane & 31;
  const int half = lane >> 5;

  // page ids (paged) or first rows (flat) of the workgroup's visible blocks
  for (int i = tid; i < t_act - t_beg; i += 256) {
    const int t = t_beg + i;
    lds.page[i] = p.paged ? p.page_table[(int64_t)b * p.pt_width + t] : p.cu_k[b] + kBlock * t;
  }

  int row_[NT], pos_[NT];
  bf16x8 qf[NT][8];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = 32 * nt + col;
    row_[nt] = r;
    const int tk = r / G, hh = r % G;
    pos_[nt] = r < nrows ? query_pos(p.qpos.rows, p.qpos.mode, p.qpos.base, q0 + tk, tk, lq, lk) : 0;
    if (r < nrows) {
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(
          p.q + ((int64_t)(q0 + tk) * p.hq + g * G + hh) * kHeadDim) + 128 * half;
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[nt][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * s));
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[nt][s] = as_bf16x8(u32x4{0, 0, 0, 0});
    }
  }

  // blocks of the chunk with no visible key: -inf (pre-filled when reducing)
  if (!REDUCE && !FUSE && half == 0) {
    for (int t = t_act + wave; t < t_end; t += 4) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int r = row_[nt];
        if (r < nrows)
          p.out[((int64_t)(g * G + r % G) * p.max_k_tiles + t) * p.total_q + q0 + r / G] = -INFINITY;
      }
    }
  }
  // settle the Q loads; page ids visible
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 w = __builtin_bit_cast(u32x4, qf[nt][s]);
      asm volatile("" : "+v"(w));
      qf[nt][s] = as_bf16x8(w);
    }
  __syncthreads();

  const int64_t kst = p.k_st.token;
  const uint32_t wring = __builtin_amdgcn_readfirstlane(lds_addr32(lds.ring)) +
                         wave * Geo::kStage;
  // this wave's blocks: t_beg + wave + 4 i, i < nb
  const int nb = t_act - t_beg > wave ? (t_act - t_beg - wave + 3) / 4 : 0;

  // stage block i of this wave: load nn writes LDS bytes [1024 nn, +1024),
  // rows RPL nn .. (RPL rows per load, LPR lanes per row), XOR-swizzled in
  // 16-byte chunks (conflict-free operand reads)
  constexpr int LPR = Geo::kRow / 16;          // lanes per row
  constexpr int RPL = 64 / LPR;                // rows per load
  constexpr int SW = FMT == kFmtFp8 ? 8 : 16;  // swizzle period (rows)
  // chunk c (keys 32 c .. 32 c + 31) of block i of this wave: loads
  // QL c .. QL c + QL - 1 (scalar block base + 32-bit lane offsets; token
  // strides are at most 16 MiB); rows past the sequence end load row 0
  // (masked)
  auto issue = [&](int i, int c) {
    const int t = t_beg + wave + 4 * i;
    const int pg = __builtin_amdgcn_readfirstlane(lds.page[t - t_beg]);
    const int nvalid = min(kBlock, lk - kBlock * t);
    const uint8_t* base = reinterpret_cast<const uint8_t*>(uniform64((unsigned long long)(
        p.paged ? p.k + (int64_t)pg * p.k_st.page + g * p.k_st.head
                : p.k + (int64_t)pg * kst + g * p.k_st.head)));
#pragma unroll
    for (int n2 = 0; n2 < QL; ++n2) {
      const int nn = QL * c + n2;
      const int row = RPL * nn + lane / LPR;
      const int c = (lane % LPR) ^ (row % SW);
      const int rr = row < nvalid ? row : 0;
      g2lds16_sv(base, (uint32_t)(rr * kst) + 16u * (uint32_t)c, wring + 1024 * nn);
    }
  };

  constexpr int LB = Geo::kLaneBytes / 16;   // 16-byte pieces per lane and chunk
  // lane's key row 32 c + col of chunk c: bytes of head dims 64 half ..
  // 64 half + 63
  auto read_chunk = [&](uint32_t sb, int c, u32x4 (&kr)[LB]) {
    const int row = 32 * c + col;
#pragma unroll
    for (int j0 = 0; j0 < LB; j0 += 4) {
      uint32_t a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int lc = LB * half + j0 + j;   // logical 16-byte chunk of the row
        const int pc = FMT == kFmtFp8 ? (lc ^ (row & 7)) : (lc ^ (row & 15));
        a[j] = sb + row * Geo::kRow + 16 * pc;
      }
      u32x4 w[4];
      lds_rd4(w, a);
#pragma unroll
      for (int j = 0; j < 4; ++j) kr[j0 + j] = w[j];
    }
  };

  // block max of chunk c into bm: NT independent accumulator chains
  auto score_chunk = [&](int t, int c, const u32x4 (&kr)[LB], float (&bm)[NT]) {
    const int nvalid = min(kBlock, lk - kBlock * t);
    const bool full = nvalid == kBlock && (!p.causal || pos_min >= kBlock * t + kBlock - 1);
    f32x16 acc[NT];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 a;
      if constexpr (FMT == kFmtFp8) {
        const u32x4 w = kr[s >> 1];
        a = (s & 1) ? fp8x8_bf16(w[2], w[3]) : fp8x8_bf16(w[0], w[1]);
      } else {
        a = as_bf16x8(kr[s]);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (s == 0) {
          f32x16 z;
#pragma unroll
          for (int r = 0; r < 16; ++r) z[r] = 0.f;
          acc[nt] = mm32<FMT>(a, qf[nt][s], z);
        } else {
          acc[nt] = mm32<FMT>(a, qf[nt][s], acc[nt]);
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (!full) {
        int lim = nvalid - 1;
        if (p.causal) lim = min(lim, pos_[nt] - kBlock * t);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * c + 8 * (r >> 2) + 4 * half + (r & 3);
          acc[nt][r] = key <= lim ? acc[nt][r] : -INFINITY;
        }
      }
      bm[nt] = fmaxf(bm[nt], max16(acc[nt]));
    }
  };

  // wait until at most `left` quarters of this wave's loads are outstanding
  auto wait_left = [&](int left) {
    if (left >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * QL) : "memory");
    else if (left == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * QL) : "memory");
    else if (left == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(QL) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  if (nb > 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) issue(0, c);
  }
  for (int i = 0; i < nb; ++i) {
    const bool next = i + 1 < nb;
    const int t = t_beg + wave + 4 * i;
    float bm[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bm[nt] = -INFINITY;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // chunk c landed: behind it in flight are the block's later chunks
      // and the next block's chunks requested so far (three in all)
      wait_left(next ? 3 : 3 - c);
      u32x4 kr[LB];
      read_chunk(wring, c, kr);
      if (next) issue(i + 1, c);   // read: the chunk's rows take the next block's
      score_chunk(t, c, kr, bm);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float v = xor_max(bm[nt], 32);
      if (half == 0) lds.res[wave][i][32 * nt + col] = v;
    }
  }

  if constexpr (FUSE) {
    // ---- the chunk's top-K per query: every wave's block maxima visible
    __syncthreads();
    const int K = p.topk;
    const int nch = t_end - t_beg;                 // <= 32 blocks: lane = block
    const int sel = p.reduce == 1 ? 0 : g;         // selection row
    const int Hg = p.reduce == 1 ? p.hkv : 1;      // KV heads folded into it
    const int hgi = p.reduce == 1 ? g : 0;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    for (int tk = wave; tk < lq; tk += 4) {
      const int t = t_beg + lane;
      float s = -INFINITY;
      if (lane < nch && t < t_act) {
        // block t = t_beg + w + 4 i was scored by wave w, slot i
        const int w = lane & 3, i = lane >> 2;
        for (int hh = 0; hh < G; ++hh) s = fmaxf(s, lds.res[w][i][tk * G + hh]);
      }
      uint32_t key[1];
      bool valid[1], chosen[1];
      valid[0] = lane < nch && (__float_as_uint(s) & 0x7F800000u) != 0x7F800000u;
      key[0] = valid[0] ? ordered_f32(s) : 0u;
      select_topk<1>(key, valid, K, lane, chosen);
      const int64_t base =
          (((int64_t)sel * p.total_q + q0 + tk) * Hg + hgi) * p.block_chunks * K + (int64_t)chunk * K;
      const unsigned long long m = __ballot(chosen[0]);
      if (chosen[0]) {
        const int pos = popc64(m & below);
        p.cand_s[base + pos] = s;
        p.cand_id[base + pos] = t;
      }
      for (int k = popc64(m) + lane; k < K; k += kWave) {
        p.cand_s[base + k] = -INFINITY;
        p.cand_id[base + k] = -1;
      }
    }
    return;
  }

  // ---- results of this wave's blocks (its own LDS rows: no barrier)
  for (int i = 0; i < nb; ++i) {
    const int t = t_beg + wave + 4 * i;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = row_[nt];
      const int tk = r / G, hh = r % G;
      float v = lds.res[wave][i][32 * nt + col];
      if constexpr (!REDUCE) {
        if (half == 0 && r < nrows)
          p.out[((int64_t)(g * G + hh) * p.max_k_tiles + t) * p.total_q + q0 + tk] = v;
      } else {
        // max over the G heads of a token when they share 32 lanes, then
        // across KV heads (other workgroups) by atomic max
        if ((G & (G - 1)) == 0 && G <= 32) {
          for (int off = 1; off < G; off <<= 1) v = xor_max(v, off);
          if (half == 0 && r < nrows && hh == 0)
            atomic_max_f32(&p.out[(rbase + t) * p.total_q + q0 + tk], v);
        } else if (half == 0 && r < nrows) {
          atomic_max_f32(&p.out[(rbase + t) * p.total_q + q0 + tk], v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill-shaped proxy (many query rows): MFMA-bound.  A workgroup scores
// tiles of 256 query rows (4 waves x 64, token x head of one KV head)
// against an equal share of a row-tile pair's visible KV blocks (see the
// work mapping below).  Each block's K streams global -> LDS with
// global_load_lds (raw bytes, XOR-swizzled rows, double buffered, one
// barrier per block); lane (key l % 32, half l / 32) reads its key row's
// bytes for head dims 64 half .. 64 half + 63 in the A-operand layout of
// 32x32x16 MFMA (Q uses the same head-dim permutation), fp8 converted in
// registers.  Per block and wave: 4 key subtiles x 2 row tiles x 8 k-steps,
// the two row tiles' chains interleaved, and the previous subtile's row
// maxima issued between them; block maxima go out as coalesced rows.
// ---------------------------------------------------------------------------
template <int FMT, bool REDUCE>
__global__ __launch_bounds__(256, 2) void msa_proxy_wide_kernel(ProxyParams p) {
  using Geo = RowsGeom<FMT>;
  constexpr int LB = Geo::kLaneBytes / 16;   // 16-byte pieces per lane and key subtile
  constexpr int LOADS = Geo::kStage / 4096;  // 1 KiB loads per wave per block
  constexpr int SW = FMT == kFmtFp8 ? 8 : 16;
  __shared__ __attribute__((aligned(16))) uint8_t ring[2][Geo::kStage];
  __shared__ int64_t kbase[kWideMaxSeg];

  // Workgroup -> (request, KV head, row-tile pair, piece).  Row tile rt is
  // paired with its reflection R - 1 - rt: under the causal mask their
  // visible blocks add up to about the same count for every pair, so cutting
  // each pair's blocks into P equal pieces gives every workgroup the same
  // work (two per CU, both busy to the end).  A pair's pieces run on one XCD,
  // so its Q tiles and K blocks are fetched into that L2 once.
  const int pairs = (p.row_tiles + 1) / 2;
  const int P = p.pieces;
  const int units = p.batch * p.hkv;
  int unit, pi, piece;
  if (units <= 8 && 8 % units == 0) {
    // each (request, KV head) keeps to 8 / units XCDs
    const int xpu = 8 / units;
    const int x = blockIdx.x % 8, k = blockIdx.x / 8;
    unit = x / xpu;
    pi = (k / P) * xpu + x % xpu;
    piece = k % P;
    if (pi >= pairs) return;
  } else {
    const int lid = xcd_remap(blockIdx.x, units * pairs * P);
    if (lid < 0) return;
    piece = lid % P;
    pi = (lid / P) % pairs;
    unit = lid / P / pairs;
  }
  const int g = unit % p.hkv;
  const int b = unit / p.hkv;

  const int G = p.group;
  // reduced output row block: all heads -> row 0, group of KV head g -> row g
  const int64_t rbase = p.reduce == 2 ? (int64_t)g * p.max_k_tiles : 0;
  const int q0 = p.cu_q[b];
  const int lq = p.cu_q[b + 1] - q0;
  const int nrows = lq * G;
  const int lk = p.paged ? p.seqused_k[b] : (p.cu_k[b + 1] - p.cu_k[b]);
  const int nblk = max(0, (lk + kBlock - 1) / kBlock);
  const bool rowpos = p.qpos.mode == 2;
  const int pos0 = query_pos(p.qpos.rows, p.qpos.mode, p.qpos.base, q0, 0, lq, lk);
  // blocks 0 .. visible(rt) - 1 hold a key some row of tile rt may see;
  // per-row positions have no order, so they bound nothing
  auto visible = [&](int rt) {
    const int r0 = rt * 256;
    if (r0 >= nrows) return 0;
    const int pos_max = rowpos ? INT_MAX : pos0 + (min(r0 + 256, nrows) - 1) / G;
    int v = min(nblk, p.max_k_tiles);
    if (p.paged) v = min(v, p.pt_width);
    if (p.causal) v = min(v, pos_max < 0 ? 0 : pos_max / kBlock + 1);
    return max(v, 0);
  };
  const int rta = pi, rtb = p.row_tiles - 1 - pi;
  const int va = visible(rta);
  const int vb = rtb != rta ? visible(rtb) : 0;
  const int64_t cost = (int64_t)va + vb;
  // The piece that runs over from tile rta into rtb pays a second start (its
  // Q rows and first K block): it is counted as kSegSwitch blocks more, so
  // that piece takes fewer blocks (the cut points move over a virtual gap at
  // the tile boundary; every block still falls in exactly one piece).
  const int pen = (va > 0 && vb > 0) ? kSegSwitch : 0;
  const int64_t ext = cost + pen;
  auto cut = [&](int64_t x) { return (int)(x < va ? x : (x < va + pen ? va : x - pen)); };
  const int s_lo = cut(ext * piece / P), s_hi = cut(ext * (piece + 1) / P);

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int64_t kst = p.k_st.token;
  // lane quantities are recomputed from the lane id where they are used
  // (read through a volatile asm, so not hoisted): kept from the prologue
  // they would hold registers through the block loop
  auto lane_id = [] {
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    return ln;
  };

  // blocks with no visible key: -inf (pre-filled when reducing), written by
  // the pair's first piece
  if (!REDUCE && piece == 0 && lane_id() < 32) {
    const int col = lane_id() & 31;
    for (int h2 = 0; h2 < (rtb != rta ? 2 : 1); ++h2) {
      const int r0 = (h2 ? rtb : rta) * 256;
      for (int t = h2 ? vb : va; t < p.max_k_tiles; ++t) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int r = r0 + 64 * wave + 32 * nt + col;
          if (r < nrows)
            p.out[((int64_t)(g * G + r % G) * p.max_k_tiles + t) * p.total_q + q0 + r / G] = -INFINITY;
        }
      }
    }
  }

  // the piece's blocks: [s_lo, s_hi) of tile rta's visible blocks followed
  // by tile rtb's
  for (int seg = 0; seg < 2; ++seg) {
  const int rt = seg ? rtb : rta;
  const int t_beg = seg ? max(s_lo - va, 0) : s_lo;
  const int t_act = seg ? s_hi - va : min(s_hi, va);
  if (t_beg >= t_act) continue;
  const int r0 = rt * 256;
  const int pos_min = rowpos ? INT_MIN : pos0 + r0 / G;
  const int lane = lane_id();
  const int tid = wave * kWave + lane;
  const int col = lane & 31;
  const int half = lane >> 5;

  for (int i = tid; i < t_act - t_beg; i += 256) {
    const int t = t_beg + i;
    if (p.paged) {
      const int64_t page = p.page_table[(int64_t)b * p.pt_width + t];
      kbase[i] = page * p.k_st.page + g * p.k_st.head;
    } else {
      kbase[i] = ((int64_t)p.cu_k[b] + kBlock * t) * kst + g * p.k_st.head;
    }
  }

  // rows of this wave: r0 + 64 wave + 32 nt + col
  int pos_[2];
  bf16x8 qf[2][8];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = r0 + 64 * wave + 32 * nt + col;
    const int tk = r / G, hh = r % G;
    pos_[nt] = r < nrows ? query_pos(p.qpos.rows, p.qpos.mode, p.qpos.base, q0 + tk, tk, lq, lk) : 0;
    if (r < nrows) {
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(
          p.q + ((int64_t)(q0 + tk) * p.hq + g * G + hh) * kHeadDim) + 128 * half;
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[nt][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * s));
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[nt][s] = as_bf16x8(u32x4{0, 0, 0, 0});
    }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 w = __builtin_bit_cast(u32x4, qf[nt][s]);
      asm volatile("" : "+v"(w));
      qf[nt][s] = as_bf16x8(w);
    }
  __syncthreads();   // kbase visible; Q loads and stores settled

  // staging: load nn of wave w fills LDS bytes [1024 (4 nn + w), + 1024) of
  // the buffer; rows of kRow bytes, XOR-swizzled in 16-byte chunks
  constexpr int LPR = Geo::kRow / 16;   // lanes per row
  constexpr int RPL = 64 / LPR;         // rows per load
  const uint32_t ring0 = __builtin_amdgcn_readfirstlane(lds_addr32(&ring[0][0]));
  // (scalar block base + 32-bit lane offsets; token strides are at most
  // 16 MiB)
  static_assert((4 * RPL) % SW == 0, "a wave's staged rows keep one swizzle phase");
  auto issue = [&](int t, int buf) {
    const int i = t - t_beg;
    const int nvalid = min(kBlock, lk - kBlock * t);
    const uint8_t* base = p.k + (int64_t)uniform64((unsigned long long)kbase[i]);
    // lane offsets recomputed per block from the lane id, read again here
    // (volatile, so not hoisted): kept from the prologue, it and the offsets
    // would hold registers through the MFMAs
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    if (nvalid == kBlock) {
      // load nn of wave w stages rows RPL (4 nn + w) + l / LPR: their
      // swizzle phase is the same for every nn, so one lane offset serves
      // all loads and the row step goes into the scalar base
      const int row0 = RPL * wave + ln / LPR;
      const uint32_t voff = (uint32_t)((ln / LPR) * kst) + 16u * (uint32_t)((ln % LPR) ^ (row0 % SW));
#pragma unroll
      for (int nn = 0; nn < LOADS; ++nn) {
        const int ld = 4 * nn + wave;
        g2lds16_sv(base + (int64_t)(RPL * ld) * kst, voff, ring0 + buf * Geo::kStage + 1024 * ld);
      }
    } else {
#pragma unroll
      for (int nn = 0; nn < LOADS; ++nn) {
        const int ld = 4 * nn + wave;
        const int row = RPL * ld + ln / LPR;
        const int c = (ln % LPR) ^ (row % SW);
        const int rr = row < nvalid ? row : 0;   // past the end: row 0 (masked)
        g2lds16_sv(base, (uint32_t)(rr * kst) + 16 * c, ring0 + buf * Geo::kStage + 1024 * ld);
      }
    }
  };

  if (t_beg < t_act) issue(t_beg, 0);
  for (int t = t_beg; t < t_act; ++t) {
    const int buf = (t - t_beg) & 1;
    if (t + 1 < t_act) {
      issue(t + 1, buf ^ 1);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    const int nvalid = min(kBlock, lk - kBlock * t);
    const bool full = nvalid == kBlock && (!p.causal || pos_min >= kBlock * t + kBlock - 1);
    const uint32_t sb = ring0 + buf * Geo::kStage;
    float bm[2] = {-INFINITY, -INFINITY};
    // Software pipeline over the 4 key subtiles: the LDS reads of subtile
    // kt + 1 and the row maxima of subtile kt - 1 overlap the MFMAs of kt.
    u32x4 kr[2][LB];
    // lane's row col of subtile 0; subtile kt is 32 kt rows further, with
    // the same swizzle phase (32 is a multiple of SW), so its reads take
    // the same addresses plus an immediate offset
    uint32_t ka[LB];
#pragma unroll
    for (int j = 0; j < LB; ++j) ka[j] = sb + col * Geo::kRow + 16 * ((LB * half + j) ^ (col % SW));
    // (kt is a constant once the subtile loop is unrolled)
    auto kread = [&](int kt, u32x4 (&dst)[LB]) {
#pragma unroll
      for (int j0 = 0; j0 < LB; j0 += 4) {
        const uint32_t a[4] = {ka[j0], ka[j0 + 1], ka[j0 + 2], ka[j0 + 3]};
        u32x4 w[4];
        switch (kt) {
          case 0: lds_rd4_issue_at<0>(w, a); break;
          case 1: lds_rd4_issue_at<32 * Geo::kRow>(w, a); break;
          case 2: lds_rd4_issue_at<64 * Geo::kRow>(w, a); break;
          default: lds_rd4_issue_at<96 * Geo::kRow>(w, a); break;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j0 + j] = w[j];
      }
    };
    auto kwait = [&](u32x4 (&dst)[LB]) {
#pragma unroll
      for (int j0 = 0; j0 < LB; j0 += 4) {
        u32x4 w[4] = {dst[j0], dst[j0 + 1], dst[j0 + 2], dst[j0 + 3]};
        lds_wait4(w);
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j0 + j] = w[j];
      }
    };
    // Whole blocks (no key masked) and the others take separate copies of
    // the subtile loop, so that the whole-block copy is straight-line code
    // whose MFMAs, row maxima and LDS reads can be interleaved.
    auto body = [&](auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
      auto reduce = [&](int kt, f32x16 (&acc)[2]) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          if constexpr (!FULL) {
            int lim = nvalid - 1;
            if (p.causal) lim = min(lim, pos_[nt] - kBlock * t);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
              acc[nt][r] = key <= lim ? acc[nt][r] : -INFINITY;
            }
          }
          bm[nt] = fmaxf(bm[nt], max16(acc[nt]));
        }
      };
      f32x16 acc[2][2];
      kread(0, kr[0]);
      kwait(kr[0]);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int cur = kt & 1;
        if (kt < 3) kread(kt + 1, kr[cur ^ 1]);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          bf16x8 a;
          if constexpr (FMT == kFmtFp8) {
            const u32x4 w = kr[cur][s >> 1];
            a = (s & 1) ? fp8x8_bf16(w[2], w[3]) : fp8x8_bf16(w[0], w[1]);
          } else {
            a = as_bf16x8(kr[cur][s]);
          }
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            if (s == 0) {
              f32x16 z;
#pragma unroll
              for (int r = 0; r < 16; ++r) z[r] = 0.f;
              acc[cur][nt] = mm32<FMT>(a, qf[nt][s], z);
            } else {
              acc[cur][nt] = mm32<FMT>(a, qf[nt][s], acc[cur][nt]);
            }
          }
        }
        if (kt > 0) reduce(kt - 1, acc[cur ^ 1]);
        if constexpr (FULL) {
          if (kt > 0) {
            // the previous subtile's row maxima between this one's MFMAs
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (kt < 3) kwait(kr[cur ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      reduce(3, acc[1]);
    };
    if (full) body(std::true_type{});
    else body(std::false_type{});
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float v = xor_max(bm[nt], 32);
      const int r = r0 + 64 * wave + 32 * nt + (lane_id() & 31);
      const int tk = r / G, hh = r % G;
      if constexpr (!REDUCE) {
        if (half == 0 && r < nrows)
          p.out[((int64_t)(g * G + hh) * p.max_k_tiles + t) * p.total_q + q0 + tk] = v;
      } else {
        if ((G & (G - 1)) == 0 && G <= 32) {
          for (int off = 1; off < G; off <<= 1) v = xor_max(v, off);
          if (half == 0 && r < nrows && hh == 0)
            atomic_max_f32(&p.out[(rbase + t) * p.total_q + q0 + tk], v);
        } else if (half == 0 && r < nrows) {
          atomic_max_f32(&p.out[(rbase + t) * p.total_q + q0 + tk], v);
        }
      }
    }
    // every wave's reads of this buffer done before it is refilled
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  }  // segments
}

__global__ void msa_fill_kernel(float* __restrict__ out, int64_t n, float v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) out[i] = v;
}

template <int FMT>
static hipError_t launch_proxy_wide_t(const ProxyParams& p, hipStream_t stream) {
  const int units = p.batch * p.hkv;
  const int pairs = (p.row_tiles + 1) / 2;
  const int n = units * pairs * p.pieces;
  if (n <= 0) return hipSuccess;
  const int grid = units <= 8 && 8 % units == 0
                       ? 8 * ((pairs + 8 / units - 1) / (8 / units)) * p.pieces
                       : 8 * ((n + 7) / 8);
  if (p.reduce) {
    const int64_t total = (int64_t)(p.reduce == 2 ? p.hkv : 1) * p.max_k_tiles * p.total_q;
    if (total > 0) {
      int fb = (int)std::min<int64_t>((total + 255) / 256, 4096);
      hipLaunchKernelGGL(msa_fill_kernel, dim3(fb), dim3(256), 0, stream, p.out, total, -INFINITY);
    }
    hipLaunchKernelGGL((msa_proxy_wide_kernel<FMT, true>), dim3(grid), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL((msa_proxy_wide_kernel<FMT, false>), dim3(grid), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

template <int NT, int FMT>
static hipError_t launch_proxy_rows_t(const ProxyParams& p, hipStream_t stream) {
  const int n = p.batch * p.hkv * p.block_chunks;
  if (n <= 0) return hipSuccess;
  if (p.reduce) {
    const int64_t total = (int64_t)(p.reduce == 2 ? p.hkv : 1) * p.max_k_tiles * p.total_q;
    if (total > 0) {
      int fb = (int)std::min<int64_t>((total + 255) / 256, 4096);
      hipLaunchKernelGGL(msa_fill_kernel, dim3(fb), dim3(256), 0, stream, p.out, total, -INFINITY);
    }
    hipLaunchKernelGGL((msa_proxy_rows_kernel<NT, FMT, true>), dim3(n), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL((msa_proxy_rows_kernel<NT, FMT, false>), dim3(n), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

// Running top-K on the decode-shaped path: candidates instead of scores.
template <int NT, int FMT>
static hipError_t launch_proxy_cand_t(const ProxyParams& p, hipStream_t stream) {
  const int n = p.batch * p.hkv * p.block_chunks;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL((msa_proxy_rows_kernel<NT, FMT, true, true>), dim3(n), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_proxy_candidates(const ProxyParams& p, int fmt, hipStream_t stream) {
  if (p.rows_per_tile <= 32)
    return fmt == kFmtFp8 ? launch_proxy_cand_t<1, kFmtFp8>(p, stream)
         : fmt == kFmtF16 ? launch_proxy_cand_t<1, kFmtF16>(p, stream)
                          : launch_proxy_cand_t<1, kFmtBf16>(p, stream);
  return fmt == kFmtFp8 ? launch_proxy_cand_t<2, kFmtFp8>(p, stream)
       : fmt == kFmtF16 ? launch_proxy_cand_t<2, kFmtF16>(p, stream)
                        : launch_proxy_cand_t<2, kFmtBf16>(p, stream);
}

// wide_rows: 1 -> 256 rows per workgroup (msa_proxy_wide_kernel); 0 -> at
// most 64 rows per (request, KV head) (msa_proxy_rows_kernel; p.rows_per_tile
// holds the row count rounded up to 32).
hipError_t launch_proxy(const ProxyParams& p, int fmt, int wide_rows, hipStream_t stream) {
  if (wide_rows) {
    return fmt == kFmtFp8 ? launch_proxy_wide_t<kFmtFp8>(p, stream)
         : fmt == kFmtF16 ? launch_proxy_wide_t<kFmtF16>(p, stream)
                          : launch_proxy_wide_t<kFmtBf16>(p, stream);
  }
  if (p.rows_per_tile <= 32)
    return fmt == kFmtFp8 ? launch_proxy_rows_t<1, kFmtFp8>(p, stream)
         : fmt == kFmtF16 ? launch_proxy_rows_t<1, kFmtF16>(p, stream)
                          : launch_proxy_rows_t<1, kFmtBf16>(p, stream);
  return fmt == kFmtFp8 ? launch_proxy_rows_t<2, kFmtFp8>(p, stream)
       : fmt == kFmtF16 ? launch_proxy_rows_t<2, kFmtF16>(p, stream)
                        : launch_proxy_rows_t<2, kFmtBf16>(p, stream);
}

}  // namespace msa
