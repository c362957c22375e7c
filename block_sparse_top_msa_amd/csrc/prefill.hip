// MSA sparse attention, prefill shape, bf16 K/V (msa_sparse_attention page,
// summary: query tiles, each running one online softmax over the union of
// the blocks its tokens selected, writing the output directly).
//
// gfx950 design:
//  * Tile = TOK query tokens of one request x the G query heads of one KV
//    head, as token-major rows cut into 32-row slots; each of NW waves owns
//    SPW slots.  32-row slots because v_mfma_f32_32x32x16_bf16 runs at twice
//    the FLOP rate of the 16x16x32 shape on this chip (measured: ~2.4 vs
//    ~1.3 PFLOP/s) and reads half the LDS bytes per FLOP.
//  * The tile's block union is built in LDS (tile_union.hpp).  Each union
//    block (128 keys of K and V, 64 KiB) is staged global -> LDS with
//    global_load_lds (16 B per lane, no VGPR staging), double buffered: block
//    u+1 streams in while block u is computed.  Rows are XOR-swizzled in
//    16-byte chunks so every operand read is bank-conflict free with an
//    unpadded 256-byte row pitch.
//  * Per 32-key chunk: S^T = K Q^T (keys on the MFMA M axis, query rows on
//    N), the softmax update, and O^T += V^T P^T with P taken straight from
//    the S^T registers.  The chunk's K and V^T fragments are read into
//    registers once and reused by every active slot of the wave; V^T comes
//    from row-major V through the transposing ds_read_b64_tr_b16.
//  * Softmax: p = exp2(s * c - m) is one FMA + one exp per score against a
//    per-row reference max m set by the row's first scores and moved again
//    (rescaling O and l) only if a score exceeds it by more than 2^64, which
//    the fp32 accumulators absorb; row sums stay per lane until the end.  A slot none of whose tokens chose a
//    block skips it (one scalar branch per slot and chunk).
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

// Transposed reads (outputs early-clobber, see kfrag_load) of the V^T operand
// of one 32-key chunk, for the four
// 32-column head-dim tiles dt and the two 16-key k-steps: rows r, r + 8
// (first k-step) and r + 16, r + 24 (second), i.e. byte offsets 0, 2048,
// 4096, 6144.  In each group of 16 lanes, lane j receives element j % 4 of
// the 8 bytes at lane 4e + j / 4's address, for e = 0..3: four consecutive
// keys of one head-dim column.
__device__ __forceinline__ void vtr_issue(u32x2 (&v)[16], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %3, %16 offset:6144\n\t"
      "ds_read_b64_tr_b16 %4, %17\n\t"
      "ds_read_b64_tr_b16 %5, %17 offset:2048\n\t"
      "ds_read_b64_tr_b16 %6, %17 offset:4096\n\t"
      "ds_read_b64_tr_b16 %7, %17 offset:6144\n\t"
      "ds_read_b64_tr_b16 %8, %18\n\t"
      "ds_read_b64_tr_b16 %9, %18 offset:2048\n\t"
      "ds_read_b64_tr_b16 %10, %18 offset:4096\n\t"
      "ds_read_b64_tr_b16 %11, %18 offset:6144\n\t"
      "ds_read_b64_tr_b16 %12, %19\n\t"
      "ds_read_b64_tr_b16 %13, %19 offset:2048\n\t"
      "ds_read_b64_tr_b16 %14, %19 offset:4096\n\t"
      "ds_read_b64_tr_b16 %15, %19 offset:6144"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
        "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]),
        "=&v"(v[14]), "=&v"(v[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}

// The eight K operand fragments of one 32-key chunk (ds_read_b128 each),
// issued without waiting (outputs early-clobber: a load may return while
// later loads of the group still read their address registers).
__device__ __forceinline__ void kfrag_issue(u32x4 (&k)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %14\n\t"
      "ds_read_b128 %7, %15"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]),
        "=&v"(k[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
}

// Waits for every outstanding LDS read; naming the K registers orders their
// uses after it.
__device__ __forceinline__ void kfrag_wait(u32x4 (&k)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]), "+v"(k[4]), "+v"(k[5]),
                 "+v"(k[6]), "+v"(k[7]));
}

// Waits for the reads above; naming the registers orders their uses after it.
__device__ __forceinline__ void vtr_wait(u32x2 (&v)[16]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
                 "+v"(v[6]), "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]),
                 "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15]));
}

__device__ __forceinline__ float swap32_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float swap32_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

}  // namespace

template <int NW, int SPW>
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
    pos_[s] = lk - lq + i0 + tk;
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

  float m_[SPW], l_[SPW];
  f32x16 o_[SPW][4];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    m_[s] = -INFINITY;
    l_[s] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o_[s][dt][r] = 0.f;
  }
  __syncthreads();  // kbase / vbase visible; q loads done

  // Staging: lane l of wave w loads the 16-byte chunk (row r_i, logical
  // chunk c) for physical position (r_i, l % 16), r_i = 4 w + l / 16 + 16 i.
  const int lr0 = 4 * wave + (lane >> 4);
  const int64_t koff0 = lr0 * kst + 16 * swz_k(lr0, lane & 15);
  const int64_t voff0 = lr0 * vst + 16 * swz_v(lr0, lane & 15);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds.kv[0])) + wave * 1024;

  auto issue = [&](int u, int buf) {
    const int t = __builtin_amdgcn_readfirstlane(lds.un.list[u]);
    const int nvalid = min(kBlock, lk - kBlock * t);
    const uint8_t* kb = p.k + lds.kbase[u];
    const uint8_t* vb = p.v + lds.vbase[u];
    const uint32_t dst = lds0 + buf * (2 * kTileBytes);
    if (nvalid == kBlock) {
#pragma unroll
      for (int i = 0; i < KLOADS; ++i)
        g2lds16(kb + koff0 + (int64_t)(4 * NW * i) * kst, dst + i * NW * 1024);
#pragma unroll
      for (int i = 0; i < KLOADS; ++i)
        g2lds16(vb + voff0 + (int64_t)(4 * NW * i) * vst, dst + kTileBytes + i * NW * 1024);
    } else {
      // partial last block: rows past Lk read the block's row 0 instead
      // (finite values; those keys are masked and their P is 0)
#pragma unroll
      for (int i = 0; i < KLOADS; ++i) {
        const bool in = lr0 + 4 * NW * i < nvalid;
        g2lds16(kb + (in ? koff0 + (int64_t)(4 * NW * i) * kst : koff0 - lr0 * kst),
                dst + i * NW * 1024);
      }
#pragma unroll
      for (int i = 0; i < KLOADS; ++i) {
        const bool in = lr0 + 4 * NW * i < nvalid;
        g2lds16(vb + (in ? voff0 + (int64_t)(4 * NW * i) * vst : voff0 - lr0 * vst),
                dst + kTileBytes + i * NW * 1024);
      }
    }
  };

  const float C = p.scale_log2;
  if (ucount > 0) issue(0, 0);

  // per-lane constant parts of the transposed V reads: 16-lane group q16
  // covers key half q16 / 2 and head-dim columns 16 * (q16 % 2) + 0..15 of a
  // 32-column tile; its lane 4e + q reads row 4 * half + e, columns 4q..4q+3
  uint32_t koffs[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) koffs[ks] = l32 * 256 + 16 * swz_k(l32, 2 * ks + hf);
  const int q16 = lane >> 4;
  const int vrow = 4 * (q16 >> 1) + ((lane & 15) >> 2);
  const int vchunk = 2 * (q16 & 1) + ((lane & 3) >> 1);
  const int vbyte = 8 * (lane & 1);

  static_assert(SPW == 1, "the software-pipelined loop runs one slot per wave");
  const unsigned long long tokmask0 = tokmask[0];
  const int tk0 = tk_[0];
  const int pos0 = pos_[0];

  for (int u = 0; u < ucount; ++u) {
    const int buf = u & 1;
    const int t = __builtin_amdgcn_readfirstlane(lds.un.list[u]);
    const unsigned long long umask = uniform64(lds.un.mask[u]);
    const int nvalid = min(kBlock, lk - kBlock * t);
    // this wave's loads of block u done (block u+1's stay in flight), then
    // every wave's
    if (u + 1 < ucount) {
      issue(u + 1, buf ^ 1);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    block_barrier();

    const uint32_t kt_lds = lds_addr(lds.kv[buf]);
    const uint32_t vt_lds = kt_lds + kTileBytes;
    const bool rowsel = (tk0 < ntok) && ((umask >> tk0) & 1ull);
    int lim = nvalid - 1;
    if (p.causal) lim = min(lim, pos0 - kBlock * t);

    if ((umask & tokmask0) != 0ull) {
      // Software pipeline over the block's four 32-key chunks: S^T of chunk
      // c + 1 and O^T += V^T P^T of chunk c are issued back to back, so the
      // matrix core works through them while the softmax of chunk c + 1 runs
      // on the vector ALU.
      u32x4 kw[8];
      {
        uint32_t a[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) a[ks] = kt_lds + koffs[ks];
        kfrag_issue(kw, a);
        kfrag_wait(kw);
      }
      f32x16 s_next;
#pragma unroll
      for (int r = 0; r < 16; ++r) s_next[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s_next = mfma32(as_bf16x8(kw[ks]), qf[0][ks], s_next);

#pragma unroll
      for (int c = 0; c < 4; ++c) {
        f32x16 acc = s_next;
        // V^T fragments of chunk c and K fragments of chunk c + 1, in flight
        // during the softmax
        u32x2 vv[16];
        {
          const int r = 32 * c + vrow;
          uint32_t a[4];
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
            a[dt] = vt_lds + r * 256 + 16 * swz_v(r, 4 * dt + vchunk) + vbyte;
          vtr_issue(vv, a);
        }
        if (c < 3) {
          uint32_t a[8];
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) a[ks] = kt_lds + 32 * (c + 1) * 256 + koffs[ks];
          kfrag_issue(kw, a);
        }
        // ---- mask (diagonal / partial block only)
        if (__ballot(rowsel && lim < 32 * c + 31) != 0ull) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * c + 8 * (r >> 2) + 4 * hf + (r & 3);
            acc[r] = key <= lim ? acc[r] : -INFINITY;
          }
        }
        float mx = fmaxf(fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])),
                         fmaxf(fmaxf(acc[4], acc[5]), fmaxf(acc[6], acc[7])));
        mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(acc[8], acc[9]), fmaxf(acc[10], acc[11])),
                             fmaxf(fmaxf(acc[12], acc[13]), fmaxf(acc[14], acc[15]))));
        mx = rowsel ? mx * C : -INFINITY;
        // first scores of a row: take the max as the reference (O and l are
        // still zero); afterwards move it only when it grows past the slack
        if (__ballot(mx > m_[0] + kRescaleSlack) != 0ull) {
          const float mr = swap32_max(mx);
          if (__ballot(mr > m_[0] + kRescaleSlack && m_[0] > -INFINITY) != 0ull) {
            const float alpha =
                mr > m_[0] + kRescaleSlack ? __builtin_amdgcn_exp2f(m_[0] - mr) : 1.0f;
            l_[0] *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) o_[0][dt] *= alpha;
          }
          m_[0] = mr > m_[0] + kRescaleSlack ? mr : m_[0];
        }
        const float mu = (rowsel && m_[0] > -INFINITY) ? m_[0] : INFINITY;
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[r], C, -mu));
        l_[0] += (((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]))) +
                 (((e[8] + e[9]) + (e[10] + e[11])) + ((e[12] + e[13]) + (e[14] + e[15])));
        u32x4 pw0, pw1;  // P^T for the two 16-key k-steps
        pw0[0] = cvt_pk_bf16(e[0], e[1]);
        pw0[1] = cvt_pk_bf16(e[2], e[3]);
        pw0[2] = cvt_pk_bf16(e[4], e[5]);
        pw0[3] = cvt_pk_bf16(e[6], e[7]);
        pw1[0] = cvt_pk_bf16(e[8], e[9]);
        pw1[1] = cvt_pk_bf16(e[10], e[11]);
        pw1[2] = cvt_pk_bf16(e[12], e[13]);
        pw1[3] = cvt_pk_bf16(e[14], e[15]);
        vtr_wait(vv);
        if (c < 3) {
          kfrag_wait(kw);
#pragma unroll
          for (int r = 0; r < 16; ++r) s_next[r] = 0.f;
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) s_next = mfma32(as_bf16x8(kw[ks]), qf[0][ks], s_next);
        }
        // ---- O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const u32x4 w0 = {vv[4 * dt][0], vv[4 * dt][1], vv[4 * dt + 1][0], vv[4 * dt + 1][1]};
          const u32x4 w1 = {vv[4 * dt + 2][0], vv[4 * dt + 2][1], vv[4 * dt + 3][0],
                            vv[4 * dt + 3][1]};
          o_[0][dt] = mfma32(as_bf16x8(w0), as_bf16x8(pw0), o_[0][dt]);
          o_[0][dt] = mfma32(as_bf16x8(w1), as_bf16x8(pw1), o_[0][dt]);
        }
      }
    }
    // every wave's LDS reads of buffer `buf` are done before it is refilled
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    block_barrier();
  }

  // ---- epilogue: out = O / l * v_gs (bf16), lse = (m + log2 l) * ln 2
  const int out_row0 = q0 + i0;
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const float lsum = swap32_sum(l_[s]);
    const int slot = wave * SPW + s;
    const int tk = tk_[s];
    if (tk >= ntok) continue;
    const int hh = (32 * slot + l32) % G;
    const int64_t row = (int64_t)(out_row0 + tk) * p.hq + g * G + hh;
    const float inv = lsum > 0.f ? p.v_gs / lsum : 0.f;
    uint16_t* op = p.out + row * kHeadDim + 4 * hf;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x2*>(op + 32 * dt + 8 * q) =
            u32x2{pack_bf16x2(o_[s][dt][4 * q] * inv, o_[s][dt][4 * q + 1] * inv),
                  pack_bf16x2(o_[s][dt][4 * q + 2] * inv, o_[s][dt][4 * q + 3] * inv)};
    if (p.lse && hf == 0)
      p.lse[row] = lsum > 0.f ? (m_[s] + __log2f(lsum)) * kLn2f : -INFINITY;
  }
}

template <int NW, int SPW>
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
  hipLaunchKernelGGL((msa_prefill_kernel<NW, SPW>), dim3(grid), dim3(NW * kWave), 0, stream, p);
  return hipGetLastError();
}

// Tiles of 256 rows: 8 waves x one 32-row slot.
hipError_t launch_prefill_bf16(const AttnParams& p, int spw, hipStream_t stream) {
  (void)spw;
  return launch_prefill_t<8, 1>(p, stream);
}

}  // namespace msa
