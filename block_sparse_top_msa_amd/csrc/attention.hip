// MSA sparse attention on gfx950: one online softmax per query tile over the
// union of the blocks its tokens selected (msa_sparse_attention page,
// summary), with K/V blocks gathered by index into LDS, QK^T and PV on bf16
// MFMA, and in-register fp8 / E2M1 dequantisation while staging.
//
// This kernel serves prefill-shaped calls with fp8 / E2M1 K/V (bf16 prefill
// runs the asynchronous kernel in prefill.hip, decode shapes the kernel in
// decode.hip): each wave owns SPW 16-row slots (token x head rows of one KV
// head) and runs every union block over all 128 keys.  A slot whose tokens
// did not select a block skips it; rows of tokens that did not select it are
// masked.
//
// Orientation: S^T = K Q^T puts keys on the MFMA M axis and query rows on N,
// so a query's scores sit in one lane group and row max / sum need only two
// cross-lane steps; O^T = V^T P^T then takes P straight from the S^T
// registers as the B operand.
#include "common.hpp"
#include "internal.hpp"
#include "temperature.hpp"
#include "tile_union.hpp"

namespace msa {

constexpr int kKPitch = 136;  // bf16 per K row in LDS (272 B: conflict-free b128 reads)
constexpr int kVPitch = 132;  // bf16 per transposed V row (264 B: conflict-free b64 reads)
constexpr float kLn2 = 0.69314718055994530942f;

struct KvTile {
  uint16_t k[kBlock * kKPitch];
  uint16_t vt[kHeadDim * kVPitch];
};

struct AttnLds {
  KvTile kv;
  UnionLds un;
};

__device__ __forceinline__ u32x4 ld16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld8(const uint8_t* p) {
  return *reinterpret_cast<const u32x2*>(p);
}
__device__ __forceinline__ uint32_t bf16_elem(const u32x4& v, int e) {
  uint32_t w = v[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Where the rows of one KV block of one KV head start.
struct BlockAddr {
  const uint8_t* k;
  const uint8_t* v;
  const uint8_t* ks;
  const uint8_t* vs;
  int nvalid;  // keys of the block below Lk
};

// ---------------------------------------------------------------------------
// Staging: global -> registers (issued one block ahead) -> LDS (dequantised
// to bf16; V transposed to [d][key]).  Rows at or past Lk are zero-filled and
// never read from memory.
// ---------------------------------------------------------------------------
template <int FMT, int NT>
struct Stage;

template <int NT>
struct Stage<kFmtBf16, NT> {
  static constexpr int KT = 2048 / NT;  // 16-B K chunks per thread
  static constexpr int VT = 512 / NT;   // (4 keys x 16 B) V tasks per thread
  u32x4 kr[KT];
  u32x4 vr[VT][4];

  __device__ void issue(const BlockAddr& a, const AttnParams& p) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      int task = i * NT + tid, row = task >> 4, c = task & 15;
      kr[i] = row < a.nvalid ? ld16(a.k + row * p.k_st.token + 16 * c) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VT; ++i) {
      int task = i * NT + tid, j = task & 31, c = task >> 5;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        int row = 4 * j + rr;
        vr[i][rr] = row < a.nvalid ? ld16(a.v + row * p.v_st.token + 16 * c) : u32x4{0, 0, 0, 0};
      }
    }
  }

  __device__ void store(KvTile& t) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      int task = i * NT + tid, row = task >> 4, c = task & 15;
      *reinterpret_cast<u32x4*>(&t.k[row * kKPitch + 8 * c]) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < VT; ++i) {
      int task = i * NT + tid, j = task & 31, c = task >> 5;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t lo = bf16_elem(vr[i][0], e) | (bf16_elem(vr[i][1], e) << 16);
        uint32_t hi = bf16_elem(vr[i][2], e) | (bf16_elem(vr[i][3], e) << 16);
        *reinterpret_cast<u32x2*>(&t.vt[(8 * c + e) * kVPitch + 4 * j]) = u32x2{lo, hi};
      }
    }
  }
};

template <int NT>
struct Stage<kFmtFp8, NT> {
  static constexpr int KT = 1024 / NT;  // 16-B (16 value) K chunks per thread
  static constexpr int VT = 256 / NT;   // (4 keys x 16 B) V tasks per thread
  u32x4 kr[KT];
  u32x4 vr[VT][4];

  __device__ void issue(const BlockAddr& a, const AttnParams& p) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      int task = i * NT + tid, row = task >> 3, c = task & 7;
      kr[i] = row < a.nvalid ? ld16(a.k + row * p.k_st.token + 16 * c) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VT; ++i) {
      int task = i * NT + tid, j = task & 31, c = task >> 5;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        int row = 4 * j + rr;
        vr[i][rr] = row < a.nvalid ? ld16(a.v + row * p.v_st.token + 16 * c) : u32x4{0, 0, 0, 0};
      }
    }
  }

  __device__ static uint32_t byte_of(const u32x4& v, int e) { return (v[e >> 2] >> (8 * (e & 3))) & 0xFFu; }

  __device__ void store(KvTile& t) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      int task = i * NT + tid, row = task >> 3, c = task & 7;
      u32x4 w0, w1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0[e] = pack_bf16x2(e4m3_to_f32(byte_of(kr[i], 2 * e)), e4m3_to_f32(byte_of(kr[i], 2 * e + 1)));
        w1[e] = pack_bf16x2(e4m3_to_f32(byte_of(kr[i], 8 + 2 * e)), e4m3_to_f32(byte_of(kr[i], 9 + 2 * e)));
      }
      *reinterpret_cast<u32x4*>(&t.k[row * kKPitch + 16 * c]) = w0;
      *reinterpret_cast<u32x4*>(&t.k[row * kKPitch + 16 * c + 8]) = w1;
    }
#pragma unroll
    for (int i = 0; i < VT; ++i) {
      int task = i * NT + tid, j = task & 31, c = task >> 5;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        uint32_t lo = pack_bf16x2(e4m3_to_f32(byte_of(vr[i][0], e)), e4m3_to_f32(byte_of(vr[i][1], e)));
        uint32_t hi = pack_bf16x2(e4m3_to_f32(byte_of(vr[i][2], e)), e4m3_to_f32(byte_of(vr[i][3], e)));
        *reinterpret_cast<u32x2*>(&t.vt[(16 * c + e) * kVPitch + 4 * j]) = u32x2{lo, hi};
      }
    }
  }
};

template <int NT>
struct Stage<kFmtE2m1, NT> {
  // K rows: 64 B of nibbles (4 chunks of 32 values) + 8 scale bytes.
  // V tasks: 4 keys x 8 B (16 values, one scale each).
  static constexpr int KT = 512 / NT;
  static constexpr int VT = 256 / NT;
  u32x4 kr[KT];
  uint32_t ksc[KT];     // two scale bytes for the chunk
  u32x2 vr[VT][4];
  uint32_t vsc[VT][4];  // one scale byte per key

  __device__ void issue(const BlockAddr& a, const AttnParams& p) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      int task = i * NT + tid, row = task >> 2, c = task & 3;
      bool ok = row < a.nvalid;
      kr[i] = ok ? ld16(a.k + row * p.k_st.token + 16 * c) : u32x4{0, 0, 0, 0};
      ksc[i] = ok ? *reinterpret_cast<const uint16_t*>(a.ks + row * p.ks_st.token + 2 * c) : 0u;
    }
#pragma unroll
    for (int i = 0; i < VT; ++i) {
      int task = i * NT + tid, j = task & 31, c = task >> 5;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        int row = 4 * j + rr;
        bool ok = row < a.nvalid;
        vr[i][rr] = ok ? ld8(a.v + row * p.v_st.token + 8 * c) : u32x2{0, 0};
        vsc[i][rr] = ok ? a.vs[row * p.vs_st.token + c] : 0u;
      }
    }
  }

  __device__ void store(KvTile& t) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      int task = i * NT + tid, row = task >> 2, c = task & 3;
      float s0 = e4m3_to_f32(ksc[i] & 0xFFu), s1 = e4m3_to_f32((ksc[i] >> 8) & 0xFFu);
#pragma unroll
      for (int h = 0; h < 4; ++h) {  // 8 values per 32-bit word
        uint32_t w = kr[i][h];
        float sc = h < 2 ? s0 : s1;
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = pack_bf16x2(e2m1_to_f32((w >> (8 * e)) & 0xFu) * sc,
                             e2m1_to_f32((w >> (8 * e + 4)) & 0xFu) * sc);
        }
        *reinterpret_cast<u32x4*>(&t.k[row * kKPitch + 32 * c + 8 * h]) = o;
      }
    }
#pragma unroll
    for (int i = 0; i < VT; ++i) {
      int task = i * NT + tid, j = task & 31, c = task >> 5;
      float sc[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sc[rr] = e4m3_to_f32(vsc[i][rr]);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          uint32_t w = vr[i][rr][e >> 3];
          x[rr] = e2m1_to_f32((w >> (4 * (e & 7))) & 0xFu) * sc[rr];
        }
        *reinterpret_cast<u32x2*>(&t.vt[(16 * c + e) * kVPitch + 4 * j]) =
            u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      }
    }
  }
};

__device__ __forceinline__ BlockAddr block_addr(const AttnParams& p, int b, int g, int t, int lk) {
  BlockAddr a;
  a.nvalid = min(kBlock, lk - kBlock * t);
  if (p.paged) {
    int64_t page = p.page_table[(int64_t)b * p.pt_width + t];
    a.k = p.k + page * p.k_st.page + g * p.k_st.head;
    a.v = p.v + page * p.v_st.page + g * p.v_st.head;
    a.ks = p.ks ? p.ks + page * p.ks_st.page + g * p.ks_st.head : nullptr;
    a.vs = p.vs ? p.vs + page * p.vs_st.page + g * p.vs_st.head : nullptr;
  } else {
    int64_t row0 = (int64_t)p.cu_k[b] + kBlock * t;
    a.k = p.k + row0 * p.k_st.token + g * p.k_st.head;
    a.v = p.v + row0 * p.v_st.token + g * p.v_st.head;
    a.ks = p.ks ? p.ks + row0 * p.ks_st.token + g * p.ks_st.head : nullptr;
    a.vs = p.vs ? p.vs + row0 * p.vs_st.token + g * p.vs_st.head : nullptr;
  }
  return a;
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
// lse_t (nullable): also the temperature LSE, ln sum_j exp(tau * z_j) over
// the same keys, accumulated against the row's running max (tau > 0).
template <int NW, int SPW, int FMT>
__global__ __launch_bounds__(NW * kWave) void msa_attention_kernel(AttnParams p, float* lse_t,
                                                                   float tau) {
  constexpr int NT = NW * kWave;
  constexpr int NKT = kBlock / 16;      // 16-key S^T subtiles
  constexpr int NKS = kBlock / 32;      // 32-key PV steps

  __shared__ AttnLds lds;

  const int n_units = p.batch * p.hkv * p.tiles_per_req;
  const int lid = xcd_remap(blockIdx.x, n_units);
  if (lid < 0) return;
  int rest = lid;
  const int jr = rest % p.tiles_per_req;
  rest /= p.tiles_per_req;
  const int g = rest % p.hkv;
  const int b = rest / p.hkv;
  const int j = p.tiles_per_req - 1 - jr;  // later tiles (more visible blocks) first

  const int q0 = p.cu_q[b];
  const int lq = p.cu_q[b + 1] - q0;
  const int i0 = j * p.tok_per_tile;
  if (i0 >= lq) return;
  const int ntok = min(p.tok_per_tile, lq - i0);
  const int lk = p.paged ? p.seqused_k[b] : (p.cu_k[b + 1] - p.cu_k[b]);
  const int nblk = max(0, min((lk + kBlock - 1) / kBlock, p.max_k_tiles));

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int lq16 = lane & 15;
  const int lg = lane >> 4;
  const int sg = wave;            // slot group
  const int G = p.group;

  const int32_t* rows = p.q2k + ((int64_t)g * p.total_q + q0 + i0) * p.topk;
  const int ucount = build_tile_union<NT>(lds.un, rows, ntok, p.topk, nblk);
  const int u0 = 0, u1 = ucount;

  // Per-slot, per-lane row data.  Row r of the tile = token r / G, head r % G.
  bf16x8 qf[SPW][4];
  int tk_[SPW], pos_[SPW];
  unsigned long long slot_tokmask[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int slot = sg * SPW + s;
    const int r = 16 * slot + lq16;
    const int tk = r / G;
    const int hh = r % G;
    tk_[s] = tk;
    pos_[s] = tk < ntok ? query_pos(p.qpos.rows, p.qpos.mode, p.qpos.base, q0 + i0 + tk, i0 + tk,
                                    lq, lk)
                        : 0;
    const int tfirst = (16 * slot) / G;
    const int tlast = min((16 * slot + 15) / G, ntok - 1);
    unsigned long long m = 0;
    for (int t = tfirst; t <= tlast && t < 64; ++t) m |= 1ull << t;
    slot_tokmask[s] = (tfirst < ntok) ? m : 0ull;
    if (tk < ntok) {
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(
          p.q + ((int64_t)(q0 + i0 + tk) * p.hq + g * G + hh) * kHeadDim);
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) qf[s][ds] = as_bf16x8(ld16(qp + 2 * (32 * ds + 8 * lg)));
    } else {
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) qf[s][ds] = as_bf16x8(u32x4{0, 0, 0, 0});
    }
  }

  float m_[SPW], l_[SPW], lt_[SPW];
  f32x4 o_[SPW][8];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    m_[s] = -INFINITY;
    l_[s] = 0.f;
    lt_[s] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o_[s][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  Stage<FMT, NT> stage;
  if (u0 < u1) stage.issue(block_addr(p, b, g, lds.un.list[u0], lk), p);

  const int kbase = 0;
  for (int u = u0; u < u1; ++u) {
    const int t = lds.un.list[u];
    const unsigned long long umask = lds.un.mask[u];
    const int nvalid = min(kBlock, lk - kBlock * t);
    __syncthreads();                 // previous block fully consumed
    stage.store(lds.kv);
    __syncthreads();
    if (u + 1 < u1) stage.issue(block_addr(p, b, g, lds.un.list[u + 1], lk), p);

#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      if (!(umask & slot_tokmask[s])) continue;  // no token of this slot chose t
      f32x4 acc[NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
              &lds.kv.k[(kbase + 16 * kt + lq16) * kKPitch + 32 * ds + 8 * lg]));
          acc[kt] = mfma16(a, qf[s][ds], acc[kt]);
        }
      }
      // scale into the log2 domain and mask: a key is visible to this lane's
      // row iff key <= lim (lim = -1 when the row's token did not select t).
      // Branch-free on purpose: one compare + select per accumulator value.
      const bool sel = (tk_[s] < ntok) && ((umask >> tk_[s]) & 1ull);
      int lim = nvalid - 1;
      if (p.causal) lim = min(lim, pos_[s] - kBlock * t);
      lim = sel ? lim : -1;
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kbase + 16 * kt + 4 * lg + r;
          const float x = key <= lim ? acc[kt][r] * p.scale_log2 : -INFINITY;
          acc[kt][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = xor_max(mx, 16);
      mx = xor_max(mx, 32);
      const float m_new = fmaxf(m_[s], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_[s] - m_use);
      float sum = 0.f, sum_t = 0.f;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float xv = acc[kt][r];
          if (lse_t) sum_t += __builtin_amdgcn_exp2f(tau * (xv - m_use));
          float e = __builtin_amdgcn_exp2f(xv - m_use);
          acc[kt][r] = e;
          sum += e;
        }
      }
      sum = xor_sum(sum, 16);
      sum = xor_sum(sum, 32);
      l_[s] = l_[s] * alpha + sum;
      if (lse_t) {
        sum_t = xor_sum(sum_t, 16);
        sum_t = xor_sum(sum_t, 32);
        lt_[s] = lt_[s] * __builtin_amdgcn_exp2f(tau * (m_[s] - m_use)) + sum_t;
      }
      m_[s] = m_new;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o_[s][dt] *= alpha;

#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        u32x4 pw;
        pw[0] = pack_bf16x2(acc[2 * ks][0], acc[2 * ks][1]);
        pw[1] = pack_bf16x2(acc[2 * ks][2], acc[2 * ks][3]);
        pw[2] = pack_bf16x2(acc[2 * ks + 1][0], acc[2 * ks + 1][1]);
        pw[3] = pack_bf16x2(acc[2 * ks + 1][2], acc[2 * ks + 1][3]);
        const bf16x8 pb = as_bf16x8(pw);
        const int kcol = kbase + 32 * ks + 4 * lg;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const uint16_t* vrow = &lds.kv.vt[(16 * dt + lq16) * kVPitch];
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + kcol);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + kcol + 16);
          o_[s][dt] = mfma16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb, o_[s][dt]);
        }
      }
    }
  }

  // epilogue: each wave writes its own rows
  const int out_row0 = q0 + i0;
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int slot = sg * SPW + s;
    const int tk = tk_[s];
    if (tk >= ntok) continue;
    const int hh = (16 * slot + lq16) % G;
    const int64_t row = (int64_t)(out_row0 + tk) * p.hq + g * G + hh;
    const float inv = l_[s] > 0.f ? p.v_gs / l_[s] : 0.f;
    uint16_t* op = p.out + row * kHeadDim + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      *reinterpret_cast<u32x2*>(op + 16 * dt) =
          u32x2{pack_bf16x2(o_[s][dt][0] * inv, o_[s][dt][1] * inv),
                pack_bf16x2(o_[s][dt][2] * inv, o_[s][dt][3] * inv)};
    }
    if (p.lse && lg == 0)
      p.lse[row] = l_[s] > 0.f ? (m_[s] + __log2f(l_[s])) * kLn2 : -INFINITY;
    if (lse_t && lg == 0)
      lse_t[row] = l_[s] > 0.f ? (tau * m_[s] + __log2f(lt_[s])) * kLn2 : -INFINITY;
  }
}

template <int NW, int SPW, int FMT>
static hipError_t launch_one(const AttnParams& p, hipStream_t stream, float* lse_t = nullptr,
                             float tau = 1.f) {
  const int n = p.batch * p.hkv * p.tiles_per_req;
  if (n <= 0) return hipSuccess;
  const int grid = 8 * ((n + 7) / 8);
  hipLaunchKernelGGL((msa_attention_kernel<NW, SPW, FMT>), dim3(grid), dim3(NW * kWave), 0, stream,
                     p, lse_t, tau);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnParams& p, int fmt, const AttnPlan& plan,
                            hipStream_t stream) {
  if (plan.decode) return launch_decode(p, fmt, stream);
  switch (fmt) {
    case kFmtBf16:
      if (plan.async_bf16) return launch_prefill_bf16(p, plan.spw, stream);
      return launch_one<4, 2, kFmtBf16>(p, stream);
    case kFmtF16:   // the 16-bit prefill kernel, fp16 instantiation (p.out_f16)
      return launch_prefill_bf16(p, plan.spw, stream);
    case kFmtFp8: return launch_one<4, 2, kFmtFp8>(p, stream);
    default: return launch_one<4, 2, kFmtE2m1>(p, stream);
  }
}

hipError_t launch_attention_temperature(const AttnParams& p, int fmt, float* lse_t, float tau,
                                        hipStream_t stream) {
  switch (fmt) {
    case kFmtBf16: return launch_one<4, 2, kFmtBf16>(p, stream, lse_t, tau);
    case kFmtFp8: return launch_one<4, 2, kFmtFp8>(p, stream, lse_t, tau);
    case kFmtE2m1: return launch_one<4, 2, kFmtE2m1>(p, stream, lse_t, tau);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Tile union export (same builder as the attention kernel).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void msa_tile_union_kernel(
    const int32_t* __restrict__ q2k, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ len_k, int total_q, int hkv, int topk, int tiles_per_req,
    int max_k_tiles, int tile_tokens, int max_union, int32_t* __restrict__ ublocks,
    unsigned long long* __restrict__ umasks, int32_t* __restrict__ ucount) {
  __shared__ UnionLds un;
  const int tile = blockIdx.x % tiles_per_req;
  const int g = (blockIdx.x / tiles_per_req) % hkv;
  const int b = blockIdx.x / (tiles_per_req * hkv);
  const int q0 = cu_q[b];
  const int lq = cu_q[b + 1] - q0;
  const int i0 = tile * tile_tokens;
  const int64_t out_idx = ((int64_t)g * (gridDim.x / hkv) + (int64_t)b * tiles_per_req + tile);
  int32_t* ob = ublocks + out_idx * max_union;
  unsigned long long* om = umasks + out_idx * max_union;
  int cnt = 0;
  if (i0 < lq) {
    const int ntok = min(tile_tokens, lq - i0);
    const int nblk = max(0, min((len_k[b] + kBlock - 1) / kBlock, max_k_tiles));
    cnt = build_tile_union<256>(un, q2k + ((int64_t)g * total_q + q0 + i0) * topk, ntok, topk, nblk);
    for (int i = threadIdx.x; i < cnt; i += 256) {
      ob[i] = un.list[i];
      om[i] = un.mask[i];
    }
  }
  for (int i = cnt + threadIdx.x; i < max_union; i += 256) {
    ob[i] = -1;
    om[i] = 0ull;
  }
  if (threadIdx.x == 0) ucount[out_idx] = cnt;
}

hipError_t launch_tile_union(const int32_t* q2k, const int32_t* cu_q, const int32_t* len_k,
                             int batch, int total_q, int hkv, int topk, int max_seqlen_q,
                             int max_k_tiles, int tile_tokens, int max_union,
                             int32_t* ublocks, uint64_t* umasks, int32_t* ucount,
                             hipStream_t stream) {
  const int tiles = (max_seqlen_q + tile_tokens - 1) / tile_tokens;
  const int n = batch * hkv * tiles;
  if (n <= 0) return hipSuccess;
  // the kernel indexes outputs as [g][b][tile]; gridDim.x / hkv == batch * tiles
  hipLaunchKernelGGL(msa_tile_union_kernel, dim3(n), dim3(256), 0, stream, q2k, cu_q, len_k,
                     total_q, hkv, topk, tiles, max_k_tiles, tile_tokens, max_union, ublocks,
                     reinterpret_cast<unsigned long long*>(umasks), ucount);
  return hipGetLastError();
}

}  // namespace msa
