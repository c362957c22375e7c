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
// step.  With reduce_heads the max over query heads happens in-kernel: within
// a wave across the G heads of a token, then across KV heads with an exact
// order-independent atomic max into an output pre-filled with -inf.
#include "common.hpp"
#include "internal.hpp"

namespace msa {

constexpr int kPKPitch = 136;  // bf16 per K row in LDS

template <int FMT>
struct ProxyStage;

template <>
struct ProxyStage<kFmtBf16> {
  static constexpr int KT = 2048 / 256;
  u32x4 kr[KT];
  __device__ void issue(const uint8_t* kb, int64_t st, int nvalid) {
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      int task = i * 256 + threadIdx.x, row = task >> 4, c = task & 15;
      kr[i] = row < nvalid ? *reinterpret_cast<const u32x4*>(kb + row * st + 16 * c)
                           : u32x4{0, 0, 0, 0};
    }
  }
  __device__ void store(uint16_t* k) const {
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      int task = i * 256 + threadIdx.x, row = task >> 4, c = task & 15;
      *reinterpret_cast<u32x4*>(&k[row * kPKPitch + 8 * c]) = kr[i];
    }
  }
};

template <>
struct ProxyStage<kFmtFp8> {
  static constexpr int KT = 1024 / 256;
  u32x4 kr[KT];
  __device__ void issue(const uint8_t* kb, int64_t st, int nvalid) {
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      int task = i * 256 + threadIdx.x, row = task >> 3, c = task & 7;
      kr[i] = row < nvalid ? *reinterpret_cast<const u32x4*>(kb + row * st + 16 * c)
                           : u32x4{0, 0, 0, 0};
    }
  }
  __device__ static uint32_t byte_of(const u32x4& v, int e) {
    return (v[e >> 2] >> (8 * (e & 3))) & 0xFFu;
  }
  __device__ void store(uint16_t* k) const {
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      int task = i * 256 + threadIdx.x, row = task >> 3, c = task & 7;
      u32x4 w0, w1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0[e] = pack_bf16x2(e4m3_to_f32(byte_of(kr[i], 2 * e)), e4m3_to_f32(byte_of(kr[i], 2 * e + 1)));
        w1[e] = pack_bf16x2(e4m3_to_f32(byte_of(kr[i], 8 + 2 * e)), e4m3_to_f32(byte_of(kr[i], 9 + 2 * e)));
      }
      *reinterpret_cast<u32x4*>(&k[row * kPKPitch + 16 * c]) = w0;
      *reinterpret_cast<u32x4*>(&k[row * kPKPitch + 16 * c + 8]) = w1;
    }
  }
};

// NTW: 32-row N tiles per wave.  KSW: 32-key subtiles per wave (of 4 per block).
template <int NTW, int KSW, int FMT, bool REDUCE>
__global__ __launch_bounds__(256) void msa_proxy_kernel(ProxyParams p) {
  constexpr int KG = 4 / KSW;          // waves sharing the same rows
  constexpr int RG = 4 / KG;           // row groups
  constexpr int RW = RG * NTW * 32;    // rows per workgroup
  __shared__ uint16_t klds[kBlock * kPKPitch];
  __shared__ float red[KG][RW];

  const int n = p.batch * p.hkv * p.row_tiles * p.block_chunks;
  const int lid = xcd_remap(blockIdx.x, n);
  if (lid < 0) return;
  const int chunk = lid % p.block_chunks;
  int rest = lid / p.block_chunks;
  const int rt = rest % p.row_tiles;
  rest /= p.row_tiles;
  const int g = rest % p.hkv;
  const int b = rest / p.hkv;

  const int G = p.group;
  const int q0 = p.cu_q[b];
  const int lq = p.cu_q[b + 1] - q0;
  const int nrows = lq * G;
  const int r0 = rt * RW;
  if (r0 >= nrows) return;
  const int lk = p.paged ? p.seqused_k[b] : (p.cu_k[b + 1] - p.cu_k[b]);
  const int nblk = max(0, (lk + kBlock - 1) / kBlock);
  const int t_beg = chunk * p.blocks_per_wg;
  const int t_end = min(t_beg + p.blocks_per_wg, p.max_k_tiles);
  if (t_beg >= t_end) return;

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int rgp = wave / KG;
  const int kgp = wave % KG;

  const int r_last = min(r0 + RW, nrows) - 1;
  const int pos_max = lk - lq + r_last / G;
  // blocks with at least one visible key for some row of the tile
  int t_act = min(t_end, nblk);
  if (p.paged) t_act = min(t_act, p.pt_width);
  if (p.causal) t_act = min(t_act, pos_max < 0 ? 0 : pos_max / kBlock + 1);
  t_act = max(t_act, t_beg);

  // rows of this wave
  int row_[NTW], pos_[NTW];
  bf16x8 qf[NTW][8];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int r = r0 + (rgp * NTW + nt) * 32 + col;
    row_[nt] = r;
    const int tk = r / G, hh = r % G;
    pos_[nt] = lk - lq + tk;
    if (r < nrows) {
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(
          p.q + ((int64_t)(q0 + tk) * p.hq + g * G + hh) * kHeadDim);
#pragma unroll
      for (int s = 0; s < 8; ++s)
        qf[nt][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 2 * (16 * s + 8 * half)));
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[nt][s] = as_bf16x8(u32x4{0, 0, 0, 0});
    }
  }

  // fully masked blocks of the chunk: -inf (pre-filled when reducing)
  if (!REDUCE && kgp == 0 && half == 0) {
    for (int t = t_act; t < t_end; ++t) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int r = row_[nt];
        if (r < nrows) {
          const int tk = r / G, hh = r % G;
          p.out[((int64_t)(g * G + hh) * p.max_k_tiles + t) * p.total_q + q0 + tk] = -INFINITY;
        }
      }
    }
  }

  auto kbase_of = [&](int t) -> const uint8_t* {
    if (p.paged) {
      int64_t page = p.page_table[(int64_t)b * p.pt_width + t];
      return p.k + page * p.k_st.page + g * p.k_st.head;
    }
    return p.k + ((int64_t)p.cu_k[b] + kBlock * t) * p.k_st.token + g * p.k_st.head;
  };

  ProxyStage<FMT> stage;
  if (t_beg < t_act) stage.issue(kbase_of(t_beg), p.k_st.token, min(kBlock, lk - kBlock * t_beg));

  for (int t = t_beg; t < t_act; ++t) {
    const int nvalid = min(kBlock, lk - kBlock * t);
    __syncthreads();
    stage.store(klds);
    __syncthreads();
    if (t + 1 < t_act) stage.issue(kbase_of(t + 1), p.k_st.token, min(kBlock, lk - kBlock * (t + 1)));

    float cm[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) cm[nt] = -INFINITY;
#pragma unroll
    for (int ktl = 0; ktl < KSW; ++ktl) {
      const int kt = kgp * KSW + ktl;
      f32x16 acc[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
            &klds[(32 * kt + col) * kPKPitch + 16 * s + 8 * half]));
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) acc[nt] = mfma32(a, qf[nt][s], acc[nt]);
      }
      // Visible keys of this block for a row: key <= lim.  Written without
      // short-circuit logic so the select stays a plain compare + cndmask on
      // the accumulator values.
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        int lim = nvalid - 1;
        if (p.causal) lim = min(lim, pos_[nt] - kBlock * t);
        float m = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
          const float v = acc[nt][r];
          m = fmaxf(m, key <= lim ? v : -INFINITY);
        }
        m = xor_max(m, 32);
        cm[nt] = fmaxf(cm[nt], m);
      }
    }
    if constexpr (KG > 1) {
      if (half == 0) {
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) red[kgp][(rgp * NTW + nt) * 32 + col] = cm[nt];
      }
      __syncthreads();
      if (kgp != 0) continue;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int k = 1; k < KG; ++k) cm[nt] = fmaxf(cm[nt], red[k][(rgp * NTW + nt) * 32 + col]);
    }
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int r = row_[nt];
      const int tk = r / G, hh = r % G;
      if constexpr (!REDUCE) {
        if (half == 0 && r < nrows)
          p.out[((int64_t)(g * G + hh) * p.max_k_tiles + t) * p.total_q + q0 + tk] = cm[nt];
      } else {
        float v = cm[nt];
        // max over the G heads of a token when they share this 32-lane half
        if ((G & (G - 1)) == 0 && G <= 32) {
          for (int off = 1; off < G; off <<= 1) v = xor_max(v, off);
          if (half == 0 && r < nrows && hh == 0)
            atomic_max_f32(&p.out[(int64_t)t * p.total_q + q0 + tk], v);
        } else if (half == 0 && r < nrows) {
          atomic_max_f32(&p.out[(int64_t)t * p.total_q + q0 + tk], v);
        }
      }
    }
  }
}

__global__ void msa_fill_kernel(float* __restrict__ out, int64_t n, float v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) out[i] = v;
}

template <int NTW, int KSW, int FMT>
static hipError_t launch_proxy_t(const ProxyParams& p, hipStream_t stream) {
  const int n = p.batch * p.hkv * p.row_tiles * p.block_chunks;
  if (n <= 0) return hipSuccess;
  const int grid = 8 * ((n + 7) / 8);
  if (p.reduce) {
    const int64_t total = (int64_t)p.max_k_tiles * p.total_q;
    if (total > 0) {
      int fb = (int)std::min<int64_t>((total + 255) / 256, 4096);
      hipLaunchKernelGGL(msa_fill_kernel, dim3(fb), dim3(256), 0, stream, p.out, total, -INFINITY);
    }
    hipLaunchKernelGGL((msa_proxy_kernel<NTW, KSW, FMT, true>), dim3(grid), dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL((msa_proxy_kernel<NTW, KSW, FMT, false>), dim3(grid), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

// wide_rows: 1 -> 256 rows per workgroup (4 row groups x 64); 0 -> 64 rows
// shared by 4 waves that split each block's keys.
hipError_t launch_proxy(const ProxyParams& p, int fmt, int wide_rows, hipStream_t stream) {
  if (wide_rows) {
    return fmt == kFmtFp8 ? launch_proxy_t<2, 4, kFmtFp8>(p, stream)
                          : launch_proxy_t<2, 4, kFmtBf16>(p, stream);
  }
  return fmt == kFmtFp8 ? launch_proxy_t<2, 1, kFmtFp8>(p, stream)
                        : launch_proxy_t<2, 1, kFmtBf16>(p, stream);
}

}  // namespace msa
