// Internal launch interfaces between the C ABI layer (api.cpp) and the HIP
// kernels.  Not installed; the public surface is include/msa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

enum KvFmt : int { kFmtBf16 = 0, kFmtFp8 = 1, kFmtE2m1 = 2, kFmtF16 = 3 };  // kFmtF16: fp16 Q, K, V, out

// Largest union a tile may hold (entries), and largest block-id bitmap.
constexpr int kMaxUnion = 512;
constexpr int kMaxBitmapWords = 512;   // block ids < 16384 (2M tokens)
constexpr int kMaxTopk = 64;

struct Strides {
  int64_t page, head, token;  // bytes
};

// Causal position of the queries: mode 0 right-aligned (Lk - Lq + iq),
// 1 base + iq, 2 rows[i] for query row i.
struct QueryPos {
  const int32_t* rows;
  int mode;
  int base;
};

struct AttnParams {
  const uint16_t* q;          // bf16 [total_q, Hq, 128]
  const uint8_t* k;
  const uint8_t* v;
  const uint8_t* ks;          // E2M1 block scales
  const uint8_t* vs;
  Strides k_st, v_st, ks_st, vs_st;
  const int32_t* q2k;
  const int32_t* cu_q;
  const int32_t* cu_k;        // flat route
  const int32_t* page_table;  // paged route
  const int32_t* seqused_k;
  int pt_width;
  int paged;
  uint16_t* out;
  int out_f16;                // out (and Q) are fp16 rather than bf16
  float* lse;                 // may be null
  int batch, total_q, hq, hkv, group, topk, causal;
  int max_k_tiles;            // bound on ceil(Lk / 128)
  int tok_per_tile;           // query tokens per tile
  int tiles_per_req;          // ceil(max_seqlen_q / tok_per_tile)
  int splits;                 // split-KV partials per tile (1 = none)
  float scale_log2;           // softmax_scale * k_global_scale * log2(e)
  float v_gs;
  float* ws_o;                // [units, splits, rows, 128] fp32 split partials (O / l)
  float* ws_lse;              // [units, splits, rows_pad] their natural-log LSE
  int ws_rows;                // rows per unit (tok_per_tile * group)
  int ws_lse_rows;            // rows_pad: rows rounded up to 32
  QueryPos qpos;              // causal positions of the queries
  // temperature LSE (ln sum_j exp(tau z_j)), written when lse_t is set
  float* lse_t;
  float tau;                  // lse_temperature_scale
  float tslack;               // rescale slack (log2 units) keeping 2^(tau (x - m)) <= 2^64
  float* ws_lse_t;            // [units, splits, rows_pad] split partials of lse_t
  uint32_t* ws_count;         // [units] split arrival counters, zero between launches
};

// Split-KV arrival counters sit in the last kCounterBytes of the caller's
// workspace (every workspace size the library reports reserves them, and
// nothing else writes there): zero-filled before first use, each unit's
// counter is reset by the workgroup that merges it.
constexpr size_t kCounterBytes = 64 * 1024;
constexpr int kMaxCounterUnits = (int)(kCounterBytes / 4);

// Kernel family selection for one attention call.
struct AttnPlan {
  int decode;       // 1: decode kernel (<= 64 rows per token tile), 0: prefill tiles
  int tok_per_tile;
  int splits;
};

// 16-bit (bf16, or fp16 with p.out_f16) prefill tiles of 256 rows: 8 waves x 1 slot
hipError_t launch_prefill_bf16(const AttnParams& p, hipStream_t stream);

// decode kernel (+ split merge when p.splits > 1); workgroups one CU holds
hipError_t launch_decode(const AttnParams& p, int fmt, hipStream_t stream);
int decode_workgroups_per_cu(int fmt, int rows);

struct ProxyParams {
  const uint16_t* q;
  const uint8_t* k;
  Strides k_st;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* page_table;
  const int32_t* seqused_k;
  int pt_width, paged;
  float* out;
  int batch, total_q, hq, hkv, group, causal, reduce;
  int max_k_tiles;
  int rows_per_tile;          // query rows (token x head) per workgroup
  int row_tiles;              // ceil(max_seqlen_q * group / rows_per_tile)
  int blocks_per_wg;          // KV blocks per workgroup (decode-shaped path)
  int block_chunks;           // ceil(max_k_tiles / blocks_per_wg)
  int pieces;                 // prefill-shaped path: workgroups per row-tile pair
  QueryPos qpos;              // causal positions of the queries
  // running top-K (decode shapes): each workgroup writes the top-K of its
  // chunk per query instead of scores, [sel_rows, total_q, Hg, chunks, topk]
  float* cand_s;
  int32_t* cand_id;
  int topk;
};

// Most KV blocks of one row tile a prefill-shaped proxy workgroup scores.
constexpr int kWideMaxSeg = 64;
// Blocks a prefill-shaped proxy piece is charged for running over from one
// row tile into the next (a second start: Q rows, first K block).
constexpr int kSegSwitch = 2;

hipError_t launch_proxy(const ProxyParams& p, int fmt, int wide_rows, hipStream_t stream);
// decode-shaped proxy (<= 64 rows per request and KV head) writing per-chunk
// top-K candidates (p.cand_s, p.cand_id) instead of scores
hipError_t launch_proxy_candidates(const ProxyParams& p, int fmt, hipStream_t stream);

hipError_t launch_topk(const float* scores, int score_heads, int T, int total_q, int topk,
                       int hkv, int mode, int32_t* q2k, hipStream_t stream);

// q2k from per-chunk top-K candidates ([sel_rows, total_q, n_cand] scores
// and block ids, -1 padded): ids folded by max score, then the top-K; shared:
// one selection written to every KV head's row.
hipError_t launch_topk_merge(const float* cand_s, const int32_t* cand_id, int n_cand, int T,
                             int total_q, int topk, int hkv, int shared, int32_t* q2k,
                             hipStream_t stream);

struct QsaParams {
  const uint16_t* q;          // bf16 [total_q, hq, 256]
  const uint16_t* k;          // bf16 rows of 256, addressed by token and head strides
  const uint16_t* v;
  int64_t k_row_stride, k_head_stride, v_row_stride, v_head_stride;   // bytes
  const int32_t* indices;     // [total_q, width] (indexed source)
  const uint8_t* bitmap;      // [total_q, num_blocks] (bitmap source) or null
  int num_blocks, num_kv_tokens;
  uint16_t* out;              // bf16 [total_q, hq, 256]
  float* out_f32;             // fp32 [total_q, hq, 256] or null
  float* lse;                 // fp32 [hq, total_q] or null
  int total_q, hq, hkv, group, width;
  float scale_log2;           // softmax_scale * log2(e)
};

hipError_t launch_qsa(const QsaParams& p, hipStream_t stream);   // bitmap source when p.bitmap

hipError_t launch_tile_union(const int32_t* q2k, const int32_t* cu_q, const int32_t* len_k,
                             int batch, int total_q, int hkv, int topk, int max_seqlen_q,
                             int max_k_tiles, int tile_tokens, int max_union,
                             int32_t* ublocks, uint64_t* umasks, int32_t* ucount,
                             hipStream_t stream);

}  // namespace msa
