// C ABI of the MSA library: host-side validation, launch planning and
// dispatch.  No device memory is allocated and the host never waits on the
// device; every launch goes to the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/msa.h"
#include "internal.hpp"
#include "stage16.hpp"
#include "validate.hpp"

namespace {

thread_local char g_last_error[512] = "";

msa_status_t fail(msa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

msa_status_t ok() {
  g_last_error[0] = '\0';
  return MSA_OK;
}

msa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// q_offset_mode / q_offset_value / q_offset of the attention and proxy
// arguments -> the kernels' query positions.
msa_status_t resolve_qpos(int32_t mode, int32_t value, const int32_t* rows, bool need_ptrs,
                          msa::QueryPos* out) {
  if (mode < 0 || mode > 2)
    return fail(MSA_ERR_UNSUPPORTED, "q_offset_mode must be 0 (right-aligned), 1 (q_offset_value "
                "+ iq) or 2 (per-row q_offset), got %d", mode);
  if (mode == 1 && (value < -(1 << 30) || value > (1 << 30)))
    return fail(MSA_ERR_SHAPE, "q_offset_value %d is outside [-2^30, 2^30]", value);
  if (mode == 2 && need_ptrs && !rows)
    return fail(MSA_ERR_NULL, "q_offset_mode 2 needs the q_offset tensor");
  out->mode = mode;
  out->base = mode == 1 ? value : 0;
  out->rows = mode == 2 ? rows : nullptr;
  return MSA_OK;
}

constexpr int64_t kMaxTokenStride = (int64_t)1 << 24;

// Longest query (tokens per request) that takes the decode kernel with one
// token per tile (G >= 16); longer queries take the prefill tiles.
constexpr int kDecodeMaxTokens = 64;

// Resolve a stride triple for a tensor with `row_bytes` contiguous bytes per
// token row.  Dense layout for zeros.  Rejects unaligned views.
msa_status_t resolve_strides(const char* name, const msa_strides_t& in, bool paged, int hkv,
                             int64_t row_bytes, int64_t align, msa::Strides* out) {
  msa::Strides s;
  s.token = in.token ? in.token : row_bytes;
  if (paged) {
    s.head = in.head ? in.head : (int64_t)128 * s.token;
    s.page = in.page ? in.page : (int64_t)hkv * s.head;
  } else {
    s.head = in.head ? in.head : row_bytes;
    s.token = in.token ? in.token : (int64_t)hkv * row_bytes;
    s.page = 0;
  }
  // (kernels address a 128-token block as base + 32-bit per-lane offset)
  if (s.token < row_bytes || s.token > kMaxTokenStride || s.token % align || s.head % align ||
      s.page % align || s.head < 0 || s.page < 0)
    return fail(MSA_ERR_UNSUPPORTED,
                "%s: strides (page %lld, head %lld, token %lld bytes) are not a readable view "
                "(rows of %lld contiguous bytes, %lld-byte aligned, token stride <= %lld); "
                "views are never copied",
                name, (long long)s.page, (long long)s.head, (long long)s.token,
                (long long)row_bytes, (long long)align, (long long)kMaxTokenStride);
  *out = s;
  return MSA_OK;
}

int kv_row_bytes(int fmt) {
  return (fmt == MSA_KV_BF16 || fmt == MSA_KV_F16) ? 256 : (fmt == MSA_KV_FP8_E4M3 ? 128 : 64);
}

struct Resolved {
  msa::AttnParams p;
  msa::AttnPlan plan;
  size_t ws_bytes;
  bool stage16;   // fp8 / E2M1 prefill: K/V staged to bf16 pages in the workspace
  int stage_slots; // staged pages per request when only selected blocks are staged, else 0
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

msa_status_t resolve_attention(const msa_attn_args_t* a, Resolved* r, bool need_ptrs) {
  if (!a) return fail(MSA_ERR_NULL, "args is NULL");
  if (a->batch < 0 || a->total_q < 0)
    return fail(MSA_ERR_SHAPE, "batch (%d) and total_q (%d) must be >= 0", a->batch, a->total_q);
  if (a->head_dim != 128) return fail(MSA_ERR_SHAPE, "head_dim must be 128 (got %d)", a->head_dim);
  if (a->num_qo_heads <= 0 || a->num_kv_heads <= 0 || a->num_qo_heads % a->num_kv_heads)
    return fail(MSA_ERR_SHAPE, "num_qo_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                a->num_qo_heads, a->num_kv_heads);
  if (a->topk < 1 || a->topk > msa::kMaxTopk)
    return fail(MSA_ERR_SHAPE, "topk must be in [1, %d] (got %d)", msa::kMaxTopk, a->topk);
  if (a->max_seqlen_q < 0 || a->max_k_tiles < 0)
    return fail(MSA_ERR_SHAPE, "max_seqlen_q and max_k_tiles must be >= 0");
  if (a->max_k_tiles > msa::kMaxBitmapWords * 32)
    return fail(MSA_ERR_SHAPE, "max_k_tiles %d exceeds %d blocks", a->max_k_tiles,
                msa::kMaxBitmapWords * 32);
  if (a->kv_dtype < MSA_KV_BF16 || a->kv_dtype > MSA_KV_F16)
    return fail(MSA_ERR_DTYPE, "unknown kv_dtype %d", a->kv_dtype);
  const bool paged = a->page_table != nullptr;
  if (paged) {
    if (a->cu_seqlens_k && a->seqused_k)
      return fail(MSA_ERR_CONFLICT,
                  "paged route: both cu_seqlens_k and seqused_k were given; seqused_k is the "
                  "only source of KV lengths and the call is declined rather than choosing one");
    if (!a->seqused_k) return fail(MSA_ERR_NULL, "paged route needs seqused_k");
    if (a->page_table_width < a->max_k_tiles || a->page_table_width <= 0)
      return fail(MSA_ERR_SHAPE, "page_table_width (%d) must be >= max_k_tiles (%d) and > 0",
                  a->page_table_width, a->max_k_tiles);
  } else {
    if (!a->cu_seqlens_k) return fail(MSA_ERR_NULL, "flat route needs cu_seqlens_k");
  }
  if (need_ptrs && a->kv_dtype == MSA_KV_E2M1X2 && (!a->k_scale || !a->v_scale))
    return fail(MSA_ERR_NULL, "packed E2M1 K/V needs k_scale and v_scale");
  if (a->kv_dtype != MSA_KV_E2M1X2 && (a->k_scale || a->v_scale))
    return fail(MSA_ERR_UNSUPPORTED, "k_scale/v_scale are only read with packed E2M1 K/V");
  if (need_ptrs && a->total_q > 0 && a->batch > 0) {
    if (!a->q || !a->k || !a->v || !a->q2k || !a->cu_seqlens_q || !a->out)
      return fail(MSA_ERR_NULL, "q, k, v, q2k, cu_seqlens_q and out must be non-NULL");
    if (!aligned(a->q, 16) || !aligned(a->out, 16) || !aligned(a->k, 16) || !aligned(a->v, 16))
      return fail(MSA_ERR_UNSUPPORTED, "q, k, v and out must be 16-byte aligned");
  }

  msa::AttnParams& p = r->p;
  std::memset(&p, 0, sizeof(p));
  const int fmt = a->kv_dtype;   // msa_kv_dtype_t values are the kernels' formats
  p.out_f16 = a->kv_dtype == MSA_KV_F16 ? 1 : 0;
  const int rb = kv_row_bytes(fmt);
  msa_status_t st;
  if ((st = resolve_strides("k", a->k_strides, paged, a->num_kv_heads, rb, 16, &p.k_st))) return st;
  if ((st = resolve_strides("v", a->v_strides, paged, a->num_kv_heads, rb, 16, &p.v_st))) return st;
  if (fmt == MSA_KV_E2M1X2) {
    if ((st = resolve_strides("k_scale", a->k_scale_strides, paged, a->num_kv_heads, 8, 8, &p.ks_st)))
      return st;
    if ((st = resolve_strides("v_scale", a->v_scale_strides, paged, a->num_kv_heads, 8, 8, &p.vs_st)))
      return st;
    // paged: the decode kernel stages a head's scale rows two at a time (16
    // bytes), so they must be contiguous within the page; flat scales (any
    // (token, head) strides of 8-byte rows) are read row by row by the
    // general kernel
    if (paged && (p.ks_st.token != 8 || p.vs_st.token != 8 || p.ks_st.page % 16 ||
                  p.vs_st.page % 16 ||
                  (a->num_kv_heads > 1 && (p.ks_st.head % 16 || p.vs_st.head % 16))))
      return fail(MSA_ERR_UNSUPPORTED,
                  "paged k_scale/v_scale: a head's token rows must be contiguous (8 bytes) and "
                  "page/head strides multiples of 16 bytes");
    if (need_ptrs && (!aligned(a->k_scale, 16) || !aligned(a->v_scale, 16)))
      return fail(MSA_ERR_UNSUPPORTED, "k_scale/v_scale must be 16-byte aligned");
  }

  const int G = a->num_qo_heads / a->num_kv_heads;
  p.q = static_cast<const uint16_t*>(a->q);
  p.k = static_cast<const uint8_t*>(a->k);
  p.v = static_cast<const uint8_t*>(a->v);
  p.ks = static_cast<const uint8_t*>(a->k_scale);
  p.vs = static_cast<const uint8_t*>(a->v_scale);
  p.q2k = a->q2k;
  p.cu_q = a->cu_seqlens_q;
  p.cu_k = a->cu_seqlens_k;
  p.page_table = a->page_table;
  p.seqused_k = a->seqused_k;
  p.pt_width = a->page_table_width;
  p.paged = paged;
  p.out = static_cast<uint16_t*>(a->out);
  p.lse = a->lse;
  p.batch = a->batch;
  p.total_q = a->total_q;
  p.hq = a->num_qo_heads;
  p.hkv = a->num_kv_heads;
  p.group = G;
  p.topk = a->topk;
  p.causal = a->causal ? 1 : 0;
  p.max_k_tiles = a->max_k_tiles;
  const float scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.0f / std::sqrt(128.0f);
  const float kgs = a->k_global_scale > 0.f ? a->k_global_scale : 1.0f;
  p.scale_log2 = scale * kgs * 1.4426950408889634f;
  p.v_gs = a->v_global_scale > 0.f ? a->v_global_scale : 1.0f;
  if ((st = resolve_qpos(a->q_offset_mode, a->q_offset_value, a->q_offset,
                         need_ptrs && a->total_q > 0 && a->batch > 0, &p.qpos)))
    return st;

  // ---- plan ----
  msa::AttnPlan& plan = r->plan;
  plan = msa::AttnPlan{};
  r->stage16 = false;
  const int lqmax = std::max(1, a->max_seqlen_q);
  const int rows_req = lqmax * G;
  // packed E2M1 in the flat layout takes the prefill tiles at every shape:
  // the decode kernel stages block-scale rows two at a time, which needs a
  // head's rows contiguous and stays inside a 128-row page, but could pass
  // the end of a flat tensor
  const bool flat_e2m1 = !paged && a->kv_dtype == MSA_KV_E2M1X2;
  // the temperature LSE is accumulated by the decode and prefill kernels
  // beside the row sum
  const bool temp = a->lse_t != nullptr;
  if (temp && !(a->lse_temperature_scale > 0.f && std::isfinite(a->lse_temperature_scale)))
    return fail(MSA_ERR_UNSUPPORTED, "lse_temperature_scale must be finite and > 0 (got %g)",
                (double)a->lse_temperature_scale);
  p.lse_t = a->lse_t;
  p.tau = temp ? a->lse_temperature_scale : 1.0f;
  {
    // 2^(tau (x - m)) <= 2^64 for every accepted score: the reference max
    // moves once a score passes it by 64 / tau (and at most by the format's
    // own slack)
    const float base = a->kv_dtype == MSA_KV_F16 ? 15.0f : 64.0f;
    p.tslack = std::min(base, 64.0f / p.tau);
  }
  // When one token's G heads fill a 16-row MFMA tile, every token of a short
  // query is a decode tile of its own: it streams just the pages it selected
  // (a union over the request's tokens would make each page cost all of
  // their row tiles), with less state per workgroup.
  const bool per_token = G >= 16 && G <= 64 && lqmax > 1 && lqmax <= kDecodeMaxTokens;
  const int dec_rows = per_token ? G : rows_req;
  // a decode tile holds all of a request's tokens: their selections must fit
  // the union list, else the prefill tiles (which shrink to fit) take them
  const bool dec_union_fits = (per_token ? 1 : lqmax) * a->topk <= msa::kMaxUnion;
  if (dec_rows <= 64 && !flat_e2m1 && dec_union_fits) {
    // decode shape: one workgroup per (request, KV head, token tile, split);
    // its waves split every page's keys
    plan.decode = 1;
    plan.tok_per_tile = per_token ? 1 : lqmax;
    const int tiles = (lqmax + plan.tok_per_tile - 1) / plan.tok_per_tile;
    const int units = std::max(1, a->batch * a->num_kv_heads * tiles);
    const int union_max = std::min(plan.tok_per_tile * a->topk, std::max(1, a->max_k_tiles));
    int splits;
    if (a->splits > 0) {
      splits = a->splits;
    } else {
      // fill every CU (256) with as many workgroups as its LDS holds, with at
      // least 8 pages per split (fewer leave a wave's page ring too short to
      // hide its own latencies: 4 splits of 4 pages ran slower than 2 of 8)
      const int target =
          256 * msa::decode_workgroups_per_cu(a->kv_dtype, plan.tok_per_tile * G);
      splits = std::max(1, std::min((target + units - 1) / units, union_max / 8));
      splits = std::min(splits, 16);
    }
    plan.splits = std::max(1, std::min(splits, 64));
  } else {
    plan.decode = 0;
    // fp8 / E2M1 K/V: converted to bf16 pages once, then the bf16 kernel
    r->stage16 = a->kv_dtype == MSA_KV_FP8_E4M3 || a->kv_dtype == MSA_KV_E2M1X2;
    // 8 waves x one 32-row slot (two waves per SIMD overlap MFMA and
    // softmax work)
    const int rows = 256;
    if (G > rows)
      return fail(MSA_ERR_SHAPE,
                  "num_qo_heads / num_kv_heads = %d exceeds the %d query rows of a prefill tile",
                  G, rows);
    plan.tok_per_tile = std::max(1, std::min(64, rows / G));
    plan.splits = 1;
  }
  if (plan.tok_per_tile * a->topk > msa::kMaxUnion) {
    if (plan.decode)
      return fail(MSA_ERR_SHAPE, "seqlen_q (%d) x topk (%d) exceeds the %d-entry tile union",
                  lqmax, a->topk, msa::kMaxUnion);
    plan.tok_per_tile = std::max(1, msa::kMaxUnion / a->topk);
  }
  p.tok_per_tile = plan.tok_per_tile;
  p.tiles_per_req = (lqmax + plan.tok_per_tile - 1) / plan.tok_per_tile;
  p.splits = plan.splits;

  r->ws_bytes = 0;
  r->stage_slots = 0;
  if (r->stage16) {
    r->stage_slots = msa::stage16_slots(a->max_seqlen_q, a->num_kv_heads, a->topk, a->max_k_tiles);
    r->ws_bytes = msa::stage16_bytes(a->batch, a->max_k_tiles, a->num_kv_heads, r->stage_slots);
  }
  if (plan.splits > 1) {
    if ((int64_t)a->batch * a->num_kv_heads * p.tiles_per_req > msa::kMaxCounterUnits)
      return fail(MSA_ERR_SHAPE, "split-KV over %lld (request, KV head, token tile) units: at most "
                  "%d are counted; use splits = 1", (long long)a->batch * a->num_kv_heads *
                  p.tiles_per_req, msa::kMaxCounterUnits);
    // [partial LSE][partial O][partial temperature LSE (with lse_t)]
    const int rows = plan.tok_per_tile * G;
    const int rows_pad = (rows + 31) / 32 * 32;
    const size_t units = (size_t)a->batch * a->num_kv_heads * p.tiles_per_req;
    p.ws_rows = rows;
    p.ws_lse_rows = rows_pad;
    const size_t l_bytes = round_up(units * plan.splits * rows_pad * sizeof(float), 256);
    r->ws_bytes = l_bytes + round_up(units * plan.splits * rows * 128 * sizeof(float), 256) +
                  (temp ? l_bytes : 0);
  }
  // every nonzero workspace keeps the split counters' tail free: the data
  // ends on a 256-byte boundary, and the counters take the last
  // kCounterBytes of the (256-byte rounded-down) buffer, past any data
  if (r->ws_bytes) r->ws_bytes = round_up(r->ws_bytes, 256) + msa::kCounterBytes;
  return MSA_OK;
}

}  // namespace

extern "C" {

const char* msa_status_string(msa_status_t s) {
  switch (s) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_NULL: return "MSA_ERR_NULL";
    case MSA_ERR_SHAPE: return "MSA_ERR_SHAPE";
    case MSA_ERR_DTYPE: return "MSA_ERR_DTYPE";
    case MSA_ERR_CONFLICT: return "MSA_ERR_CONFLICT";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
    case MSA_ERR_CONTRACT: return "MSA_ERR_CONTRACT";
  }
  return "MSA_ERR_UNKNOWN";
}

const char* msa_last_error(void) { return g_last_error; }

const char* msa_version(void) { return "0.1.0"; }

msa_status_t msa_sparse_attention_workspace_size(const msa_attn_args_t* args, size_t* bytes) {
  if (!bytes) return fail(MSA_ERR_NULL, "bytes is NULL");
  Resolved r;
  msa_status_t st = resolve_attention(args, &r, false);
  if (st) return st;
  *bytes = r.ws_bytes;
  return ok();
}

msa_status_t msa_sparse_attention_plan(const msa_attn_args_t* args, int32_t* decode_route,
                                       int32_t* splits) {
  if (!decode_route || !splits) return fail(MSA_ERR_NULL, "decode_route and splits must be non-NULL");
  Resolved r;
  msa_status_t st = resolve_attention(args, &r, false);
  if (st) return st;
  *decode_route = r.plan.decode;
  *splits = r.plan.splits;
  return ok();
}

msa_status_t msa_validate_attention(const msa_attn_args_t* a, void* stream) {
  Resolved r;
  msa_status_t st = resolve_attention(a, &r, true);
  if (st) return st;
  if (a->total_q == 0 || a->batch == 0) return ok();
  msa::ValidateParams v;
  v.batch = a->batch;
  v.total_q = a->total_q;
  v.hkv = a->num_kv_heads;
  v.topk = a->topk;
  v.max_seqlen_q = a->max_seqlen_q;
  v.max_k_tiles = a->max_k_tiles;
  v.paged = a->page_table != nullptr;
  v.pt_width = v.paged ? a->page_table_width : 0;
  v.q2k = a->q2k;
  v.cu_q = a->cu_seqlens_q;
  v.cu_k = a->cu_seqlens_k;
  v.page_table = a->page_table;
  v.seqused = a->seqused_k;
  unsigned long long word = ~0ull;
  if ((st = hip_status(msa::run_validate(v, static_cast<hipStream_t>(stream), &word),
                       "msa_validate_attention")))
    return st;
  if (word == ~0ull) return ok();
  const int kind = (int)(word >> 48);
  const long long pos = (long long)(word & ((1ull << 48) - 1));
  switch (kind) {
    case msa::kValCuQ:
      return fail(MSA_ERR_CONTRACT, "cu_seqlens_q at request %lld: must start at 0, end at "
                  "total_q (%d) and give lengths in [0, max_seqlen_q = %d]", pos, a->total_q,
                  a->max_seqlen_q);
    case msa::kValCuK:
      return fail(MSA_ERR_CONTRACT, "cu_seqlens_k decreases after request %lld", pos);
    case msa::kValKvLen:
      return fail(MSA_ERR_CONTRACT, "KV length of request %lld is outside [0, 128 * %d]", pos,
                  v.paged ? std::min(a->max_k_tiles, a->page_table_width) : a->max_k_tiles);
    case msa::kValPage:
      return fail(MSA_ERR_CONTRACT, "page_table[%lld, %lld] is negative inside the request's "
                  "pages", pos / v.pt_width, pos % v.pt_width);
    case msa::kValQ2kPad:
    case msa::kValQ2kOrder: {
      const long long row = pos / a->topk, e = pos % a->topk;
      return fail(MSA_ERR_CONTRACT, "q2k[g=%lld, i=%lld] entry %lld %s", row / a->total_q,
                  row % a->total_q, e,
                  kind == msa::kValQ2kPad ? "follows -1 padding (padding must be trailing)"
                                          : "is not above the previous block id (rows ascend "
                                            "without repeats)");
    }
  }
  return fail(MSA_ERR_CONTRACT, "contract violation kind %d at %lld", kind, pos);
}

}  // extern "C"

namespace {

// Launches a resolved attention call with `workspace` (already checked for
// size when r.ws_bytes > 0).
msa_status_t run_attention(const msa_attn_args_t* args, Resolved& r, void* workspace,
                           size_t workspace_bytes, void* stream) {
  msa_status_t st;
  // debug path: check the device-side contracts first (synchronises the stream)
  const char* env = std::getenv("MSA_VALIDATE");
  if (env && env[0] == '1' && (st = msa_validate_attention(args, stream))) return st;
  if (r.ws_bytes) {
    if (!workspace || workspace_bytes < r.ws_bytes)
      return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu at %p)", r.ws_bytes,
                  workspace_bytes, workspace);
    if (!aligned(workspace, 256)) return fail(MSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  if (r.ws_bytes && !r.stage16) {
    // layout: [partial LSE][partial O][partial temperature LSE]
    const size_t units = (size_t)args->batch * args->num_kv_heads * r.p.tiles_per_req;
    const size_t l_bytes = round_up(units * r.plan.splits * r.p.ws_lse_rows * sizeof(float), 256);
    const size_t o_bytes =
        round_up(units * r.plan.splits * r.p.ws_rows * 128 * sizeof(float), 256);
    char* base = static_cast<char*>(workspace);
    r.p.ws_lse = reinterpret_cast<float*>(base);
    r.p.ws_o = reinterpret_cast<float*>(base + l_bytes);
    r.p.ws_lse_t = args->lse_t ? reinterpret_cast<float*>(base + l_bytes + o_bytes) : nullptr;
    // the counters: the last kCounterBytes of the caller's buffer
    r.p.ws_count = reinterpret_cast<uint32_t*>(base + workspace_bytes / 256 * 256 -
                                               msa::kCounterBytes);
  }
  if (args->total_q == 0 || args->batch == 0) return ok();
  if (r.stage16) {
    msa::AttnParams pq;
    msa_status_t st2 = hip_status(msa::launch_stage16(r.p, args->kv_dtype, r.stage_slots, workspace, &pq,
                                                      static_cast<hipStream_t>(stream)),
                                  "msa_sparse_attention staging launch");
    if (st2) return st2;
    return hip_status(msa::launch_prefill_bf16(pq, static_cast<hipStream_t>(stream)),
                      "msa_sparse_attention launch");
  }
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  return hip_status(r.plan.decode ? msa::launch_decode(r.p, args->kv_dtype, hs)
                                  : msa::launch_prefill_bf16(r.p, hs),
                    "msa_sparse_attention launch");
}

// Scratch of the allocation-free entry point: one array per GPU the library
// runs on, held until the process ends.  Host code never passes `scratch`
// itself (in host code the name is not a device address): it looks up each
// device's address once with hipGetSymbolAddress and passes that.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on its first use.
msa_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MSA_ERR_UNSUPPORTED, "device %d is past the %d devices the scratch table holds",
                dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

}  // namespace

extern "C" {

msa_status_t msa_sparse_attention(const msa_attn_args_t* args, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  Resolved r;
  msa_status_t st = resolve_attention(args, &r, true);
  if (st) return st;
  return run_attention(args, r, workspace, workspace_bytes, stream);
}

msa_status_t msa_sparse_attention_noalloc(const msa_attn_args_t* args, void* stream) {
  Resolved r;
  msa_status_t st = resolve_attention(args, &r, true);
  if (st) return st;
  if (r.ws_bytes > kScratchBytes)
    return fail(MSA_ERR_WORKSPACE,
                "these arguments need %zu bytes of workspace; the allocation-free entry point "
                "holds %zu (use msa_sparse_attention with a caller workspace)",
                r.ws_bytes, kScratchBytes);
  void* ws = nullptr;
  if (r.ws_bytes && (st = scratch_address(&ws))) return st;
  return run_attention(args, r, ws, r.ws_bytes ? kScratchBytes : 0, stream);
}

}  // extern "C"

namespace {

// Checks and launch parameters of a proxy call (the arguments of
// msa_proxy_score; out is required only when need_out).  *empty: nothing to
// compute.  *wide_out: the prefill-shaped kernel (> 64 rows per request and
// KV head) rather than the decode-shaped one.
msa_status_t resolve_proxy(const msa_proxy_args_t* a, bool need_out, msa::ProxyParams* pp,
                           int* wide_out, bool* empty) {
  if (!a) return fail(MSA_ERR_NULL, "args is NULL");

  if (a->head_dim != 128) return fail(MSA_ERR_SHAPE, "head_dim must be 128 (got %d)", a->head_dim);
  if (a->batch < 0 || a->total_q < 0 || a->max_k_tiles < 0 || a->max_seqlen_q < 0)
    return fail(MSA_ERR_SHAPE, "sizes must be >= 0");
  if (a->num_qo_heads <= 0 || a->num_kv_heads <= 0 || a->num_qo_heads % a->num_kv_heads)
    return fail(MSA_ERR_SHAPE, "num_qo_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                a->num_qo_heads, a->num_kv_heads);
  if (a->kv_dtype != MSA_KV_BF16 && a->kv_dtype != MSA_KV_FP8_E4M3 && a->kv_dtype != MSA_KV_F16)
    return fail(MSA_ERR_DTYPE, "proxy K must be bf16, fp16 or fp8 E4M3 (got kv_dtype %d)",
                a->kv_dtype);
  const bool paged = a->page_table != nullptr;
  if (paged) {
    if (!a->seqused_k) return fail(MSA_ERR_NULL, "paged K needs page_table and seqused_k together");
    if (a->cu_seqlens_k)
      return fail(MSA_ERR_CONFLICT, "paged K takes seqused_k; cu_seqlens_k must be NULL");
    if (a->page_table_width <= 0)
      return fail(MSA_ERR_SHAPE, "page_table_width must be > 0 (got %d)", a->page_table_width);
  } else if (!a->cu_seqlens_k) {
    return fail(MSA_ERR_NULL, "flat K needs cu_seqlens_k");
  } else if (a->seqused_k) {
    return fail(MSA_ERR_UNSUPPORTED, "seqused_k is read only with a page_table");
  }
  *empty = a->total_q == 0 || a->batch == 0 || a->max_k_tiles == 0;
  if (*empty) return ok();
  if (!a->q || !a->k || !a->cu_seqlens_q || (need_out && !a->out))
    return fail(MSA_ERR_NULL, "q, k, cu_seqlens_q%s must be non-NULL", need_out ? " and out" : "");
  if (!aligned(a->q, 16) || !aligned(a->k, 16))
    return fail(MSA_ERR_UNSUPPORTED, "q and k must be 16-byte aligned");
  msa::ProxyParams& p = *pp;
  std::memset(&p, 0, sizeof(p));
  msa_status_t st;
  const int rb = kv_row_bytes(a->kv_dtype);
  if ((st = resolve_strides("k", a->k_strides, paged, a->num_kv_heads, rb, 16, &p.k_st))) return st;
  const int G = a->num_qo_heads / a->num_kv_heads;
  p.q = static_cast<const uint16_t*>(a->q);
  p.k = static_cast<const uint8_t*>(a->k);
  p.cu_q = a->cu_seqlens_q;
  p.cu_k = a->cu_seqlens_k;
  p.page_table = a->page_table;
  p.seqused_k = a->seqused_k;
  p.pt_width = a->page_table_width;
  p.paged = paged;
  p.out = a->out;
  p.batch = a->batch;
  p.total_q = a->total_q;
  p.hq = a->num_qo_heads;
  p.hkv = a->num_kv_heads;
  p.group = G;
  p.causal = a->causal ? 1 : 0;
  if (a->reduce_heads < 0 || a->reduce_heads > 2)
    return fail(MSA_ERR_UNSUPPORTED, "reduce_heads must be 0, 1 (all heads) or 2 (per KV head group), got %d",
                a->reduce_heads);
  p.reduce = a->reduce_heads;
  p.max_k_tiles = a->max_k_tiles;
  if ((st = resolve_qpos(a->q_offset_mode, a->q_offset_value, a->q_offset, true, &p.qpos)))
    return st;
  const int lqmax = std::max(1, a->max_seqlen_q);
  const int rows = lqmax * G;
  const int wide = rows > 64;
  *wide_out = wide;
  p.rows_per_tile = wide ? 256 : (rows <= 32 ? 32 : 64);
  p.row_tiles = (rows + p.rows_per_tile - 1) / p.rows_per_tile;
  const int base = std::max(1, a->batch * a->num_kv_heads * p.row_tiles);
  if (wide) {
    // pieces per row-tile pair: about two workgroups per CU in all, each
    // piece at most kWideMaxSeg blocks of a row tile (a pair's blocks plus
    // the tile-switch charge, cut into equal pieces)
    const int pairs = std::max(1, a->batch * a->num_kv_heads * ((p.row_tiles + 1) / 2));
    p.pieces = std::max((512 + pairs - 1) / pairs,
                        (2 * a->max_k_tiles + msa::kSegSwitch + msa::kWideMaxSeg - 1) /
                            msa::kWideMaxSeg);
    p.pieces = std::max(1, p.pieces);
    p.blocks_per_wg = 0;
    p.block_chunks = 0;
    return MSA_OK;
  }
  // aim for ~3072 workgroups (24-block chunks measured 3.5 % faster than 32
  // on the MTP decode proxy and 16 slower), a multiple of 4 blocks each (the
  // 4 waves take every 4th block)
  const int chunks = std::max(1, (3072 + base - 1) / base);
  int bpw = std::max(4, (a->max_k_tiles + chunks - 1) / chunks);
  bpw = std::min(32, (bpw + 3) / 4 * 4);
  p.blocks_per_wg = bpw;
  p.block_chunks = (a->max_k_tiles + bpw - 1) / bpw;
  p.pieces = 0;
  return MSA_OK;
}

int proxy_fmt(int kv_dtype) {
  return kv_dtype == MSA_KV_FP8_E4M3 ? msa::kFmtFp8
       : kv_dtype == MSA_KV_F16      ? msa::kFmtF16
                                     : msa::kFmtBf16;
}

// Workspace of msa_proxy_topk: fused (decode shapes): [sel_rows, total_q, Hg,
// chunks, topk] candidate scores then ids; else the score buffer
// [H_s, max_k_tiles, total_q] fp32.
size_t proxy_topk_bytes(const msa_proxy_args_t* a, const msa::ProxyParams& p, int wide,
                        int topk) {
  if (!wide) {
    const int sel_rows = a->reduce_heads == 1 ? 1 : a->num_kv_heads;
    const int hg = a->reduce_heads == 1 ? a->num_kv_heads : 1;
    const size_t n = (size_t)sel_rows * a->total_q * hg * p.block_chunks * topk;
    return round_up(n * 4, 256) * 2;
  }
  const int hs = a->reduce_heads == 1 ? 1 : (a->reduce_heads == 2 ? a->num_kv_heads
                                                                    : a->num_qo_heads);
  return round_up((size_t)hs * a->max_k_tiles * a->total_q * 4, 256);
}

}  // namespace

extern "C" {

msa_status_t msa_proxy_score(const msa_proxy_args_t* a, void* stream) {
  msa::ProxyParams p;
  int wide = 0;
  bool empty = false;
  msa_status_t st = resolve_proxy(a, true, &p, &wide, &empty);
  if (st || empty) return st;
  return hip_status(msa::launch_proxy(p, proxy_fmt(a->kv_dtype), wide,
                                      static_cast<hipStream_t>(stream)),
                    "msa_proxy_score launch");
}

msa_status_t msa_proxy_topk_workspace_size(const msa_proxy_args_t* a, int32_t topk,
                                           size_t* bytes) {
  if (!bytes) return fail(MSA_ERR_NULL, "bytes is NULL");
  if (topk < 1 || topk > msa::kMaxTopk)
    return fail(MSA_ERR_SHAPE, "topk must be in [1, %d] (got %d)", msa::kMaxTopk, topk);
  msa::ProxyParams p;
  int wide = 0;
  bool empty = false;
  msa_status_t st = resolve_proxy(a, false, &p, &wide, &empty);
  if (st) return st;
  *bytes = empty ? 0 : proxy_topk_bytes(a, p, wide, topk);
  return ok();
}

msa_status_t msa_proxy_topk(const msa_proxy_args_t* a, int32_t topk, int32_t* q2k,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (topk < 1 || topk > msa::kMaxTopk)
    return fail(MSA_ERR_SHAPE, "topk must be in [1, %d] (got %d)", msa::kMaxTopk, topk);
  msa::ProxyParams p;
  int wide = 0;
  bool empty = false;
  msa_status_t st = resolve_proxy(a, false, &p, &wide, &empty);
  if (st) return st;
  if (a->total_q == 0 || a->batch == 0) return ok();
  if (!q2k) return fail(MSA_ERR_NULL, "q2k must be non-NULL");
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (empty) {   // no blocks: every row is padding
    return hip_status(msa::launch_topk(nullptr, 1, 0, a->total_q, topk, a->num_kv_heads, 1, q2k,
                                       hs),
                      "msa_proxy_topk launch");
  }
  const size_t need = proxy_topk_bytes(a, p, wide, topk);
  if (!workspace || workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu at %p)", need,
                workspace_bytes, workspace);
  if (!aligned(workspace, 256)) return fail(MSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const int fmt = proxy_fmt(a->kv_dtype);
  if (!wide) {
    // running top-K in the proxy kernel, then the merge of the candidates
    const int sel_rows = a->reduce_heads == 1 ? 1 : a->num_kv_heads;
    const int hg = a->reduce_heads == 1 ? a->num_kv_heads : 1;
    const size_t n = (size_t)sel_rows * a->total_q * hg * p.block_chunks * topk;
    p.cand_s = static_cast<float*>(workspace);
    p.cand_id = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + round_up(n * 4, 256));
    p.topk = topk;
    p.reduce = a->reduce_heads == 1 ? 1 : 2;
    if ((st = hip_status(msa::launch_proxy_candidates(p, fmt, hs), "msa_proxy_topk launch")))
      return st;
    return hip_status(msa::launch_topk_merge(p.cand_s, p.cand_id, hg * p.block_chunks * topk,
                                             a->max_k_tiles, a->total_q, topk, a->num_kv_heads,
                                             a->reduce_heads == 1, q2k, hs),
                      "msa_proxy_topk merge launch");
  }
  // prefill shapes: scores into the workspace, then the select
  p.out = static_cast<float*>(workspace);
  if ((st = hip_status(msa::launch_proxy(p, fmt, wide, hs), "msa_proxy_topk launch"))) return st;
  const int sh = a->reduce_heads == 1 ? 1 : (a->reduce_heads == 2 ? a->num_kv_heads
                                                                   : a->num_qo_heads);
  const int mode = a->reduce_heads == 1 ? 1 : (sh == a->num_kv_heads ? 0 : 2);
  return hip_status(msa::launch_topk(p.out, sh, a->max_k_tiles, a->total_q, topk,
                                     a->num_kv_heads, mode, q2k, hs),
                    "msa_proxy_topk select launch");
}

msa_status_t msa_topk_select(const float* scores, int32_t score_heads, int32_t max_k_tiles,
                             int32_t total_q, int32_t topk, int32_t num_kv_heads, int32_t mode,
                             int32_t* q2k, void* stream) {
  if (topk < 1 || topk > msa::kMaxTopk)
    return fail(MSA_ERR_SHAPE, "topk must be in [1, %d] (got %d)", msa::kMaxTopk, topk);
  if (score_heads <= 0 || num_kv_heads <= 0 || total_q < 0 || max_k_tiles < 0)
    return fail(MSA_ERR_SHAPE, "bad sizes (score_heads %d, num_kv_heads %d, total_q %d, T %d)",
                score_heads, num_kv_heads, total_q, max_k_tiles);
  if (max_k_tiles > 16384)
    return fail(MSA_ERR_UNSUPPORTED, "top-K select reads at most 16384 blocks per row (got %d)",
                max_k_tiles);
  if (mode == MSA_REDUCE_NONE && score_heads != num_kv_heads)
    return fail(MSA_ERR_SHAPE, "mode NONE needs score_heads == num_kv_heads (%d vs %d)",
                score_heads, num_kv_heads);
  if (mode == MSA_REDUCE_GROUP && score_heads % num_kv_heads)
    return fail(MSA_ERR_SHAPE, "mode GROUP needs score_heads %% num_kv_heads == 0");
  if (mode < MSA_REDUCE_NONE || mode > MSA_REDUCE_GROUP)
    return fail(MSA_ERR_UNSUPPORTED, "unknown reduce mode %d", mode);
  if (total_q == 0) return ok();
  if (!scores || !q2k) return fail(MSA_ERR_NULL, "scores and q2k must be non-NULL");
  return hip_status(msa::launch_topk(scores, score_heads, max_k_tiles, total_q, topk, num_kv_heads,
                                     mode, q2k, static_cast<hipStream_t>(stream)),
                    "msa_topk_select launch");
}

msa_status_t msa_tile_union(const int32_t* q2k, const int32_t* cu_seqlens_q,
                            const int32_t* lengths_k, int32_t batch, int32_t total_q,
                            int32_t num_kv_heads, int32_t topk, int32_t max_seqlen_q,
                            int32_t max_k_tiles, int32_t tile_tokens, int32_t max_union,
                            int32_t* union_blocks, uint64_t* union_masks, int32_t* union_count,
                            void* stream) {
  if (tile_tokens < 1 || tile_tokens > 64)
    return fail(MSA_ERR_SHAPE, "tile_tokens must be in [1, 64] (got %d)", tile_tokens);
  if (topk < 1 || topk > msa::kMaxTopk) return fail(MSA_ERR_SHAPE, "topk must be in [1, 64]");
  if (max_k_tiles < 0 || max_k_tiles > msa::kMaxBitmapWords * 32)
    return fail(MSA_ERR_SHAPE, "max_k_tiles must be in [0, %d]", msa::kMaxBitmapWords * 32);
  if (tile_tokens * topk > msa::kMaxUnion)
    return fail(MSA_ERR_SHAPE, "tile_tokens x topk must be <= %d", msa::kMaxUnion);
  if (max_union < std::min(tile_tokens * topk, max_k_tiles) || max_union > 1024)
    return fail(MSA_ERR_SHAPE, "max_union (%d) must be >= min(tile_tokens*topk, max_k_tiles) and <= 1024",
                max_union);
  if (batch < 0 || total_q < 0 || num_kv_heads <= 0 || max_seqlen_q < 0)
    return fail(MSA_ERR_SHAPE, "bad sizes");
  if (batch == 0 || max_seqlen_q == 0) return ok();
  if (!q2k || !cu_seqlens_q || !lengths_k || !union_blocks || !union_masks || !union_count)
    return fail(MSA_ERR_NULL, "all pointers must be non-NULL");
  return hip_status(msa::launch_tile_union(q2k, cu_seqlens_q, lengths_k, batch, total_q,
                                           num_kv_heads, topk, max_seqlen_q, max_k_tiles,
                                           tile_tokens, max_union, union_blocks, union_masks,
                                           union_count, static_cast<hipStream_t>(stream)),
                    "msa_tile_union launch");
}

static msa_status_t qsa_forward(const msa_qsa_args_t* a, bool bitmap, void* stream) {
  const char* name = bitmap ? "msa_qsa_bitmap_forward" : "msa_qsa_indexed_forward";
  if (!a) return fail(MSA_ERR_NULL, "%s: args is NULL", name);
  if (a->head_dim != 256) return fail(MSA_ERR_UNSUPPORTED, "QSA needs head_dim 256 (got %d)", a->head_dim);
  if (a->total_q < 0 || a->num_kv_heads <= 0 || a->num_qo_heads <= 0 ||
      a->num_qo_heads % a->num_kv_heads)
    return fail(MSA_ERR_SHAPE, "num_qo_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                a->num_qo_heads, a->num_kv_heads);
  if (a->num_qo_heads / a->num_kv_heads > 16)
    return fail(MSA_ERR_UNSUPPORTED, "at most 16 query heads per KV head (got %d)",
                a->num_qo_heads / a->num_kv_heads);
  if (!bitmap && (a->width < 4 || a->width % 4 || a->width > 2052))
    return fail(MSA_ERR_SHAPE, "width must be a multiple of 4 in [4, 2052] (got %d)", a->width);
  if (bitmap && (a->num_kv_tokens < 0 || a->num_kv_tokens > INT32_MAX - 4))
    return fail(MSA_ERR_SHAPE, "num_kv_tokens out of range (got %d)", a->num_kv_tokens);
  if (a->total_q == 0) return ok();
  // a bitmap over no KV tokens selects nothing: k, v and bitmap are never read
  const bool no_kv = bitmap && a->num_kv_tokens == 0;
  if (!a->q || !a->out || (!no_kv && (!a->k || !a->v || (bitmap ? !a->bitmap : !a->indices))))
    return fail(MSA_ERR_NULL, "q, k, v, %s and out must be non-NULL", bitmap ? "bitmap" : "indices");
  const int64_t row = 256 * 2;
  const int64_t kt = a->k_strides.token ? a->k_strides.token : row * a->num_kv_heads;
  const int64_t kh = a->k_strides.head ? a->k_strides.head : row;
  const int64_t vt = a->v_strides.token ? a->v_strides.token : row * a->num_kv_heads;
  const int64_t vh = a->v_strides.head ? a->v_strides.head : row;
  if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->out, 16) ||
      !aligned(a->out_f32, 16) || kt % 16 || kh % 16 || vt % 16 || vh % 16)
    return fail(MSA_ERR_UNSUPPORTED, "q, k, v, out, out_f32 and the k/v strides must be 16-byte aligned");
  msa::QsaParams p;
  p.q = static_cast<const uint16_t*>(a->q);
  p.k = static_cast<const uint16_t*>(a->k);
  p.v = static_cast<const uint16_t*>(a->v);
  p.k_row_stride = kt;
  p.k_head_stride = kh;
  p.v_row_stride = vt;
  p.v_head_stride = vh;
  p.indices = bitmap ? nullptr : a->indices;
  p.bitmap = bitmap ? a->bitmap : nullptr;
  p.num_kv_tokens = bitmap ? a->num_kv_tokens : 0;
  p.num_blocks = bitmap ? (a->num_kv_tokens + 3) / 4 : 0;
  p.out = static_cast<uint16_t*>(a->out);
  p.out_f32 = a->out_f32;
  p.lse = a->lse;
  p.total_q = a->total_q;
  p.hq = a->num_qo_heads;
  p.hkv = a->num_kv_heads;
  p.group = a->num_qo_heads / a->num_kv_heads;
  p.width = bitmap ? 0 : a->width;
  const float scale = a->softmax_scale > 0.f ? a->softmax_scale : 1.0f / 16.0f;
  p.scale_log2 = scale * 1.4426950408889634f;
  char what[64];
  snprintf(what, sizeof what, "%s launch", name);
  return hip_status(msa::launch_qsa(p, static_cast<hipStream_t>(stream)), what);
}

msa_status_t msa_qsa_indexed_forward(const msa_qsa_args_t* a, void* stream) {
  return qsa_forward(a, false, stream);
}

msa_status_t msa_qsa_bitmap_forward(const msa_qsa_args_t* a, void* stream) {
  return qsa_forward(a, true, stream);
}

}  // extern "C"
