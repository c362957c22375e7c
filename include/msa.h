/*
 * msa.h — C ABI of the MI355X (gfx950) MiniMax Sparse Attention hot path.
 *
 * The operations follow the MSA documentation pages:
 *   msa_proxy_score       msa_proxy_score page (summary, Parameters, Returns)
 *   msa_topk_select       the top-K block select that feeds q2k_indices
 *                         (msa_proxy_score page, summary: "feeds directly into
 *                         msa_topk_select"; msa_sparse_attention page,
 *                         Parameters: q2k_indices)
 *   msa_sparse_attention  msa_sparse_attention page (summary, Parameters,
 *                         Returns); the paged decode route of
 *                         prepare_msa_nvfp4_sparse_decode page (Parameters)
 *   msa_tile_union        the per-tile union the attention builds internally
 *                         (msa_sparse_attention page, summary), exported so it
 *                         can be checked on its own
 *
 * Conventions for every entry point:
 *   - Every tensor pointer is a DEVICE pointer.  The argument structs and the
 *     integers in them are HOST memory, read during the call only.
 *   - All buffers are caller-owned.  The library never allocates or frees
 *     device memory and never synchronises with the host; it only enqueues
 *     kernels on `stream` (a hipStream_t; NULL = the null stream).
 *   - Host-side validation runs before any HIP call.  A non-OK return
 *     enqueues nothing; msa_last_error() then holds a message for the calling
 *     thread.  MSA_ERR_HIP means a launch was rejected by the runtime.
 *   - Device-side contents (sequence boundaries, indices, page ids) are
 *     caller contracts and are not copied to the host for checking on the
 *     timed path.  msa_validate_attention checks them on the device; with
 *     the environment variable MSA_VALIDATE=1, msa_sparse_attention runs that
 *     check first (and then synchronises the stream: a debug mode, not for
 *     graph capture).
 *   - head_dim is 128 and the KV block / page size is 128 tokens.
 *   - Strides are in BYTES; a stride of 0 selects the dense layout.  The last
 *     (head_dim) dimension must be contiguous and every row 16-byte aligned
 *     (8-byte for E4M3 block-scale rows), and the token stride at most
 *     16 MiB; other views are rejected with MSA_ERR_UNSUPPORTED, never copied.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_NULL = 1,        /* a required pointer is NULL                     */
  MSA_ERR_SHAPE = 2,       /* sizes inconsistent or outside the envelope     */
  MSA_ERR_DTYPE = 3,       /* unknown or unsupported storage format          */
  MSA_ERR_CONFLICT = 4,    /* both cu_seqlens_k and seqused_k on the paged route */
  MSA_ERR_UNSUPPORTED = 5, /* a view or option this library does not read   */
  MSA_ERR_WORKSPACE = 6,   /* workspace missing or too small                 */
  MSA_ERR_HIP = 7,         /* the HIP runtime rejected a launch              */
  MSA_ERR_CONTRACT = 8     /* a device-side caller contract is broken (found
                              only by msa_validate_attention / MSA_VALIDATE=1) */
} msa_status_t;

/* K/V storage formats (msa_sparse_attention page, Parameters: k). */
typedef enum {
  MSA_KV_BF16 = 0,      /* bf16 values                                        */
  MSA_KV_FP8_E4M3 = 1,  /* OCP float8 E4M3FN bytes, upconverted in-kernel     */
  MSA_KV_E2M1X2 = 2,    /* packed E2M1, two per byte (element 2i = low nibble),
                           with E4M3 block scales, one per 16 values          */
  MSA_KV_F16 = 3        /* fp16 values; q and out are fp16 too (the page's
                           "bf16/fp16" q, k and v)                            */
} msa_kv_dtype_t;

/* How score heads map to the per-KV-head selections of q2k_indices. */
typedef enum {
  MSA_REDUCE_NONE = 0,  /* one score head per KV head                         */
  MSA_REDUCE_ALL = 1,   /* max over every score head; the one shared selection
                           is written for every KV head (msa_proxy_score page,
                           Parameters: reduce_heads)                          */
  MSA_REDUCE_GROUP = 2  /* per-query-head scores; max over the G = Hq/Hkv heads
                           of each KV head (per-group analogue of reduce_heads) */
} msa_reduce_t;

/* Byte strides of a K/V (or block-scale) tensor.  Flat layout
 * (total_k, Hkv, d'): `token` and `head` are used, `page` is ignored.  Paged
 * layout (num_pages, Hkv, 128, d'): all three are used.  0 = dense. */
typedef struct {
  int64_t page;
  int64_t head;
  int64_t token;
} msa_strides_t;

/* ------------------------------------------------------------------------ */
/* Sparse attention                                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
  /* host integers */
  int32_t batch;          /* B                                                */
  int32_t total_q;        /* rows of q                                        */
  int32_t num_qo_heads;   /* Hq                                               */
  int32_t num_kv_heads;   /* Hkv; Hq % Hkv == 0 (query head h reads KV head
                             h / (Hq / Hkv))                                   */
  int32_t head_dim;       /* must be 128                                      */
  int32_t topk;           /* width of q2k_indices rows, 1..64                 */
  int32_t max_seqlen_q;   /* >= every per-request query length               */
  int32_t max_k_tiles;    /* >= every ceil(Lk / 128); paged: <= page_table_width */
  int32_t page_table_width; /* paged: columns of page_table                   */
  int32_t causal;         /* 1: right-aligned causal mask, query i of a request
                             sits at KV position Lk - Lq + i                  */
  float softmax_scale;    /* <= 0 selects head_dim^-0.5                       */
  float k_global_scale;   /* <= 0 selects 1; folds into the softmax scale     */
  float v_global_scale;   /* <= 0 selects 1; multiplies the output            */
  int32_t kv_dtype;       /* msa_kv_dtype_t                                   */
  int32_t splits;         /* 0: library choice; > 0 forces that many split-KV
                             partials per (request, KV head) on the decode
                             route; ignored on the prefill route              */
  /* device tensors */
  const void* q;          /* bf16 [total_q, Hq, 128], contiguous (fp16 when
                             kv_dtype is MSA_KV_F16)                          */
  const void* k;          /* flat [total_k, Hkv, d'] or paged [pages, Hkv, 128, d'];
                             d' = 128 (bf16, fp16, fp8) or 64 bytes (E2M1)    */
  const void* v;          /* same layout rules as k                           */
  const void* k_scale;    /* E2M1 only: E4M3 bytes, one per 16 values of a row,
                             16-byte aligned base.  Paged [pages, Hkv, 128, 8]:
                             a head's rows contiguous (8 bytes), page/head
                             strides multiples of 16.  Flat [total_k, Hkv, 8]
                             in (token, head) order or any view of 8-byte rows
                             (strides multiples of 8); flat E2M1 takes the
                             prefill route at every shape.  The E4M3 NaN
                             bytes (0x7F, 0xFF) are outside the caller
                             contract: outputs are NaN, the LSE unspecified   */
  const void* v_scale;    /* E2M1 only: same, stored linearly                 */
  msa_strides_t k_strides, v_strides, k_scale_strides, v_scale_strides;
  const int32_t* q2k;     /* [Hkv, total_q, topk] block ids, ascending, -1 padded */
  const int32_t* cu_seqlens_q; /* [B + 1]                                     */
  const int32_t* cu_seqlens_k; /* flat route: [B + 1]; must be NULL when paged */
  const int32_t* page_table;   /* paged route: [B, page_table_width]          */
  const int32_t* seqused_k;    /* paged route: [B] valid KV tokens per request */
  void* out;              /* bf16 [total_q, Hq, 128], written (fp16 with
                             MSA_KV_F16)                                      */
  float* lse;             /* NULL or fp32 [total_q, Hq], natural log, written;
                             -inf for a row with no attended key (out = 0)    */
  float* lse_t;           /* NULL or fp32 [total_q, Hq]: the temperature LSE
                             ln sum_j exp(lse_temperature_scale * z_j) over the
                             attended keys (z_j the logits of lse), -inf for an
                             empty row (msa_sparse_attention page, Parameters:
                             return_temperature_lse, lse_temperature_scale).
                             Accumulated by the same decode and prefill
                             kernels beside the row sum, every format        */
  float lse_temperature_scale; /* finite and > 0 when lse_t is set (1 gives
                             lse), else MSA_ERR_UNSUPPORTED                   */
  /* Causal positions of the queries (msa_sparse_attention page, Parameters:
     q_offset; the page calls it a per-query offset tensor and defines it no
     further).  Reading: q_offset_mode 0 (default): right-aligned, query iq
     of a request at KV position Lk - Lq + iq; 1: query iq of every request
     at q_offset_value + iq; 2: query row i at q_offset[i] (device int32
     [total_q]).  Key j is visible iff j <= that position (and j < Lk); a
     position below 0 leaves the row empty (out 0, lse -inf).  Read only
     with causal; other modes are MSA_ERR_UNSUPPORTED. */
  int32_t q_offset_mode;
  int32_t q_offset_value;
  const int32_t* q_offset;
} msa_attn_args_t;

/* Bytes of workspace msa_sparse_attention needs for these arguments: the
 * fp32 split-KV partials (O / l per row) and their LSE, and with lse_t their
 * temperature LSE (prepare_msa_nvfp4_sparse_decode page, Parameters:
 * workspace_buffer), or, for fp8 / E2M1 K/V on the prefill route, the bf16
 * pages their blocks are converted to: 2 * batch * S * Hkv * 32 KiB plus the
 * page table and lengths, with S = max_k_tiles (every visible block), or,
 * when max_seqlen_q * Hkv * topk <= 2048, S = min(that product,
 * max_k_tiles) (only the blocks some query of the request selected).  0 for
 * bf16 / fp16 K/V on the prefill route and for decode shapes whose plan uses
 * one split.  Every nonzero size includes 64 KiB at the end of the buffer
 * for the split-KV arrival counters: each split's workgroup counts its
 * arrival there, and the last of a (request, KV head, token tile) merges
 * the partials and resets its counter (the page's runner likewise resets its
 * completion counters after every merge).  So the buffer must be zero-filled
 * before its first use; the library keeps the last 64 KiB of any buffer it
 * is given at zero between launches and writes nothing else there.  At most
 * 16384 units can be split (MSA_ERR_SHAPE beyond).  The buffer is 256-byte
 * aligned and owned by the caller; apart from the counters every launch
 * writes what it reads later on the same stream.  Launches that may run
 * concurrently need separate workspaces. */
msa_status_t msa_sparse_attention_workspace_size(const msa_attn_args_t* args,
                                                 size_t* bytes);

/* The launch plan msa_sparse_attention would use for these arguments: the
 * route (1: the paged/flat decode kernel, 0: a prefill-tile kernel) and the
 * split-KV factor (1 when not split; prepare_msa_nvfp4_sparse_decode page:
 * the runner reports the chosen factor).  Host-side only; the same checks
 * and statuses as msa_sparse_attention_workspace_size. */
msa_status_t msa_sparse_attention_plan(const msa_attn_args_t* args, int32_t* decode_route,
                                       int32_t* splits);

/* Forward sparse attention (msa_sparse_attention page).  Each query token,
 * per KV head, attends only to the 128-token KV blocks listed in its q2k row;
 * query tiles run one online softmax over the union of their tokens' blocks
 * and write out (and lse) directly, or through split-KV partials merged by
 * LSE on the decode route.  q2k entries outside [0, ceil(Lk/128)) and -1 are
 * ignored; rows must be ascending without duplicates (caller contract).
 * Route: the decode kernel when max_seqlen_q * G <= 64 and the tile's
 * selections fit its union (max_seqlen_q * topk <= 512), or, with
 * G = Hq / Hkv in [16, 64], when max_seqlen_q <= 64 (one token per tile);
 * flat E2M1 always takes prefill tiles.  A prefill tile holds 256 query
 * rows: a larger G is MSA_ERR_SHAPE.  `workspace` may be NULL when the size query returned 0. */
msa_status_t msa_sparse_attention(const msa_attn_args_t* args, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* msa_sparse_attention for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc): the workspace is the library's own scratch array of 32 MiB per
 * GPU (a file-scope device array, held until the process ends), so the
 * caller passes only inputs and outputs.  Nothing is allocated or freed.
 * Arguments whose workspace size query exceeds 32 MiB return
 * MSA_ERR_WORKSPACE before any launch (msa_sparse_attention with a caller
 * workspace takes them).  Every call on one GPU shares that GPU's array:
 * calls that may overlap on one GPU (different streams or threads) race and
 * must be serialised by the caller.  The scratch needs no clearing: every
 * launch writes what it later reads.  Same statuses otherwise. */
msa_status_t msa_sparse_attention_noalloc(const msa_attn_args_t* args, void* stream);

/* Debug check of the device-side caller contracts of msa_sparse_attention
 * with these arguments (msa_sparse_attention page, Parameters: cu_seqlens_q,
 * cu_seqlens_k, q2k_indices, page_table, seqused_k): cu_seqlens_q starts at
 * 0, ends at total_q and gives lengths in [0, max_seqlen_q]; cu_seqlens_k
 * does not decrease; every KV length is in [0, 128 * max_k_tiles] (paged:
 * also <= 128 * page_table_width); page_table[b, t] >= 0 for
 * t < ceil(seqused_k[b] / 128); in every q2k row the non-negative block ids
 * ascend without repeats and -1 padding is trailing.  Page ids are not
 * bounded above (the pool size is not an argument).  Runs the host checks of
 * msa_sparse_attention, then one small kernel on `stream`, and waits for it
 * (synchronises the stream); concurrent checks in one process are
 * serialised (they share one result word per device).  Returns MSA_ERR_CONTRACT, with the first
 * violation (kind, then position) in msa_last_error(), or MSA_OK; never
 * launches the attention. */
msa_status_t msa_validate_attention(const msa_attn_args_t* args, void* stream);

/* ------------------------------------------------------------------------ */
/* Proxy score (stage 1)                                                     */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t batch, total_q, num_qo_heads, num_kv_heads, head_dim;
  int32_t max_seqlen_q;   /* >= every per-request query length               */
  int32_t max_k_tiles;    /* columns t of the output                          */
  int32_t page_table_width;
  int32_t causal;         /* right-aligned, applied before the block max      */
  int32_t kv_dtype;       /* K: MSA_KV_BF16 or MSA_KV_FP8_E4M3 (bf16 q), or
                             MSA_KV_F16 (fp16 q and K)                        */
  int32_t reduce_heads;   /* 0: per query head, output (Hq, T, total_q);
                             1: max over all query heads, output (1, T, total_q);
                             2: max over the G query heads of each KV head,
                                output (Hkv, T, total_q); else MSA_ERR_UNSUPPORTED */
  const void* q;          /* bf16 or fp16 [total_q, Hq, 128] (the proxy Q)    */
  const void* k;          /* flat [total_k, Hkv, 128] or paged [pages, Hkv, 128, 128] */
  msa_strides_t k_strides;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;   /* flat route                               */
  const int32_t* page_table;     /* paged route, with seqused_k              */
  const int32_t* seqused_k;
  float* out;             /* fp32 [Hq | 1 | Hkv, max_k_tiles, total_q], written in full */
  /* Causal positions of the queries (msa_proxy_score page, Parameters:
     q_offset, an int or a tensor used by the causal alignment), as in
     msa_attn_args_t: mode 0 right-aligned, 1 q_offset_value + iq, 2
     q_offset[i] per query row. */
  int32_t q_offset_mode;
  int32_t q_offset_value;
  const int32_t* q_offset;
} msa_proxy_args_t;

/* max_score[h, t, i]: the max over the keys of block t of the UNSCALED dot
 * products q[i, h] . k[j, h / G], after the causal mask; -inf where no key of
 * the block is visible or the block is past the sequence (msa_proxy_score
 * page, summary).  With reduce_heads the max over h (all heads, or the heads
 * of each KV head's group) is taken in-kernel, so the per-head scores are
 * never written (msa_proxy_score page, Parameters: reduce_heads).  q and k
 * hold finite values (NaN or infinite inputs leave the scores unspecified). */
msa_status_t msa_proxy_score(const msa_proxy_args_t* args, void* stream);

/* Proxy score, head reduction and top-K block select in one call, with the
 * selection kept running inside the proxy pass where the query is short
 * (msa_proxy_score page, Parameters: reduce_heads, on folding the reduction
 * into the kernel so that no score buffer is materialised).  Writes q2k int32
 * [num_kv_heads, total_q, topk] exactly as msa_proxy_score followed by
 * msa_topk_select would: reduce_heads 1 selects on the max over all query
 * heads and writes that shared selection to every KV head's row; 0 and 2
 * select per KV head on the max over its query heads.  args->out is not
 * read (may be NULL).  Decode shapes (max_seqlen_q * G <= 64): each proxy
 * workgroup writes, per query, the top-K (score, block id) of its own chunk
 * of blocks over its KV head's head-group maximum, and a merge kernel folds
 * every chunk's and KV head's candidates by block id (largest score) and
 * selects the top-K; no score buffer exists.  Other shapes: the scores go to
 * the workspace, then the select.  workspace: caller-owned, 256-byte
 * aligned, msa_proxy_topk_workspace_size bytes, no initialisation needed.
 * 1 <= topk <= 64; the other checks as msa_proxy_score. */
msa_status_t msa_proxy_topk_workspace_size(const msa_proxy_args_t* args, int32_t topk,
                                           size_t* bytes);
msa_status_t msa_proxy_topk(const msa_proxy_args_t* args, int32_t topk, int32_t* q2k,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Top-K block select                                                        */
/* ------------------------------------------------------------------------ */

/* scores: fp32 [score_heads, max_k_tiles, total_q].  Writes q2k int32
 * [num_kv_heads, total_q, topk]: per (KV head, query) the `topk` blocks with
 * the largest finite score (equal scores, with -0 == +0, go to the lower block
 * id), ascending, -1 padded.  -inf and NaN scores are never selected.
 * mode: MSA_REDUCE_NONE needs score_heads == num_kv_heads; MSA_REDUCE_ALL
 * takes the max over all score heads and writes the shared selection to every
 * KV head; MSA_REDUCE_GROUP needs score_heads % num_kv_heads == 0.
 * 1 <= topk <= 64 and max_k_tiles <= 16384, else MSA_ERR_SHAPE /
 * MSA_ERR_UNSUPPORTED with nothing launched. */
msa_status_t msa_topk_select(const float* scores, int32_t score_heads,
                             int32_t max_k_tiles, int32_t total_q, int32_t topk,
                             int32_t num_kv_heads, int32_t mode, int32_t* q2k,
                             void* stream);

/* ------------------------------------------------------------------------ */
/* Tile union (the attention kernel's own builder, exported for checking)    */
/* ------------------------------------------------------------------------ */

/* For every tile of `tile_tokens` consecutive query tokens of one request and
 * one KV head (tiles never cross requests; tile j of request b covers local
 * queries [j * tile_tokens, ...)), writes the ascending union of the valid
 * selected blocks (0 <= id < n_blocks_b, n_blocks_b = ceil(Lk_b / 128)) and,
 * per union entry, the bit mask of tile tokens that selected it.
 *   q2k          [Hkv, total_q, topk]
 *   cu_seqlens_q [B + 1]; lengths_k [B] KV tokens per request
 *   union_blocks int32  [Hkv, B, tiles_per_req, max_union], -1 padded
 *   union_masks  uint64 [Hkv, B, tiles_per_req, max_union], 0 padded
 *   union_count  int32  [Hkv, B, tiles_per_req]
 * tiles_per_req = ceil(max_seqlen_q / tile_tokens); tile_tokens in 1..64;
 * max_union >= min(tile_tokens * topk, max_k_tiles) and <= 1024. */
msa_status_t msa_tile_union(const int32_t* q2k, const int32_t* cu_seqlens_q,
                            const int32_t* lengths_k, int32_t batch,
                            int32_t total_q, int32_t num_kv_heads, int32_t topk,
                            int32_t max_seqlen_q, int32_t max_k_tiles,
                            int32_t tile_tokens, int32_t max_union,
                            int32_t* union_blocks, uint64_t* union_masks,
                            int32_t* union_count, void* stream);

/* ------------------------------------------------------------------------ */
/* QSA: packed query sparse attention over caller-selected tokens            */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t total_q;        /* T: packed query tokens                           */
  int32_t num_qo_heads;   /* Hq; Hq % Hkv == 0 and Hq / Hkv <= 16 (12/1, 24/2) */
  int32_t num_kv_heads;   /* Hkv                                               */
  int32_t head_dim;       /* 256 (the only head dimension the qsa page names) */
  int32_t width;          /* W: index entries per query, W % 4 == 0, W <= 2052 */
  float softmax_scale;    /* <= 0: head_dim^-0.5                               */
  const void* q;          /* bf16 [T, Hq, 256], contiguous                     */
  const void* k;          /* bf16 rows of 256 values: row t of head g at
                             k + t * k_strides.token + g * k_strides.head      */
  const void* v;          /* same layout as k (its own strides)                */
  msa_strides_t k_strides, v_strides;   /* bytes; token and head used; 0 =
                             dense [Tk, Hkv, 256]                              */
  const int32_t* indices; /* [T, W]: absolute packed token ids (rows of k/v) in
                             groups of four, -1 padding; query i attends the
                             set of its non-negative entries                   */
  void* out;              /* bf16 [T, Hq, 256]                                 */
  float* out_f32;         /* nullable: fp32 [T, Hq, 256], the output before
                             the bf16 cast                                     */
  float* lse;             /* nullable: fp32 [Hq, T], natural log               */
  /* bitmap entry point only (ignored by the indexed one):                    */
  const uint8_t* bitmap;  /* [T, ceil(Tk / 4)]: a non-zero byte b of row i
                             selects packed tokens 4 b .. 4 b + 3 (those < Tk)
                             for query i                                       */
  int32_t num_kv_tokens;  /* Tk: rows of k/v the bitmap covers                 */
} msa_qsa_args_t;

/* out[i, h] = softmax over the keys j listed in indices[i] of
 * (softmax_scale * q[i, h] . k[j, h / G]) applied to v[j, h / G]; lse the
 * natural-log normaliser; a query with no listed key gets zero output and
 * -inf LSE (qsa page: the indexed API, outputs and LSE, empty selections).
 * Causality is the caller's, carried by the indices.  Index values are a
 * caller contract (distinct, < Tk), not validated on the device; k and v
 * must hold at least one row (-1 padding entries may read row 0, with
 * weight 0).  Host-side checks return MSA_ERR_SHAPE / MSA_ERR_NULL /
 * MSA_ERR_UNSUPPORTED (head_dim != 256, Hq / Hkv > 16, misaligned pointers)
 * before any launch.
 * Work split: one workgroup per tile of min(16, 128 / G) consecutive query
 * tokens and KV head.  A tile whose listed keys fall in at most 64 windows
 * of 16384 keys and whose key union U is small against its L listed entries
 * (5 * U * ceil(S / 4) <= 8 * L, S = ceil(tokens * G / 16) row slots) reads
 * each union key once and computes its rows over the union in ascending
 * key order (window by window), masking the keys a row's token did not
 * list; any other tile
 * computes each token over its own keys in index order.  Results are
 * bitwise repeatable. */
msa_status_t msa_qsa_indexed_forward(const msa_qsa_args_t* args, void* stream);

/* The same attention with the key set of query i given by row i of a block
 * bitmap over the packed K/V (qsa page: the bitmap API over 4-token blocks):
 * keys are the tokens of the selected blocks, in ascending order, the last
 * block cut at Tk.  The selected blocks are compacted on the device (per
 * tile or per token, as for the indexed entry point, which gives bitwise
 * equal results on the equivalent ascending index rows), so nothing is
 * allocated and no index scratch is written; width and indices are
 * ignored, any number of blocks may be selected.
 * Host-side checks as for the indexed entry point, plus bitmap non-NULL
 * (when T > 0 and Tk > 0; with Tk == 0 nothing is selected and k, v and
 * bitmap may be NULL) and 0 <= Tk < 2^31 - 4 (MSA_ERR_SHAPE). */
msa_status_t msa_qsa_bitmap_forward(const msa_qsa_args_t* args, void* stream);

/* ------------------------------------------------------------------------ */
/* Diagnostics                                                               */
/* ------------------------------------------------------------------------ */

const char* msa_status_string(msa_status_t status);
/* Message for the last non-OK return on the calling thread ("" if none). */
const char* msa_last_error(void);
/* Library version, e.g. "0.1.0". */
const char* msa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
