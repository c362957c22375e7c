// fp8 E4M3 / packed E2M1 K/V on the prefill route: the blocks each request
// can see (or, for short queries, only the blocks they selected) are
// converted once to bf16 pages in the workspace (exactly: every E4M3 value,
// and every E2M1 value times its E4M3 block scale, is a bf16 value), then
// the bf16 prefill kernel reads them as a paged cache.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "internal.hpp"

namespace msa {

// Requests whose q2k rows hold at most this many entries (max_seqlen_q x
// hkv x topk) stage only the blocks their queries selected.
constexpr int kStageSelectMax = 2048;

// Pages per request in the pool when only selected blocks are staged
// (min(entries, max_k_tiles)); 0 when every visible block is staged.
int stage16_slots(int max_seqlen_q, int hkv, int topk, int max_k_tiles);

// Workspace bytes for B requests of at most max_k_tiles blocks and hkv KV
// heads: K and V pools of B * (slots or max_k_tiles) pages, the page table
// [B, max_k_tiles] and the lengths.
size_t stage16_bytes(int batch, int max_k_tiles, int hkv, int slots);

// Converts (p: the caller's fp8 / E2M1 arguments, fmt kFmtFp8 or kFmtE2m1)
// into `ws` (256-byte aligned, stage16_bytes long) and writes to *pq a copy
// of p that reads the bf16 pages.
hipError_t launch_stage16(const AttnParams& p, int fmt, int slots, void* ws, AttnParams* pq,
                          hipStream_t stream);

}  // namespace msa
