// Device-side caller-contract check of the sparse attention arguments
// (debug path, never on the timed path).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

// Kinds in report order; the reported word is kind << 48 | position,
// all ones when every check passed.
enum ValidateKind {
  kValCuQ = 1,       // cu_seqlens_q: [0] != 0, [B] != total_q, a length < 0 or > max_seqlen_q (b)
  kValCuK = 2,       // cu_seqlens_k decreases (b)
  kValKvLen = 3,     // a KV length outside [0, 128 * max_k_tiles] (b)
  kValPage = 4,      // a negative page id among a request's pages (b * width + t)
  kValQ2kPad = 5,    // a block id after -1 padding (row * topk + entry)
  kValQ2kOrder = 6,  // a block id not above the previous one (row * topk + entry)
};

struct ValidateParams {
  int batch, total_q, hkv, topk, max_seqlen_q, max_k_tiles, pt_width;
  bool paged;
  const int32_t* q2k;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* page_table;
  const int32_t* seqused;
};

// Runs the check on `stream`, copies the report to *word and waits for it.
hipError_t run_validate(const ValidateParams& p, hipStream_t stream, unsigned long long* word);

}  // namespace msa
