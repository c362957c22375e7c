/* The C ABI used from plain C (C11; no C++, no Python): status strings, the
 * version, host-side rejection of bad arguments, and the launch plan of two
 * shapes.  Host-only calls: no device memory is read and nothing launches,
 * so it runs without a GPU.  Exit status 0 when every check holds. */
#include <stdio.h>
#include <string.h>

#include "msa.h"

static int failures = 0;

static void check(int ok, const char* what) {
  if (!ok) {
    printf("FAIL: %s (%s)\n", what, msa_last_error());
    ++failures;
  }
}

int main(void) {
  /* stand for 16-byte aligned device buffers: never read here */
  static _Alignas(16) const int32_t fake[4] = {0};
  static _Alignas(16) int32_t fake_out[4];
  msa_attn_args_t a;
  int32_t route = -1, splits = -1;
  size_t bytes = 0;

  check(strcmp(msa_status_string(MSA_OK), "MSA_OK") == 0, "status string");
  check(strcmp(msa_status_string(MSA_ERR_SHAPE), "MSA_ERR_SHAPE") == 0, "status string");

  /* paged bf16 decode: 64 requests, one query token, 64 q / 4 KV heads */
  memset(&a, 0, sizeof(a));
  a.batch = 64;
  a.total_q = 64;
  a.num_qo_heads = 64;
  a.num_kv_heads = 4;
  a.head_dim = 128;
  a.topk = 16;
  a.max_seqlen_q = 1;
  a.max_k_tiles = 512;
  a.page_table_width = 512;
  a.causal = 1;
  a.kv_dtype = MSA_KV_BF16;
  a.q = fake;
  a.k = fake;
  a.v = fake;
  a.q2k = fake;
  a.out = fake_out;
  a.cu_seqlens_q = fake;
  a.page_table = fake;
  a.seqused_k = fake;
  check(msa_sparse_attention_plan(&a, &route, &splits) == MSA_OK, "decode plan");
  check(route == 1 && splits >= 1, "decode route");
  check(msa_sparse_attention_workspace_size(&a, &bytes) == MSA_OK, "decode workspace size");

  /* a prefill of 2048 tokens takes the prefill tiles and no workspace */
  a.batch = 1;
  a.total_q = 2048;
  a.max_seqlen_q = 2048;
  a.max_k_tiles = 16;
  a.page_table_width = 16;
  check(msa_sparse_attention_plan(&a, &route, &splits) == MSA_OK, "prefill plan");
  check(route == 0, "prefill route");
  check(msa_sparse_attention_workspace_size(&a, &bytes) == MSA_OK && bytes == 0,
        "prefill workspace size");

  /* host checks reject a bad head_dim before any launch */
  a.head_dim = 64;
  check(msa_sparse_attention_plan(&a, &route, &splits) == MSA_ERR_SHAPE, "head_dim rejected");
  check(strstr(msa_last_error(), "head_dim") != NULL, "error detail names head_dim");

  if (failures == 0) printf("C ABI checks passed\n");
  return failures ? 1 : 0;
}
