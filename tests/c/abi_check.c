/* A C11 client of the library's C ABI, with no C++ or HIP on its side:
 * compiles against include/msa.h, links libmsa.so, takes the address of
 * every declared entry point (so that the linker must resolve each of them)
 * and exercises the host-side checks that run before any GPU work: the
 * workspace size of a valid and an invalid problem, argument errors with
 * their message, the status strings and the version string. Prints "ok" on
 * success; otherwise names the failed check and exits with status 1. */
#include <stdio.h>
#include <string.h>

#include "msa.h"

#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);        \
      return 1;                                                           \
    }                                                                     \
  } while (0)

typedef void (*entry_t)(void);

int main(void) {
  const entry_t entries[] = {
      (entry_t)msa_workspace_size,        (entry_t)msa_indexer_scores,
      (entry_t)msa_pool_select_blocks,    (entry_t)msa_sparse_attn_decode,
      (entry_t)msa_decode_layer,          (entry_t)msa_decode_layer_traced,
      (entry_t)msa_decode_layer_single,   (entry_t)msa_decode_layer_gave_up,
      (entry_t)msa_decode_layer_single_static, (entry_t)msa_decode_layer_single_traced,
      (entry_t)msa_kv_insert,             (entry_t)msa_debug_dequant_nvfp4,
      (entry_t)msa_debug_dequant_fp8,     (entry_t)msa_debug_read_bandwidth,
      (entry_t)msa_debug_layer_spin_limit, (entry_t)msa_debug_layer_splits,
      (entry_t)msa_status_string,         (entry_t)msa_last_error,
      (entry_t)msa_version};
  size_t i;
  for (i = 0; i < sizeof(entries) / sizeof(entries[0]); i++) CHECK(entries[i] != NULL);

  /* one sequence of 4,096 tokens, 8/1 heads, 4 indexer heads, bf16 caches */
  msa_params_t p;
  memset(&p, 0, sizeof(p));
  p.num_seqs = 1;
  p.q_len = 1;
  p.num_q_heads = 8;
  p.num_kv_heads = 1;
  p.head_dim = 128;
  p.idx_heads = 4;
  p.idx_dim = 64;
  p.block_size = 128;
  p.top_k = 16;
  p.keep_last = 1;
  p.max_blocks_per_seq = 32;
  p.num_pages = 32;
  p.softmax_scale = 0.0f;
  p.kv_dtype = MSA_KV_BF16;
  p.idx_dtype = MSA_IDX_BF16;

  const size_t ws = msa_workspace_size(&p);
  CHECK(ws > 0 && ws % 256 == 0);

  /* a missing cache is refused before anything is enqueued, with a message */
  CHECK(msa_decode_layer(&p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == MSA_ERR_INVALID_ARG);
  CHECK(msa_last_error() != NULL && strlen(msa_last_error()) > 0);
  CHECK(msa_decode_layer_single(&p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) != MSA_OK);

  /* head_dim must be 128: no workspace size, and the layer refuses it */
  p.head_dim = 64;
  CHECK(msa_workspace_size(&p) == 0);
  p.head_dim = 128;

  /* debug switches reject values outside their range */
  CHECK(msa_debug_layer_splits(3) == MSA_ERR_INVALID_ARG);
  CHECK(msa_debug_layer_splits(0) == MSA_OK);

  {
    int s;
    for (s = MSA_OK; s <= MSA_ERR_HIP; s++) {
      const char* str = msa_status_string((msa_status_t)s);
      CHECK(str != NULL && strlen(str) > 0);
    }
    CHECK(strcmp(msa_status_string(MSA_OK), msa_status_string(MSA_ERR_INVALID_ARG)) != 0);
  }
  CHECK(msa_version() != NULL && strlen(msa_version()) > 0);
  printf("ok %s\n", msa_version());
  return 0;
}
