/* Uses the library from plain C99 through include/dsa_indexer.h: host-only
 * entry points and argument errors (no device memory is touched). */
#include <stdio.h>
#include <string.h>

#include "dsa_indexer.h"

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

int main(void) {
  static const int expect_full[16] = {0,  1,  5,  9,  13, 17, 21, 25,
                                      29, 33, 37, 41, 45, 49, 53, 57};
  uint8_t skip[61];
  int full = 0, i;
  CHECK(dsa_version() >= 100);
  /* vLLM IndexCache practical guide, section 4 (method 1): 61 layers,
   * offset 2, freq 4 compute at layers 0, 1, 5, 9, ..., 57 */
  CHECK(dsa_index_cache_mask(NULL, 4, 2, 0, 61, -1, 0, 0, skip) == DSA_OK);
  for (i = 0; i < 61; ++i) {
    if (skip[i] == 0) {
      CHECK(full < 16 && expect_full[full] == i);
      ++full;
    }
  }
  CHECK(full == 16);
  /* MTP layer 61 at draft step 1 with the reuse switch: S */
  CHECK(dsa_index_cache_mask(NULL, 1, 2, 61, 1, 61, 1, 1, skip) == DSA_OK);
  CHECK(skip[0] == 1);
  /* a bad pattern character is an error with a message */
  CHECK(dsa_index_cache_mask("FX", 1, 2, 0, 2, -1, 0, 0, skip) ==
        DSA_ERR_INVALID_ARG);
  CHECK(strlen(dsa_last_error()) > 0);
  /* logits budget: 1M columns, 32K rows, 30 % of 288 GB */
  {
    const size_t budget = dsa_logits_budget_bytes(288000000000ull, -1.0, 1.0);
    const int64_t rows = dsa_logits_chunk_rows(32768, 1048576, budget);
    CHECK(budget == 86400000000ull);
    CHECK(rows == (int64_t)(budget / (1048576ull * 4)));
    CHECK(dsa_logits_chunk_rows(7, 1 << 20, 1) == 7);
  }
  /* argument errors are caught before any device work */
  CHECK(dsa_indexer_topk(NULL, 300, NULL, 4, 8, NULL, 8, NULL, 0, NULL) ==
        DSA_ERR_INVALID_ARG);                       /* ld % 256 != 0 */
  CHECK(dsa_quantize_q(NULL, 4, 4, 64, NULL, NULL, NULL) ==
        DSA_ERR_UNSUPPORTED);                       /* head_dim 64 */
  CHECK(dsa_forward_workspace_size(0, 64, 8192, 2048) == 0);
  printf("c abi ok\n");
  return 0;
}
