/* Host-side fuzz of the C ABI: every size query and host rule with extreme,
 * negative and random arguments, and every device entry point with null
 * pointers or zero rows, which must be rejected (or be a no-op) on the host
 * without touching a device.  Meant to run under AddressSanitizer and
 * UndefinedBehaviorSanitizer (host code only); it checks return codes, not
 * values. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dsa_indexer.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void) {               /* splitmix64 */
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static const int64_t kEdges[] = {0,
                                 1,
                                 -1,
                                 2,
                                 63,
                                 64,
                                 65,
                                 255,
                                 256,
                                 257,
                                 2048,
                                 65536,
                                 65537,
                                 (int64_t)1 << 30,
                                 ((int64_t)1 << 31) - 1,
                                 (int64_t)1 << 31,
                                 (int64_t)1 << 40,
                                 INT64_MAX,
                                 INT64_MIN};

static int64_t pick64(void) {
  const uint64_t r = next_u64();
  const size_t n = sizeof(kEdges) / sizeof(kEdges[0]);
  if (r % 3 == 0) return (int64_t)(next_u64() >> (next_u64() % 64));
  if (r % 3 == 1) return -(int64_t)(next_u64() >> (1 + next_u64() % 63));
  return kEdges[(r >> 8) % n];
}

static int pick32(void) {
  const int64_t v = pick64();
  return (int)(v > INT32_MAX ? INT32_MAX : v < INT32_MIN ? INT32_MIN : v);
}

#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "failed at line %d (iteration %d): %s\n", __LINE__, \
              it, #cond);                                                  \
      return 1;                                                            \
    }                                                                      \
  } while (0)

int main(void) {
  static uint8_t skip[4096];
  static char pattern[300];
  int it;
  for (it = 0; it < 20000; ++it) {
    const int64_t T = pick64(), ld = pick64(), rpc = pick64();
    const int H = pick32(), k = pick32(), R = pick32();
    size_t s;
    int64_t rows;
    /* size queries: any arguments, no crash */
    s = dsa_topk_workspace_size(T, ld, k);
    s += dsa_forward_workspace_size(T, H, ld, k);
    s += dsa_forward_chunked_workspace_size(T, R, H, ld, k, rpc);
    s += dsa_run_workspace_size(T, R, H, ld, k, rpc);
    (void)s;
    if (T <= 0 || T > ((int64_t)1 << 31) || ld <= 0 || ld > ((int64_t)1 << 30))
      EXPECT(dsa_topk_workspace_size(T, ld, k) == 0 &&
             dsa_forward_workspace_size(T, H, ld, k) == 0 &&
             dsa_run_workspace_size(T, R, H, ld, k, rpc) == 0);
    /* logits budget and chunk rule */
    {
      const double frac = (double)(int64_t)(next_u64() % 3000) / 1000.0 - 1.0;
      const double odd[] = {NAN, 1e300, -1e300, -0.0};
      const size_t budget = dsa_logits_budget_bytes(
          (size_t)next_u64() >> (next_u64() % 64), frac, frac + 0.5);
      EXPECT(budget >= 1);
      EXPECT(dsa_logits_budget_bytes((size_t)pick64(), odd[it & 3],
                                     odd[(it >> 2) & 3]) >= 1);
      rows = dsa_logits_chunk_rows(T, ld, budget);
      EXPECT((T <= 0 || ld <= 0) ? rows == 0 : (rows >= 1 && rows <= T));
    }
    /* layer mask: random patterns (sometimes with a bad character) */
    {
      const int n = (int)(next_u64() % 290);
      const int num_layers = (int)(next_u64() % 4096);
      int i;
      for (i = 0; i < n; ++i) pattern[i] = (next_u64() & 1) ? 'F' : 'S';
      if (n > 0 && next_u64() % 5 == 0) pattern[next_u64() % n] = 'x';
      pattern[n] = '\0';
      (void)dsa_index_cache_mask((next_u64() & 1) ? pattern : NULL, pick32(),
                                 pick32(), pick32(), num_layers, pick32(),
                                 pick32(), pick32() & 1, skip);
      EXPECT(dsa_index_cache_mask(NULL, 1, 2, 0, 5, -1, 0, 0, NULL) ==
             DSA_ERR_INVALID_ARG);
    }
    /* device entry points: null pointers with rows are rejected */
    if (T > 0) {
      EXPECT(dsa_quantize_q(NULL, T, 64, 128, NULL, NULL, NULL) < 0);
      EXPECT(dsa_indexer_logits(NULL, NULL, NULL, NULL, 16, NULL, 4, NULL,
                                NULL, T, 1, 64, 128, 64, NULL, 256,
                                NULL) < 0);
      EXPECT(dsa_indexer_topk(NULL, 256, NULL, T, 8, NULL, 8, NULL, 0,
                              NULL) < 0);
      EXPECT(dsa_indexer_forward(NULL, NULL, NULL, 16, NULL, 4, NULL, NULL,
                                 T, 1, 64, 128, 64, NULL, 256, 8, NULL, 8,
                                 NULL, 0, NULL) < 0);
      EXPECT(dsa_indexer_forward_chunked(NULL, NULL, NULL, 16, NULL, 4, NULL,
                                         NULL, T, 1, 64, 128, 64, 256, 8,
                                         NULL, 8, rpc, NULL, 0, NULL) < 0);
      EXPECT(dsa_slot_mapping(NULL, 4, NULL, 1, NULL, T, NULL, NULL) < 0);
      EXPECT(dsa_compressed_slot_mapping(NULL, 4, NULL, 1, NULL, T, 4, 16,
                                         NULL, NULL, NULL) < 0);
      EXPECT(dsa_indexer_k_write(NULL, T, 128, NULL, NULL, 16, NULL) < 0);
      EXPECT(dsa_topk_to_slots(NULL, T, 8, 8, NULL, 4, NULL, 1, NULL,
                               NULL) < 0);
      EXPECT(dsa_topk_mask(NULL, T, 8, 8, NULL, 256, NULL) < 0);
      EXPECT(dsa_index_cache_run(NULL, 1, 2, 0, 3, -1, 0, 0, NULL, NULL, 4,
                                 NULL, NULL, T, 1, 64, 256, 8, 0, NULL, T,
                                 NULL, NULL, NULL, NULL, NULL, 0, NULL) < 0);
    }
    /* random shape arguments with null pointers: rejected or a no-op,
     * never a device call (T == 0 is a no-op) */
    {
      const int64_t t0 = (next_u64() & 1) ? 0 : T;
      const int r1 = dsa_indexer_logits(NULL, NULL, NULL, NULL, pick64(),
                                        NULL, pick64(), NULL, NULL, t0, R, H,
                                        pick32(), pick32(), NULL, ld, NULL);
      const int r2 = dsa_indexer_topk(NULL, ld, NULL, t0, k, NULL, pick64(),
                                      NULL, (size_t)pick64(), NULL);
      const int r3 = dsa_topk_mask(NULL, t0, k, pick64(), NULL, ld, NULL);
      EXPECT(r1 <= 0 && r2 <= 0 && r3 <= 0);
      EXPECT(t0 != 0 || r1 != DSA_ERR_HIP);
    }
    /* options: unknown keys are errors, known ones round-trip */
    EXPECT(dsa_set_option("no_such_option", 1) == DSA_ERR_INVALID_ARG);
    EXPECT(dsa_set_option(NULL, 1) == DSA_ERR_INVALID_ARG);
    EXPECT(dsa_set_option("topk_kernel", -3) == DSA_ERR_INVALID_ARG);
  }
  {
    const char* keys[] = {"logits_kernel", "row_pages_per_wave",
                          "row_head_waves", "tile_pages_per_split",
                          "topk_kernel"};
    size_t i;
    it = -1;
    for (i = 0; i < sizeof(keys) / sizeof(keys[0]); ++i) {
      EXPECT(dsa_set_option(keys[i], 3) >= 0);
      EXPECT(dsa_set_option(keys[i], 0) == 3);
    }
  }
  EXPECT(dsa_set_option("no_such_option", 1) == DSA_ERR_INVALID_ARG);
  EXPECT(strlen(dsa_last_error()) > 0);
  printf("host fuzz ok\n");
  return 0;
}
