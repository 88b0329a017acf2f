/* Host-side entry points of the library exercised from C, for a build with
 * the host compiler's address and undefined-behaviour sanitizers (no GPU
 * needed: nothing here launches a kernel).  Exits non-zero on the first
 * failed check. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fastocr.h"

#define EXPECT(cond)                                                 \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                      \
    }                                                                \
  } while (0)

static uint32_t lcg = 7u;
static uint32_t next_u32(void) {
  lcg = lcg * 1664525u + 1013904223u;
  return lcg >> 8;
}

int main(void) {
  /* kept counts: k in [1, n], ceil(tau * n) for exact products */
  EXPECT(fastocr_kept_count(0.1, 256) == 26);
  EXPECT(fastocr_kept_count(0.05, 16384) == 820);
  EXPECT(fastocr_kept_count(0.5, 0) == 0);
  EXPECT(fastocr_kept_count(1.5, 10) == FASTOCR_ERR_INVALID_ARG);
  for (int n = 1; n < 2000; n += 7) {
    const int32_t k = fastocr_kept_count(0.05, n);
    EXPECT(k >= 1 && k <= n);
  }

  /* image-first maps of random span sets: a permutation, image rows first */
  for (int trial = 0; trial < 500; ++trial) {
    const int rows = 1 + (int)(next_u32() % 300);
    int32_t spans[16];
    int ns = 0, at = 0;
    while (ns < 8 && at < rows) {
      const int gap = (int)(next_u32() % 20), len = (int)(next_u32() % 40);
      if (at + gap + len > rows) break;
      spans[2 * ns] = at + gap;
      spans[2 * ns + 1] = len;
      at += gap + len;
      ++ns;
    }
    int32_t* map = malloc(sizeof(int32_t) * (size_t)rows);
    char* seen = calloc((size_t)rows, 1);
    const int32_t n = fastocr_image_first_map(spans, ns, rows, map);
    EXPECT(n >= 0 && n <= rows);
    for (int i = 0; i < rows; ++i) {
      EXPECT(map[i] >= 0 && map[i] < rows && !seen[map[i]]);
      seen[map[i]] = 1;
      if (i > 0 && i != n) EXPECT(map[i] > map[i - 1]);
    }
    free(map);
    free(seen);
  }
  {
    int32_t bad[4] = {5, 4, 2, 1}, map[20];
    EXPECT(fastocr_image_first_map(bad, 2, 20, map) == FASTOCR_ERR_INVALID_ARG);
    EXPECT(fastocr_image_first_map(NULL, 1, 20, map) == FASTOCR_ERR_INVALID_ARG);
    EXPECT(fastocr_image_first_map(NULL, 0, 0, map) == 0);
  }

  /* focal layers: ascending, the largest ratios, ties to the lower layer */
  for (int trial = 0; trial < 500; ++trial) {
    const int L = 1 + (int)(next_u32() % 40), c = 1 + (int)(next_u32() % (uint32_t)L);
    double r[40];
    int32_t out[40];
    for (int l = 0; l < L; ++l) r[l] = (double)(next_u32() % 5) / 5.0;
    EXPECT(fastocr_choose_focal_layers(r, L, c, out) == FASTOCR_OK);
    for (int i = 1; i < c; ++i) EXPECT(out[i] > out[i - 1]);
    double worst_in = 2.0, best_out = -1.0;
    for (int l = 0, j = 0; l < L; ++l) {
      if (j < c && out[j] == l) {
        worst_in = r[l] < worst_in ? r[l] : worst_in;
        ++j;
      } else {
        best_out = r[l] > best_out ? r[l] : best_out;
      }
    }
    EXPECT(worst_in >= best_out);
  }
  EXPECT(fastocr_choose_focal_layers(NULL, 4, 2, NULL) == FASTOCR_ERR_INVALID_ARG);

  /* configuration checks and argument validation (no kernel runs) */
  fastocr_config cfg;
  memset(&cfg, 0, sizeof(cfg));
  cfg.tau = 0.1;
  cfg.num_layers = 4;
  cfg.num_q_heads = 4;
  cfg.num_kv_heads = 2;
  cfg.head_dim = 96; /* invalid */
  cfg.batch = 1;
  cfg.max_seq_len = 304;
  cfg.max_img_tokens = 256;
  cfg.dtype = FASTOCR_DTYPE_F32;
  cfg.num_focal = 2;
  cfg.warmup_steps = 4;
  fastocr_handle* h = NULL;
  EXPECT(fastocr_create(&cfg, NULL, &h) == FASTOCR_ERR_INVALID_ARG && h == NULL);
  EXPECT(fastocr_create(NULL, NULL, &h) == FASTOCR_ERR_INVALID_ARG);
  EXPECT(fastocr_attend(NULL, 0, NULL, NULL, NULL, NULL, NULL) == FASTOCR_ERR_INVALID_ARG);
  EXPECT(fastocr_destroy(NULL) == FASTOCR_OK);
  EXPECT(fastocr_pack_rows(NULL, NULL, NULL, NULL, 1, 1, 8, 64, FASTOCR_DTYPE_BF16, NULL, NULL) ==
         FASTOCR_ERR_INVALID_ARG);
  for (int code = 1; code >= -5; --code) EXPECT(fastocr_error_string(code) != NULL);
  printf("host checks ok\n");
  return 0;
}
