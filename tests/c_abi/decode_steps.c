/* A decode run driven through the C ABI alone (no Python, no torch): the
 * caller allocates its buffers with the HIP runtime, fills them from a
 * fixed-seed generator, runs the warm-up, the focal-layer profile and
 * pruned steps, and writes every step's outputs to a file for comparison
 * with the same run through the Python binding.
 *
 * usage: decode_steps OUT_FILE
 * Shapes: fp32, L = 3 layers, 4 query / 2 KV heads, head_dim 64, batch 2,
 * capacity 96 rows, 40 image tokens per sequence, 20 prompt rows, w = 2
 * warm-up steps, 2 focal layers, tau = 0.25, 6 steps in all. */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "fastocr.h"

enum { L = 3, HQ = 4, HKV = 2, D = 64, B = 2, S = 96, NIMG = 40, NPROMPT = 20, W = 2, STEPS = 6 };

static uint64_t rng_state = 12345u;
static float next_value(void) { /* xorshift64*, uniform in [-1, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  const uint64_t x = rng_state * 2685821657736338717ull;
  return (float)((double)(x >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

#define CHECK_HIP(call)                                                    \
  do {                                                                     \
    if ((call) != hipSuccess) {                                            \
      fprintf(stderr, "HIP error at %s:%d\n", __FILE__, __LINE__);        \
      return 2;                                                            \
    }                                                                      \
  } while (0)
#define CHECK_OCR(call)                                                    \
  do {                                                                     \
    int rc_ = (call);                                                      \
    if (rc_ != FASTOCR_OK) {                                               \
      fprintf(stderr, "%s failed: %s\n", #call, fastocr_error_string(rc_)); \
      return 3;                                                            \
    }                                                                      \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 2) return 1;
  const size_t kv_elems = (size_t)B * HKV * S * D, q_elems = (size_t)B * HQ * D;
  float* host_kv = malloc(kv_elems * sizeof(float));
  float* host_q = malloc(q_elems * sizeof(float));
  float* host_out = malloc(q_elems * sizeof(float));
  float *k[L], *v[L], *q, *out;
  int32_t* lens;
  for (int l = 0; l < L; ++l) {
    CHECK_HIP(hipMalloc((void**)&k[l], kv_elems * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&v[l], kv_elems * sizeof(float)));
    for (size_t i = 0; i < kv_elems; ++i) host_kv[i] = next_value();
    CHECK_HIP(hipMemcpy(k[l], host_kv, kv_elems * sizeof(float), hipMemcpyHostToDevice));
    for (size_t i = 0; i < kv_elems; ++i) host_kv[i] = next_value();
    CHECK_HIP(hipMemcpy(v[l], host_kv, kv_elems * sizeof(float), hipMemcpyHostToDevice));
  }
  CHECK_HIP(hipMalloc((void**)&q, q_elems * sizeof(float)));
  CHECK_HIP(hipMalloc((void**)&out, q_elems * sizeof(float)));
  CHECK_HIP(hipMalloc((void**)&lens, B * 2 * sizeof(int32_t)));

  fastocr_config cfg = {0};
  cfg.tau = 0.25;
  cfg.num_layers = L;
  cfg.num_q_heads = HQ;
  cfg.num_kv_heads = HKV;
  cfg.head_dim = D;
  cfg.batch = B;
  cfg.max_seq_len = S;
  cfg.max_img_tokens = NIMG;
  cfg.dtype = FASTOCR_DTYPE_F32;
  cfg.num_focal = 2;
  cfg.warmup_steps = W;
  cfg.mode = FASTOCR_MODE_PRUNED;
  fastocr_handle* h = NULL;
  CHECK_OCR(fastocr_create(&cfg, NULL, &h));
  FILE* f = fopen(argv[1], "wb");
  if (!f) return 4;
  int32_t focal[2] = {-1, -1};
  for (int t = 0; t < STEPS; ++t) {
    if (t == W) CHECK_OCR(fastocr_profile_warmup(h, focal));
    int32_t host_lens[B * 2];
    for (int b = 0; b < B; ++b) {
      host_lens[2 * b] = NIMG;
      host_lens[2 * b + 1] = NIMG + NPROMPT + t + 1;
    }
    CHECK_HIP(hipMemcpy(lens, host_lens, sizeof(host_lens), hipMemcpyHostToDevice));
    for (int l = 0; l < L; ++l) {
      for (size_t i = 0; i < q_elems; ++i) host_q[i] = 2.0f * next_value();
      CHECK_HIP(hipMemcpy(q, host_q, q_elems * sizeof(float), hipMemcpyHostToDevice));
      CHECK_OCR(fastocr_attend(h, l, q, k[l], v[l], lens, out));
      CHECK_HIP(hipMemcpy(host_out, out, q_elems * sizeof(float), hipMemcpyDeviceToHost));
      fwrite(host_out, sizeof(float), q_elems, f);
    }
  }
  int32_t flags = -1;
  CHECK_OCR(fastocr_get_status(h, &flags));
  CHECK_OCR(fastocr_destroy(h));
  fclose(f);
  printf("focal %d %d flags %d\n", focal[0], focal[1], flags);
  return flags == 0 ? 0 : 5;
}
