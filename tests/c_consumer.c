/* A plain C consumer of libsanala's C-ABI: the header compiles as C11, every entry point links from C,
 * and calls with bad arguments return their status codes on the host before any HIP call (so this runs
 * without a GPU).  Exits 0 when every check holds, else prints the first failed check and exits 1. */
#include <stdio.h>
#include <string.h>

#include "sanala.h"

static int fails = 0;
#define EXPECT(cond)                                           \
  do {                                                         \
    if (!(cond)) {                                             \
      fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
      fails++;                                                 \
    }                                                          \
  } while (0)

int main(void) {
  /* fake, 16-byte aligned device addresses: every call below is rejected before they are used */
  void* q = (void*)0x1000;
  void* k = (void*)0x2000000;
  void* v = (void*)0x4000000;
  const float* gq = (const float*)0x6000000;
  const float* gk = (const float*)0x6001000;
  void* out = (void*)0x8000000;
  hipStream_t s = 0;

  EXPECT(strcmp(sana_status_string(SANA_OK), sana_status_string(SANA_ERR_HIP)) != 0);
  EXPECT(sana_linear_attn_fwd(NULL, k, v, gq, gk, 1, 16, 2, 32, 1e-6f, out, s, SANA_BF16) == SANA_ERR_INVALID_ARG);
  EXPECT(sana_linear_attn_fwd(q, k, v, gq, gk, 1, 16, 2, 16, 1e-6f, out, s, SANA_BF16) == SANA_ERR_UNSUPPORTED);
  EXPECT(sana_linear_attn_fwd(q, k, v, gq, NULL, 1, 16, 2, 32, 1e-6f, out, s, SANA_BF16) == SANA_ERR_INVALID_ARG);
  EXPECT(sana_linear_attn_fwd(q, k, v, gq, gk, 0, 16, 2, 32, 1e-6f, out, s, SANA_F32) == SANA_ERR_INVALID_ARG);
  EXPECT(sana_linear_attn_fwd(q, k, v, gq, gk, 1, 16, 2, 32, -1.0f, out, s, SANA_F16) == SANA_ERR_INVALID_ARG);
  EXPECT(sana_linear_attn_fwd((char*)q + 2, k, v, gq, gk, 1, 16, 2, 32, 1e-6f, out, s, SANA_BF16) ==
         SANA_ERR_MISALIGNED);
  EXPECT(sana_linear_attn_fwd_noalloc(q, k, v, gq, gk, 1, 16, 2, 32, 1e-6f, NULL, s, SANA_BF16) ==
         SANA_ERR_INVALID_ARG);
  EXPECT(sana_qkv_linear_attn_fwd(NULL, k, gq, gk, 1, 16, 2, 32, 1e-6f, out, s) == SANA_ERR_INVALID_ARG);
  EXPECT(sana_qkv_w8a8_linear_attn_fwd(q, NULL, gq, gq, gk, 1, 16, 2, 32, 1e-6f, out, s) == SANA_ERR_INVALID_ARG);
  EXPECT(sana_pack_weight_i8(NULL, 96, 64, out, s) == SANA_ERR_INVALID_ARG);
  EXPECT(sana_quantize_rows_i8(NULL, 4, 64, out, (float*)v, s) == SANA_ERR_INVALID_ARG);
  EXPECT(sana_mix_ffn_fwd(NULL, k, v, q, 1, 4, 4, 64, 64, out, s) == SANA_ERR_INVALID_ARG);
  EXPECT(sana_cross_attn_fwd(NULL, k, v, gq, gk, NULL, 1, 16, 8, 2, 32, 1e-6f, out, s, SANA_BF16) ==
         SANA_ERR_INVALID_ARG);
  if (fails == 0) printf("c consumer: all checks passed\n");
  return fails == 0 ? 0 : 1;
}
