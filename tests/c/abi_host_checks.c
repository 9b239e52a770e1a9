/* Host-side checks of the C ABI from plain C (no GPU, no kernel launched).
 *
 * Compiled with gcc against include/tbq4.h and linked against libtbq4.so by
 * tests/test_abi_c.py: the header is valid C, every call links, and the
 * documented host-side contract holds -- sizes, the sign vector, and the
 * status codes of invalid calls (checked before anything is launched).
 * Prints one line per failed check and exits with the number of failures. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tbq4.h"

static int failures = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      printf("FAILED line %d: %s\n", __LINE__, #cond);                     \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

int main(void) {
  /* never dereferenced: every call below fails its host-side checks */
  uint8_t *const fake = (uint8_t *)(uintptr_t)0x10000;

  CHECK(tbq4_version() != NULL && strlen(tbq4_version()) >= 5);
  CHECK(strcmp(tbq4_status_str(TBQ4_OK), tbq4_status_str(TBQ4_ERR_CAPACITY)) != 0);

  /* 66 bytes per head vector: 262144 tokens x 128 (layer, KV head) pairs */
  CHECK(tbq4_cache_bytes(1, 128, 262144) == (size_t)262144 * 128 * 66);
  CHECK(tbq4_cache_bytes(-1, 1, 8) == 0);
  CHECK(tbq4_format_row_bytes(TBQ4_FMT_TBQ4) == TBQ4_BLOCK_BYTES);
  CHECK(tbq4_format_row_bytes(TBQ4_FMT_F16) == 2 * TBQ4_HEAD_DIM);
  CHECK(tbq4_format_row_bytes(TBQ4_FMT_TBQ3) == 50);
  CHECK(tbq4_format_row_bytes(TBQ4_FMT_Q8_0) == 136);
  CHECK(tbq4_format_row_bytes(99) == 0);

  /* sign vector: 128 bits, a function of the seed only */
  uint8_t s0[16], s0b[16], s1[16];
  CHECK(tbq4_sign_vector(0, s0) == TBQ4_OK);
  CHECK(tbq4_sign_vector(0, s0b) == TBQ4_OK);
  CHECK(tbq4_sign_vector(1, s1) == TBQ4_OK);
  CHECK(memcmp(s0, s0b, 16) == 0 && memcmp(s0, s1, 16) != 0);
  CHECK(tbq4_sign_vector(0, NULL) == TBQ4_ERR_INVALID_ARG);

  /* workspace sizes and split counts */
  const int32_t p = tbq4_decode_auto_splits(4, 8, 131072);
  CHECK(p >= 1 && p <= 1024);
  CHECK(tbq4_decode_workspace_bytes(4, 8, 64, 131072, 16) == (size_t)4 * 64 * 16 * 130 * 4);
  CHECK(tbq4_decode_workspace_bytes(4, 8, 64, 131072, 1025) == 0);

  /* invalid calls return their status and touch nothing */
  tbq4_cache c = {fake, fake, 1, 2, 128, 64, 0};
  CHECK(tbq4_quantize_append(NULL, fake, fake, TBQ4_F32, 0, 1, NULL) == TBQ4_ERR_INVALID_ARG);
  CHECK(tbq4_quantize_append(&c, fake, fake, TBQ4_F32, 60, 5, NULL) == TBQ4_ERR_CAPACITY);
  CHECK(tbq4_quantize_append(&c, fake, fake, TBQ4_F32, 0, 0, NULL) == TBQ4_OK);   /* no-op */
  tbq4_cache bad = c;
  bad.head_dim = 64;
  CHECK(tbq4_quantize_append(&bad, fake, fake, TBQ4_F32, 0, 1, NULL) == TBQ4_ERR_UNSUPPORTED);
  bad = c;
  bad.capacity = 60;
  CHECK(tbq4_quantize_append(&bad, fake, fake, TBQ4_F32, 0, 1, NULL) == TBQ4_ERR_ALIGNMENT);
  CHECK(tbq4_attn_decode(&c, fake, TBQ4_F32, 8, 65, 1.0f, fake, TBQ4_F16, 0, fake, 1 << 20,
                         NULL) == TBQ4_ERR_CAPACITY);
  CHECK(tbq4_attn_decode(&c, fake, TBQ4_F32, 8, 10, 1.0f, fake, TBQ4_F16, 0, fake, 16, NULL) ==
        TBQ4_ERR_WORKSPACE);
  CHECK(tbq4_attn_prefill_chunk(&c, fake, TBQ4_F32, 16, 60, 5, 0.1f, fake, TBQ4_F16, NULL) ==
        TBQ4_ERR_CAPACITY);
  CHECK(tbq4_attn_verify(&c, fake, TBQ4_F32, 16, 10, 5, 1.0f, fake, TBQ4_F16, 0, fake, 1 << 20,
                         NULL) == TBQ4_ERR_UNSUPPORTED);
  CHECK(tbq4_decode_step_workspace_bytes(1, 2, 8, 64, 4) == ((size_t)8 * 5 * 130 * 4 + 255) / 256 * 256);
  CHECK(tbq4_decode_step(&c, fake, fake, TBQ4_F32, 64, NULL, fake, TBQ4_F32, 8, 1.0f, fake,
                         TBQ4_F16, 4, fake, 1 << 20, NULL) == TBQ4_ERR_CAPACITY);
  CHECK(tbq4_decode_step(&c, fake, fake, TBQ4_F32, 10, NULL, fake, TBQ4_F32, 8, 1.0f, fake,
                         TBQ4_F16, 4, fake, 8 * 4 * 130 * 4, NULL) == TBQ4_ERR_WORKSPACE);
  tbq4_mixed_cache m = {fake, fake, TBQ4_FMT_TBQ4, TBQ4_FMT_Q8_0, 1, 2, 128, 64, 0};
  CHECK(tbq4_mixed_append(&m, fake, fake, TBQ4_F32, 60, 5, NULL) == TBQ4_ERR_CAPACITY);
  m.v_format = 7;
  CHECK(tbq4_mixed_append(&m, fake, fake, TBQ4_F32, 0, 1, NULL) == TBQ4_ERR_UNSUPPORTED);

  if (failures == 0) printf("all host-side ABI checks passed\n");
  return failures;
}
