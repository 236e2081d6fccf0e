/* A plain C99 caller of libgqa: checks that the header compiles as C and that the host-side entry
 * points answer as documented without a GPU (every call here returns before any HIP call). */
#include <stdio.h>
#include <string.h>

#include "gqa.h"

static int failures = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    printf("FAIL: %s\n", what);
    ++failures;
  }
}

int main(void) {
  /* the 70B-shaped layer: B32 Hq64 Hkv8 d128 L8192, bf16 everywhere */
  gqa_shape_t s = {32, 64, 8, 8192, 128, GQA_BF16, GQA_BF16, GQA_BF16, 1.0f, 1.0f, 0};
  expect(gqa_shape_check(&s) == GQA_OK, "valid shape");
  const size_t n = gqa_decode_workspace_bytes(&s);
  expect(n > ((size_t)1 << 20) && n % 16 == 0, "workspace: the 1 MiB counter area plus partial slots");

  gqa_shape_t bad = s;
  bad.Hq = 60; /* not a multiple of Hkv */
  expect(gqa_shape_check(&bad) == GQA_ERR_INVALID_ARG, "Hq % Hkv != 0 rejected");
  expect(gqa_decode_workspace_bytes(&bad) == 0, "no workspace for an invalid shape");
  bad = s;
  bad.d = 96;
  expect(gqa_shape_check(&bad) == GQA_ERR_UNSUPPORTED, "head dim 96 unsupported");

  /* null pointers are refused before anything is enqueued */
  expect(gqa_decode(NULL, NULL, NULL, NULL, 0.088f, NULL, &s, NULL, 0, NULL) == GQA_ERR_INVALID_ARG,
         "null pointers");

  /* the pages' KV-bytes formula: 2 * layers * kv_heads * head_dim * dtype_bytes */
  expect(gqa_kv_bytes_per_token(80, 8, 128, 2) == 327680u, "70B GQA-8: 320 KiB per token");
  expect(gqa_kv_bytes_per_token(32, 8, 128, 2) == 131072u, "8B-class GQA-8: 128 KiB per token");

  expect(strncmp(gqa_status_string(GQA_ERR_WORKSPACE), "GQA_ERR_WORKSPACE", 17) == 0, "status text");

  gqa_paged_shape_t ps = {32, 64, 8, 128, 16, 512, 14024, GQA_BF16, GQA_BF16, GQA_BF16, 1.0f, 1.0f, 0};
  expect(gqa_paged_shape_check(&ps) == GQA_OK, "valid paged shape");
  ps.block_size = 24;
  expect(gqa_paged_shape_check(&ps) == GQA_ERR_UNSUPPORTED, "block size not a power of two");

  if (failures == 0) printf("ok\n");
  return failures == 0 ? 0 : 1;
}
