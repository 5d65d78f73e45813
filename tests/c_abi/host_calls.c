/* Plain C99 client of libs4kv.so: the public headers compile as C, the library
 * links without C++ or HIP headers on the client side, and the host-only calls
 * (shape validation, sizes, argument refusals) behave as documented. No GPU
 * work is enqueued: every call here either is host-only or fails validation
 * before any launch. Prints "ok" and exits 0 on success. */
#include <stdio.h>
#include <stdint.h>

#include "s4kv.h"
#include "s4kv_probe.h"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      printf("check failed at line %d: %s\n", __LINE__, #c);       \
      return 1;                                                    \
    }                                                              \
  } while (0)

int main(void) {
  s4kv_shape s = {4, 32, 8, S4KV_HEAD_DIM, S4KV_PAGE_SIZE, 100, 64};
  CHECK(s4kv_validate(&s) == S4KV_OK);
  CHECK(s4kv_validate(NULL) == S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_pool_bytes(&s) == (size_t)100 * 8 * S4KV_CHUNK_STRIDE);
  CHECK(s4kv_kivi2_pool_bytes(&s) == (size_t)100 * 8 * S4KV_K2_CHUNK_STRIDE);
  CHECK(s4kv_fp16_pool_bytes(&s) == (size_t)100 * 8 * S4KV_F16_CHUNK_BYTES);
  CHECK(s4kv_fp8_pool_bytes(&s) == (size_t)100 * 8 * S4KV_FP8_CHUNK_BYTES);
  CHECK(s4kv_tail_bytes(&s) == (size_t)4 * 8 * 16 * 128 * 2);
  CHECK(s4kv_decode_workspace_bytes(&s, 1000) > 0);
  CHECK(s4kv_mq_workspace_bytes(&s, 1000, 4) > s4kv_decode_workspace_bytes(&s, 1000));
  CHECK(s4kv_mq_workspace_bytes(&s, 1000, 5) > s4kv_mq_workspace_bytes(&s, 1000, 4));
  CHECK(s4kv_mq_workspace_bytes(&s, 1000, 70000) == 0);

  s4kv_shape bad = s;
  bad.head_dim = 96;
  CHECK(s4kv_validate(&bad) == S4KV_ERR_UNSUPPORTED);
  CHECK(s4kv_pool_bytes(&bad) == 0);
  /* refused before any launch: null pointers, bad sizes */
  CHECK(s4kv_quantize_append(&s, NULL, NULL, NULL, NULL, 1, NULL, NULL, NULL, NULL, NULL) ==
        S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_paged_decode(&bad, NULL, NULL, NULL, NULL, NULL, NULL, 16, 0.088f, NULL, NULL, 0,
                          NULL) == S4KV_ERR_UNSUPPORTED);
  CHECK(s4kv_paged_decode_append(&s, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 16, 0.088f,
                                 NULL, NULL, 0, NULL) == S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_fp8_paged_decode(&s, NULL, NULL, NULL, NULL, 0, 0.088f, NULL, NULL, NULL, NULL, 0,
                              NULL) == S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_probe_read(NULL, 4096, NULL, 1, 1, 1, NULL) == S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_status_string(S4KV_ERR_WORKSPACE)[0] != '\0');
  printf("ok\n");
  return 0;
}
