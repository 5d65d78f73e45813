/* Host-only driver of the C ABI (csrc/api.cpp linked against stub
 * launchers): every entry point with valid arguments reaches its launcher
 * exactly once; null pointers, refused shapes, out-of-range bounds and short
 * workspaces return their status and launch nothing. Shapes at the int32
 * limits exercise the overflow checks. Built with ASan and UBSan (no
 * recovery), so an out-of-bounds access or undefined arithmetic in the
 * validation aborts the run. Prints "ok" on success. */
#include <stdint.h>
#include <stdio.h>

#include "s4kv.h"

int stub_launches(void);

#define CHECK(c)                                               \
  do {                                                         \
    if (!(c)) {                                                \
      printf("check failed at line %d: %s\n", __LINE__, #c);   \
      return 1;                                                \
    }                                                          \
  } while (0)

/* fake device pointers: the stubs never dereference them */
static char dev_buf[64];
#define P ((void*)dev_buf)
#define IP ((const int32_t*)(void*)dev_buf)
#define FP ((const float*)(void*)dev_buf)

static int launched(int before) { return stub_launches() - before; }

int main(void) {
  const s4kv_shape s = {4, 32, 8, S4KV_HEAD_DIM, S4KV_PAGE_SIZE, 100, 64};
  const size_t ws = s4kv_decode_workspace_bytes(&s, 1000);
  const size_t mws = s4kv_mq_workspace_bytes(&s, 1000, 4);
  int n;
  CHECK(ws > 0 && mws > 0);

  /* valid calls: one launch each */
  n = stub_launches();
  CHECK(s4kv_quantize_append(&s, P, P, IP, IP, 16, IP, P, P, P, NULL) == S4KV_OK);
  CHECK(s4kv_kivi2_quantize_append(&s, P, P, IP, IP, 16, IP, P, P, P, NULL) == S4KV_OK);
  CHECK(s4kv_paged_decode(&s, P, P, P, P, IP, IP, 1000, 0.088f, P, P, ws, NULL) == S4KV_OK);
  CHECK(s4kv_kivi2_paged_decode(&s, P, P, P, P, IP, IP, 1000, 0.088f, P, P, ws, NULL) == S4KV_OK);
  CHECK(s4kv_paged_decode_append(&s, P, P, P, P, P, P, IP, IP, 1000, 0.088f, P, P, ws, NULL) ==
        S4KV_OK);
  CHECK(s4kv_paged_attention_mq(&s, P, IP, 4, 16, P, P, P, IP, IP, 1000, 0.088f, P, P, mws, NULL) ==
        S4KV_OK);
  CHECK(s4kv_fp16_append(&s, P, P, IP, IP, 16, IP, P, NULL) == S4KV_OK);
  CHECK(s4kv_fp16_paged_decode(&s, P, P, IP, IP, 1000, 0.088f, P, P, ws, NULL) == S4KV_OK);
  CHECK(s4kv_fp8_append(&s, P, P, IP, IP, 16, IP, FP, FP, P, NULL) == S4KV_OK);
  CHECK(s4kv_fp8_paged_decode(&s, P, P, IP, IP, 1000, 0.088f, FP, FP, P, P, ws, NULL) == S4KV_OK);
  CHECK(s4kv_paged_decode_append_noalloc(&s, P, P, P, P, P, P, IP, IP, 1000, 0.088f, P, NULL) ==
        S4KV_OK);
  CHECK(s4kv_check_tables(&s, IP, IP, 1000, (int32_t*)P, NULL) == S4KV_OK);
  CHECK(s4kv_check_tables(&s, IP, IP, 0, (int32_t*)P, NULL) == S4KV_OK);
  CHECK(launched(n) == 13);
  /* max_new 0 appends nothing and launches nothing */
  n = stub_launches();
  CHECK(s4kv_quantize_append(&s, P, P, IP, IP, 0, IP, P, P, P, NULL) == S4KV_OK);
  CHECK(launched(n) == 0);

  /* refusals: nothing launched */
  n = stub_launches();
  CHECK(s4kv_quantize_append(NULL, P, P, IP, IP, 1, IP, P, P, P, NULL) == S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_quantize_append(&s, NULL, P, IP, IP, 1, IP, P, P, P, NULL) == S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_quantize_append(&s, P, P, IP, IP, -1, IP, P, P, P, NULL) == S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_quantize_append(&s, P, P, IP, IP, 64 * 16 + 1, IP, P, P, P, NULL) ==
        S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_paged_decode(&s, P, P, P, P, IP, IP, 0, 0.088f, P, P, ws, NULL) == S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_paged_decode(&s, P, P, P, P, IP, IP, 64 * 16 + 1, 0.088f, P, P, ws, NULL) ==
        S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_paged_decode(&s, P, P, P, P, IP, IP, 1000, 0.088f, P, P, ws - 1, NULL) ==
        S4KV_ERR_WORKSPACE);
  CHECK(s4kv_paged_decode(&s, P, P, P, P, IP, IP, 1000, 0.088f, P, NULL, ws, NULL) ==
        S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_paged_decode_append(&s, P, NULL, P, P, P, P, IP, IP, 1000, 0.088f, P, P, ws, NULL) ==
        S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_paged_decode_append(&s, P, P, P, P, P, P, IP, IP, 1000, 0.088f, P, P, ws - 1, NULL) ==
        S4KV_ERR_WORKSPACE);
  CHECK(s4kv_paged_attention_mq(&s, P, IP, 70000, 16, P, P, P, IP, IP, 1000, 0.088f, P, P, mws,
                                NULL) == S4KV_ERR_UNSUPPORTED);
  CHECK(s4kv_paged_attention_mq(&s, P, IP, 4, 17, P, P, P, IP, IP, 1000, 0.088f, P, P, mws, NULL) ==
        S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_paged_attention_mq(&s, P, IP, 4, 16, P, P, P, IP, IP, 1000, 0.088f, P, P, mws - 1,
                                NULL) == S4KV_ERR_WORKSPACE);
  CHECK(s4kv_fp8_append(&s, P, P, IP, IP, 16, IP, NULL, FP, P, NULL) == S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_fp16_paged_decode(&s, P, P, IP, IP, 1000, 0.088f, P, P, 0, NULL) == S4KV_ERR_WORKSPACE);
  CHECK(s4kv_paged_decode_append_noalloc(&s, NULL, P, P, P, P, P, IP, IP, 1000, 0.088f, P, NULL) ==
        S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_check_tables(&s, NULL, IP, 1000, (int32_t*)P, NULL) == S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_check_tables(&s, IP, IP, 1000, NULL, NULL) == S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_check_tables(&s, IP, IP, -1, (int32_t*)P, NULL) == S4KV_ERR_INVALID_ARG);
  CHECK(s4kv_check_tables(NULL, IP, IP, 1000, (int32_t*)P, NULL) == S4KV_ERR_INVALID_ARG);
  {
    /* a shape whose workspace exceeds the static scratch array */
    const s4kv_shape wide = {65535, 16, 16, S4KV_HEAD_DIM, S4KV_PAGE_SIZE, 100, 64};
    CHECK(s4kv_validate(&wide) == S4KV_OK);
    CHECK(s4kv_decode_workspace_bytes(&wide, 1000) > (size_t)S4KV_NOALLOC_SCRATCH_BYTES);
    CHECK(s4kv_paged_decode_append_noalloc(&wide, P, P, P, P, P, P, IP, IP, 1000, 0.088f, P,
                                           NULL) == S4KV_ERR_SCRATCH_LIMIT);
  }
  CHECK(launched(n) == 0);

  /* shapes at and past the limits: validation arithmetic must not overflow */
  {
    s4kv_shape b = s;
    const int32_t big[] = {INT32_MAX, INT32_MAX - 1, 65535, 65536, 1 << 30};
    unsigned i, j;
    for (i = 0; i < sizeof big / sizeof big[0]; ++i) {
      for (j = 0; j < 5; ++j) {
        b = s;
        switch (j) {
          case 0: b.num_seqs = big[i]; break;
          case 1: b.num_pages = big[i]; break;
          case 2: b.max_pages_per_seq = big[i]; break;
          case 3: b.num_kv_heads = big[i]; b.num_q_heads = big[i]; break;
          default: b.num_pages = big[i]; b.num_kv_heads = 16; b.num_q_heads = 256; break;
        }
        n = stub_launches();
        (void)s4kv_validate(&b);
        (void)s4kv_pool_bytes(&b);
        (void)s4kv_tail_bytes(&b);
        (void)s4kv_decode_workspace_bytes(&b, INT32_MAX);
        (void)s4kv_mq_workspace_bytes(&b, INT32_MAX, INT32_MAX);
        if (s4kv_validate(&b) != S4KV_OK) {
          CHECK(s4kv_paged_decode(&b, P, P, P, P, IP, IP, 1000, 0.088f, P, P, (size_t)-1, NULL) !=
                S4KV_OK);
          CHECK(launched(n) == 0);
        }
      }
    }
    b = s;
    b.head_dim = 64;
    CHECK(s4kv_validate(&b) == S4KV_ERR_UNSUPPORTED);
    b = s;
    b.num_q_heads = 8 * 17;
    CHECK(s4kv_validate(&b) == S4KV_ERR_UNSUPPORTED);
    b = s;
    b.num_seqs = -5;
    CHECK(s4kv_validate(&b) == S4KV_ERR_INVALID_ARG);
    CHECK(s4kv_mq_workspace_bytes(&s, 1000, INT32_MAX) == 0);
  }
  for (n = -2; n < 8; ++n) CHECK(s4kv_status_string((s4kv_status)n) != NULL);
  printf("ok\n");
  return 0;
}
