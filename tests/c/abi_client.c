/* A plain C99 client of the C ABI: it includes only cpattn.h, links
 * libcpattn.so and calls the entry points that need no device (version,
 * order selection, workspace sizes, argument validation).  Exit status 0
 * when every check holds; each failed check prints a line. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "cpattn.h"

static int failures = 0;
#define CHECK(cond)                                            \
  do {                                                         \
    if (!(cond)) {                                             \
      printf("check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                              \
    }                                                          \
  } while (0)

static cpattn_tensor bshd(int dtype, int64_t B, int64_t S, int64_t H, int64_t D) {
  cpattn_tensor t;
  memset(&t, 0, sizeof t);
  t.data = (void*)(uintptr_t)0x100000; /* never dereferenced by these calls */
  t.dtype = dtype;
  t.B = B;
  t.S = S;
  t.H = H;
  t.D = D;
  t.stride_h = D;
  t.stride_s = H * D;
  t.stride_b = S * H * D;
  return t;
}

int main(void) {
  const char* v = cpattn_version();
  CHECK(v != NULL && strncmp(v, "cpattn ", 7) == 0);

  /* 2048 new tokens on a 131072-token context, 16 ranks, 16/1 heads, D = 128 */
  cpattn_tensor q = bshd(CPATTN_BF16, 1, 2048, 16, 128);
  cpattn_tensor k = bshd(CPATTN_BF16, 1, 133120, 1, 128);
  int order = -1;
  uint64_t b_kv = 0, b_q = 0;
  CHECK(cpattn_ring_select_order(&q, &k, 16, 1, &order, &b_kv, &b_q) == CPATTN_OK);
  CHECK(order == CPATTN_PASS_Q);
  CHECK(b_kv == 1022361600u && b_q == 379453440u);

  /* equal lengths: Pass-KV moves less; 136 causal pair slots of 8192 rows */
  cpattn_tensor q2 = bshd(CPATTN_BF16, 1, 131072, 16, 128);
  cpattn_tensor k2 = bshd(CPATTN_BF16, 1, 131072, 1, 128);
  CHECK(cpattn_ring_select_order(&q2, &k2, 16, 1, &order, NULL, NULL) == CPATTN_OK);
  CHECK(order == CPATTN_PASS_KV);
  size_t ws = cpattn_ring_prefill_workspace_size(&q2, NULL, 16, 1);
  CHECK(ws >= (size_t)136 * 8192 * 16 * 129 * 4);

  /* invalid: chunk count that does not divide the sequence */
  CHECK(cpattn_ring_prefill_workspace_size(&q2, NULL, 7, 1) == 0);
  const char* err = cpattn_last_error();
  CHECK(err != NULL && strlen(err) > 0);

  /* no place for the result */
  CHECK(cpattn_ring_select_order(&q2, &k2, 16, 1, NULL, NULL, NULL) == CPATTN_ERR_INVALID_ARG);

  if (failures == 0) printf("abi client ok: %s\n", v);
  return failures == 0 ? 0 : 1;
}
