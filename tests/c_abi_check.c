/* Calls libmala's C ABI from plain C99: the header compiles as C, and the
 * queries and argument checks that need no GPU behave as documented. Built
 * and run by test_abi.py (exit status 0 = every check passed). */
#include <stdio.h>
#include <string.h>

#include "mala.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main(void) {
  int32_t bq = 0, bk = 0, chunk = -1;
  CHECK(strstr(mala_version(), "gfx950") != NULL);

  CHECK(mala_get_tiling(MALA_OP_FWD, MALA_BF16, 128, &bq, &bk, &chunk) == MALA_OK);
  CHECK(bq == 32 && bk == 64 && chunk == 0);
  CHECK(mala_get_tiling(MALA_OP_BWD, MALA_BF16, 128, &bq, &bk, &chunk) == MALA_OK);
  CHECK(bq == 32 && bk == 16);
  CHECK(mala_get_tiling(MALA_OP_DECODE, MALA_BF16, 128, &bq, &bk, &chunk) == MALA_OK);
  CHECK(bq == 1 && bk == 64 && chunk == 256);
  CHECK(mala_get_tiling(7, MALA_BF16, 128, &bq, &bk, &chunk) == MALA_ERR_INVALID_ARG);
  CHECK(strlen(mala_last_error()) > 0);

  mala_problem p;
  memset(&p, 0, sizeof p);
  p.batch = 1; p.n_q_heads = 8; p.n_kv_heads = 2; p.n_q = 1000; p.n_k = 1000;
  p.head_dim = 128; p.dtype = MALA_BF16; p.causal = 1; p.tau = 1e-4f;
  p.softmax_scale = 0.088388f;
  CHECK(mala_bwd_workspace_size(&p) > 0);
  p.tau = -1.0f;                                   /* rejected: tau < 0 */
  CHECK(mala_bwd_workspace_size(&p) == 0);
  CHECK(mala_fwd(&p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == MALA_ERR_INVALID_ARG);
  CHECK(strstr(mala_last_error(), "tau") != NULL);
  CHECK(mala_fwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == MALA_ERR_INVALID_ARG);
  p.tau = 1e-4f;                                   /* the nested backward needs the flag */
  CHECK(mala_bwd_nested(&p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                        NULL, NULL, NULL) == MALA_ERR_INVALID_ARG);
  CHECK(strstr(mala_last_error(), "MALA_FLAG_GATE_PASS") != NULL);
  CHECK(mala_bwd_auto(&p, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                      NULL, NULL, NULL) == MALA_ERR_INVALID_ARG);  /* no forward counters */
  CHECK(strstr(mala_last_error(), "fwd_kept_tiles") != NULL);

  mala_decode_problem d;
  memset(&d, 0, sizeof d);
  d.batch = 8; d.n_q_heads = 8; d.n_kv_heads = 1; d.head_dim = 128;
  d.cache_capacity = 131073; d.max_n_k = 131073; d.dtype = MALA_BF16;
  d.tau = 1e-4f; d.softmax_scale = 0.088388f;
  CHECK(mala_decode_split_keys(&d) == 256);        /* split_keys = 0: the default */
  d.split_keys = MALA_DECODE_SPLIT_AUTO;
  CHECK(mala_decode_split_keys(&d) == 1280);
  d.split_keys = 1 << 20;                          /* longer than the sequence */
  CHECK(mala_decode_split_keys(&d) == 131136);
  d.split_keys = 100;                              /* not a multiple of 64 */
  CHECK(mala_decode_split_keys(&d) == 0);
  CHECK(mala_decode_workspace_size(&d) == 0);

  if (failures == 0) printf("c abi ok\n");
  return failures == 0 ? 0 : 1;
}
