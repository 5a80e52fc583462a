/* A plain C99 caller of the library's C ABI (built and run by
 * tests/test_c_abi.py on the host, no GPU): the header compiles as C, the
 * library links, and the host-only calls behave as include/mcs.h states. */
#include <stdio.h>
#include <string.h>

#include "mcs.h"

static int failures = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

int main(void) {
  mcs_problem p;
  size_t bytes = 0, min_bytes = 0;
  mcs_status s;
  memset(&p, 0, sizeof p);
  p.B = 1; p.H = 12; p.Nq = 32760; p.Nkv = 32760; p.d = 128; p.group_size = 64; p.k = 1638;
  p.scale = 0.08838834764831845f; p.pddp_iters = 32; p.dtype = MCS_BF16;
  CHECK(p.r_dtype == MCS_F32); /* zero-initialised: float32 residual */
  CHECK(sizeof(mcs_problem) == 14 * sizeof(int32_t));
  CHECK(p.anchor_mode == MCS_ANCHOR_AUTO);

  CHECK(mcs_version() > 0);
  CHECK(strcmp(mcs_status_string(MCS_OK), "MCS_OK") == 0);

  s = mcs_workspace_size(&p, MCS_WS_ANCHOR, &bytes, &min_bytes);
  CHECK(s == MCS_OK);
  CHECK(min_bytes > 0 && min_bytes <= bytes);
  s = mcs_workspace_size(&p, MCS_WS_GROUP, &bytes, &min_bytes);
  CHECK(s == MCS_OK && bytes > 0);

  /* an unsupported head dimension is refused on the host, with a message */
  p.d = 96;
  s = mcs_workspace_size(&p, MCS_WS_ANCHOR, &bytes, &min_bytes);
  CHECK(s == MCS_ERR_UNSUPPORTED);
  CHECK(strlen(mcs_last_error()) > 0);
  p.d = 128;

  /* a bf16 residual needs bf16 inputs */
  p.dtype = MCS_F32; p.r_dtype = MCS_BF16;
  s = mcs_workspace_size(&p, MCS_WS_ANCHOR, &bytes, &min_bytes);
  CHECK(s == MCS_ERR_UNSUPPORTED);
  p.dtype = MCS_BF16;
  s = mcs_workspace_size(&p, MCS_WS_ANCHOR, &bytes, &min_bytes);
  CHECK(s == MCS_OK);
  p.r_dtype = MCS_F32;

  /* a NULL pointer is refused before any launch */
  s = mcs_dense_attn(&p, NULL, NULL, NULL, NULL, NULL, NULL);
  CHECK(s == MCS_ERR_INVALID_ARG);

  /* an empty query set is a no-op that needs no pointers */
  p.Nq = 0;
  s = mcs_dense_attn(&p, NULL, NULL, NULL, NULL, NULL, NULL);
  CHECK(s == MCS_OK);

  if (failures == 0) printf("c abi ok (version %d)\n", (int)mcs_version());
  return failures == 0 ? 0 : 1;
}
