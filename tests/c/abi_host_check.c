/* A plain C99 caller of libep (include/ep.h): sizing, status strings and
 * the argument checks that return before anything is enqueued, with no
 * device memory involved.  Built and run by tests/test_abi_c.py. */
#include <stdio.h>
#include <string.h>

#include "ep.h"

static int failures = 0;

static void expect(int ok, const char* what) {
  if (!ok) {
    printf("FAIL %s\n", what);
    ++failures;
  }
}

int main(void) {
  ep_problem p;
  memset(&p, 0, sizeof p);
  p.num_ranks = 8;
  p.num_tokens = 4096;
  p.hidden = 7168;
  p.num_experts = 256;
  p.num_topk = 8;
  p.expert_alignment = 1;
  p.mode = EP_MODE_NORMAL;
  p.quant = EP_QUANT_NONE;
  p.region_bytes = 2 << 20;
  p.epoch = 1;

  /* worst-case receive rows: R*T*K (alignment 1) */
  expect(ep_max_recv_rows(&p) == (int64_t)8 * 4096 * 8, "normal worst-case rows");
  expect(ep_workspace_bytes(&p) > 0, "normal workspace");
  p.mode = EP_MODE_LOW_LATENCY;
  expect(ep_max_recv_rows(&p) == (int64_t)256 * 8 * 4096, "low-latency rows E*R*T");
  p.mode = EP_MODE_RANK_MAJOR;
  expect(ep_max_recv_rows(&p) == (int64_t)8 * 4096 * 8, "rank-major rows R*T*min(K,R)");
  p.mode = EP_MODE_NORMAL;

  /* invalid problems: no workspace size, no rows */
  p.num_experts = 255; /* not a multiple of R */
  expect(ep_workspace_bytes(&p) == 0 && ep_max_recv_rows(&p) == -1, "E % R rejected");
  p.num_experts = 256;
  p.quant = EP_QUANT_FP8_F32;
  p.hidden = 200; /* quantised rows need H % 128 == 0 */
  expect(ep_workspace_bytes(&p) == 0, "FP8 hidden % 128 rejected");
  p.hidden = 7168;
  p.quant = EP_QUANT_NONE;
  p.reserved = 1;
  expect(ep_workspace_bytes(&p) == 0, "reserved field must be 0");
  p.reserved = 0;

  /* argument errors return before any launch */
  expect(ep_get_layout(&p, NULL, NULL, NULL, 0, NULL) == EP_ERR_NULL, "layout without outputs");
  expect(ep_get_layout(NULL, NULL, NULL, NULL, 0, NULL) == EP_ERR_NULL, "layout without problem");
  expect(ep_combine(&p, NULL, NULL, 0, NULL, NULL, NULL) != EP_OK, "combine without arguments");

  /* every status has a message */
  for (int s = EP_ERR_HIP; s <= EP_OK; ++s)
    expect(ep_status_string(s) != NULL && strlen(ep_status_string(s)) > 0, "status string");

  printf("%s\n", failures ? "abi check failed" : "abi check ok");
  return failures ? 1 : 0;
}
