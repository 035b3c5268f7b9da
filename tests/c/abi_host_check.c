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

  /* message sizing, host only.  The 64-rank message shape: a region of n
   * tokens is 32 bytes (header, flag) plus a body of n*7168 codes, n*56*4
   * scale bytes, 2 * n*8*4 bytes of weights and ids, n*4 token bytes (all
   * multiples of 16 at n = 256).  Worst case: every pair carries T = 256
   * tokens: a region of 1,909,792 bytes; a rank's 64 regions rounded up
   * to 2 MiB are 59 regions; a body spans at most one 2 MiB boundary, so a
   * message has at most 1 + 2*1 payload pieces, a header and a flag. */
  {
    ep_problem m = p;
    int64_t sb = -1, rb = -1, nd = -1;
    m.num_ranks = 64;
    m.num_tokens = 256;
    m.mode = EP_MODE_MESSAGES;
    m.quant = EP_QUANT_FP8_F32;
    expect(ep_messages_capacity(&m, NULL, &sb, &rb, &nd) == EP_OK, "message sizing ok");
    expect(sb == (int64_t)64 * 59 * (2 << 20) && rb == sb, "worst-case arena bytes");
    expect(nd == (int64_t)64 * 64 * 5, "worst-case descriptors");
    static int32_t counts[64 * 64];
    memset(counts, 0, sizeof counts);
    expect(ep_messages_capacity(&m, counts, &sb, &rb, &nd) == EP_OK && sb == 0 && rb == 0 &&
               nd == 0,
           "no messages, no bytes");
    /* one message of one token: region 32 + 7168 + 224 + 32 + 32 + 16 bytes,
     * rounded up to one 2 MiB region on each side; three pieces */
    counts[3 * 64 + 5] = 1;
    expect(ep_messages_capacity(&m, counts, &sb, &rb, &nd) == EP_OK && sb == (2 << 20) &&
               rb == (2 << 20) && nd == 3,
           "one message");
    counts[3 * 64 + 5] = 257; /* more than T tokens */
    expect(ep_messages_capacity(&m, counts, &sb, &rb, &nd) == EP_ERR_SHAPE, "count above T");
    m.mode = EP_MODE_NORMAL;
    expect(ep_messages_capacity(&m, NULL, &sb, &rb, &nd) == EP_ERR_MODE, "sizing outside messages");
  }

  /* every status has a message */
  for (int s = EP_ERR_HIP; s <= EP_OK; ++s)
    expect(ep_status_string(s) != NULL && strlen(ep_status_string(s)) > 0, "status string");

  printf("%s\n", failures ? "abi check failed" : "abi check ok");
  return failures ? 1 : 0;
}
