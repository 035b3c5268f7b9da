/* A plain C caller of libep on the GPU, with device memory from the HIP
 * runtime and no Python: the layout, dispatch and combine of a small
 * normal-mode bf16 problem through ep_get_layout / ep_dispatch / ep_combine,
 * then the fused low-latency FP8 call (ep_dispatch_fused), then message
 * mode end to end (sizing, packer and descriptors, delivery, receiver),
 * each result compared with the oracle's C functions (oracle/ep_oracle.h).  Built and
 * run by tests/test_gpu_c_roundtrip.py. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep.h"
#include "ep_oracle.h"

static int failures = 0;

static void expect(int ok, const char* what) {
  if (!ok) {
    if (failures < 20) printf("FAIL %s\n", what);
    ++failures;
  }
}

#define HIP_OK(call)                                                    \
  do {                                                                  \
    hipError_t e_ = (call);                                             \
    if (e_ != hipSuccess) {                                             \
      printf("HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__);   \
      exit(2);                                                          \
    }                                                                   \
  } while (0)

/* seeded inputs (a linear congruential generator) */
static uint32_t seed = 20261202u;
static uint32_t next_u32(void) {
  seed = seed * 1664525u + 1013904223u;
  return seed >> 8;
}

/* bf16 bits of a float, nearest-even (input generation only) */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static double from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* K distinct experts per token, about one entry in ten masked (-1) */
static void gen_routing(int R, int T, int E, int K, int32_t* topk) {
  for (int i = 0; i < R * T; ++i) {
    for (int k = 0; k < K; ++k) {
      int e, dup;
      do {
        e = (int)(next_u32() % (uint32_t)E);
        dup = 0;
        for (int k2 = 0; k2 < k; ++k2) dup |= topk[i * K + k2] == e;
      } while (dup);
      topk[i * K + k] = e;
    }
    for (int k = 0; k < K; ++k)
      if (next_u32() % 10 == 0) topk[i * K + k] = -1;
  }
}

static void* dev(size_t bytes) {
  void* p = NULL;
  HIP_OK(hipMalloc(&p, bytes < 16 ? 16 : bytes));
  HIP_OK(hipMemset(p, 0x5A, bytes < 16 ? 16 : bytes));
  return p;
}

static void* host_of(const void* d, size_t bytes) {
  void* h = malloc(bytes < 16 ? 16 : bytes);
  HIP_OK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
  return h;
}

/* device layout buffers and their host copies */
typedef struct {
  ep_layout l;
  int R, T, E, K;
} dev_layout;

static void layout_alloc(dev_layout* d, int R, int T, int E, int K, int64_t cap) {
  memset(d, 0, sizeof *d);
  d->R = R;
  d->T = T;
  d->E = E;
  d->K = K;
  d->l.num_tokens_per_rank = dev(sizeof(int32_t) * R * R);
  d->l.num_tokens_per_expert = dev(sizeof(int32_t) * R * E);
  d->l.is_token_in_rank = dev((size_t)R * T * R);
  d->l.rank_prefix_matrix = dev(sizeof(int32_t) * R * R);
  d->l.recv_tokens_per_expert = dev(sizeof(int32_t) * E);
  d->l.expert_start = dev(sizeof(int32_t) * E);
  d->l.rows_per_rank = dev(sizeof(int32_t) * R);
  d->l.row_base = dev(sizeof(int32_t) * (R + 1));
  d->l.send_pos = dev(sizeof(int32_t) * R * T * K);
  d->l.send_head = dev(sizeof(int32_t) * R * T * R);
  d->l.recv_src_idx = dev(sizeof(int32_t) * (size_t)cap);
  d->l.recv_capacity = cap;
  d->l.err = dev(sizeof(int32_t));
}

static int same_i32(const void* d, const int32_t* o, int64_t n) {
  int32_t* h = host_of(d, sizeof(int32_t) * (size_t)n);
  const int ok = memcmp(h, o, sizeof(int32_t) * (size_t)n) == 0;
  free(h);
  return ok;
}

/* every layout output against the oracle's (recv_src_idx at the rows the
 * routed entries name) */
static void check_layout(const dev_layout* d, const orc_problem* op, const int32_t* topk,
                         int64_t cap, int32_t** send_pos_out, const char* name) {
  const int R = d->R, T = d->T, E = d->E, K = d->K;
  int32_t* cnt_rank = malloc(sizeof(int32_t) * R * R);
  int32_t* cnt_expert = malloc(sizeof(int32_t) * R * E);
  uint8_t* in_rank = malloc((size_t)R * T * R);
  int32_t* rpm = malloc(sizeof(int32_t) * R * R);
  int32_t* recv_pe = malloc(sizeof(int32_t) * E);
  int32_t* start = malloc(sizeof(int32_t) * E);
  int32_t* rows = malloc(sizeof(int32_t) * R);
  int32_t* base = malloc(sizeof(int32_t) * (R + 1));
  int32_t* send_pos = malloc(sizeof(int32_t) * R * T * K);
  int32_t* send_head = malloc(sizeof(int32_t) * R * T * R);
  int32_t* src_idx = malloc(sizeof(int32_t) * (size_t)cap);
  for (int64_t i = 0; i < cap; ++i) src_idx[i] = -7;
  const int oerr = orc_layout(op, topk, cnt_rank, cnt_expert, in_rank, rpm, recv_pe, start, rows,
                              base, send_pos, send_head, src_idx, cap);
  char what[128];
  snprintf(what, sizeof what, "%s: error word", name);
  expect(same_i32(d->l.err, &oerr, 1), what);
  snprintf(what, sizeof what, "%s: num_tokens_per_rank", name);
  expect(same_i32(d->l.num_tokens_per_rank, cnt_rank, R * R), what);
  snprintf(what, sizeof what, "%s: num_tokens_per_expert", name);
  expect(same_i32(d->l.num_tokens_per_expert, cnt_expert, R * E), what);
  snprintf(what, sizeof what, "%s: rank_prefix_matrix", name);
  expect(same_i32(d->l.rank_prefix_matrix, rpm, R * R), what);
  snprintf(what, sizeof what, "%s: recv_tokens_per_expert", name);
  expect(same_i32(d->l.recv_tokens_per_expert, recv_pe, E), what);
  snprintf(what, sizeof what, "%s: expert_start", name);
  expect(same_i32(d->l.expert_start, start, E), what);
  snprintf(what, sizeof what, "%s: rows_per_rank", name);
  expect(same_i32(d->l.rows_per_rank, rows, R), what);
  snprintf(what, sizeof what, "%s: row_base", name);
  expect(same_i32(d->l.row_base, base, R + 1), what);
  if (d->l.send_pos) { /* message mode's layout has no receive rows */
    snprintf(what, sizeof what, "%s: send_pos", name);
    expect(same_i32(d->l.send_pos, send_pos, R * T * K), what);
  }
  snprintf(what, sizeof what, "%s: send_head", name);
  expect(same_i32(d->l.send_head, send_head, R * T * R), what);
  uint8_t* g_in = host_of(d->l.is_token_in_rank, (size_t)R * T * R);
  snprintf(what, sizeof what, "%s: is_token_in_rank", name);
  expect(memcmp(g_in, in_rank, (size_t)R * T * R) == 0, what);
  free(g_in);
  /* filled rows: every row a routed entry names */
  if (d->l.recv_src_idx) {
    int32_t* g_src = host_of(d->l.recv_src_idx, sizeof(int32_t) * (size_t)cap);
    int ok = 1;
    for (int64_t i = 0; i < (int64_t)R * T * K; ++i)
      if (send_pos[i] >= 0) ok &= g_src[send_pos[i]] == src_idx[send_pos[i]];
    snprintf(what, sizeof what, "%s: recv_src_idx", name);
    expect(ok, what);
    free(g_src);
  }
  *send_pos_out = send_pos;
  free(cnt_rank);
  free(cnt_expert);
  free(in_rank);
  free(rpm);
  free(recv_pe);
  free(start);
  free(rows);
  free(base);
  free(send_head);
  free(src_idx);
}

static ep_problem problem(int R, int T, int H, int E, int K, int mode, int quant) {
  ep_problem p;
  memset(&p, 0, sizeof p);
  p.num_ranks = R;
  p.num_tokens = T;
  p.hidden = H;
  p.num_experts = E;
  p.num_topk = K;
  p.expert_alignment = 1;
  p.mode = mode;
  p.quant = quant;
  p.region_bytes = 2 << 20;
  p.epoch = 1;
  return p;
}

static orc_problem oproblem(const ep_problem* p) {
  orc_problem o;
  memset(&o, 0, sizeof o);
  o.R = p->num_ranks;
  o.T = p->num_tokens;
  o.H = p->hidden;
  o.E = p->num_experts;
  o.K = p->num_topk;
  o.align = p->expert_alignment;
  o.mode = p->mode;
  o.quant = p->quant;
  o.region_bytes = p->region_bytes;
  o.epoch = p->epoch;
  return o;
}

/* normal mode, bf16: layout, dispatch, combine of the identity expert */
static void normal_bf16(void) {
  const int R = 4, T = 100, H = 256, E = 16, K = 4, N = R * T;
  ep_problem p = problem(R, T, H, E, K, EP_MODE_NORMAL, EP_QUANT_NONE);
  orc_problem op = oproblem(&p);
  int32_t* topk = malloc(sizeof(int32_t) * N * K);
  uint16_t* x = malloc(sizeof(uint16_t) * (size_t)N * H);
  float* w = malloc(sizeof(float) * N * K);
  gen_routing(R, T, E, K, topk);
  for (int64_t i = 0; i < (int64_t)N * H; ++i)
    x[i] = to_bf16(((float)(next_u32() % 40001u) - 20000.0f) / 10000.0f);
  for (int i = 0; i < N * K; ++i) w[i] = (float)(next_u32() % 1000u + 1u) / 1000.0f;

  const int64_t cap = ep_max_recv_rows(&p);
  const size_t ws_bytes = ep_workspace_bytes(&p);
  void* ws = dev(ws_bytes);
  void* d_topk = dev(sizeof(int32_t) * N * K);
  void* d_x = dev(sizeof(uint16_t) * (size_t)N * H);
  void* d_w = dev(sizeof(float) * N * K);
  HIP_OK(hipMemcpy(d_topk, topk, sizeof(int32_t) * N * K, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_x, x, sizeof(uint16_t) * (size_t)N * H, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_w, w, sizeof(float) * N * K, hipMemcpyHostToDevice));
  dev_layout d;
  layout_alloc(&d, R, T, E, K, cap);
  ep_recv recv;
  memset(&recv, 0, sizeof recv);
  recv.x = dev(sizeof(uint16_t) * (size_t)cap * H);
  recv.capacity = cap;
  void* d_out = dev(sizeof(uint16_t) * (size_t)N * H);

  expect(ep_get_layout(&p, d_topk, &d.l, ws, ws_bytes, NULL) == EP_OK, "normal: ep_get_layout");
  expect(ep_dispatch(&p, &d.l, d_x, NULL, NULL, &recv, NULL, ws, ws_bytes, NULL) == EP_OK,
         "normal: ep_dispatch");
  /* identity expert: the combine reads the receive rows themselves */
  expect(ep_combine(&p, &d.l, recv.x, cap, d_w, d_out, NULL) == EP_OK, "normal: ep_combine");
  HIP_OK(hipDeviceSynchronize());

  int32_t* send_pos;
  check_layout(&d, &op, topk, cap, &send_pos, "normal");
  /* receive rows: bit for bit */
  uint16_t* orecv = calloc((size_t)cap * H, sizeof(uint16_t));
  orc_dispatch(&op, x, topk, send_pos, orecv, NULL, cap);
  uint16_t* grecv = host_of(recv.x, sizeof(uint16_t) * (size_t)cap * H);
  int ok = 1;
  for (int64_t i = 0; i < (int64_t)N * K; ++i)
    if (send_pos[i] >= 0)
      ok &= memcmp(grecv + (int64_t)send_pos[i] * H, orecv + (int64_t)send_pos[i] * H,
                   sizeof(uint16_t) * H) == 0;
  expect(ok, "normal: receive rows");
  /* combine: within 1e-2 relative, plus one part in 2^16 of the summed
   * magnitudes (the fp32 sum's rounding under cancellation) */
  uint16_t* oout = malloc(sizeof(uint16_t) * (size_t)N * H);
  orc_combine(&op, orecv, cap, w, send_pos, NULL, 0, oout);
  uint16_t* gout = host_of(d_out, sizeof(uint16_t) * (size_t)N * H);
  ok = 1;
  for (int t = 0; t < N; ++t)
    for (int c = 0; c < H; ++c) {
      double mag = 0.0;
      for (int k = 0; k < K; ++k)
        if (send_pos[t * K + k] >= 0)
          mag += fabs(w[t * K + k] * from_bf16(orecv[(int64_t)send_pos[t * K + k] * H + c]));
      const double g = from_bf16(gout[(int64_t)t * H + c]);
      const double o = from_bf16(oout[(int64_t)t * H + c]);
      ok &= fabs(g - o) <= 1e-2 * fabs(o) + mag / 65536.0;
    }
  expect(ok, "normal: combine");
  free(gout);
  free(oout);
  free(grecv);
  free(orecv);
  free(send_pos);
  free(topk);
  free(x);
  free(w);
}

/* low-latency FP8 (fp32 scales), layout and dispatch in one call, large
 * enough (8,192 entries) for the chunked layout the dispatch finishes */
static void ll_fp8_fused(void) {
  const int R = 8, T = 128, H = 512, E = 64, K = 8, N = R * T, G = H / 128;
  ep_problem p = problem(R, T, H, E, K, EP_MODE_LOW_LATENCY, EP_QUANT_FP8_F32);
  orc_problem op = oproblem(&p);
  int32_t* topk = malloc(sizeof(int32_t) * N * K);
  uint16_t* x = malloc(sizeof(uint16_t) * (size_t)N * H);
  gen_routing(R, T, E, K, topk);
  for (int64_t i = 0; i < (int64_t)N * H; ++i)
    x[i] = to_bf16(((float)(next_u32() % 40001u) - 20000.0f) / 1000.0f);
  const int64_t cap = ep_max_recv_rows(&p); /* E * R * T */
  const size_t ws_bytes = ep_workspace_bytes(&p);
  void* ws = dev(ws_bytes);
  void* d_topk = dev(sizeof(int32_t) * N * K);
  void* d_x = dev(sizeof(uint16_t) * (size_t)N * H);
  HIP_OK(hipMemcpy(d_topk, topk, sizeof(int32_t) * N * K, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_x, x, sizeof(uint16_t) * (size_t)N * H, hipMemcpyHostToDevice));
  dev_layout d;
  layout_alloc(&d, R, T, E, K, cap);
  ep_recv recv;
  memset(&recv, 0, sizeof recv);
  recv.x = dev((size_t)cap * H);
  recv.scales = dev(sizeof(float) * (size_t)E * G * R * T);
  recv.capacity = cap;
  expect(ep_dispatch_fused(&p, d_topk, &d.l, d_x, &recv, ws, ws_bytes, NULL) == EP_OK,
         "low-latency: ep_dispatch_fused");
  HIP_OK(hipDeviceSynchronize());

  int32_t* send_pos;
  check_layout(&d, &op, topk, cap, &send_pos, "low-latency");
  uint8_t* ocodes = calloc((size_t)cap * H, 1);
  float* oscales = calloc((size_t)E * G * R * T, sizeof(float));
  orc_dispatch(&op, x, topk, send_pos, ocodes, oscales, cap);
  uint8_t* gcodes = host_of(recv.x, (size_t)cap * H);
  float* gscales = host_of(recv.scales, sizeof(float) * (size_t)E * G * R * T);
  int ok_codes = 1, ok_scales = 1;
  for (int64_t i = 0; i < (int64_t)N * K; ++i) {
    const int32_t r = send_pos[i];
    if (r < 0) continue;
    ok_codes &= memcmp(gcodes + (int64_t)r * H, ocodes + (int64_t)r * H, H) == 0;
    const int e = r / (R * T), pos = r % (R * T);
    for (int g = 0; g < G; ++g) {
      const int64_t si = ((int64_t)e * G + g) * R * T + pos;
      ok_scales &= memcmp(&gscales[si], &oscales[si], sizeof(float)) == 0;
    }
  }
  expect(ok_codes, "low-latency: e4m3 codes");
  expect(ok_scales, "low-latency: scales");
  free(gcodes);
  free(gscales);
  free(ocodes);
  free(oscales);
  free(send_pos);
  free(topk);
  free(x);
}

/* message mode, FP8 with fp32 scales: packer and descriptors, loopback
 * delivery, receiver; sizes from ep_messages_capacity on read-back counts */
static void messages_path(void) {
  const int R = 4, T = 40, H = 256, E = 16, K = 4, N = R * T, G = H / 128, RT = R * T;
  ep_problem p = problem(R, T, H, E, K, EP_MODE_MESSAGES, EP_QUANT_FP8_F32);
  p.region_bytes = 512; /* puts are cut at every 512-byte boundary */
  p.epoch = 7;
  orc_problem op = oproblem(&p);
  int32_t* topk = malloc(sizeof(int32_t) * N * K);
  uint16_t* x = malloc(sizeof(uint16_t) * (size_t)N * H);
  float* w = malloc(sizeof(float) * N * K);
  gen_routing(R, T, E, K, topk);
  for (int64_t i = 0; i < (int64_t)N * H; ++i)
    x[i] = to_bf16(((float)(next_u32() % 40001u) - 20000.0f) / 1000.0f);
  for (int i = 0; i < N * K; ++i) w[i] = (float)(next_u32() % 1000u + 1u) / 1000.0f;
  const size_t ws_bytes = ep_workspace_bytes(&p);
  void* ws = dev(ws_bytes);
  void* d_topk = dev(sizeof(int32_t) * N * K);
  void* d_x = dev(sizeof(uint16_t) * (size_t)N * H);
  void* d_w = dev(sizeof(float) * N * K);
  HIP_OK(hipMemcpy(d_topk, topk, sizeof(int32_t) * N * K, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_x, x, sizeof(uint16_t) * (size_t)N * H, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_w, w, sizeof(float) * N * K, hipMemcpyHostToDevice));
  dev_layout d;
  layout_alloc(&d, R, T, E, K, 16);
  HIP_OK(hipFree(d.l.send_pos));
  HIP_OK(hipFree(d.l.recv_src_idx));
  d.l.send_pos = NULL; /* message mode: no receive rows, only send_head */
  d.l.recv_src_idx = NULL;
  d.l.recv_capacity = 0;
  expect(ep_get_layout(&p, d_topk, &d.l, ws, ws_bytes, NULL) == EP_OK, "messages: ep_get_layout");
  HIP_OK(hipDeviceSynchronize());
  int32_t* counts = host_of(d.l.num_tokens_per_rank, sizeof(int32_t) * R * R);
  int64_t send_bytes = 0, recv_bytes = 0, ndesc = 0;
  expect(ep_messages_capacity(&p, counts, &send_bytes, &recv_bytes, &ndesc) == EP_OK,
         "messages: ep_messages_capacity");
  ep_messages m;
  memset(&m, 0, sizeof m);
  m.send_arena = dev((size_t)send_bytes);
  m.send_capacity = send_bytes;
  m.table = dev(sizeof(int64_t) * R * R * 8);
  m.arena_base = dev(sizeof(int64_t) * 2 * (R + 1));
  m.descriptors = dev((size_t)ndesc * 64);
  m.desc_capacity = ndesc;
  m.num_descriptors = dev(sizeof(int64_t));
  expect(ep_dispatch(&p, &d.l, d_x, d_topk, d_w, NULL, &m, ws, ws_bytes, NULL) == EP_OK,
         "messages: ep_dispatch");
  uint8_t* recv_arena = dev((size_t)recv_bytes);
  int32_t* err = dev(sizeof(int32_t));
  HIP_OK(hipMemset(err, 0, sizeof(int32_t)));
  expect(ep_messages_execute(&p, &m, recv_arena, recv_bytes, 0, err, NULL) == EP_OK,
         "messages: ep_messages_execute");
  ep_recv out;
  memset(&out, 0, sizeof out);
  out.x = dev((size_t)E * RT * H);
  out.scales = dev(sizeof(float) * (size_t)E * G * RT);
  out.capacity = (int64_t)E * RT;
  int32_t* d_count = dev(sizeof(int32_t) * E);
  int32_t* d_src = dev(sizeof(int32_t) * E * RT);
  expect(ep_messages_unpack(&p, &m, recv_arena, recv_bytes, d.l.num_tokens_per_expert, &out,
                            d_count, d_src, 0, err, NULL) == EP_OK,
         "messages: ep_messages_unpack");
  HIP_OK(hipDeviceSynchronize());

  int32_t* send_pos;
  check_layout(&d, &op, topk, 0, &send_pos, "messages");
  /* the oracle's packer, delivery and receiver */
  uint8_t* o_send = calloc((size_t)send_bytes, 1);
  int64_t* o_table = malloc(sizeof(int64_t) * R * R * 8);
  int64_t* o_base = malloc(sizeof(int64_t) * 2 * (R + 1));
  uint8_t* o_desc = calloc((size_t)ndesc, 64);
  int64_t o_nd = 0;
  expect(orc_messages(&op, x, topk, w, o_send, send_bytes, o_table, o_base, o_desc, ndesc,
                      &o_nd) == 0, "messages: oracle packer");
  int64_t* g_table = host_of(m.table, sizeof(int64_t) * R * R * 8);
  int64_t* g_base = host_of(m.arena_base, sizeof(int64_t) * 2 * (R + 1));
  int64_t* g_nd = host_of(m.num_descriptors, sizeof(int64_t));
  uint8_t* g_desc = host_of(m.descriptors, (size_t)ndesc * 64);
  uint8_t* g_send = host_of(m.send_arena, (size_t)send_bytes);
  expect(memcmp(g_table, o_table, sizeof(int64_t) * R * R * 8) == 0, "messages: table");
  expect(memcmp(g_base, o_base, sizeof(int64_t) * 2 * (R + 1)) == 0, "messages: arena bases");
  expect(*g_nd == o_nd && o_nd == ndesc, "messages: descriptor count");
  expect(memcmp(g_desc, o_desc, (size_t)o_nd * 64) == 0, "messages: descriptors");
  int ok = 1;
  for (int i = 0; i < R * R; ++i)
    if (o_table[i * 8 + 2] > 0)
      ok &= memcmp(g_send + o_table[i * 8], o_send + o_table[i * 8], (size_t)o_table[i * 8 + 2]) == 0;
  expect(ok, "messages: message regions");
  uint8_t* o_recv = calloc((size_t)recv_bytes, 1);
  expect(orc_messages_execute(&op, o_send, send_bytes, o_base, o_desc, o_nd, o_recv, recv_bytes)
             == 0, "messages: oracle delivery");
  uint8_t* g_recv = host_of(recv_arena, (size_t)recv_bytes);
  ok = 1;
  for (int i = 0; i < R * R; ++i)
    if (o_table[i * 8 + 2] > 0)
      ok &= memcmp(g_recv + o_table[i * 8 + 1], o_recv + o_table[i * 8 + 1],
                   (size_t)o_table[i * 8 + 2]) == 0;
  expect(ok, "messages: delivered regions");
  int32_t* cnt_expert = host_of(d.l.num_tokens_per_expert, sizeof(int32_t) * R * E);
  uint8_t* o_codes = calloc((size_t)E * RT * H, 1);
  float* o_scales = calloc((size_t)E * G * RT, sizeof(float));
  int32_t* o_count = malloc(sizeof(int32_t) * E);
  int32_t* o_src = malloc(sizeof(int32_t) * E * RT);
  for (int i = 0; i < E * RT; ++i) o_src[i] = -1;
  expect(orc_messages_unpack(&op, o_recv, recv_bytes, o_table, cnt_expert, o_codes, o_scales,
                             o_count, o_src) == 0, "messages: oracle receiver");
  int32_t* g_err = host_of(err, sizeof(int32_t));
  expect(*g_err == 0, "messages: delivery and receiver error word");
  expect(same_i32(d_count, o_count, E), "messages: receive counts");
  uint8_t* g_codes = host_of(out.x, (size_t)E * RT * H);
  float* g_scales = host_of(out.scales, sizeof(float) * (size_t)E * G * RT);
  int32_t* g_src = host_of(d_src, sizeof(int32_t) * E * RT);
  int ok_rows = 1, ok_sc = 1, ok_src = 1, filled = 0;
  for (int r = 0; r < E * RT; ++r) {
    if (o_src[r] < 0) continue;
    ++filled;
    ok_src &= g_src[r] == o_src[r];
    ok_rows &= memcmp(g_codes + (int64_t)r * H, o_codes + (int64_t)r * H, H) == 0;
    const int e = r / RT, pos = r % RT;
    for (int g = 0; g < G; ++g) {
      const int64_t si = ((int64_t)e * G + g) * RT + pos;
      ok_sc &= memcmp(&g_scales[si], &o_scales[si], sizeof(float)) == 0;
    }
  }
  expect(filled > 0, "messages: rows were unpacked");
  expect(ok_src, "messages: unpacked source indices");
  expect(ok_rows, "messages: unpacked codes");
  expect(ok_sc, "messages: unpacked scales");
  free(g_codes); free(g_scales); free(g_src); free(g_err); free(o_codes); free(o_scales);
  free(o_count); free(o_src); free(cnt_expert); free(g_recv); free(o_recv); free(g_send);
  free(g_desc); free(g_nd); free(g_base); free(g_table); free(o_desc); free(o_base);
  free(o_table); free(o_send); free(counts); free(send_pos); free(topk); free(x); free(w);
}

int main(void) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
    printf("no GPU\n");
    return 3;
  }
  normal_bf16();
  ll_fp8_fused();
  messages_path();
  if (failures) {
    printf("%d checks failed\n", failures);
    return 1;
  }
  printf("gpu roundtrip ok\n");
  return 0;
}
