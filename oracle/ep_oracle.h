/*
 * ep_oracle.h -- plain single-threaded CPU oracle for MoE token dispatch /
 * combine on simulated ranks.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes,
 * links or calls this code; only the tests, the smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no source, header, table or
 * helper with the HIP implementation.
 *
 * Sources (the web pages this method is described on):
 *   [DEEP]  "DeepEP" deep dive (llm-infra-atlas, moe/06_deepep):
 *           sec. 1.1 / 1.2 (normal vs. low-latency modes, packed masked
 *           layout, FP8 dispatch with column-major scales),
 *           sec. 2.1 (notify_dispatch: per-rank / per-expert counts, the
 *           rank prefix matrix, receive counts rounded to expert_alignment),
 *           sec. 2.3 (prefix matrix as the receiver's address book, handle),
 *           sec. 3.2 (dst_rank = expert / num_local_experts),
 *           sec. 4.3 (psum of per-expert receive counts = segment offsets).
 *   [EAAS]  "Eaas_server" notes: packing kernel (16-byte aligned payload,
 *           header first) and the three puts per server (payload, header,
 *           completion flag); only servers with load get a message.
 *   [IBGDA] "ibgda_device.cuh" notes, sec. 1 (chunking so that one RDMA
 *           write never spans two memory regions) and sec. 3 (WQE control /
 *           remote-address / data segments, big-endian fields).
 *   [GIC]   "GPU-Initiated Communication: Dissecting Down to the Bone",
 *           WQE anatomy (16-byte segments in 64-byte basic blocks) and
 *           Ordering (payload visible before the announcing store).
 *
 * Where the pages leave a step open, the reading taken is stated at the
 * function that takes it.  Parity pins for every function live in the
 * CPU test-suite; the message layout and descriptor byte format are this
 * library's own specification (the pages give no field values) and are
 * pinned only by structural invariants and a brute-force re-derivation.
 *
 * Precision: integers are exact; FP8 quantisation is done in IEEE fp32
 * (the decision it feeds is an integer code, so both sides take it in
 * fp32); the combine sum is accumulated in fp64 and rounded once to bf16.
 */
#ifndef EP_ORACLE_H
#define EP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* receive-layout modes */
#define ORC_MODE_NORMAL 0 /* contiguous, expert-major per destination rank   */
#define ORC_MODE_LL 1     /* packed masked [E][R*T] rows                       */
#define ORC_MODE_MSG 2    /* one message per (source, destination) rank pair   */
#define ORC_MODE_RANK 3   /* rank-major: one row per (token, destination rank) */

/* payload quantisation */
#define ORC_Q_NONE 0      /* bf16 rows                                        */
#define ORC_Q_FP8_F32 1   /* e4m3 codes, fp32 scale = amax / 448              */
#define ORC_Q_FP8_UE8M0 2 /* e4m3 codes, power-of-two scale stored as 8-bit exponent */

/* error bits (returned, OR-ed together) */
#define ORC_ERR_TOPK_RANGE 1  /* an index outside [-1, E)                    */
#define ORC_ERR_LL_OVERFLOW 2 /* low-latency position >= R*T                  */
#define ORC_ERR_CAPACITY 4    /* output buffer smaller than the data          */
#define ORC_ERR_MESSAGE 8     /* a descriptor or received message is malformed */

typedef struct {
  int32_t R;        /* simulated ranks                                     */
  int32_t T;        /* tokens per rank                                     */
  int32_t H;        /* hidden size (channels)                              */
  int32_t E;        /* experts; E % R == 0, L = E / R per rank              */
  int32_t K;        /* top-k                                               */
  int32_t align;    /* expert_alignment (>= 1), normal mode only           */
  int32_t mode;     /* ORC_MODE_*                                          */
  int32_t quant;    /* ORC_Q_*                                             */
  int64_t region_bytes; /* message mode: descriptor split granularity      */
  uint32_t epoch;   /* message mode: completion-flag value                 */
  int32_t pad_;
} orc_problem;

/* ---- scalar codecs -------------------------------------------------- */
uint8_t orc_e4m3_encode(float v);
float orc_e4m3_decode(uint8_t code);
uint16_t orc_bf16_from_double(double v);
double orc_bf16_to_double(uint16_t b);
float orc_fp8_scale_f32(float amax);       /* amax floor, then amax / 448   */
uint8_t orc_fp8_scale_ue8m0(float amax);   /* biased exponent of the scale  */
/* bulk forms, for exhaustive tests */
void orc_e4m3_encode_array(const float* v, uint8_t* out, int64_t n);

/* ---- layout (counts, prefix matrix, slots) -------------------------- */
/* Total receive rows of the layout (normal: aligned sum; LL: E*R*T);
 * message mode: 0. */
int64_t orc_recv_rows(const orc_problem* p, const int32_t* topk);

int orc_layout(const orc_problem* p, const int32_t* topk /*[R][T][K]*/,
               int32_t* cnt_rank /*[R][R]*/, int32_t* cnt_expert /*[R][E]*/,
               uint8_t* in_rank /*[R][T][R]*/, int32_t* rank_prefix /*[R][R]*/,
               int32_t* recv_per_expert /*[E]*/, int32_t* expert_start /*[E]*/,
               int32_t* rows /*[R]*/, int32_t* row_base /*[R+1]*/,
               int32_t* send_pos /*[R][T][K]*/, int32_t* send_head /*[R][T][R]*/,
               int32_t* recv_src_idx /*[cap]*/, int64_t recv_cap);

/* ---- rank-major receive metadata ------------------------------------ */
/* For every row of the rank-major layout (mode ORC_MODE_RANK), the token's
 * top-k as the destination rank d sees it: recv_topk_idx[row][k] = e - d*L
 * when expert e = topk[s][t][k] lives on d, else -1; recv_topk_weights
 * [row][k] = w[s][t][k] when it does, else 0.                             */
int orc_rank_topk(const orc_problem* p, const int32_t* topk, const float* w,
                  const int32_t* send_pos, int64_t cap, int32_t* recv_topk_idx /*[cap][K]*/,
                  float* recv_topk_weights /*[cap][K]*/);

/* ---- dispatch (normal / LL) ----------------------------------------- */
/* recv: bf16 rows [cap][H] (quant NONE) or e4m3 codes [cap][H] (FP8).
 * scales: FP8_F32 -> float, FP8_UE8M0 -> uint8; column-major:
 *   normal: scales[g * cap + row]
 *   LL:     scales[(e * G + g) * (R*T) + pos],  row = e*(R*T) + pos        */
int orc_dispatch(const orc_problem* p, const uint16_t* x /*[R][T][H]*/,
                 const int32_t* topk, const int32_t* send_pos,
                 void* recv, void* scales, int64_t cap);

/* identity expert on an FP8 receive buffer: y = bf16(decode(code) * scale) */
void orc_dequant_rows(const orc_problem* p, const uint8_t* codes, const void* scales,
                      int64_t cap, const int32_t* row_list, int64_t nrows,
                      uint16_t* y /*[nrows][H]*/);

/* ---- combine -------------------------------------------------------- */
/* out[s][t][:] = bf16( sum_k w[s][t][k] * y[send_pos[s][t][k]][:] ), fp64 sum.
 * token_list (may be NULL = all tokens) restricts the tokens computed;
 * out then holds only those rows, in list order. */
int orc_combine(const orc_problem* p, const uint16_t* y, int64_t y_rows,
                const float* w /*[R][T][K]*/, const int32_t* send_pos,
                const int64_t* token_list, int64_t ntok, uint16_t* out);

/* ---- messages + descriptors ----------------------------------------- */
/* Per-(s,d) table, 8 int64 per entry:
 *   [0] send offset of the message region (global send arena, -1 if none)
 *   [1] recv offset of the message region (global recv arena, -1 if none)
 *   [2] region bytes (16 + body + 16), 0 if none
 *   [3] token count n
 *   [4] body bytes
 *   [5] first descriptor index
 *   [6] descriptor count
 *   [7] 0
 * arena_base: [2][R+1]: send bases then recv bases (region-aligned).     */
int64_t orc_msg_body_bytes(const orc_problem* p, int64_t n, int64_t sec_off[6]);
int orc_messages(const orc_problem* p, const uint16_t* x, const int32_t* topk,
                 const float* w, uint8_t* send_arena, int64_t send_cap,
                 int64_t* table /*[R][R][8]*/, int64_t* arena_base /*[2][R+1]*/,
                 uint8_t* desc /*[desc_cap][64]*/, int64_t desc_cap,
                 int64_t* num_desc);

/* ---- message delivery (loopback) and receive ------------------------- */
/* Executes the write descriptors in order: each copies its length of bytes
 * from byte laddr of source rank (lkey >> 16)'s send arena to byte raddr of
 * destination rank (rkey >> 16)'s receive arena (arena bases from
 * arena_base).  A descriptor naming a rank outside [0, R) sets
 * ORC_ERR_MESSAGE; one reaching past either rank's arena or the buffers
 * sets ORC_ERR_CAPACITY; neither is executed.                              */
int orc_messages_execute(const orc_problem* p, const uint8_t* send_arena, int64_t send_cap,
                         const int64_t* arena_base, const uint8_t* desc, int64_t num_desc,
                         uint8_t* recv_arena, int64_t recv_cap);

/* Receiver: for every destination d and source s with a message (table
 * [s][d]), checks the header {s, d, n, body} and the completion flag
 * {epoch, 0, 0, 0} in the receive arena (mismatch: ORC_ERR_MESSAGE, the
 * message is skipped) and unpacks its tokens into the low-latency layout:
 * the entry (token j, k) of the message with expert e on d gets slot
 *   pos = sum_{s' < s} cnt_expert[s'][e] + (entries of the message before it
 *         with expert e),
 * i.e. (source, token, k) order, row = e*(R*T) + pos; codes/rows and scales
 * are stored as low-latency dispatch stores them, recv_src_idx[row] =
 * s*T + t (t from the message), recv_count[e] = sum_s cnt_expert[s][e].
 * pos >= R*T sets ORC_ERR_LL_OVERFLOW (not stored).                         */
int orc_messages_unpack(const orc_problem* p, const uint8_t* recv_arena, int64_t recv_cap,
                        const int64_t* table /*[R][R][8]*/, const int32_t* cnt_expert /*[R][E]*/,
                        void* recv /*[E*R*T][H] bf16 or codes*/, void* scales,
                        int32_t* recv_count /*[E]*/, int32_t* recv_src_idx /*[E*R*T]*/);

#ifdef __cplusplus
}
#endif
#endif
