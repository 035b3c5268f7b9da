/*
 * ep.h -- C ABI of libep: MoE token dispatch / combine on simulated ranks
 * that live as partitions of one MI355X's HBM (gfx950).
 *
 * The method (web pages it is described on):
 *   "DeepEP" deep dive (llm-infra-atlas, moe/06_deepep)
 *     sec. 1.1  normal mode: contiguous per-expert receive layout, FP8
 *               dispatch with bf16 combine, receive size known only after
 *               the count exchange (or a worst-case capacity);
 *     sec. 1.2  low-latency mode: packed masked layout
 *               [local experts][max tokens per rank * ranks][hidden] plus a
 *               per-expert receive count; FP8 scales fp32 or power of two
 *               (UE8M0), column-major;
 *     sec. 2.1  get_dispatch_layout counts (tokens per rank, per expert,
 *               is_token_in_rank) and notify_dispatch (prefix sum over
 *               source ranks = rank_prefix_matrix; per-expert receive
 *               counts rounded up to expert_alignment);
 *     sec. 2.3  rank_prefix_matrix[i][j] = tokens sent to rank j by ranks
 *               <= i; the handle (send_head, recv_src_idx) lets combine walk
 *               dispatch's addresses backwards;
 *     sec. 3.2  destination rank of expert e = e / num_local_experts;
 *     sec. 4.3  psum of per-expert receive counts = segment offsets.
 *   "Eaas_server" notes: 16-byte aligned per-destination message with a
 *     header, then payload, then a completion flag; only loaded
 *     destinations get one; three puts (payload, header, flag).
 *   "ibgda_device.cuh" notes, sec. 1 and 3: a write is cut so that no
 *     piece spans two memory regions; a write work-queue entry is a
 *     control, a remote-address and a data segment, big-endian fields.
 *   "GPU-Initiated Communication: Dissecting Down to the Bone", WQE
 *     anatomy: 16-byte segments in 64-byte basic blocks.
 *
 * Conventions for every entry point:
 *  - All array arguments are DEVICE pointers owned by the caller.  Row
 *    buffers (x, receive rows, y, out, send arena, descriptors) must be
 *    16-byte aligned, other arrays naturally aligned; arrays with one entry
 *    per token may be NULL when R*T == 0.  Struct arguments themselves are host memory,
 *    read during the call only.  The library allocates nothing, keeps no
 *    state between calls and is reentrant; calls that write the same
 *    buffers must not overlap.  (The one exception is
 *    ep_dispatch_fused_noalloc, below: its scratch is a fixed array inside
 *    the library, shared by every call on a GPU, whose device address is
 *    looked up once per GPU and kept.)
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *    enqueued asynchronously on it; nothing is synchronised.
 *  - Return: EP_OK (0) or a negative EP_ERR_* code.  Argument errors are
 *    detected on the host before anything is enqueued.  Errors that depend
 *    on device data (an expert id out of range, a capacity overflow) set
 *    bits in the caller's device error word (EP_DEVERR_*) and the offending
 *    write is skipped; read the word after synchronising.
 *  - Sizes: R = num_ranks, T = num_tokens (per rank), H = hidden,
 *    E = num_experts, K = num_topk, L = E / R, G = H / 128.
 *    Limits: 1 <= R <= 256, R <= E <= 2048, E % R == 0, 1 <= K <= 64,
 *    T >= 0, 8 <= H <= 32768, H % 8 == 0 (bf16 rows are whole 16-byte
 *    vectors), H % 128 == 0 when quantised, R*T*K < 2^31, receive rows
 *    < 2^31.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* receive layouts */
#define EP_MODE_NORMAL 0      /* contiguous, expert-major per destination rank */
#define EP_MODE_LOW_LATENCY 1 /* packed masked: E blocks of R*T rows           */
#define EP_MODE_MESSAGES 2    /* one packed message per (source, destination)  */
#define EP_MODE_RANK_MAJOR 3  /* one row per (token, destination rank), in (source, token)
                                 order per destination: the V1 receive buffer       */

/* payload formats */
#define EP_QUANT_NONE 0      /* bf16 rows                                      */
#define EP_QUANT_FP8_F32 1   /* e4m3 codes + fp32 scale (amax / 448) per 128 channels */
#define EP_QUANT_FP8_UE8M0 2 /* e4m3 codes + power-of-two scale stored as a biased 8-bit exponent */

/* host-side status codes */
#define EP_OK 0
#define EP_ERR_NULL (-1)        /* a required pointer is NULL              */
#define EP_ERR_ALIGN (-2)       /* a pointer is not suitably aligned       */
#define EP_ERR_SHAPE (-3)       /* inconsistent or out-of-limit sizes      */
#define EP_ERR_MODE (-4)        /* unknown mode / quant, or a combination not offered */
#define EP_ERR_WORKSPACE (-5)   /* workspace smaller than ep_workspace_bytes */
#define EP_ERR_CAPACITY (-6)    /* a capacity that is too small on its face */
#define EP_ERR_HIP (-7)         /* the HIP runtime reported a launch error */
#define EP_ERR_SCRATCH (-8)     /* ep_dispatch_fused_noalloc: the problem needs more scratch
                                   than EP_NOALLOC_SCRATCH_BYTES */

/* size of the library's fixed scratch array (ep_dispatch_fused_noalloc) */
#define EP_NOALLOC_SCRATCH_BYTES (64u << 20)

/* device error word bits */
#define EP_DEVERR_TOPK_RANGE 1  /* a topk_idx entry outside [-1, E): entry skipped */
#define EP_DEVERR_LL_OVERFLOW 2 /* low-latency position >= R*T (duplicate ids): skipped */
#define EP_DEVERR_CAPACITY 4    /* a row or byte offset past the caller's capacity: skipped */
#define EP_DEVERR_MESSAGE 8     /* a descriptor names a rank outside [0, R), or a received
                                   message's header or completion flag does not match: skipped */

typedef struct ep_problem {
  int32_t num_ranks;        /* R                                           */
  int32_t num_tokens;       /* T, tokens per source rank                   */
  int32_t hidden;           /* H                                           */
  int32_t num_experts;      /* E                                           */
  int32_t num_topk;         /* K                                           */
  int32_t expert_alignment; /* >= 1; normal mode rounds each expert's rows up to it */
  int32_t mode;             /* EP_MODE_*                                   */
  int32_t quant;            /* EP_QUANT_*                                  */
  int64_t region_bytes;     /* messages: descriptor split granularity (> 0, multiple of 16) */
  uint32_t epoch;           /* messages: value of the completion flag      */
  int32_t reserved;         /* must be 0                                   */
} ep_problem;

/* Outputs of ep_get_layout (the dispatch "handle").  Rows are receive-
 * buffer rows: normal mode packs the R destination partitions back to
 * back (partition d = rows [row_base[d], row_base[d+1])), each holding its
 * L experts' segments in order, each segment ordered by (source rank,
 * token, k); low-latency mode gives expert e the rows [e*R*T, (e+1)*R*T).
 * A row index is int32. */
typedef struct ep_layout {
  int32_t* num_tokens_per_rank;    /* [R][R]  [s][d]: tokens of s with >= 1 expert on d   */
  int32_t* num_tokens_per_expert;  /* [R][E]  [s][e]: (token, k) entries of s routed to e  */
  uint8_t* is_token_in_rank;       /* [R][T][R] 0/1 (any alignment)                        */
  int32_t* rank_prefix_matrix;     /* [R][R]  [i][j] = sum_{s <= i} num_tokens_per_rank[s][j] */
  int32_t* recv_tokens_per_expert; /* [E]     entries routed to e (low-latency recv_count) */
  int32_t* expert_start;           /* [E]     first row of e's segment                      */
  int32_t* rows_per_rank;          /* [R]     rows of partition d (aligned)                 */
  int32_t* row_base;               /* [R+1]   first row of partition d; [R] = total rows    */
  int32_t* send_pos;               /* [R][T][K] row of each entry, -1 if none (normal / LL) */
  int32_t* send_head;              /* [R][T][R] index of token t in the (s, d) stream in token
                                      order, -1 if not sent; may be NULL except in messages mode */
  int32_t* recv_src_idx;           /* [recv_capacity] s*T+t of each filled row; normal mode
                                      writes -1 in alignment padding rows; may be NULL      */
  int64_t recv_capacity;           /* rows available in recv_src_idx (and the receive buffer) */
  int32_t* err;                    /* [1] device error word; ep_get_layout resets it to 0  */
} ep_layout;

/* Receive side of normal / low-latency dispatch. */
typedef struct ep_recv {
  void* x;          /* [capacity][H]: bf16 (EP_QUANT_NONE) or e4m3 codes (1 byte)          */
  void* scales;     /* FP8 only, column-major: normal [G][capacity];
                       low-latency [E][G][R*T].  fp32 (FP8_F32) or uint8 exponents
                       (FP8_UE8M0: scale = 2^(byte - 127)); 4-byte aligned               */
  int64_t capacity; /* rows of x; low-latency needs >= E*R*T                              */
  int32_t* topk_idx;    /* rank-major only, may be NULL: [capacity][K], the row's token's
                           experts on this rank as local ids (e - d*L), else -1          */
  float* topk_weights;  /* rank-major only, may be NULL: [capacity][K], their weights,
                           else 0                                                       */
} ep_recv;

/* Send side of message mode. */
typedef struct ep_messages {
  uint8_t* send_arena;     /* [send_capacity] bytes: all ranks' send arenas, back to back  */
  int64_t send_capacity;
  int64_t* table;          /* [R][R][8] per (s, d): send offset, recv offset, region bytes,
                              token count n, body bytes, first descriptor, descriptor count, 0
                              (offsets -1 and sizes 0 when n == 0)                         */
  int64_t* arena_base;     /* [2][R+1]: send-arena bases, then receive-arena bases         */
  uint8_t* descriptors;    /* [desc_capacity][64] write descriptors                        */
  int64_t desc_capacity;
  int64_t* num_descriptors; /* [1] descriptors produced (may exceed the capacity)          */
} ep_messages;

/* Bytes of scratch device memory ep_get_layout / ep_dispatch need for this
 * problem (0 on invalid input).  Any 256-byte aligned buffer of at least
 * this size; its contents need not be initialised and are dead after the
 * stream reaches the end of the call. */
size_t ep_workspace_bytes(const ep_problem* p);

/* Worst-case receive rows for normal mode (every entry valid, every
 * expert padded by expert_alignment - 1), E*R*T for low-latency,
 * R*T*min(K, R) for rank-major (every token on K distinct ranks). */
int64_t ep_max_recv_rows(const ep_problem* p);

/* Buffer sizes of message mode ("Eaas_server" notes: one region per loaded
 * (source, destination) pair -- header, 16-byte padded body, flag -- packed
 * into per-rank arenas that start on region boundaries; "ibgda_device.cuh"
 * notes, sec. 1: every put is cut where it would cross a region boundary of
 * either arena, one descriptor per piece).  Host only: launches nothing and
 * reads no device memory.
 *   counts: host [R][R] int32, tokens of source s sent to rank d (the
 *           num_tokens_per_rank of ep_get_layout, read back), or NULL for
 *           bounds that hold for every routing (every token sent to every
 *           rank: the host-sizing alternative to the read-back, "DeepEP"
 *           sec. 2.1).
 *   *send_bytes:  bytes of all send arenas together (arena_base[0][R]);
 *   *recv_bytes:  bytes of all receive arenas together (arena_base[1][R]);
 *   *descriptors: descriptors ep_dispatch writes (*num_descriptors).
 * Exact with counts, upper bounds without.  Output pointers may be NULL.
 * Returns EP_ERR_MODE unless p->mode is EP_MODE_MESSAGES, EP_ERR_SHAPE for
 * an invalid problem or a count outside [0, T]; outputs are then untouched. */
int ep_messages_capacity(const ep_problem* p, const int32_t* counts, int64_t* send_bytes,
                         int64_t* recv_bytes, int64_t* descriptors);

/* Routing layout ("DeepEP" sec. 2.1, 2.3, 3.2, 4.3): histograms per rank
 * and per expert, is_token_in_rank, the rank prefix matrix, per-expert
 * receive counts and segment starts, and the slot of every routed entry
 * (send_pos) and of every sent token within its destination stream
 * (send_head).  topk_idx: [R][T][K] int32, -1 = no expert.  Slot order is
 * deterministic: within an expert's segment by (source rank, token, k).
 * Rank-major mode ("DeepEP" sec. 2.3, the V1 receive buffer and its
 * address book): partition d holds one row per token with an expert on d,
 * source s's tokens from row row_base[d] + rank_prefix_matrix[s][d] -
 * num_tokens_per_rank[s][d] on, in (s, d) stream order (send_head);
 * send_pos[s][t][k] is the token's row on the rank of expert k;
 * rows_per_rank / row_base count these rows; expert_start[e] is the first
 * row of e's rank; recv_src_idx has one entry per row.
 * Resets *err to 0, then may set EP_DEVERR_TOPK_RANGE, _LL_OVERFLOW,
 * _CAPACITY (recv_src_idx too small). */
int ep_get_layout(const ep_problem* p, const int32_t* topk_idx, const ep_layout* out,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Dispatch.
 * normal / low-latency ("DeepEP" sec. 1.1, 1.2): every routed entry
 *   (s, t, k) writes token x[s][t] to row send_pos[s][t][k] of recv->x,
 *   as bf16 or as e4m3 codes with one scale per 128-channel group (the
 *   group's largest magnitude maps to 448; UE8M0 rounds the scale up to a
 *   power of two).  Uses layout->send_pos; `msgs` may be NULL.
 * messages ("Eaas_server" notes; "ibgda_device.cuh" sec. 1, 3): for every
 *   (s, d) with num_tokens_per_rank[s][d] > 0, one region in s's send arena:
 *   16-byte header {s, d, n, body bytes} (u32 LE), body = codes n*H |
 *   scales n*G | weights n*K f32 | expert ids n*K i32 | source token n i32,
 *   each section zero-padded to 16 bytes, then a 16-byte completion flag
 *   {epoch, 0, 0, 0}, written after the rest of the region.  Then the
 *   64-byte write descriptors of the payload, header and flag puts, cut at
 *   every region_bytes boundary of either arena.  Uses layout->send_head,
 *   num_tokens_per_rank; `recv` may be NULL.
 * rank-major: each token is written once per destination rank, to row
 *   send_pos[s][t][k] (the first k on that rank); when recv->topk_idx /
 *   topk_weights are given, the row's top-k as that rank sees it (local
 *   expert ids or -1, weights or 0); FP8 scales column-major [G][capacity].
 * x: [R][T][H] bf16.  topk_idx / topk_weights ([R][T][K]) are read in
 * messages mode, and in rank-major mode for the row metadata (may be NULL
 * otherwise). */
int ep_dispatch(const ep_problem* p, const ep_layout* layout, const uint16_t* x,
                const int32_t* topk_idx, const float* topk_weights, const ep_recv* recv,
                const ep_messages* msgs, void* workspace, size_t workspace_bytes,
                void* stream);

/* Layout and dispatch in one call ("DeepEP" sec. 4.6: V2 folds the
 * layout's notify step into the dispatch kernel): the outputs of
 * ep_get_layout and of ep_dispatch, with the last step of the layout (each
 * entry's row, send_pos, recv_src_idx, send_head, the segment starts) taken
 * by the dispatch kernel itself, so the call issues one launch fewer than
 * ep_get_layout followed by ep_dispatch (as many for problems small enough
 * for the one-launch layout, which it then runs before the dispatch).
 * Arguments as for ep_get_layout and ep_dispatch; normal and low-latency
 * modes (EP_ERR_MODE otherwise).  The workspace is used by both steps. */
int ep_dispatch_fused(const ep_problem* p, const int32_t* topk_idx, const ep_layout* layout,
                      const uint16_t* x, const ep_recv* recv, void* workspace,
                      size_t workspace_bytes, void* stream);

/* ep_dispatch_fused without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops and harnesses
 * that forbid allocation.  Calls no hipMalloc / hipFree and no allocating
 * routine.  Its scratch memory is a fixed array of EP_NOALLOC_SCRATCH_BYTES
 * (64 MiB) inside the library: each GPU the library is loaded on holds its
 * own copy until the process ends.  A problem whose ep_workspace_bytes
 * exceeds that size returns EP_ERR_SCRATCH before anything is enqueued.
 * Every call on one GPU uses that GPU's one array, which keeps the last
 * call's contents (nothing in it needs to start at zero): calls whose work
 * may overlap on one GPU -- streams with no ordering between them, or host
 * threads enqueueing concurrently onto different streams -- race and give
 * wrong results; calls ordered on one stream are safe.  The first call on
 * a GPU looks up the array's device address (hipGetSymbolAddress with that
 * GPU current, the caller's current device restored); `stream`'s device
 * decides which GPU.  Arguments and results otherwise as ep_dispatch_fused. */
int ep_dispatch_fused_noalloc(const ep_problem* p, const int32_t* topk_idx,
                              const ep_layout* layout, const uint16_t* x, const ep_recv* recv,
                              void* stream);

/* Combine ("DeepEP" sec. 2.3: the handle walked backwards): out[s][t] =
 * bf16( sum_k topk_weights[s][t][k] * y[send_pos[s][t][k]] ), accumulated in
 * fp32 in k order, rounded to nearest-even; tokens with no routed entry
 * get 0.  y: expert outputs, bf16, in the receive layout ([y_rows][H]).
 * Normal / low-latency modes.  Rank-major mode: out[s][t] = bf16( sum of
 * y over the token's distinct rows (one per destination rank), in order of
 * first k ), unweighted -- the expert stage on each rank has applied the
 * weights of its experts; topk_weights may be NULL. */
int ep_combine(const ep_problem* p, const ep_layout* layout, const uint16_t* y,
               int64_t y_rows, const float* topk_weights, uint16_t* out, void* stream);

/* Loopback delivery of message mode's descriptors ("ibgda_device.cuh" notes,
 * sec. 1; "GPU-Initiated Communication: Dissecting Down to the Bone", WQE
 * anatomy and Ordering).  Descriptor i (i < min(*m->num_descriptors,
 * m->desc_capacity)) copies its length of bytes from byte laddr of rank
 * (lkey >> 16)'s send arena to byte raddr of rank (rkey >> 16)'s receive
 * arena, the arena bases taken from m->arena_base (receive arena of rank d
 * = recv_arena[arena_base[1][d] ...]).  The last descriptor of every
 * message (m->table: first index + count - 1) is its completion flag.
 * recv_arena: [recv_capacity] bytes, 16-byte aligned (arena_base[1][R]
 * bytes suffice).  Errors are OR-ed into *err (not reset):
 * EP_DEVERR_MESSAGE for a rank outside [0, R), EP_DEVERR_CAPACITY for a put
 * past either rank's arena or either buffer; such a put is skipped.
 * p->mode must be EP_MODE_MESSAGES.
 * publish_batch: when the flags go out (same page, Doorbell Batching and
 * Sharing a QP; "ibgda_device.cuh" notes, sec. 4: a doorbell after every
 * few requests).  0: every flag in a second launch, after every payload and
 * header of the call.  B >= 1: one launch; each workgroup takes a run of
 * messages in reservation order (the table's (source, destination) order)
 * and, after every B of them and after its last, releases their payloads
 * and headers with a device-scope fence and then writes their flags; a
 * workgroup's batches are announced in order and no workgroup waits for
 * another.  The delivered bytes are the same for every value; < 0 returns
 * EP_ERR_SHAPE. */
int ep_messages_execute(const ep_problem* p, const ep_messages* m, uint8_t* recv_arena,
                        int64_t recv_capacity, int32_t publish_batch, int32_t* err,
                        void* stream);

/* Most polls ep_messages_unpack makes of one flag (spin_limit). */
#define EP_MAX_SPIN (1 << 24)

/* Receiver ("Eaas_server" notes; "DeepEP" sec. 1.2 and 2.1).  For every
 * (s, d) with a message (m->table[s][d]: token count n > 0), checks the
 * header {s, d, n, body bytes} and the completion flag {epoch, 0, 0, 0} at
 * the message's receive offset (a mismatch sets EP_DEVERR_MESSAGE and the
 * message is skipped; nothing waits), then unpacks it into the low-latency
 * layout, exactly as low-latency dispatch of the same routing stores it:
 * the message's entry (token j, k) with expert e of rank d takes slot
 *   pos = sum_{s' < s} num_tokens_per_expert[s'][e]
 *         + (earlier entries of the message with expert e),
 * row e*R*T + pos of out->x (codes or bf16 row), scales at
 * [(e*G + g)*R*T + pos], recv_src_idx[row] = s*T + t (t read from the
 * message).  recv_count[e] = sum_s num_tokens_per_expert[s][e].  Rows not
 * filled are left as they were.  pos >= R*T sets EP_DEVERR_LL_OVERFLOW; a
 * message past recv_capacity sets EP_DEVERR_CAPACITY; errors are OR-ed into
 * *err.  out->capacity >= E*R*T; recv_src_idx: [E*R*T]; recv_count: [E];
 * num_tokens_per_expert: [R][E] (ep_get_layout's).  m->arena_base, when
 * not NULL, only chooses the block order from the receive loads (results
 * are the same either way).  p->mode must be EP_MODE_MESSAGES (p->quant,
 * p->epoch describe the messages).
 * spin_limit in [0, EP_MAX_SPIN]: 0 checks each flag once (the delivery
 * must have completed, e.g. ordered before on the same stream); n > 0
 * first polls the flag with acquire loads ("GPU-Initiated Communication:
 * Dissecting Down to the Bone", Ordering: the flag store is the last to
 * become visible) up to n times, sleeping about 0.2 us between polls, and
 * then checks; a flag still missing sets EP_DEVERR_MESSAGE.  The wait is
 * bounded, so a delivery that never comes ends the call with the error
 * rather than a hang. */
int ep_messages_unpack(const ep_problem* p, const ep_messages* m, const uint8_t* recv_arena,
                       int64_t recv_capacity, const int32_t* num_tokens_per_expert,
                       const ep_recv* out, int32_t* recv_count, int32_t* recv_src_idx,
                       int32_t spin_limit, int32_t* err, void* stream);

/* Static text for a status code. */
const char* ep_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* EP_H */
