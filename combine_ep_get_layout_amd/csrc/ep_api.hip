// C ABI of libep: argument validation, workspace carve-up and launches.
// Declarations, semantics and the passages each call follows: include/ep.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/ep.h"
#include "ep_internal.hpp"
#include "msg_format.hpp"

namespace ep {
size_t message_ws_bytes(int R);
}

using ep::Geometry;

namespace {

#ifndef EP_LAYOUT_TARGET_CHUNKS
#define EP_LAYOUT_TARGET_CHUNKS 1024
#endif
#ifndef EP_DIRECT_MAX_ENTRIES
#define EP_DIRECT_MAX_ENTRIES 6144
#endif
constexpr int64_t kDirectMaxEntries = EP_DIRECT_MAX_ENTRIES;  // one-launch layout up to this many
constexpr int kTargetChunks = EP_LAYOUT_TARGET_CHUNKS;  // wavefronts to spread over the chip

inline size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

inline int bits_for(int n) {  // bits to represent 0..n-1
  int b = 0;
  while ((1 << b) < n) ++b;
  return b;
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

int ep::make_geometry(const ep_problem* p, Geometry* g) {
  if (!p) return EP_ERR_NULL;
  const int R = p->num_ranks, T = p->num_tokens, H = p->hidden, E = p->num_experts,
            K = p->num_topk;
  if (p->reserved != 0) return EP_ERR_SHAPE;
  if (p->mode < EP_MODE_NORMAL || p->mode > EP_MODE_RANK_MAJOR) return EP_ERR_MODE;
  if (p->quant < EP_QUANT_NONE || p->quant > EP_QUANT_FP8_UE8M0) return EP_ERR_MODE;
  if (R < 1 || R > 256 || T < 0 || K < 1 || K > 64) return EP_ERR_SHAPE;
  if (E < R || E > 2048 || E % R != 0) return EP_ERR_SHAPE;
  if (H < 8 || H % 8 != 0 || H > 32768) return EP_ERR_SHAPE;
  if (p->quant != EP_QUANT_NONE && H % 128 != 0) return EP_ERR_SHAPE;
  if (p->expert_alignment < 1) return EP_ERR_SHAPE;
  const int64_t entries = (int64_t)R * T * K;
  if (entries >= (1ll << 31) || (int64_t)R * T * R >= (1ll << 31)) return EP_ERR_SHAPE;
  if (p->mode == EP_MODE_LOW_LATENCY) {
    if ((int64_t)E * R * T >= (1ll << 31)) return EP_ERR_SHAPE;
  } else {
    // worst-case aligned rows must stay below 2^31
    if (entries + (int64_t)E * (p->expert_alignment - 1) >= (1ll << 31)) return EP_ERR_SHAPE;
  }
  if (p->mode == EP_MODE_MESSAGES) {
    // a piece's length is a 32-bit descriptor field and never exceeds a region
    if (p->region_bytes < 16 || p->region_bytes % 16 != 0 || p->region_bytes > 0xFFFFFFF0ll)
      return EP_ERR_SHAPE;
  }
  g->R = R;
  g->T = T;
  g->H = H;
  g->E = E;
  g->K = K;
  g->L = E / R;
  g->G = H / 128;
  int tb = 64 / K;
  const int cap = 2048 / R;  // LDS row buffer of tb*R ints
  if (tb > cap) tb = cap;
  if (tb < 1) tb = 1;
  g->tb = tb;
  // small problems: one launch with a block per expert and per rank, each
  // reading every entry (16 entries per thread of a 1024-thread block)
  g->direct = entries <= kDirectMaxEntries && p->mode != EP_MODE_RANK_MAJOR ? 1 : 0;
  // fewer, longer chunks only when there are plenty of them
  const int64_t batches = (int64_t)R * ((T + tb - 1) / tb);
  int64_t per = (batches + kTargetChunks - 1) / kTargetChunks;
  if (per < 1) per = 1;
  if (per > kMaxChunkBatches) per = kMaxChunkBatches;
  g->ct = tb * (int)per;
  g->C = (T + g->ct - 1) / g->ct;
  g->NC = R * g->C;
  g->ebits = bits_for(E);
  g->rbits = bits_for(R);
  size_t off = 0;
  g->off_hist_e = off;
  off += up256(sizeof(int32_t) * (size_t)E * g->NC);
  g->off_hist_r = off;
  off += up256(sizeof(int32_t) * (size_t)R * g->NC);
  g->off_local_e = off;
  off += up256(sizeof(int32_t) * (size_t)entries);
  g->off_local_r = off;
  off += up256(sizeof(int32_t) * (size_t)R * T * R);
  g->off_msg = off;
  if (p->mode == EP_MODE_MESSAGES) off += up256(message_ws_bytes(R));
  g->off_stage = off;
  if ((p->mode == EP_MODE_NORMAL || p->mode == EP_MODE_RANK_MAJOR) &&
      p->quant != EP_QUANT_NONE) {
    // row-major scale staging for the worst-case number of receive rows
    const int64_t rows = p->mode == EP_MODE_RANK_MAJOR
                             ? (int64_t)R * T * (K < R ? K : R)
                             : entries + (int64_t)E * (p->expert_alignment - 1);
    off += up256((size_t)rows * g->G * (p->quant == EP_QUANT_FP8_F32 ? 4 : 1));
  }
  g->ws_bytes = off < 256 ? 256 : off;
  return EP_OK;
}

extern "C" {

size_t ep_workspace_bytes(const ep_problem* p) {
  Geometry g;
  if (ep::make_geometry(p, &g) != EP_OK) return 0;
  return g.ws_bytes;
}

int64_t ep_max_recv_rows(const ep_problem* p) {
  Geometry g;
  if (ep::make_geometry(p, &g) != EP_OK) return -1;
  if (p->mode == EP_MODE_LOW_LATENCY) return (int64_t)g.E * g.R * g.T;
  if (p->mode == EP_MODE_RANK_MAJOR) return (int64_t)g.R * g.T * (g.K < g.R ? g.K : g.R);
  return (int64_t)g.R * g.T * g.K + (int64_t)g.E * (p->expert_alignment - 1);
}

}  // extern "C"

namespace {

// Pieces a put of len bytes from arena offset la to arena offset ra is cut
// into when no piece may cross a multiple of rb on either side: one more
// than the cut points, which are the multiples of rb strictly inside
// (la, la + len) on the local side and inside (ra, ra + len) on the remote
// side.  Both sets have period rb, so they coincide when la = ra (mod rb)
// and are disjoint otherwise.
int64_t put_pieces(int64_t la, int64_t ra, int64_t len, int64_t rb) {
  if (len <= 0) return 0;
  const int64_t cl = (la + len - 1) / rb - la / rb;
  const int64_t cr = (ra + len - 1) / rb - ra / rb;
  return 1 + cl + (la % rb == ra % rb ? 0 : cr);
}

int64_t region_bytes_of(int64_t n, const ep_problem* p) {
  return n > 0 ? 32 + ep::msg_sections(n, p->hidden, p->num_topk, p->quant).body : 0;
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

}  // namespace

extern "C" {

int ep_messages_capacity(const ep_problem* p, const int32_t* counts, int64_t* send_bytes,
                         int64_t* recv_bytes, int64_t* descriptors) {
  Geometry g;
  const int st = ep::make_geometry(p, &g);
  if (st != EP_OK) return st;
  if (p->mode != EP_MODE_MESSAGES) return EP_ERR_MODE;
  const int R = g.R;
  const int64_t rb = p->region_bytes;
  int64_t send = 0, recv = 0, desc = 0;
  if (!counts) {
    // every pair carries T tokens: the largest region, arena and body; a
    // message's header and flag are one piece each (16 bytes at 16-byte
    // aligned offsets, rb a multiple of 16), its payload at most one more
    // than the region boundaries inside it on either side
    const int64_t reg = region_bytes_of(g.T, p);
    const int64_t arena = round_up((int64_t)R * reg, rb);
    send = recv = (int64_t)R * arena;
    if (reg > 0) desc = (int64_t)R * R * (3 + 2 * ((reg - 32 + rb - 1) / rb));
  } else {
    for (int64_t i = 0; i < (int64_t)R * R; ++i)
      if (counts[i] < 0 || counts[i] > g.T) return EP_ERR_SHAPE;
    // the packer's own arithmetic: region sizes, offsets inside each rank's
    // arena (prefix over destinations for a source, over sources for a
    // destination), arenas rounded up to the region size, then the pieces
    // of each message's payload, header and flag puts
    for (int s = 0; s < R; ++s) {
      int64_t tot = 0;
      for (int d = 0; d < R; ++d) tot += region_bytes_of(counts[s * R + d], p);
      send += round_up(tot, rb);
    }
    for (int d = 0; d < R; ++d) {
      int64_t tot = 0;
      for (int s = 0; s < R; ++s) tot += region_bytes_of(counts[s * R + d], p);
      recv += round_up(tot, rb);
    }
    int64_t recv_loc[256];  // running offset inside each destination's arena (R <= 256)
    for (int d = 0; d < R; ++d) recv_loc[d] = 0;
    for (int s = 0; s < R; ++s) {
      int64_t send_loc = 0;
      for (int d = 0; d < R; ++d) {
        const int64_t reg = region_bytes_of(counts[s * R + d], p);
        if (reg > 0) {
          const int64_t la = send_loc, ra = recv_loc[d], body = reg - 32;
          desc += put_pieces(la + 16, ra + 16, body, rb) + put_pieces(la, ra, 16, rb) +
                  put_pieces(la + 16 + body, ra + 16 + body, 16, rb);
        }
        send_loc += reg;
        recv_loc[d] += reg;
      }
    }
  }
  if (send_bytes) *send_bytes = send;
  if (recv_bytes) *recv_bytes = recv;
  if (descriptors) *descriptors = desc;
  return EP_OK;
}

const char* ep_status_string(int s) {
  switch (s) {
    case EP_OK: return "ok";
    case EP_ERR_NULL: return "a required pointer is NULL";
    case EP_ERR_ALIGN: return "a pointer is not suitably aligned";
    case EP_ERR_SHAPE: return "inconsistent or out-of-limit sizes";
    case EP_ERR_MODE: return "unknown or unsupported mode / quantisation";
    case EP_ERR_WORKSPACE: return "workspace too small";
    case EP_ERR_CAPACITY: return "capacity too small";
    case EP_ERR_HIP: return "HIP runtime error";
    case EP_ERR_SCRATCH: return "problem needs more scratch than the fixed no-alloc array";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// Checks ep_get_layout's arguments and fills the kernel arguments.
int layout_args(const ep_problem* p, const Geometry& g, const int32_t* topk_idx,
                const ep_layout* out, void* workspace, size_t workspace_bytes,
                ep::LayoutArgs* a) {
  // arrays with one entry per token may be NULL when there are no tokens
  const bool toks = (int64_t)g.R * g.T > 0;
  if (!out || !out->num_tokens_per_rank || !out->num_tokens_per_expert ||
      !out->rank_prefix_matrix || !out->recv_tokens_per_expert || !out->expert_start ||
      !out->rows_per_rank || !out->row_base || !out->err || !workspace)
    return EP_ERR_NULL;
  if (toks && (!topk_idx || !out->is_token_in_rank)) return EP_ERR_NULL;
  if (toks && p->mode != EP_MODE_MESSAGES && !out->send_pos) return EP_ERR_NULL;
  if (toks && p->mode == EP_MODE_MESSAGES && !out->send_head) return EP_ERR_NULL;
  const void* ints[] = {topk_idx, out->num_tokens_per_rank, out->num_tokens_per_expert,
                        out->rank_prefix_matrix, out->recv_tokens_per_expert, out->expert_start,
                        out->rows_per_rank, out->row_base, out->send_pos, out->send_head,
                        out->recv_src_idx, out->err};
  for (const void* q : ints)
    if (q && !aligned(q, 4)) return EP_ERR_ALIGN;
  if (!aligned(workspace, 16)) return EP_ERR_ALIGN;
  if (workspace_bytes < g.ws_bytes) return EP_ERR_WORKSPACE;
  if (out->recv_src_idx && out->recv_capacity < 0) return EP_ERR_CAPACITY;

  memset(a, 0, sizeof(*a));
  a->g = g;
  a->mode = p->mode;
  a->align = p->mode == EP_MODE_NORMAL ? p->expert_alignment : 1;
  a->topk = topk_idx;
  a->cnt_rank = out->num_tokens_per_rank;
  a->cnt_expert = out->num_tokens_per_expert;
  a->in_rank = out->is_token_in_rank;
  a->rpm = out->rank_prefix_matrix;
  a->recv_per_expert = out->recv_tokens_per_expert;
  a->expert_start = out->expert_start;
  a->rows = out->rows_per_rank;
  a->row_base = out->row_base;
  a->send_pos = out->send_pos;
  a->send_head = out->send_head;
  a->recv_src_idx = out->recv_src_idx;
  a->recv_cap = out->recv_capacity;
  a->err = out->err;
  char* ws = (char*)workspace;
  a->hist_e = (int32_t*)(ws + g.off_hist_e);
  a->hist_r = (int32_t*)(ws + g.off_hist_r);
  a->local_e = (int32_t*)(ws + g.off_local_e);
  a->local_r = (int32_t*)(ws + g.off_local_r);
  return EP_OK;
}

// Checks ep_dispatch's arguments for the normal, low-latency and
// rank-major modes and fills the kernel arguments.
int dispatch_args(const ep_problem* p, const Geometry& g, const ep_layout* layout,
                  const uint16_t* x, const int32_t* topk_idx, const float* topk_weights,
                  const ep_recv* recv, void* workspace, size_t workspace_bytes,
                  ep::DispatchArgs* a) {
  const bool toks = (int64_t)g.R * g.T > 0;
  memset(a, 0, sizeof(*a));
  if (!recv) return EP_ERR_NULL;
  // receive buffers may be NULL when they have no rows
  const bool rows = recv->capacity > 0;
  if (toks && !layout->send_pos) return EP_ERR_NULL;
  if (toks && rows && !recv->x) return EP_ERR_NULL;
  if (toks && rows && p->quant != EP_QUANT_NONE && !recv->scales) return EP_ERR_NULL;
  if (!aligned(recv->x, 16) || !aligned(layout->send_pos, 4)) return EP_ERR_ALIGN;
  if (recv->scales && !aligned(recv->scales, 4)) return EP_ERR_ALIGN;
  if (recv->capacity < 0) return EP_ERR_CAPACITY;
  if (p->mode == EP_MODE_LOW_LATENCY && recv->capacity < (int64_t)g.E * g.R * g.T)
    return EP_ERR_CAPACITY;
  const bool rank_major = p->mode == EP_MODE_RANK_MAJOR;
  const bool staged =
      (p->mode == EP_MODE_NORMAL || rank_major) && p->quant != EP_QUANT_NONE;
  if (rank_major && toks) {
    // per-row metadata needs the routing (ids) and, for weights, the weights
    if ((recv->topk_idx || recv->topk_weights) && !topk_idx) return EP_ERR_NULL;
    if (recv->topk_weights && !topk_weights) return EP_ERR_NULL;
    if (!aligned(recv->topk_idx, 4) || !aligned(recv->topk_weights, 4) ||
        !aligned(topk_idx, 4) || !aligned(topk_weights, 4))
      return EP_ERR_ALIGN;
  }
  if (staged && toks) {
    if (!workspace || !layout->expert_start || !layout->recv_tokens_per_expert ||
        !layout->row_base)
      return EP_ERR_NULL;
    if (!aligned(workspace, 16)) return EP_ERR_ALIGN;
    if (workspace_bytes < g.ws_bytes) return EP_ERR_WORKSPACE;
  }
  
  a->g = g;
  a->mode = p->mode;
  a->quant = p->quant;
  a->stage = staged ? (char*)workspace + g.off_stage : nullptr;
  a->stage_rows = rank_major ? (int64_t)g.R * g.T * (g.K < g.R ? g.K : g.R)
                            : (int64_t)g.R * g.T * g.K + (int64_t)g.E * (p->expert_alignment - 1);
  // scales staged once per token when the layout's row -> token map covers
  // every receive row (the staging holds stage_rows >= R*T rows either way)
  a->row_token = staged && layout->recv_src_idx && layout->recv_capacity >= recv->capacity
                     ? layout->recv_src_idx
                     : nullptr;
  a->align = p->mode == EP_MODE_NORMAL ? p->expert_alignment : 1;
  a->rank_major = rank_major;
  a->topk = rank_major ? topk_idx : nullptr;
  a->w = rank_major ? topk_weights : nullptr;
  a->recv_topk_idx = rank_major ? recv->topk_idx : nullptr;
  a->recv_topk_weights = rank_major ? recv->topk_weights : nullptr;
  a->expert_start = layout->expert_start;
  a->recv_per_expert = layout->recv_tokens_per_expert;
  a->row_base = layout->row_base;
  a->x = x;
  a->send_pos = layout->send_pos;
  a->recv_x = recv->x;
  a->recv_scales = recv->scales;
  a->cap = recv->capacity;
  // low-latency rows never leave the E blocks of R*T rows the scales cover
  if (p->mode == EP_MODE_LOW_LATENCY) a->cap = (int64_t)g.E * g.R * g.T;
  a->err = layout->err;
  return EP_OK;
}

}  // namespace

extern "C" {

int ep_get_layout(const ep_problem* p, const int32_t* topk_idx, const ep_layout* out,
                  void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  int st = ep::make_geometry(p, &g);
  if (st != EP_OK) return st;
  ep::LayoutArgs a;
  st = layout_args(p, g, topk_idx, out, workspace, workspace_bytes, &a);
  if (st != EP_OK) return st;
  if (ep::launch_layout(a, (hipStream_t)stream) != hipSuccess) return EP_ERR_HIP;
  return EP_OK;
}

int ep_dispatch(const ep_problem* p, const ep_layout* layout, const uint16_t* x,
                const int32_t* topk_idx, const float* topk_weights, const ep_recv* recv,
                const ep_messages* msgs, void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  int st = ep::make_geometry(p, &g);
  if (st != EP_OK) return st;
  const bool toks = (int64_t)g.R * g.T > 0;
  if (!layout || !layout->err || (toks && !x)) return EP_ERR_NULL;
  if (!aligned(x, 16) || !aligned(layout->err, 4)) return EP_ERR_ALIGN;
  if (p->mode != EP_MODE_MESSAGES) {
    ep::DispatchArgs a;
    st = dispatch_args(p, g, layout, x, topk_idx, topk_weights, recv, workspace,
                       workspace_bytes, &a);
    if (st != EP_OK) return st;
    if (ep::launch_dispatch(a, (hipStream_t)stream) != hipSuccess) return EP_ERR_HIP;
    return EP_OK;
  }
  // message mode
  if (!msgs || !layout->num_tokens_per_rank || !msgs->send_arena || !msgs->table ||
      !msgs->arena_base || !msgs->descriptors || !msgs->num_descriptors || !workspace)
    return EP_ERR_NULL;
  if (toks && (!topk_idx || !topk_weights || !layout->send_head)) return EP_ERR_NULL;
  if (!aligned(msgs->send_arena, 16) || !aligned(msgs->descriptors, 16) ||
      !aligned(msgs->table, 8) || !aligned(msgs->arena_base, 8) ||
      !aligned(msgs->num_descriptors, 8) || !aligned(topk_idx, 4) || !aligned(topk_weights, 4) ||
      !aligned(layout->send_head, 4) || !aligned(layout->num_tokens_per_rank, 4) ||
      !aligned(workspace, 16))
    return EP_ERR_ALIGN;
  if (workspace_bytes < g.ws_bytes) return EP_ERR_WORKSPACE;
  if (msgs->send_capacity < 0 || msgs->desc_capacity < 0) return EP_ERR_CAPACITY;
  ep::MessageArgs a;
  a.g = g;
  a.quant = p->quant;
  a.region_bytes = p->region_bytes;
  a.epoch = p->epoch;
  a.x = x;
  a.topk = topk_idx;
  a.w = topk_weights;
  a.cnt_rank = layout->num_tokens_per_rank;
  a.send_head = layout->send_head;
  a.arena = msgs->send_arena;
  a.arena_cap = msgs->send_capacity;
  a.table = msgs->table;
  a.arena_base = msgs->arena_base;
  a.desc = msgs->descriptors;
  a.desc_cap = msgs->desc_capacity;
  a.num_desc = msgs->num_descriptors;
  a.err = layout->err;
  a.ws = (char*)workspace + g.off_msg;
  if (ep::launch_messages(a, (hipStream_t)stream) != hipSuccess) return EP_ERR_HIP;
  return EP_OK;
}

int ep_dispatch_fused(const ep_problem* p, const int32_t* topk_idx, const ep_layout* layout,
                      const uint16_t* x, const ep_recv* recv, void* workspace,
                      size_t workspace_bytes, void* stream) {
  Geometry g;
  int st = ep::make_geometry(p, &g);
  if (st != EP_OK) return st;
  if (p->mode != EP_MODE_NORMAL && p->mode != EP_MODE_LOW_LATENCY) return EP_ERR_MODE;
  const bool toks = (int64_t)g.R * g.T > 0;
  if (!layout || !layout->err || (toks && !x)) return EP_ERR_NULL;
  if (!aligned(x, 16) || !aligned(layout->err, 4)) return EP_ERR_ALIGN;
  ep::LayoutArgs la;
  st = layout_args(p, g, topk_idx, layout, workspace, workspace_bytes, &la);
  if (st != EP_OK) return st;
  ep::DispatchArgs a;
  st = dispatch_args(p, g, layout, x, topk_idx, nullptr, recv, workspace, workspace_bytes, &a);
  if (st != EP_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (g.direct || !toks) {  // small problems: the one-launch layout, then dispatch
    if (ep::launch_layout(la, s) != hipSuccess) return EP_ERR_HIP;
  } else {
    if (ep::launch_layout_counts(la, s) != hipSuccess) return EP_ERR_HIP;
    a.fused = true;
    a.la = la;
  }
  if (ep::launch_dispatch(a, s) != hipSuccess) return EP_ERR_HIP;
  return EP_OK;
}

int ep_messages_execute(const ep_problem* p, const ep_messages* m, uint8_t* recv_arena,
                        int64_t recv_capacity, int32_t publish_batch, int32_t* err,
                        void* stream) {
  Geometry g;
  int st = ep::make_geometry(p, &g);
  if (st != EP_OK) return st;
  if (p->mode != EP_MODE_MESSAGES) return EP_ERR_MODE;
  if (!m || !err || !m->table || !m->arena_base || !m->num_descriptors) return EP_ERR_NULL;
  if ((m->send_capacity > 0 && !m->send_arena) || (m->desc_capacity > 0 && !m->descriptors) ||
      (recv_capacity > 0 && !recv_arena))
    return EP_ERR_NULL;
  if (!aligned(m->send_arena, 16) || !aligned(recv_arena, 16) || !aligned(m->descriptors, 16) ||
      !aligned(m->table, 8) || !aligned(m->arena_base, 8) || !aligned(m->num_descriptors, 8) ||
      !aligned(err, 4))
    return EP_ERR_ALIGN;
  if (m->send_capacity < 0 || m->desc_capacity < 0 || recv_capacity < 0) return EP_ERR_CAPACITY;
  if (m->desc_capacity > 0x7fffffff) return EP_ERR_SHAPE;  // descriptor indices are 31-bit
  if (publish_batch < 0) return EP_ERR_SHAPE;
  ep::ExecArgs a;
  a.publish_batch = publish_batch;
  a.g = g;
  a.region_bytes = p->region_bytes;
  a.send = m->send_arena;
  a.send_cap = m->send_capacity;
  a.table = m->table;
  a.arena_base = m->arena_base;
  a.desc = m->descriptors;
  a.desc_cap = m->desc_capacity;
  a.num_desc = m->num_descriptors;
  a.recv = recv_arena;
  a.recv_cap = recv_capacity;
  a.err = err;
  if (ep::launch_execute(a, (hipStream_t)stream) != hipSuccess) return EP_ERR_HIP;
  return EP_OK;
}

int ep_messages_unpack(const ep_problem* p, const ep_messages* m, const uint8_t* recv_arena,
                       int64_t recv_capacity, const int32_t* num_tokens_per_expert,
                       const ep_recv* out, int32_t* recv_count, int32_t* recv_src_idx,
                       int32_t spin_limit, int32_t* err, void* stream) {
  Geometry g;
  int st = ep::make_geometry(p, &g);
  if (st != EP_OK) return st;
  if (p->mode != EP_MODE_MESSAGES) return EP_ERR_MODE;
  if (spin_limit < 0 || spin_limit > EP_MAX_SPIN) return EP_ERR_SHAPE;
  const int64_t rows = (int64_t)g.E * g.R * g.T;
  if (!m || !m->table || !out || !err || !recv_count || !num_tokens_per_expert)
    return EP_ERR_NULL;
  if (rows > 0 && (!out->x || !recv_src_idx || (p->quant != EP_QUANT_NONE && !out->scales)))
    return EP_ERR_NULL;
  if (recv_capacity > 0 && !recv_arena) return EP_ERR_NULL;
  if (!aligned(recv_arena, 16) || !aligned(out->x, 16) || !aligned(out->scales, 4) ||
      !aligned(m->table, 8) || !aligned(num_tokens_per_expert, 4) || !aligned(recv_count, 4) ||
      !aligned(recv_src_idx, 4) || !aligned(err, 4))
    return EP_ERR_ALIGN;
  if (recv_capacity < 0 || out->capacity < rows) return EP_ERR_CAPACITY;
  ep::UnpackArgs a;
  a.g = g;
  a.quant = p->quant;
  a.epoch = p->epoch;
  a.arena = recv_arena;
  a.recv_cap = recv_capacity;
  a.table = m->table;
  a.arena_base = aligned(m->arena_base, 8) ? m->arena_base : nullptr;
  a.cnt_expert = num_tokens_per_expert;
  a.recv_x = out->x;
  a.recv_scales = out->scales;
  a.recv_count = recv_count;
  a.recv_src_idx = recv_src_idx;
  a.spin_limit = spin_limit;
  a.err = err;
  if (ep::launch_unpack(a, (hipStream_t)stream) != hipSuccess) return EP_ERR_HIP;
  return EP_OK;
}

int ep_combine(const ep_problem* p, const ep_layout* layout, const uint16_t* y, int64_t y_rows,
               const float* topk_weights, uint16_t* out, void* stream) {
  Geometry g;
  int st = ep::make_geometry(p, &g);
  if (st != EP_OK) return st;
  if (p->mode == EP_MODE_MESSAGES) return EP_ERR_MODE;
  const bool toks = (int64_t)g.R * g.T > 0;
  if (!layout || !layout->err) return EP_ERR_NULL;
  const bool rank_major = p->mode == EP_MODE_RANK_MAJOR;  // unweighted: no weights read
  if (toks && (!layout->send_pos || (!topk_weights && !rank_major) || !out || (!y && y_rows > 0)))
    return EP_ERR_NULL;
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(topk_weights, 4) ||
      !aligned(layout->send_pos, 4) || !aligned(layout->err, 4))
    return EP_ERR_ALIGN;
  if (y_rows < 0) return EP_ERR_CAPACITY;
  ep::CombineArgs a;
  a.g = g;
  a.y = y;
  a.y_rows = y_rows;
  a.send_pos = layout->send_pos;
  a.w = rank_major ? nullptr : topk_weights;
  a.rank_major = rank_major;
  a.out = out;
  a.err = layout->err;
  if (ep::launch_combine(a, (hipStream_t)stream) != hipSuccess) return EP_ERR_HIP;
  return EP_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// ep_dispatch_fused_noalloc: ep_dispatch_fused with the library's own fixed
// scratch array in place of the caller's workspace, for callers that cannot
// allocate.  Every GPU the library runs on holds its own copy of the array
// (EP_NOALLOC_SCRATCH_BYTES) until the process ends.  In host code the
// array's name is only a stand-in for the symbol: its device address on each
// GPU is looked up once, with that GPU current, and cached; kernels receive
// that address as their workspace.

static __device__ __align__(256) uint8_t scratch[EP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on device `dev` (first call on a device: one
// hipGetSymbolAddress with that device current, the caller's current device
// restored afterwards).
int scratch_on_device(int dev, void** out) {
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return EP_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return EP_ERR_HIP;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return EP_ERR_HIP;
    if (e != hipSuccess || !p) return EP_ERR_HIP;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return EP_OK;
}

}  // namespace

extern "C" int ep_dispatch_fused_noalloc(const ep_problem* p, const int32_t* topk_idx,
                                         const ep_layout* layout, const uint16_t* x,
                                         const ep_recv* recv, void* stream) {
  Geometry g;
  const int st = ep::make_geometry(p, &g);
  if (st != EP_OK) return st;
  if (g.ws_bytes > (size_t)EP_NOALLOC_SCRATCH_BYTES) return EP_ERR_SCRATCH;
  int dev = 0;
  const hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) return EP_ERR_HIP;
  void* ws = nullptr;
  const int sst = scratch_on_device(dev, &ws);
  if (sst != EP_OK) return sst;
  return ep_dispatch_fused(p, topk_idx, layout, x, recv, ws, (size_t)EP_NOALLOC_SCRATCH_BYTES,
                           stream);
}
