// Host/device shared declarations internal to libep (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ep.h"

namespace ep {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Token chunking used by the layout kernels: one wavefront walks a chunk of
// consecutive tokens of one source rank in batches of `tb` tokens (tb*K
// entries <= 64, one entry per lane), at most kMaxChunkBatches batches per
// chunk, whose expert ids it loads together and then counts one batch after
// another.  Measured on MI355X at the FP8 training shape (131,072 tokens,
// top-8): 16 batches per chunk, count 22.3 us + scan 4.9 us; 8 batches
// (twice the chunks), 15.5 + 6.0 us; 4 batches, 13.7 + 11.5 us.
constexpr int kMaxChunkBatches = 8;

struct Geometry {
  int R, T, H, E, K, L, G;
  int tb;      // tokens per batch
  int ct;      // tokens per chunk
  int C;       // chunks per source rank
  int NC;      // R * C
  int ebits;   // bits of an expert id
  int rbits;   // bits of a rank id
  int direct;  // small problem: the whole layout in one launch, no chunks
  // workspace carve-up (byte offsets from the workspace base)
  size_t off_hist_e, off_hist_r, off_local_e, off_local_r, off_msg, off_stage, ws_bytes;
};

int make_geometry(const ep_problem* p, Geometry* g);  // EP_OK or EP_ERR_*

struct LayoutArgs {
  Geometry g;
  int mode, align;
  const int32_t* topk;
  int32_t* cnt_rank;       // [R][R]
  int32_t* cnt_expert;     // [R][E]
  uint8_t* in_rank;        // [R][T][R]
  int32_t* rpm;            // [R][R]
  int32_t* recv_per_expert;// [E]
  int32_t* expert_start;   // [E]
  int32_t* rows;           // [R]
  int32_t* row_base;       // [R+1]
  int32_t* send_pos;       // [R][T][K] or NULL
  int32_t* send_head;      // [R][T][R] or NULL
  int32_t* recv_src_idx;   // or NULL
  int64_t recv_cap;
  int32_t* err;
  // workspace
  int32_t* hist_e;         // [E][NC]
  int32_t* hist_r;         // [R][R][C]
  int32_t* local_e;        // [R][T][K]
  int32_t* local_r;        // [R][T][R]
};

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream);
// The counting and scanning launches only (chunked path), for dispatch
// kernels that take the final step themselves.
hipError_t launch_layout_counts(const LayoutArgs& a, hipStream_t stream);

struct DispatchArgs {
  Geometry g;
  int mode, quant;
  const uint16_t* x;
  const int32_t* send_pos;
  void* recv_x;
  void* recv_scales;
  int64_t cap;
  int32_t* err;
  // normal-mode FP8: row-major scale staging (workspace) and the layout's
  // segment starts / counts / row bases used to transpose it column-major
  void* stage;
  int64_t stage_rows;  // rows the staging buffer holds
  // the layout's recv_src_idx when it covers every receive row: the
  // staging then holds each token's scales once ([N][G]) and the transpose
  // gathers them per row; NULL: one staged copy per receive row
  const int32_t* row_token;
  int align;           // expert_alignment (normal mode; 1 otherwise)
  const int32_t* expert_start;
  const int32_t* recv_per_expert;
  const int32_t* row_base;
  // rank-major: one row per (token, destination rank); optional per-row
  // top-k metadata from the routing and weights
  bool rank_major;
  const int32_t* topk;
  const float* w;
  int32_t* recv_topk_idx;
  float* recv_topk_weights;
  // layout fused into dispatch: the kernel derives each token's rows from
  // the scanned chunk histograms (la) instead of reading send_pos, and
  // writes the layout's remaining outputs itself
  bool fused;
  LayoutArgs la;
};

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream);

struct CombineArgs {
  Geometry g;
  const uint16_t* y;
  int64_t y_rows;
  const int32_t* send_pos;
  const float* w;          // NULL in rank-major mode
  bool rank_major;         // sum the token's distinct rows, unweighted
  uint16_t* out;
  int32_t* err;
};

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

struct MessageArgs {
  Geometry g;
  int quant;
  int64_t region_bytes;
  uint32_t epoch;
  const uint16_t* x;
  const int32_t* topk;
  const float* w;
  const int32_t* cnt_rank;   // [R][R]
  const int32_t* send_head;  // [R][T][R]
  uint8_t* arena;
  int64_t arena_cap;
  int64_t* table;            // [R][R][8]
  int64_t* arena_base;       // [2][R+1]
  uint8_t* desc;
  int64_t desc_cap;
  int64_t* num_desc;
  int32_t* err;
  void* ws;                  // message workspace
};

hipError_t launch_messages(const MessageArgs& a, hipStream_t stream);

// Loopback execution of message mode's descriptors.
struct ExecArgs {
  Geometry g;
  int64_t region_bytes;
  const uint8_t* send;       // send arenas
  int64_t send_cap;
  const int64_t* table;      // [R][R][8]
  const int64_t* arena_base; // [2][R+1]
  const uint8_t* desc;       // [desc_cap][64]
  int64_t desc_cap;
  const int64_t* num_desc;
  uint8_t* recv;             // receive arenas
  int64_t recv_cap;
  int publish_batch;         // 0: flags in a second launch; B >= 1: every B messages
  int32_t* err;
};

hipError_t launch_execute(const ExecArgs& a, hipStream_t stream);

// Receiver: delivered messages -> low-latency layout.
struct UnpackArgs {
  Geometry g;
  int quant;
  uint32_t epoch;
  const uint8_t* arena;        // receive arenas
  int64_t recv_cap;
  const int64_t* table;        // [R][R][8]
  const int64_t* arena_base;   // [2][R+1] or NULL (receive loads, for the block order)
  const int32_t* cnt_expert;   // [R][E]
  void* recv_x;                // [E*R*T][H] bf16 or codes
  void* recv_scales;           // [E][G][R*T]
  int32_t* recv_count;         // [E]
  int32_t* recv_src_idx;       // [E*R*T]
  int spin_limit;              // extra polls of a message's flag before giving up
  int32_t* err;
};

hipError_t launch_unpack(const UnpackArgs& a, hipStream_t stream);

}  // namespace ep
