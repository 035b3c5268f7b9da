// Per-destination message packer and 64-byte write descriptors (gfx950).
//
// "Eaas_server" notes: a packing kernel lays each loaded destination's data
// out 16-byte aligned behind a header, then three puts go out per
// destination: payload, header, completion flag.  "ibgda_device.cuh" notes,
// sec. 1: a put is cut so that no piece spans two memory regions; sec. 3: a
// write work-queue entry is a control, a remote-address and a data segment
// with big-endian fields.  "GPU-Initiated Communication: Dissecting Down to
// the Bone", WQE anatomy (16-byte segments in a 64-byte block) and Ordering
// (payload stores visible before the store that announces them).
//
// Four launches:
//   1. offsets: one block per source (region sizes from the token counts,
//               compact offsets in its send arena: prefix over destinations)
//               and one per destination (offsets in its receive arena: prefix
//               over sources; descriptor count of each message).
//   2. rows   : one block per source: arena bases rounded to the region size,
//               first descriptor of each message, the table row.
//   3. pack   : one wavefront per token row piece, four tokens per block,
//               each die taking a contiguous run of tokens.  The row is read
//               once and quantised once, then stored into every message that
//               carries the token, at index send_head[s][t][d] within the
//               message, with the token's scales, weights, expert ids and
//               index.
//   4. finish : one thread per message: section padding, header, then (after
//               a fence) the completion flag, then the descriptors.
#include "ep_device.hpp"
#include "ep_internal.hpp"
#include "msg_format.hpp"
#include "quant.hpp"

namespace ep {

// Number of pieces a put [la, la+len) -> [ra, ra+len) is cut into when no
// piece may cross a multiple of rb on either side.
__device__ inline int64_t count_chunks(int64_t la, int64_t ra, int64_t len, int64_t rb) {
  int64_t n = 0;
  while (len > 0) {
    int64_t c = len;
    const int64_t l = rb - la % rb, r = rb - ra % rb;
    if (l < c) c = l;
    if (r < c) c = r;
    la += c;
    ra += c;
    len -= c;
    ++n;
  }
  return n;
}

struct MsgWs {
  int64_t* region;    // [R*R] region bytes (0 = no message)
  int64_t* send_loc;  // [R*R] offset within the source's arena
  int64_t* recv_loc;  // [R*R] offset within the destination's arena
  int64_t* dcount;    // [R*R] descriptors of the message
  int64_t* send_tot;  // [R] bytes of each source's messages
  int64_t* recv_tot;  // [R] bytes of each destination's messages
};

__device__ inline MsgWs msg_ws(void* ws, int R) {
  MsgWs w;
  int64_t* p = (int64_t*)ws;
  const int64_t rr = (int64_t)R * R;
  w.region = p;
  w.send_loc = p + rr;
  w.recv_loc = p + 2 * rr;
  w.dcount = p + 3 * rr;
  w.send_tot = p + 4 * rr;
  w.recv_tot = p + 4 * rr + R;
  return w;
}

__device__ __forceinline__ int64_t region_of(int64_t n, int H, int K, int quant) {
  return n > 0 ? 32 + msg_sections(n, H, K, quant).body : 0;
}

// Exclusive scan of one int64 per thread over the block; *total = sum.
__device__ int64_t block_scan64(int64_t v, int64_t* total) {
  __shared__ int64_t wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t incl = v;
  for (int o = 1; o < kWave; o <<= 1) {
    const int64_t t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int64_t before = 0, all = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    if (w < wave) before += wsum[w];
    all += wsum[w];
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

__device__ __forceinline__ int64_t message_descriptors(int64_t reg, int64_t la, int64_t ra,
                                                       int64_t rb) {
  if (reg == 0) return 0;
  const int64_t body = reg - 32;
  return count_chunks(la + 16, ra + 16, body, rb) + count_chunks(la, ra, 16, rb) +
         count_chunks(la + 16 + body, ra + 16 + body, 16, rb);
}

// Blocks [0, R): source s: region sizes of its messages and their offsets
// in s's arena (prefix over destinations).  Blocks [R, 2R): destination d:
// offsets in d's arena (prefix over sources) and the descriptor count of
// every message to d (its send offset re-derived from s's row).
// One thread per rank (R <= 256 = blockDim).
__global__ __launch_bounds__(256) void msg_offsets(MessageArgs a) {
  const Geometry& g = a.g;
  const int R = g.R;
  MsgWs w = msg_ws(a.ws, R);
  const int i = threadIdx.x;
  if ((int)blockIdx.x < R) {
    const int s = blockIdx.x;
    const int64_t reg = i < R ? region_of(a.cnt_rank[s * R + i], g.H, g.K, a.quant) : 0;
    int64_t tot;
    const int64_t off = block_scan64(reg, &tot);
    if (i < R) {
      w.region[s * R + i] = reg;
      w.send_loc[s * R + i] = off;
    }
    if (i == 0) w.send_tot[s] = tot;
  } else {
    const int d = blockIdx.x - R;
    const int64_t reg = i < R ? region_of(a.cnt_rank[i * R + d], g.H, g.K, a.quant) : 0;
    int64_t tot;
    const int64_t roff = block_scan64(reg, &tot);
    if (i < R) {
      w.recv_loc[i * R + d] = roff;
      // offset of (i, d) in source i's arena: the regions of i's messages to
      // destinations before d, their counts loaded sixteen at a time (one
      // memory latency per sixteen instead of one per destination)
      int64_t soff = 0;
      const int32_t* crow = a.cnt_rank + i * R;
      for (int d0 = 0; d0 < d; d0 += 16) {
        int n[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) n[q] = d0 + q < d ? crow[d0 + q] : 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) soff += region_of(n[q], g.H, g.K, a.quant);
      }
      w.dcount[i * R + d] = message_descriptors(reg, soff, roff, a.region_bytes);
    }
    if (i == 0) w.recv_tot[d] = tot;
  }
}

// Block s: arena bases (every block re-derives them), the first descriptor
// of each of s's messages (descriptors of all earlier sources, then a
// prefix over destinations) and s's table row.
// (Measured on MI355X at 64 ranks, kernel traces: 7.43 -> 7.03 us against
// eight loads issued after the arena-base scans.)
constexpr int kRowsLoads = 16;  // descriptor counts in flight per thread

__global__ __launch_bounds__(256) void msg_rows(MessageArgs a) {
  __shared__ int64_t base_s[257], base_r[257];
  const Geometry& g = a.g;
  const int R = g.R;
  MsgWs w = msg_ws(a.ws, R);
  const int s = blockIdx.x, i = threadIdx.x;
  const int64_t rb = a.region_bytes;
  // descriptors of sources before s, kRowsLoads loads per thread in flight
  // (issued first: nothing below feeds them, and a barrier would keep
  // them from being issued earlier than it; unconditional, clamped)
  int64_t part = 0;
  const int64_t nbefore = (int64_t)s * R;
  for (int64_t j0 = i; j0 < nbefore; j0 += kRowsLoads * (int64_t)blockDim.x) {
    int64_t c[kRowsLoads];
#pragma unroll
    for (int q = 0; q < kRowsLoads; ++q) {
      const int64_t j = j0 + q * (int64_t)blockDim.x;
      const int64_t v = w.dcount[j < nbefore ? j : nbefore - 1];
      c[q] = j < nbefore ? v : 0;
    }
#pragma unroll
    for (int q = 0; q < kRowsLoads; ++q) part += c[q];
  }
  int64_t tot;
  const int64_t vs = i < R ? (w.send_tot[i] + rb - 1) / rb * rb : 0;
  const int64_t os = block_scan64(vs, &tot);
  if (i < R) base_s[i] = os;
  if (i == 0) base_s[R] = tot;
  const int64_t vr = i < R ? (w.recv_tot[i] + rb - 1) / rb * rb : 0;
  const int64_t orr = block_scan64(vr, &tot);
  if (i < R) base_r[i] = orr;
  if (i == 0) base_r[R] = tot;
  __syncthreads();
  if (s == 0)
    for (int j = i; j <= R; j += blockDim.x) {
      a.arena_base[j] = base_s[j];
      a.arena_base[R + 1 + j] = base_r[j];
    }
  int64_t before;
  block_scan64(part, &before);
  const int64_t dc = i < R ? w.dcount[s * R + i] : 0;
  int64_t row_total;
  const int64_t first = before + block_scan64(dc, &row_total);
  if (s == R - 1 && i == 0) *a.num_desc = before + row_total;
  if (i < R) {
    const int64_t sd = (int64_t)s * R + i;
    const int64_t reg = w.region[sd];
    int64_t* row = a.table + sd * 8;
    row[0] = reg > 0 ? base_s[s] + w.send_loc[sd] : -1;
    row[1] = reg > 0 ? base_r[i] + w.recv_loc[sd] : -1;
    row[2] = reg;
    row[3] = a.cnt_rank[sd];
    row[4] = reg > 0 ? reg - 32 : 0;
    row[5] = first;
    row[6] = dc;
    row[7] = 0;
  }
}

// Store the per-token sections (weights, ids, token index) of one message.
__device__ __forceinline__ void store_token_meta(uint8_t* body, const MsgSections& m, int64_t j,
                                                 int K, int lane, const float* wrow,
                                                 const int32_t* idrow, int t) {
  if (lane < K) {
    ((float*)(body + m.off[2]))[j * K + lane] = wrow[lane];
    ((int32_t*)(body + m.off[3]))[j * K + lane] = idrow[lane];
  }
  if (lane == 0) ((int32_t*)(body + m.off[4]))[j] = t;
}

// Destinations of token (s, t): walk send_head in slabs of 64 ranks, each
// lane loading one destination's slot, message offset and token count, so
// the loop below reads them with readlane instead of a load per message.
// For each destination d the token goes to, call f(d, j, off, n) with j its
// index in the (s, d) message, off the message's send offset and n its
// token count (uniform across the wave).
template <typename F>
__device__ __forceinline__ void for_each_destination(const int32_t* head_row,
                                                     const int64_t* table_row,
                                                     const int32_t* cnt_row, int R, F&& f) {
  const int lane = lane_id();
  for (int slab = 0; slab < R; slab += kWave) {
    const int d = slab + lane;
    const int h = d < R ? head_row[d] : -1;
    int64_t off = -1;
    int n = 0;
    if (h >= 0) {
      off = table_row[(int64_t)d * 8];
      n = cnt_row[d];
    }
    uint64_t mask = __ballot(h >= 0);
    while (mask) {
      const int b = __builtin_ctzll(mask);
      mask &= mask - 1;
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)off, b);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)off >> 32), b);
      f(slab + b, __builtin_amdgcn_readlane(h, b), (int64_t)(((uint64_t)hi << 32) | lo),
        (int64_t)__builtin_amdgcn_readlane(n, b));
    }
  }
}

template <int NP, int Q>
__global__ __launch_bounds__(256) void msg_pack_fp8(MessageArgs a, int P) {
  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63;
  // four tokens per block; each die takes a contiguous run of blocks, so
  // consecutive tokens of a message (adjacent scale, weight and id entries)
  // are stored from one L2 and their cache lines merge there (measured on
  // MI355X at the 64-rank message workload: the pack unchanged, the
  // delivery that reads the messages next 1% faster)
  const int nblk = (g.R * g.T + 3) / 4;
  const int blk = xcd_run(blockIdx.x, nblk);
  if (blk >= nblk) return;
  const int tok = uniform(blk * 4 + (threadIdx.x >> 6));
  if (tok >= g.R * g.T) return;
  const int piece = blockIdx.y;
  const int base = piece * kWave * NP;
  const int s = tok / g.T, t = tok % g.T;
  const u32x4* src = (const u32x4*)a.x + (int64_t)tok * (2 * (int64_t)P);
  u32x4 lo[NP], hi[NP], cv[NP];
  float scf[NP];
  uint32_t sce[NP];
  load_pairs<NP>(src, base, P, lo, hi);
#pragma unroll
  for (int i = 0; i < NP; ++i) quantise_pair<Q>(lo[i], hi[i], cv[i], scf[i], sce[i]);
  // the piece's group scales gathered into lanes 0 .. ng-1 (lane L: group
  // base/8 + L, held by lane 8*(L&7) in register L>>3), so each message
  // takes them in one store instead of one per pair (measured on MI355X at
  // the 64-rank message workload: pack 250.3 -> 241.8 us; one store for the
  // weights, ids and token index as well gained nothing more)
  const int ng = (min(base + kWave * NP, P) - base) >> 3;
  float gsf = 0.0f;
  uint32_t gse = 0;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const float vf = __shfl(scf[i], (lane & 7) * 8);
    const uint32_t ve = (uint32_t)__shfl((int)sce[i], (lane & 7) * 8);
    if ((lane >> 3) == i) {
      gsf = vf;
      gse = ve;
    }
  }
  const float* wrow = a.w + (int64_t)tok * g.K;
  const int32_t* idrow = a.topk + (int64_t)tok * g.K;
  for_each_destination(a.send_head + (int64_t)tok * g.R, a.table + (int64_t)s * g.R * 8,
                       a.cnt_rank + (int64_t)s * g.R, g.R,
                       [&](int d, int j, int64_t off, int64_t n) {
    (void)d;
    const MsgSections m = msg_sections(n, g.H, g.K, Q);
    if (off < 0 || j >= n || off + 32 + m.body > a.arena_cap) {
      if (lane == 0) set_err(a.err, EP_DEVERR_CAPACITY);
      return;
    }
    uint8_t* body = a.arena + off + 16;
    u32x4* crow = (u32x4*)(body + m.off[0] + (int64_t)j * g.H);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = base + lane + kWave * i;
      // non-temporal (measured on MI355X: plain stores make the pack 4%
      // faster and the next delivery 9% slower, as it writes them back)
      if (p < P) __builtin_nontemporal_store(cv[i], crow + p);
    }
    if (lane < ng) {
      const int64_t gi = (int64_t)j * g.G + (base >> 3) + lane;
      if (Q == EP_QUANT_FP8_F32) ((float*)(body + m.off[1]))[gi] = gsf;
      else (body + m.off[1])[gi] = (uint8_t)gse;
    }
    if (piece == 0) store_token_meta(body, m, j, g.K, lane, wrow, idrow, t);
  });
}

template <int NV>
__global__ __launch_bounds__(256) void msg_pack_bf16(MessageArgs a, int V) {
  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63;
  // the FP8 packer's die-aware block order
  const int nblk = (g.R * g.T + 3) / 4;
  const int blk = xcd_run(blockIdx.x, nblk);
  if (blk >= nblk) return;
  const int tok = uniform(blk * 4 + (threadIdx.x >> 6));
  if (tok >= g.R * g.T) return;
  const int piece = blockIdx.y;
  const int base = piece * kWave * NV;
  const int s = tok / g.T, t = tok % g.T;
  const u32x4* src = (const u32x4*)a.x + (int64_t)tok * V;
  u32x4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {  // clamped, so every load is in bounds
    const int j = min(base + lane + kWave * i, V - 1);
    v[i] = __builtin_nontemporal_load(src + j);
  }
  const float* wrow = a.w + (int64_t)tok * g.K;
  const int32_t* idrow = a.topk + (int64_t)tok * g.K;
  for_each_destination(a.send_head + (int64_t)tok * g.R, a.table + (int64_t)s * g.R * 8,
                       a.cnt_rank + (int64_t)s * g.R, g.R,
                       [&](int d, int j, int64_t off, int64_t n) {
    (void)d;
    const MsgSections m = msg_sections(n, g.H, g.K, EP_QUANT_NONE);
    if (off < 0 || j >= n || off + 32 + m.body > a.arena_cap) {
      if (lane == 0) set_err(a.err, EP_DEVERR_CAPACITY);
      return;
    }
    uint8_t* body = a.arena + off + 16;
    u32x4* crow = (u32x4*)(body + m.off[0]) + (int64_t)j * V;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int p = base + lane + kWave * i;
      if (p < V) __builtin_nontemporal_store(v[i], crow + p);
    }
    if (piece == 0) store_token_meta(body, m, j, g.K, lane, wrow, idrow, t);
  });
}


// One 64-byte descriptor: control | remote address | data | zero pad.
__device__ __forceinline__ void write_desc(uint8_t* dst, uint32_t wqe, uint32_t qpn,
                                           uint64_t raddr, uint32_t rkey, uint32_t len,
                                           uint32_t lkey, uint64_t laddr) {
  u32x4* q = (u32x4*)dst;
  q[0] = u32x4{be32((wqe << 8) | 0x08u), be32((qpn << 8) | 3u), 0x08000000u, 0u};
  q[1] = u32x4{be32((uint32_t)(raddr >> 32)), be32((uint32_t)raddr), be32(rkey), 0u};
  q[2] = u32x4{be32(len), be32(lkey), be32((uint32_t)(laddr >> 32)), be32((uint32_t)laddr)};
  q[3] = u32x4{0u, 0u, 0u, 0u};
}

__global__ __launch_bounds__(256) void msg_finish(MessageArgs a) {
  const Geometry& g = a.g;
  const int R = g.R;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)R * R) return;
  const int64_t* row = a.table + i * 8;
  const int64_t reg = row[2];
  if (reg == 0) return;
  const int s = (int)(i / R), d = (int)(i % R);
  const int64_t off = row[0], roff = row[1], n = row[3], body = row[4];
  const MsgSections m = msg_sections(n, g.H, g.K, a.quant);
  if (off + reg <= a.arena_cap) {
    uint8_t* msg = a.arena + off;
    for (int q = 0; q < 5; ++q)
      for (int64_t b = m.off[q] + m.len[q]; b < m.off[q] + pad16(m.len[q]); ++b) msg[16 + b] = 0;
    *(u32x4*)msg = u32x4{(uint32_t)s, (uint32_t)d, (uint32_t)n, (uint32_t)body};
    __threadfence();  // body (earlier launch), padding and header before the flag
    *(u32x4*)(msg + 16 + body) = u32x4{a.epoch, 0u, 0u, 0u};
  } else {
    set_err(a.err, EP_DEVERR_CAPACITY);
  }
  // descriptors: payload, header, flag; addresses relative to each rank's arena
  const int64_t rb = a.region_bytes;
  const int64_t la0 = off - a.arena_base[s], ra0 = roff - a.arena_base[R + 1 + d];
  const int64_t put_off[3] = {16, 0, 16 + body};
  const int64_t put_len[3] = {body, 16, 16};
  int64_t di = row[5];
  uint32_t wqe = 0;
  for (int u = 0; u < 3; ++u) {
    int64_t la = la0 + put_off[u], ra = ra0 + put_off[u], rem = put_len[u];
    while (rem > 0) {
      int64_t c = rem;
      const int64_t l = rb - la % rb, r = rb - ra % rb;
      if (l < c) c = l;
      if (r < c) c = r;
      if (di < a.desc_cap) {
        // a key holds the region index in 16 bits: a piece past region
        // 65535 of either arena gets keys naming no rank (the executor
        // rejects it) and raises the capacity bit
        const bool fits = la / rb <= kMaxRegionIndex && ra / rb <= kMaxRegionIndex;
        if (!fits) set_err(a.err, EP_DEVERR_CAPACITY);
        write_desc(a.desc + di * 64, wqe, (uint32_t)(s * R + d), (uint64_t)ra,
                   fits ? (uint32_t)((d << 16) | (ra / rb)) : kBadKey, (uint32_t)c,
                   fits ? (uint32_t)((s << 16) | (la / rb)) : kBadKey, (uint64_t)la);
      } else {
        set_err(a.err, EP_DEVERR_CAPACITY);
      }
      ++di;
      ++wqe;
      la += c;
      ra += c;
      rem -= c;
    }
  }
}

template <int NP, int Q>
static void launch_pack_fp8(const MessageArgs& a, hipStream_t st) {
  const int P = a.g.H / 16;
  const int npieces = (P + kWave * NP - 1) / (kWave * NP);
  const int N = a.g.R * a.g.T;
  hipLaunchKernelGGL((msg_pack_fp8<NP, Q>), dim3(xcd_blocks((N + 3) / 4), npieces), dim3(256), 0,
                     st, a, P);
}

template <int Q>
static void launch_pack_q(const MessageArgs& a, hipStream_t st) {
  const int P = a.g.H / 16;
  const int npieces = (P + kWave * 8 - 1) / (kWave * 8);
  const int np = (P + kWave * npieces - 1) / (kWave * npieces);
  switch (np) {
    case 1: launch_pack_fp8<1, Q>(a, st); break;
    case 2: launch_pack_fp8<2, Q>(a, st); break;
    case 3: launch_pack_fp8<3, Q>(a, st); break;
    case 4: launch_pack_fp8<4, Q>(a, st); break;
    case 5: launch_pack_fp8<5, Q>(a, st); break;
    case 6: launch_pack_fp8<6, Q>(a, st); break;
    case 7: launch_pack_fp8<7, Q>(a, st); break;
    default: launch_pack_fp8<8, Q>(a, st); break;
  }
}

template <int NV>
static void launch_pack_bf16(const MessageArgs& a, hipStream_t st) {
  const int V = a.g.H / 8;
  const int npieces = (V + kWave * NV - 1) / (kWave * NV);
  const int N = a.g.R * a.g.T;
  hipLaunchKernelGGL(msg_pack_bf16<NV>, dim3(xcd_blocks((N + 3) / 4), npieces), dim3(256), 0, st,
                     a, V);
}

size_t message_ws_bytes(int R) { return sizeof(int64_t) * (4 * (size_t)R * R + 2 * (size_t)R); }

hipError_t launch_messages(const MessageArgs& a, hipStream_t st) {
  const int R = a.g.R;
  hipLaunchKernelGGL(msg_offsets, dim3(2 * R), dim3(256), 0, st, a);
  hipLaunchKernelGGL(msg_rows, dim3(R), dim3(256), 0, st, a);
  if ((int64_t)a.g.R * a.g.T > 0) {
    if (a.quant == EP_QUANT_FP8_F32) {
      launch_pack_q<EP_QUANT_FP8_F32>(a, st);
    } else if (a.quant == EP_QUANT_FP8_UE8M0) {
      launch_pack_q<EP_QUANT_FP8_UE8M0>(a, st);
    } else {
      const int V = a.g.H / 8;
      const int npieces = (V + kWave * 8 - 1) / (kWave * 8);
      const int nv = (V + kWave * npieces - 1) / (kWave * npieces);
      switch (nv) {
        case 1: launch_pack_bf16<1>(a, st); break;
        case 2: launch_pack_bf16<2>(a, st); break;
        case 3: launch_pack_bf16<3>(a, st); break;
        case 4: launch_pack_bf16<4>(a, st); break;
        case 5: launch_pack_bf16<5>(a, st); break;
        case 6: launch_pack_bf16<6>(a, st); break;
        case 7: launch_pack_bf16<7>(a, st); break;
        default: launch_pack_bf16<8>(a, st); break;
      }
    }
  }
  const int64_t rr = (int64_t)R * R;
  hipLaunchKernelGGL(msg_finish, dim3((unsigned)((rr + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ep
