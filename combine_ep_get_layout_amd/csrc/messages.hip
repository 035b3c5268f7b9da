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
// Three launches:
//   1. table  : one block.  Region size per (source, destination) from the
//               token counts; compact offsets in each source's send arena
//               (prefix over destinations) and each destination's receive
//               arena (prefix over sources); arena bases rounded to the region
//               size; descriptor counts and their prefix.
//   2. pack   : one wavefront per token row piece.  The row is read once and
//               quantised once, then stored into every message that carries
//               the token, at index send_head[s][t][d] within the message,
//               with the token's scales, weights, expert ids and index.
//   3. finish : one thread per message: section padding, header, then (after
//               a fence) the completion flag, then the descriptors.
#include "ep_device.hpp"
#include "ep_internal.hpp"
#include "quant.hpp"

namespace ep {

struct MsgSections {
  int64_t off[5];  // section offsets within the body
  int64_t len[5];  // unpadded section lengths
  int64_t body;    // body bytes (sum of padded sections)
};

__host__ __device__ inline int64_t pad16(int64_t v) { return (v + 15) & ~(int64_t)15; }

// Body of a message with n tokens: codes | scales | weights | ids | token.
__host__ __device__ inline MsgSections msg_sections(int64_t n, int H, int K, int quant) {
  MsgSections m;
  const int64_t G = H / 128;
  m.len[0] = n * H * (quant == EP_QUANT_NONE ? 2 : 1);
  m.len[1] = n * G * (quant == EP_QUANT_FP8_F32 ? 4 : (quant == EP_QUANT_FP8_UE8M0 ? 1 : 0));
  m.len[2] = n * K * 4;
  m.len[3] = n * K * 4;
  m.len[4] = n * 4;
  int64_t o = 0;
  for (int i = 0; i < 5; ++i) {
    m.off[i] = o;
    o += pad16(m.len[i]);
  }
  m.body = o;
  return m;
}

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
  int64_t* region;   // [R*R]
  int64_t* send_loc; // [R*R] offset within the source's arena
  int64_t* recv_loc; // [R*R] offset within the destination's arena
  int64_t* dcount;   // [R*R]
};

__device__ inline MsgWs msg_ws(void* ws, int R) {
  MsgWs w;
  int64_t* p = (int64_t*)ws;
  const int64_t rr = (int64_t)R * R;
  w.region = p;
  w.send_loc = p + rr;
  w.recv_loc = p + 2 * rr;
  w.dcount = p + 3 * rr;
  return w;
}

// Exclusive scan of a strided sequence of n int64 by one wavefront; returns
// the total.
__device__ int64_t wave_scan_strided(const int64_t* in, int64_t* out, int n, int64_t stride) {
  const int lane = lane_id();
  int64_t carry = 0;
  for (int b = 0; b < n; b += kWave) {
    const int i = b + lane;
    const int64_t v = i < n ? in[i * stride] : 0;
    int64_t incl = v;
    for (int o = 1; o < kWave; o <<= 1) {
      const int64_t t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (i < n) out[i * stride] = carry + incl - v;
    carry += __shfl(incl, kWave - 1);
  }
  return carry;
}

__global__ __launch_bounds__(1024) void msg_table(MessageArgs a) {
  const Geometry& g = a.g;
  const int R = g.R;
  const int rr = R * R;
  MsgWs w = msg_ws(a.ws, R);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, nw = blockDim.x >> 6;
  __shared__ int64_t tot_send[257], tot_recv[257];

  for (int i = tid; i < rr; i += blockDim.x) {
    const int64_t n = a.cnt_rank[i];
    w.region[i] = n > 0 ? 32 + msg_sections(n, g.H, g.K, a.quant).body : 0;
  }
  __syncthreads();
  // send side: per source, prefix over destinations; receive side: per
  // destination, prefix over sources
  for (int s = wave; s < R; s += nw) {
    const int64_t t = wave_scan_strided(w.region + (int64_t)s * R, w.send_loc + (int64_t)s * R, R, 1);
    if (lane == 0) tot_send[s] = t;
  }
  for (int d = wave; d < R; d += nw) {
    const int64_t t = wave_scan_strided(w.region + d, w.recv_loc + d, R, R);
    if (lane == 0) tot_recv[d] = t;
  }
  __syncthreads();
  // arena bases (each rank's arena starts on a region boundary)
  if (wave == 0) {
    const int64_t rb = a.region_bytes;
    int64_t cs = 0, cr = 0;
    for (int b = 0; b < R; b += kWave) {
      const int i = b + lane;
      int64_t vs = i < R ? (tot_send[i] + rb - 1) / rb * rb : 0;
      int64_t vr = i < R ? (tot_recv[i] + rb - 1) / rb * rb : 0;
      int64_t is = vs, ir = vr;
      for (int o = 1; o < kWave; o <<= 1) {
        const int64_t ts = __shfl_up(is, o), tr = __shfl_up(ir, o);
        if (lane >= o) {
          is += ts;
          ir += tr;
        }
      }
      if (i < R) {
        a.arena_base[i] = cs + is - vs;
        a.arena_base[R + 1 + i] = cr + ir - vr;
      }
      cs += __shfl(is, kWave - 1);
      cr += __shfl(ir, kWave - 1);
    }
    if (lane == 0) {
      a.arena_base[R] = cs;
      a.arena_base[2 * R + 1] = cr;
    }
  }
  // descriptor counts
  for (int i = tid; i < rr; i += blockDim.x) {
    const int64_t reg = w.region[i];
    int64_t c = 0;
    if (reg > 0) {
      const int64_t body = reg - 32, la = w.send_loc[i], ra = w.recv_loc[i];
      c = count_chunks(la + 16, ra + 16, body, a.region_bytes) + count_chunks(la, ra, 16, a.region_bytes) +
          count_chunks(la + 16 + body, ra + 16 + body, 16, a.region_bytes);
    }
    w.dcount[i] = c;
  }
  __syncthreads();
  // prefix of descriptor counts in (s, d) order: per-thread runs + block scan
  __shared__ int64_t part[1024];
  const int per = (rr + blockDim.x - 1) / blockDim.x;
  const int lo = min(rr, tid * per), hi = min(rr, lo + per);
  int64_t sum = 0;
  for (int i = lo; i < hi; ++i) sum += w.dcount[i];
  part[tid] = sum;
  __syncthreads();
  if (wave == 0) {
    // scan of the 1024 partial sums by one wavefront (16 per lane)
    const int per_lane = blockDim.x / kWave;
    int64_t loc = 0;
    for (int q = 0; q < per_lane; ++q) loc += part[lane * per_lane + q];
    int64_t incl = loc;
    for (int o = 1; o < kWave; o <<= 1) {
      const int64_t t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    int64_t run = incl - loc;
    for (int q = 0; q < per_lane; ++q) {
      const int64_t v = part[lane * per_lane + q];
      part[lane * per_lane + q] = run;
      run += v;
    }
    if (lane == kWave - 1) *a.num_desc = incl;
  }
  __syncthreads();
  int64_t run = part[tid];
  for (int i = lo; i < hi; ++i) {
    const int s = i / R, d = i % R;
    int64_t* row = a.table + (int64_t)i * 8;
    const int64_t reg = w.region[i];
    row[0] = reg > 0 ? a.arena_base[s] + w.send_loc[i] : -1;
    row[1] = reg > 0 ? a.arena_base[R + 1 + d] + w.recv_loc[i] : -1;
    row[2] = reg;
    row[3] = a.cnt_rank[i];
    row[4] = reg > 0 ? reg - 32 : 0;
    row[5] = run;
    row[6] = w.dcount[i];
    row[7] = 0;
    run += w.dcount[i];
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

// Destinations of token (s, t): walk send_head in slabs of 64 ranks; for
// each destination d the token goes to, call f(d, j) with j its index in
// the (s, d) message (uniform across the wave).
template <typename F>
__device__ __forceinline__ void for_each_destination(const int32_t* head_row, int R, F&& f) {
  const int lane = lane_id();
  for (int slab = 0; slab < R; slab += kWave) {
    const int d = slab + lane;
    const int h = d < R ? head_row[d] : -1;
    uint64_t mask = __ballot(h >= 0);
    while (mask) {
      const int b = __builtin_ctzll(mask);
      mask &= mask - 1;
      f(slab + b, __builtin_amdgcn_readlane(h, b));
    }
  }
}

// Grid: x = token / 4 (one wavefront per token, tok = s * T + t), y = piece.
template <int NP, int Q>
__global__ __launch_bounds__(256) void msg_pack_fp8(MessageArgs a, int P) {
  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63;
  const int tok = uniform(blockIdx.x * 4 + (threadIdx.x >> 6));
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
  const float* wrow = a.w + (int64_t)tok * g.K;
  const int32_t* idrow = a.topk + (int64_t)tok * g.K;
  for_each_destination(a.send_head + (int64_t)tok * g.R, g.R, [&](int d, int j) {
    const int64_t sd = (int64_t)s * g.R + d;
    const int64_t off = a.table[sd * 8 + 0];
    const int64_t n = a.cnt_rank[sd];
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
      if (p < P) {
        __builtin_nontemporal_store(cv[i], crow + p);
        if ((lane & 7) == 0) {
          const int64_t gi = (int64_t)j * g.G + (p >> 3);
          if (Q == EP_QUANT_FP8_F32) ((float*)(body + m.off[1]))[gi] = scf[i];
          else (body + m.off[1])[gi] = (uint8_t)sce[i];
        }
      }
    }
    if (piece == 0) store_token_meta(body, m, j, g.K, lane, wrow, idrow, t);
  });
}

template <int NV>
__global__ __launch_bounds__(256) void msg_pack_bf16(MessageArgs a, int V) {
  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63;
  const int tok = uniform(blockIdx.x * 4 + (threadIdx.x >> 6));
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
  for_each_destination(a.send_head + (int64_t)tok * g.R, g.R, [&](int d, int j) {
    const int64_t sd = (int64_t)s * g.R + d;
    const int64_t off = a.table[sd * 8 + 0];
    const int64_t n = a.cnt_rank[sd];
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

__device__ __forceinline__ uint32_t be32(uint32_t v) { return __builtin_bswap32(v); }

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
        write_desc(a.desc + di * 64, wqe, (uint32_t)(s * R + d), (uint64_t)ra,
                   (uint32_t)((d << 16) | (ra / rb)), (uint32_t)c, (uint32_t)((s << 16) | (la / rb)),
                   (uint64_t)la);
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
  hipLaunchKernelGGL((msg_pack_fp8<NP, Q>), dim3((N + 3) / 4, npieces), dim3(256), 0, st, a, P);
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
  hipLaunchKernelGGL(msg_pack_bf16<NV>, dim3((N + 3) / 4, npieces), dim3(256), 0, st, a, V);
}

size_t message_ws_bytes(int R) { return sizeof(int64_t) * 4 * (size_t)R * R; }

hipError_t launch_messages(const MessageArgs& a, hipStream_t st) {
  const int R = a.g.R;
  hipLaunchKernelGGL(msg_table, dim3(1), dim3(1024), 0, st, a);
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
