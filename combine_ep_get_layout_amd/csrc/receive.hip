// Message delivery inside one GPU (loopback descriptor execution) and the
// receiver that unpacks delivered messages into the low-latency layout.
//
// "ibgda_device.cuh" notes, sec. 1, and "GPU-Initiated Communication:
// Dissecting Down to the Bone", WQE anatomy: a write descriptor names a
// local (lkey, laddr) and a remote (rkey, raddr) address and a length; the
// "wire" here is a copy between two arenas in HBM.  Same page, Ordering: the
// store that announces a message (its completion flag) must become visible
// after the message.  "Eaas_server" notes: the receiver reads a loaded
// server's message once its flag has arrived.  "DeepEP" deep dive, sec. 1.2:
// the packed low-latency layout the receiver fills (one block of R*T rows
// per expert, recv_count); sec. 2.1: the per-expert counts ranks exchange
// before the data, which give every source's first slot.
//
// Execute, publication batch 0, two launches:
//   1. every descriptor except the last one of each message (its flag), cut
//      into pieces of at most kPieceBytes; one block per (descriptor, piece)
//      copies with 16-byte vectors through LDS, 64 KiB per round;
//   2. one thread per message copies its flag.
//   The launch boundary puts every payload and header before every flag.
// Execute, publication batch B >= 1, one launch: each workgroup copies a
// run of messages and announces their flags B messages at a time, each
// batch behind a release fence (msg_exec_batched).
// Unpack, one launch: one block of eight wavefronts per (source,
// destination) message.  One thread polls the message's flag with acquire
// loads, at most 1 + spin_limit times, then checks the header and the flag
// (a message that fails is reported and skipped).  The message's
// entries are taken in segments: the wavefronts first rank the segment's
// expert ids, one local expert each, with one ballot per 64 entries (each
// match takes the next slot of its expert after the slots of earlier
// sources and segments); then all eight copy the matched tokens' rows and
// scales to their slots, the segment split evenly over them in tiles of at
// most 64 entries.
#include "ep_device.hpp"
#include "ep_internal.hpp"
#include "msg_format.hpp"

namespace ep {

// One block of 1024 threads per descriptor piece of up to 2 MiB (a whole
// descriptor at the default region size).  Measured on MI355X at the
// 64-rank message workload: 0.395 ms against 0.42-0.47 ms for 256 KiB -
// 1 MiB pieces of 256 - 512 threads (more blocks with nothing to copy) and
// for non-temporal loads and stores.
constexpr int64_t kPieceBytes = 2048 * 1024;
constexpr int kMaxPieces = 64;
constexpr int kExecThreads = 1024;

struct Put {
  int64_t src, dst, len;  // absolute offsets in the send / receive arenas
  int s, d;
};

// Descriptor i (control | remote address | data | pad, big-endian fields).
// Returns 0 when the put may run, else the error bit that rejects it.
__device__ inline int read_put(const ExecArgs& a, int64_t i, Put* p) {
  const u32x4* q = (const u32x4*)(a.desc + i * 64);
  const u32x4 r = q[1], dt = q[2];
  const uint64_t raddr = ((uint64_t)be32(r[0]) << 32) | be32(r[1]);
  const uint32_t rkey = be32(r[2]);
  const uint32_t len = be32(dt[0]);
  const uint32_t lkey = be32(dt[1]);
  const uint64_t laddr = ((uint64_t)be32(dt[2]) << 32) | be32(dt[3]);
  const int R = a.g.R;
  p->s = (int)(lkey >> 16);
  p->d = (int)(rkey >> 16);
  p->len = len;
  if (p->s >= R || p->d >= R) return EP_DEVERR_MESSAGE;
  const int64_t* send_base = a.arena_base;
  const int64_t* recv_base = a.arena_base + R + 1;
  const uint64_t send_sz = (uint64_t)(send_base[p->s + 1] - send_base[p->s]);
  const uint64_t recv_sz = (uint64_t)(recv_base[p->d + 1] - recv_base[p->d]);
  if (laddr > send_sz || len > send_sz - laddr || raddr > recv_sz || len > recv_sz - raddr)
    return EP_DEVERR_CAPACITY;
  p->src = send_base[p->s] + (int64_t)laddr;
  p->dst = recv_base[p->d] + (int64_t)raddr;
  if (p->src + p->len > a.send_cap || p->dst + p->len > a.recv_cap) return EP_DEVERR_CAPACITY;
  return 0;
}

// Copies bytes [lo, hi) of a put with the threads of the block; every
// thread of the block must call it (it synchronises the block).  Aligned
// puts go through LDS in 64 KiB rounds: the block loads a round (each
// thread one vector in flight at a time), then stores it.  Measured on
// MI355X at the 64-rank message workload: 0.7% faster than keeping four
// vectors per thread in flight in registers; 32 KiB rounds gain 0.2% and
// 128 KiB rounds (one block per CU) are 11% slower.
constexpr int kCopyRound = 4096;  // vectors of LDS per block

__device__ inline void copy_range(const ExecArgs& a, const Put& p, int64_t lo, int64_t hi) {
  const uint8_t* src = a.send + p.src;
  uint8_t* dst = a.recv + p.dst;
  if (((p.src | p.dst | lo | hi) & 15) == 0) {
    __shared__ u32x4 stage[kCopyRound];
    const u32x4* s4 = (const u32x4*)(src + lo);
    u32x4* d4 = (u32x4*)(dst + lo);
    const int64_t nv = (hi - lo) / 16;
    for (int64_t c0 = 0; c0 < nv; c0 += kCopyRound) {
      const int n = (int)min((int64_t)kCopyRound, nv - c0);
      // non-temporal loads of the send arena (measured on MI355X at the
      // 64-rank message workload: delivery 4% faster, the receiver after it
      // 1% slower, the step 0.9% faster); plain stores (non-temporal ones
      // made delivery 2% slower)
      for (int j = threadIdx.x; j < n; j += blockDim.x)
        stage[j] = __builtin_nontemporal_load(s4 + c0 + j);
      __syncthreads();
      for (int j = threadIdx.x; j < n; j += blockDim.x) d4[c0 + j] = stage[j];
      __syncthreads();
    }
  } else {
    for (int64_t o = lo + threadIdx.x; o < hi; o += blockDim.x) dst[o] = src[o];
  }
}

__device__ inline int64_t live_descriptors(const ExecArgs& a) {
  const int64_t n = *a.num_desc;
  return n < a.desc_cap ? n : a.desc_cap;
}

// Launch 1: blockIdx.y = piece; block x takes descriptors x, x + gridDim.x,
// ... (the grid is at most kExecMaxBlocks wide, whatever the descriptor
// capacity).  Flags are left to launch 2.
constexpr int64_t kExecMaxBlocks = 65536;

__global__ __launch_bounds__(kExecThreads) void msg_exec_puts(ExecArgs a, int64_t piece) {
  const int64_t live = live_descriptors(a);
  for (int64_t i = blockIdx.x; i < live; i += gridDim.x) {
    Put p;
    const int bad = read_put(a, i, &p);  // uniform across the block
    if (bad) {
      if (blockIdx.y == 0 && threadIdx.x == 0) set_err(a.err, bad);
      continue;
    }
    const int64_t* row = a.table + ((int64_t)p.s * a.g.R + p.d) * 8;
    if (i == row[5] + row[6] - 1) continue;  // the message's flag
    const int64_t lo = (int64_t)blockIdx.y * piece;
    if (lo >= p.len) continue;
    const int64_t hi = lo + piece < p.len ? lo + piece : p.len;
    copy_range(a, p, lo, hi);
  }
}

// Launch 2: one thread per (s, d) message copies the last descriptor of the
// message, its completion flag.
__global__ __launch_bounds__(256) void msg_exec_flags(ExecArgs a) {
  const int R = a.g.R;
  const int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= (int64_t)R * R) return;
  const int64_t* row = a.table + m * 8;
  if (row[3] <= 0 || row[6] <= 0) return;
  const int64_t i = row[5] + row[6] - 1;
  if (i >= live_descriptors(a)) return;
  Put p;
  const int bad = read_put(a, i, &p);
  if (bad) {
    set_err(a.err, bad);
    return;
  }
  // a flag is 16 bytes at a 16-byte aligned offset (one vector); the byte
  // loop covers any other last piece
  if (p.len == 16 && ((p.src | p.dst) & 15) == 0) {
    *(u32x4*)(a.recv + p.dst) = *(const u32x4*)(a.send + p.src);
    return;
  }
  for (int64_t o = 0; o < p.len; ++o) a.recv[p.dst + o] = a.send[p.src + o];
}

// Batched publication (publish_batch = B >= 1), one launch ("GPU-Initiated
// Communication: Dissecting Down to the Bone", Doorbell Batching: one
// notification for a batch of work requests; Sharing a QP: slots reserved,
// filled in parallel, announced in reservation order; "ibgda_device.cuh"
// notes, sec. 4: a doorbell after every few requests).  Workgroup w takes
// the table entries [w * per, (w + 1) * per) in reservation order -- the
// (source, destination) order in which the packer numbered the descriptors
// -- and copies each message's payload and header pieces with all its
// threads.  After every B messages of its run, and after the last, it
// publishes that batch: every thread releases its copies (device-scope
// fence), a workgroup barrier, then the batch's flags, one thread each.  A
// workgroup's batches are thus announced in order, each after its own data;
// no workgroup waits for another.
__device__ inline void publish_flags(const ExecArgs& a, int64_t m_lo, int64_t m_hi,
                                     int64_t live) {
  __threadfence();  // this thread's payload and header stores, device-wide
  __syncthreads();  // ... and every other thread's, before any flag
  for (int64_t m = m_lo + threadIdx.x; m < m_hi; m += blockDim.x) {
    const int64_t* row = a.table + m * 8;
    if (row[3] <= 0 || row[6] <= 0) continue;
    const int64_t i = row[5] + row[6] - 1;
    if (i >= live) continue;
    Put p;
    const int bad = read_put(a, i, &p);
    if (bad) {
      set_err(a.err, bad);
      continue;
    }
    if (p.len == 16 && ((p.src | p.dst) & 15) == 0) {
      *(u32x4*)(a.recv + p.dst) = *(const u32x4*)(a.send + p.src);
    } else {
      for (int64_t o = 0; o < p.len; ++o) a.recv[p.dst + o] = a.send[p.src + o];
    }
  }
}

__global__ __launch_bounds__(kExecThreads) void msg_exec_batched(ExecArgs a, int64_t per) {
  const int64_t rr = (int64_t)a.g.R * a.g.R;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < rr ? lo + per : rr;
  const int64_t live = live_descriptors(a);
  int64_t batch_lo = lo;
  int in_batch = 0;
  for (int64_t m = lo; m < hi; ++m) {  // uniform across the block
    const int64_t* row = a.table + m * 8;
    if (row[3] > 0 && row[6] > 0) {
      const int64_t first = row[5], flag = row[5] + row[6] - 1;
      for (int64_t i = first; i < flag && i < live; ++i) {
        Put p;
        const int bad = read_put(a, i, &p);
        if (bad) {
          if (threadIdx.x == 0) set_err(a.err, bad);
          continue;
        }
        copy_range(a, p, 0, p.len);
      }
      ++in_batch;
    }
    if (in_batch == a.publish_batch || (m == hi - 1 && in_batch > 0)) {
      publish_flags(a, batch_lo, m + 1, live);
      batch_lo = m + 1;
      in_batch = 0;
    }
  }
}

// Unpack: one block per (s, d), ranking and copying as described at the
// top of this file.  Die-aware order: workgroups are dealt to the chip's
// kXcds dies round-robin, so block b runs on die b % kXcds.  Destination d
// is given die d % kXcds, and its messages follow in source order on that
// die: the slots of an expert from consecutive sources are adjacent, and
// their column-major scale stores (4 bytes each, one cache line per
// (expert, group) column run) meet in the same L2 instead of being written
// back as partial lines from eight L2s.

constexpr int kUnpackSeg = 2048;   // entries ranked per round (LDS slots)
constexpr int kUnpackMaxL = 2048;  // local experts (E <= 2048)
constexpr int kUnpackWaves = 8;
constexpr int kUnpackChunk = 16;   // sources per die run under skewed loads

__global__ __launch_bounds__(1024) void msg_unpack(UnpackArgs a) {
  const Geometry& g = a.g;
  const int R = g.R, L = g.L, E = g.E, K = g.K, H = g.H, G = g.G, T = g.T;
  // Block -> (destination d, source s).  Balanced receive loads: each
  // destination's messages run on one die, in source order (the dies take
  // destinations round-robin).  Skewed loads (one destination receiving
  // more than twice the mean bytes, from the receive-arena bases) would
  // overload that die, so there the dies take runs of kUnpackChunk
  // sources of every destination instead.  Every block takes the same
  // decision, so the mapping stays a bijection.
  bool skewed = false;
  if (a.arena_base && R >= 2 * kUnpackChunk) {
    const int64_t* rb = a.arena_base + R + 1;
    int64_t mx = 0;
    for (int q = lane_id(); q < R; q += kWave) mx = max(mx, rb[q + 1] - rb[q]);
    for (int o = 32; o > 0; o >>= 1) mx = max(mx, (int64_t)__shfl_xor(mx, o));
    skewed = mx * R > 2 * rb[R];
  }
  int d, s;
  if (!skewed) {
    const int x = blockIdx.x % kXcds, rest = blockIdx.x / kXcds;
    d = x + kXcds * (rest / R);
    s = rest % R;
  } else {
    const int nch = (R + kUnpackChunk - 1) / kUnpackChunk;
    const int x = blockIdx.x % kXcds, m = blockIdx.x / kXcds;
    const int q = x + kXcds * (m / kUnpackChunk);
    d = q / nch;
    s = (q % nch) * kUnpackChunk + m % kUnpackChunk;
    if (s >= R) return;
  }
  if (d >= R) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int64_t rt = (int64_t)R * T;
  // recv_count of d's experts: written once, by the block of source 0
  if (s == 0) {
    for (int l = wave; l < L; l += nw) {
      int64_t c = 0;
      for (int s2 = lane; s2 < R; s2 += kWave) c += a.cnt_expert[(int64_t)s2 * E + d * L + l];
      for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
      if (lane == 0) a.recv_count[d * L + l] = (int32_t)c;
    }
  }
  const int64_t* row = a.table + ((int64_t)s * R + d) * 8;
  const int64_t n = row[3];
  if (n <= 0) return;
  const int64_t off = row[1], reg = row[2], body = row[4];
  if (off < 0 || off + reg > a.recv_cap) {
    if (threadIdx.x == 0) set_err(a.err, EP_DEVERR_CAPACITY);
    return;
  }
  const MsgSections ms = msg_sections(n, H, K, a.quant);
  const uint8_t* msg = a.arena + off;
  // Slots, in segments of kUnpackSeg entries.  Phase 1: wavefront w ranks
  // the entries of local experts w, w + nw, ... by ballot, in (token, k)
  // order, continuing each expert's count from the earlier segments
  // (run[l], LDS), and records every entry's slot (-1: not on d) and local
  // expert.  Phase 2: the segment's entries are dealt to the wavefronts in
  // equal tiles of at most 64 (a short message gives every wavefront a
  // tile), and each wavefront copies the rows, scales and source index of
  // its tiles' hits.  A tile's source tokens are loaded lane-parallel
  // before its hits, and a hit's scales are loaded with its row, so each
  // hit costs one memory round trip.  Measured on MI355X at the 64-rank
  // message workload (about 31 tokens, 246 entries per message; three
  // interleaved runs each): 0.382 ms against 0.407 ms with 64-entry tiles
  // (four wavefronts busy) and three round trips per hit; blocks of four or
  // sixteen wavefronts take 0.416 and 0.413 ms.
  __shared__ int slot[kUnpackSeg];
  __shared__ int16_t hit_l[kUnpackSeg];  // L <= kUnpackMaxL < 2^15
  __shared__ int run[kUnpackMaxL];
  __shared__ int ok;
  // slots taken by earlier sources; their loads overlap the message check
  // below, which lane 0 of the last wavefront makes
  for (int l = wave; l < L; l += nw) {
    int64_t r = 0;
    for (int s2 = lane; s2 < s; s2 += kWave) r += a.cnt_expert[(int64_t)s2 * E + d * L + l];
    for (int o = 32; o > 0; o >>= 1) r += __shfl_xor(r, o);
    if (lane == 0) run[l] = (int)r;
  }
  if (threadIdx.x == blockDim.x - kWave) {
    // the table's sizes first: they place the flag inside the region
    int good = body == ms.body && reg == 32 + body;
    if (good && a.spin_limit > 0) {
      // poll the flag's first word with acquire loads (the stores it
      // announces become visible with it) until it shows the epoch, at most
      // spin_limit times, sleeping between polls; then check as below
      uint32_t* f0 = (uint32_t*)(uintptr_t)(msg + 16 + body);
      for (int it = 0; it < a.spin_limit &&
                       __hip_atomic_load(f0, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != a.epoch;
           ++it)
        __builtin_amdgcn_s_sleep(8);
    }
    if (good) {
      const u32x4 hd = *(const u32x4*)msg;
      const u32x4 fl = *(const u32x4*)(msg + 16 + body);
      good = hd[0] == (uint32_t)s && hd[1] == (uint32_t)d && hd[2] == (uint32_t)n &&
             hd[3] == (uint32_t)body && fl[0] == a.epoch && fl[1] == 0u && fl[2] == 0u &&
             fl[3] == 0u;
    }
    if (!good) set_err(a.err, EP_DEVERR_MESSAGE);
    ok = good;
  }
  __syncthreads();
  if (!ok) return;
  const uint8_t* b = msg + 16;
  const int32_t* ids = (const int32_t*)(b + ms.off[3]);
  const int32_t* src_tok = (const int32_t*)(b + ms.off[4]);
  const int cb = a.quant == EP_QUANT_NONE ? 2 : 1;
  const int sb = a.quant == EP_QUANT_FP8_F32 ? 4 : (a.quant == EP_QUANT_FP8_UE8M0 ? 1 : 0);
  const int64_t row_bytes = (int64_t)H * cb;
  const int nvec = (int)(row_bytes / 16);
  const int64_t nent = n * K;
  for (int64_t seg0 = 0; seg0 < nent; seg0 += kUnpackSeg) {
    const int nseg = (int)min((int64_t)kUnpackSeg, nent - seg0);
    for (int i = threadIdx.x; i < nseg; i += blockDim.x) slot[i] = -1;
    __syncthreads();
    for (int l = wave; l < L; l += nw) {
      const int e = d * L + l;
      int r = run[l];
      for (int i0 = 0; i0 < nseg; i0 += 4 * kWave) {
        int v[4];  // four loads of ids in flight, then their ballots
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = i0 + q * kWave + lane;
          v[q] = i < nseg ? ids[seg0 + i] : -1;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = i0 + q * kWave + lane;
          const bool hit = v[q] == e;  // e >= 0: lanes past the segment never hit
          const uint64_t hits = __ballot(hit);
          if (hit) {
            slot[i] = r + (int)__popcll(hits & lanes_below());
            hit_l[i] = (int16_t)l;
          }
          r += (int)__popcll(hits);
        }
      }
      if (lane == 0) run[l] = r;
    }
    __syncthreads();
    // entries per tile: the segment split evenly over the wavefronts,
    // rounded up to a multiple of 8, at most 64
    const int tile = min(kWave, ((nseg + nw - 1) / nw + 7) & ~7);
    for (int i0 = wave * tile; i0 < nseg; i0 += nw * tile) {
      const int ii = i0 + lane;
      const int myslot = lane < tile && ii < nseg ? slot[ii] : -1;
      const int myl = myslot >= 0 ? hit_l[ii] : 0;
      const int myt = myslot >= 0 ? src_tok[(seg0 + ii) / K] : 0;
      uint64_t hits = __ballot(myslot >= 0);
      while (hits) {  // in (token, k) order within the tile
        const int hl = __builtin_ctzll(hits);
        hits &= hits - 1;
        const int64_t j = (seg0 + i0 + hl) / K;
        const int64_t pos = __builtin_amdgcn_readlane(myslot, hl);
        if (pos >= rt) {
          if (lane == 0) set_err(a.err, EP_DEVERR_LL_OVERFLOW);
          continue;
        }
        const int t = __builtin_amdgcn_readlane(myt, hl);
        if (t < 0 || t >= T) {
          if (lane == 0) set_err(a.err, EP_DEVERR_MESSAGE);
          continue;
        }
        const int e = d * L + __builtin_amdgcn_readlane(myl, hl);
        const int64_t r = (int64_t)e * rt + pos;
        const u32x4* sv = (const u32x4*)(b + ms.off[0] + j * row_bytes);
        u32x4* dv = (u32x4*)((uint8_t*)a.recv_x + r * row_bytes);
        const float* sf = (const float*)(b + ms.off[1]) + j * G;
        const uint8_t* su = b + ms.off[1] + j * G;
        // the first 64 scales go out with the row's loads
        const float f0 = sb == 4 && lane < G ? sf[lane] : 0.0f;
        const uint8_t u0 = sb == 1 && lane < G ? su[lane] : (uint8_t)0;
        // eight vectors per lane in flight; non-temporal loads and stores
        // keep the message bodies and unpacked rows from displacing the
        // caches.  Measured on MI355X: non-temporal stores make the next
        // step's delivery 4.5% faster.  Non-temporal loads make the unpack
        // 5.6% faster, and cut its HBM writes from 1.22 to 1.06 GB: the
        // 4-byte column-major scale stores then stay in L2 until whole lines
        // are written back.
        for (int v0 = lane; v0 < nvec; v0 += 8 * kWave) {
          u32x4 tv[8];
#pragma unroll
          for (int q = 0; q < 8; ++q)
            tv[q] = __builtin_nontemporal_load(sv + min(v0 + q * kWave, nvec - 1));
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (v0 + q * kWave < nvec) __builtin_nontemporal_store(tv[q], dv + v0 + q * kWave);
        }
        if (sb == 4) {
          float* col = (float*)a.recv_scales + (int64_t)e * G * rt + pos;
          if (lane < G) col[(int64_t)lane * rt] = f0;
          for (int q = lane + kWave; q < G; q += kWave) col[(int64_t)q * rt] = sf[q];
        } else if (sb == 1) {
          uint8_t* col = (uint8_t*)a.recv_scales + (int64_t)e * G * rt + pos;
          if (lane < G) col[(int64_t)lane * rt] = u0;
          for (int q = lane + kWave; q < G; q += kWave) col[(int64_t)q * rt] = su[q];
        }
        if (lane == 0) a.recv_src_idx[r] = (int32_t)((int64_t)s * T + t);
      }
    }
    __syncthreads();  // slot[] is reused by the next segment
  }
}

// Workgroups of the batched form: two 1024-thread groups per compute unit.
constexpr int64_t kBatchedGroups = 512;

hipError_t launch_execute(const ExecArgs& a, hipStream_t st) {
  const int R = a.g.R;
  if (a.publish_batch > 0) {
    const int64_t rr = (int64_t)R * R;
    const int64_t per = (rr + kBatchedGroups - 1) / kBatchedGroups;
    const int64_t groups = (rr + per - 1) / per;
    hipLaunchKernelGGL(msg_exec_batched, dim3((unsigned)groups), dim3(kExecThreads), 0, st, a,
                       per);
    return hipGetLastError();
  }
  // pieces of at least kPieceBytes, at most kMaxPieces per descriptor (a
  // descriptor never exceeds region_bytes)
  int64_t piece = kPieceBytes;
  const int64_t min_piece = pad16((a.region_bytes + kMaxPieces - 1) / kMaxPieces);
  if (piece < min_piece) piece = min_piece;
  const int64_t pieces = (a.region_bytes + piece - 1) / piece;
  if (a.desc_cap > 0) {
    const int64_t blocks = a.desc_cap < kExecMaxBlocks ? a.desc_cap : kExecMaxBlocks;
    hipLaunchKernelGGL(msg_exec_puts, dim3((unsigned)blocks, (unsigned)pieces),
                       dim3(kExecThreads), 0, st, a, piece);
  }
  const int64_t rr = (int64_t)R * R;
  hipLaunchKernelGGL(msg_exec_flags, dim3((unsigned)((rr + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_unpack(const UnpackArgs& a, hipStream_t st) {
  const int R = a.g.R;
  const int waves = kUnpackWaves;
  // enough blocks for either mapping of (d, s) pairs
  const int nch = (R + kUnpackChunk - 1) / kUnpackChunk;
  const int64_t by_dest = (int64_t)kXcds * ((R + kXcds - 1) / kXcds) * R;
  const int64_t by_chunk = (int64_t)kXcds * ((R * nch + kXcds - 1) / kXcds) * kUnpackChunk;
  const unsigned blocks = (unsigned)(by_dest > by_chunk ? by_dest : by_chunk);
  hipLaunchKernelGGL(msg_unpack, dim3(blocks), dim3(kWave * waves), 0, st, a);
  return hipGetLastError();
}

}  // namespace ep
