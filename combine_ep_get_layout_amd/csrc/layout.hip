// Routing layout on gfx950: per-rank / per-expert histograms, the rank
// prefix matrix, receive offsets and deterministic slots.
//
// "DeepEP" deep dive (llm-infra-atlas, moe/06_deepep), sec. 2.1 (counts,
// rank prefix matrix, expert_alignment), sec. 2.3 (send_head /
// recv_src_idx address book), sec. 3.2 (rank of an expert), sec. 4.3
// (per-expert prefix sums as segment offsets).
//
// Small problems (up to a few thousand (token, k) entries, outside
// rank-major mode): one launch (layout_direct, below).  Larger problems take
// three launches, all small next to the data movement they enable (the
// fused dispatch takes over the third):
//   1. count   : one wavefront per token chunk.  Entries of a batch (one per
//                lane, in (token, k) order) find their equal-key peers with
//                one ballot per key bit; the lowest lane of each key advances
//                that key's counter in LDS.  This gives every entry its rank
//                among same-expert entries of the chunk, and every first hit
//                of a token on a rank its rank among the chunk's tokens sent
//                there.  No atomics decide positions: slots are deterministic.
//   2. scan    : one block per expert (chunk histogram -> exclusive prefix
//                over (source rank, chunk)) and one per destination rank
//                (token counts, the rank prefix matrix column, chunk prefixes).
//   3. finalize: every block scans the per-expert counts (rounded up to
//                expert_alignment) into segment starts in LDS; slot = segment
//                start + chunk prefix + rank in chunk; block 0 publishes the
//                starts, rows per rank and row bases.  Rank-major mode: slot
//                = partition base + exclusive rank prefix + stream index.
#include "ep_device.hpp"
#include "ep_internal.hpp"
#include "layout_rows.hpp"

namespace ep {

constexpr int kLayoutWaves = 4;       // most wavefronts (chunks) per count block
constexpr int kCountBlocks = 256;     // count blocks wanted before blocks grow past one wave

// Count one chunk of source rank s (tokens [t_begin, t_end)) with one
// wavefront.  cnt_e[E], cnt_r[R] (LDS, zeroed here) end up holding the
// chunk's histograms; rowbuf[tb*R] is scratch.  Writes each entry's rank
// in its chunk (local_e) and each token's per-rank stream rank in its
// chunk (local_r, -1 when not sent), and is_token_in_rank.
__device__ void count_chunk(const LayoutArgs& a, int s, int t_begin, int t_end, int32_t* cnt_e,
                            int32_t* cnt_r, int32_t* rowbuf) {
  const Geometry& g = a.g;
  const int lane = lane_id();
  for (int i = lane; i < g.E + g.R; i += kWave) cnt_e[i] = 0;  // cnt_r follows cnt_e
  // the row buffer starts cleared; each batch's read-out clears it again
  for (int i = lane; i < g.tb * g.R; i += kWave) rowbuf[i] = -1;
  wave_lds_sync();  // zeroed counters and cleared rows before any lane reads them
  const int K = g.K;
  const int my_tok = lane / K, my_k = lane % K;
  const int nent = g.tb * K;
  // lanes of my own token below me
  const int first_lane = my_tok * K;
  const uint64_t below = lanes_below();
  const uint64_t own_below = below & ~(first_lane == 0 ? 0ull : (~0ull >> (64 - first_lane)));
  const int nb = (t_end - t_begin + g.tb - 1) / g.tb;

  // the expert ids of the chunk's batches (at most kMaxChunkBatches) are
  // loaded together, so it pays one memory latency instead of one per batch
  // (a 16-batch buffer before chunks were capped at 8 batches: 72 VGPRs
  // against 56, decode-shape count 4.50 against 4.34 us on MI355X)
  for (int b0 = 0; b0 < nb; b0 += kMaxChunkBatches) {
    int pre[kMaxChunkBatches];
#pragma unroll
    for (int q = 0; q < kMaxChunkBatches; ++q) {
      const int t = t_begin + (b0 + q) * g.tb + my_tok;
      const bool in_batch = b0 + q < nb && lane < nent && t < t_end;
      pre[q] = in_batch ? a.topk[((int64_t)s * g.T + t) * K + my_k] : -1;
    }
#pragma unroll
    for (int q = 0; q < kMaxChunkBatches; ++q) {
      if (b0 + q >= nb) break;
      const int t0 = t_begin + (b0 + q) * g.tb;
      const int t = t0 + my_tok;
      const bool in_batch = lane < nent && t < t_end;
      const int64_t ent = ((int64_t)s * g.T + t) * K + my_k;
      const int e = pre[q];
      const bool valid = in_batch && e >= 0 && e < g.E;
      const uint64_t vmask = __ballot(valid);

      // expert level: rank among same-expert entries of this chunk
      const uint64_t eq = match_key(valid ? (uint32_t)e : 0u, g.ebits, vmask);
      int slot = -1;
      if (valid) {
        slot = cnt_e[e] + rank_below(eq);
        if ((eq & below) == 0) cnt_e[e] = slot + (int)__popcll(eq);
      }
      if (in_batch) a.local_e[ent] = slot;

      // rank level: first entry of a token on each rank, and that token's
      // rank among the chunk's tokens sent to the rank
      const int r = valid ? e / g.L : 0;
      const uint64_t eqr = match_key((uint32_t)r, g.rbits, vmask);
      const bool first = valid && (eqr & own_below) == 0;
      const uint64_t eqf = eqr & __ballot(first);
      if (first) {
        const int h = cnt_r[r] + rank_below(eqf);
        rowbuf[my_tok * g.R + r] = h;
        if ((eqf & below) == 0) cnt_r[r] = h + (int)__popcll(eqf);
      }
      wave_lds_sync();  // the first hits before the row buffer is read out
      const int nt = min(g.tb, t_end - t0);
      const int64_t rbase = ((int64_t)s * g.T + t0) * g.R;
      for (int i = lane; i < nt * g.R; i += kWave) {
        const int v = rowbuf[i];
        rowbuf[i] = -1;  // cleared for the next batch (rows past nt stay cleared)
        a.in_rank[rbase + i] = v >= 0 ? 1 : 0;
        a.local_r[rbase + i] = v;
      }
      // counters advanced by one lane and the row buffer read out and
      // cleared, before the next batch reads the counters and fills it
      wave_lds_sync();
    }
  }
}

__global__ __launch_bounds__(256) void layout_count(LayoutArgs a) {
  extern __shared__ int32_t smem[];
  const Geometry& g = a.g;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.x * (blockDim.x >> 6) + wave;
  if (chunk >= g.NC) return;  // uniform per wave
  const int per_wave = g.E + g.R + g.tb * g.R;
  int32_t* cnt_e = smem + wave * per_wave;
  int32_t* cnt_r = cnt_e + g.E;
  int32_t* rowbuf = cnt_r + g.R;
  const int s = chunk / g.C, c = chunk % g.C;
  const int t_begin = c * g.ct;
  count_chunk(a, s, t_begin, min(g.T, t_begin + g.ct), cnt_e, cnt_r, rowbuf);
  for (int e = lane; e < g.E; e += kWave) a.hist_e[(int64_t)e * g.NC + chunk] = cnt_e[e];
  for (int d = lane; d < g.R; d += kWave) a.hist_r[(int64_t)d * g.NC + chunk] = cnt_r[d];
}

// Exclusive scan, in place, of a row of n = nseg * seg ints; seg_start[j]
// (LDS) receives the prefix at the start of segment j and seg_start[nseg]
// the total.  With `relative`, each element is made relative to its
// segment's start.  A thread's PER elements (PER >= per, its share) are
// loaded together into registers and each final value is stored once: a
// loop that adds each loaded element before loading the next waits for one
// memory round trip per element.  (Measured on MI355X, three interleaved
// runs each: prefill layout 23.5 -> 22.9 us, 64-rank message layout 27.1 ->
// 26.3 us; with it, 2048 or 4096 target chunks are still slower than 1024.)
template <int PER>
__device__ __forceinline__ void scan_row_reg(int32_t* row, int n, int nseg, int seg, int per, int* seg_start,
                             bool relative) {
  const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
  int v[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int x = row[min(lo + q, n - 1)];  // unconditional, in bounds (n >= 1)
    v[q] = lo + q < hi ? x : 0;
  }
  int sum = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) sum += v[q];
  int total;
  int run = block_exclusive_scan(sum, &total);
  int pre[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = lo + q;
    pre[q] = run;
    if (i < hi && i % seg == 0) seg_start[i / seg] = run;
    run += v[q];
  }
  if (threadIdx.x == 0) seg_start[nseg] = total;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = lo + q;
    if (i < hi) row[i] = relative ? pre[q] - seg_start[i / seg] : pre[q];
  }
}

__device__ __forceinline__ void scan_row_segments(int32_t* row, int nseg, int seg, int* seg_start,
                                                  bool relative) {
  const int n = nseg * seg;
  for (int j = threadIdx.x; j <= nseg; j += blockDim.x) seg_start[j] = 0;  // empty rows
  __syncthreads();
  if (n == 0) return;
  const int per = (n + blockDim.x - 1) / blockDim.x;
  if (per <= 1) return scan_row_reg<1>(row, n, nseg, seg, per, seg_start, relative);
  if (per <= 2) return scan_row_reg<2>(row, n, nseg, seg, per, seg_start, relative);
  if (per <= 4) return scan_row_reg<4>(row, n, nseg, seg, per, seg_start, relative);
  if (per <= 8) return scan_row_reg<8>(row, n, nseg, seg, per, seg_start, relative);
  // longer rows: element by element
  const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += row[i];
  int total;
  int run = block_exclusive_scan(sum, &total);
  for (int i = lo; i < hi; ++i) {
    const int v = row[i];
    row[i] = run;
    if (i % seg == 0) seg_start[i / seg] = run;
    run += v;
  }
  if (threadIdx.x == 0) seg_start[nseg] = total;
  __syncthreads();
  if (relative)
    for (int i = lo; i < hi; ++i) row[i] -= seg_start[i / seg];
}

// Blocks [0, E): expert e's chunk histogram over (source, chunk) becomes
// its exclusive prefix = rows of earlier sources and chunks; per-source
// counts and the expert's receive total fall out of the segment starts.
// Blocks [E, E+R): destination d's token histogram over (source, chunk):
// per-source totals (num_tokens_per_rank), the inclusive prefix over
// sources (rank_prefix_matrix column d), and per-source chunk prefixes.
__global__ __launch_bounds__(1024) void layout_scan(LayoutArgs a) {
  __shared__ int seg_start[257];
  const Geometry& g = a.g;
  const int b = blockIdx.x;
  // errors are raised only by the finalize launch that follows
  if (b == 0 && threadIdx.x == 0) *a.err = 0;
  if (b < g.E) {
    const int e = b;
    scan_row_segments(a.hist_e + (int64_t)e * g.NC, g.R, g.C, seg_start, false);
    for (int s = threadIdx.x; s < g.R; s += blockDim.x)
      a.cnt_expert[(int64_t)s * g.E + e] = seg_start[s + 1] - seg_start[s];
    if (threadIdx.x == 0) a.recv_per_expert[e] = seg_start[g.R];
  } else {
    const int d = b - g.E;
    scan_row_segments(a.hist_r + (int64_t)d * g.NC, g.R, g.C, seg_start, true);
    for (int s = threadIdx.x; s < g.R; s += blockDim.x) {
      a.cnt_rank[s * g.R + d] = seg_start[s + 1] - seg_start[s];
      a.rpm[s * g.R + d] = seg_start[s + 1];
    }
  }
}

// Slots: row = segment start + (source, chunk) prefix + rank in chunk, and
// the token streams' indices.  Block 0 also publishes the segment starts,
// rows per rank and row bases; padding rows get recv_src_idx = -1.
// hist_e / hist_r: the scanned chunk histograms ([E][NC], [R][NC]), in
// global memory or LDS.
struct FirstItems {
  int e, local, head;
};

__device__ void finalize_body(const LayoutArgs& a, const int* start, const int* rbase,
                              const int32_t* hist_e, const int32_t* hist_r,
                              const FirstItems& pre) {
  const Geometry& g = a.g;
  const bool rank_major = a.mode == EP_MODE_RANK_MAJOR;
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e < g.E; e += blockDim.x) a.expert_start[e] = start[e];
    for (int d = threadIdx.x; d <= g.R; d += blockDim.x) {
      const int b0 = rank_major ? rbase[d] : start[d * g.L];
      a.row_base[d] = b0;
      if (d < g.R) a.rows[d] = (rank_major ? rbase[d + 1] : start[(d + 1) * g.L]) - b0;
    }
  }
  if (a.mode == EP_MODE_NORMAL && a.recv_src_idx && a.align > 1) {
    for (int e = blockIdx.x; e < g.E; e += gridDim.x) {
      const int first = start[e] + a.recv_per_expert[e];
      for (int r = first + (int)threadIdx.x; r < start[e + 1]; r += blockDim.x)
        if (r < a.recv_cap) a.recv_src_idx[r] = -1;
    }
  }
  const int64_t n_ent = (int64_t)g.R * g.T * g.K;
  // rank-major rows come from the stream indices, needed even without send_head
  const int64_t n_head = (a.send_head || rank_major) ? (int64_t)g.R * g.T * g.R : 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // one index walks both the (token, k) entries and the (token, rank) heads,
  // so their chunk-prefix gathers are in flight together
  const int64_t n_all = n_ent > n_head ? n_ent : n_head;
  // Each iteration loads the next one's entry and head first (unconditional
  // loads, clamped into the arrays), so an item waits for one round trip,
  // its chunk-prefix gather, instead of two (measured on MI355X at 64 ranks,
  // four items per thread, kernel traces: 9.35 -> 8.90 us).
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  FirstItems cur = pre;
  for (int64_t i = i0; i < n_all; i += stride) {
    const int64_t in = i + stride;
    const int e_n = a.topk[in < n_ent ? in : 0];
    const int local_n = a.local_e[in < n_ent ? in : 0];
    const int head_n = a.local_r[in < n_head ? in : 0];
    const bool is_ent = i < n_ent, is_head = i < n_head;
    const int e = is_ent ? cur.e : 0;
    const int local = is_ent ? cur.local : -1;
    int v = is_head ? cur.head : -1;
    cur = FirstItems{e_n, in < n_ent ? local_n : -1, in < n_head ? head_n : -1};
    if (is_ent) {
      if (e < -1 || e >= g.E) set_err(a.err, EP_DEVERR_TOPK_RANGE);
      int row = -1;
      if (local >= 0) {
        const int64_t st = i / g.K;  // s * T + t
        const int s = (int)(st / g.T), t = (int)(st % g.T);
        if (rank_major) {
          // the token's row on the expert's rank: its stream index there
          const int d = e / g.L;
          const int64_t hi = st * g.R + d;
          const int head = a.local_r[hi] + hist_r[(int64_t)d * g.NC + s * g.C + t / g.ct];
          row = rbase[d] + a.rpm[s * g.R + d] - a.cnt_rank[s * g.R + d] + head;
        } else {
          row = entry_row(a, start[e], hist_e, st, e, local);
          if (row >= 0 && a.mode != EP_MODE_MESSAGES && a.recv_src_idx) {
            if (row < a.recv_cap) a.recv_src_idx[row] = (int)st;
            else set_err(a.err, EP_DEVERR_CAPACITY);
          }
        }
      }
      if (a.send_pos) a.send_pos[i] = (a.mode == EP_MODE_MESSAGES) ? -1 : row;
    }
    if (is_head) {
      if (v >= 0) {
        const int64_t st = i / g.R;
        const int d = (int)(i % g.R);
        const int s = (int)(st / g.T);
        v = stream_index(a, hist_r, st, d, v);
        if (rank_major && a.recv_src_idx) {
          const int row = rbase[d] + a.rpm[s * g.R + d] - a.cnt_rank[s * g.R + d] + v;
          if (row < a.recv_cap) a.recv_src_idx[row] = (int)st;
          else set_err(a.err, EP_DEVERR_CAPACITY);
        }
      }
      if (a.send_head) a.send_head[i] = v;
    }
  }
}

// A thread's first entry and head, loaded before the segment-start scan so
// that their memory latency overlaps it.
__device__ FirstItems first_items(const LayoutArgs& a) {
  const Geometry& g = a.g;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  FirstItems f{0, -1, -1};
  if (i0 < (int64_t)g.R * g.T * g.K) {
    f.e = a.topk[i0];
    f.local = a.local_e[i0];
  }
  if ((a.send_head || a.mode == EP_MODE_RANK_MAJOR) && i0 < (int64_t)g.R * g.T * g.R)
    f.head = a.local_r[i0];
  return f;
}

__global__ __launch_bounds__(256) void layout_finalize(LayoutArgs a) {
  __shared__ int start[2049];
  __shared__ int rbase[257];
  const FirstItems pre = first_items(a);
  if (a.mode == EP_MODE_RANK_MAJOR) rank_bases(a, start, rbase);
  else segment_starts(a, start);
  finalize_body(a, start, rbase, a.hist_e, a.hist_r, pre);
}

// Small problems (at most kDirectPer entries per thread of one 1024-thread
// block): one launch.  Each of the first ceil(E / kDirectExperts) blocks
// takes kDirectExperts experts and finds the rank of every entry routed to
// each of them among all such entries in (source, token, k) order, with one
// block scan over all entries; each of the last R blocks does the same for
// the tokens sent to one rank.  Every block reads all entries (a few tens of
// KB, served by the caches), which at this size costs less than chunk
// histograms and two more launches.  Block 0 also histograms all experts,
// derives every error condition from the histogram and writes the error
// word once.
constexpr int kDirectPer = 16;
constexpr int kDirectThreads = 1024;
constexpr int kDirectExperts = 4;

// Exclusive block scan of N ints per thread at once (kDirectThreads
// threads); total[j] receives the block sums.
template <int N>
__device__ void block_exclusive_scan_n(int (&v)[N], int (&total)[N]) {
  __shared__ int wsum[16][N];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl[N];
#pragma unroll
  for (int j = 0; j < N; ++j) incl[j] = v[j];
  for (int o = 1; o < kWave; o <<= 1) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int n = __shfl_up(incl[j], o);
      if (lane >= o) incl[j] += n;
    }
  }
  if (lane == kWave - 1)
#pragma unroll
    for (int j = 0; j < N; ++j) wsum[wave][j] = incl[j];
  __syncthreads();
  const int nw = blockDim.x >> 6;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    int before = 0, all = 0;
    for (int w = 0; w < nw; ++w) {
      const int x = wsum[w][j];
      if (w < wave) before += x;
      all += x;
    }
    total[j] = all;
    v[j] = before + incl[j] - v[j];
  }
  __syncthreads();
}

__device__ void direct_expert_block(const LayoutArgs& a, int e0, int* hist, int* starts,
                                    int (*src_prefix)[257], int* err_bits) {
  const Geometry& g = a.g;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int M = g.R * g.T * g.K, TK = g.T * g.K, rt = g.R * g.T;
  const bool ll = a.mode == EP_MODE_LOW_LATENCY, msg = a.mode == EP_MODE_MESSAGES;
  const bool first = e0 == 0;
  const bool need_hist = first || !ll;
  const int per = (M + nth - 1) / nth;  // <= kDirectPer
  const int lo = min(M, tid * per), hi = min(M, lo + per);
  int ids[kDirectPer];
#pragma unroll
  for (int q = 0; q < kDirectPer; ++q) ids[q] = lo + q < hi ? a.topk[lo + q] : -1;
  if (need_hist)
    for (int i = tid; i < g.E; i += nth) hist[i] = 0;
  if (first && tid == 0) *err_bits = 0;
  __syncthreads();
  int cnt[kDirectExperts];
#pragma unroll
  for (int j = 0; j < kDirectExperts; ++j) cnt[j] = 0;
  int bad = 0;
#pragma unroll
  for (int q = 0; q < kDirectPer; ++q) {
    if (lo + q >= hi) continue;  // lo + q only grows: every later entry is out too
    const int id = ids[q];
#pragma unroll
    for (int j = 0; j < kDirectExperts; ++j) cnt[j] += id == e0 + j;
    if (id < -1 || id >= g.E) bad = 1;
    else if (need_hist && id >= 0) atomicAdd(&hist[id], 1);
  }
  if (first && bad) atomicOr(err_bits, EP_DEVERR_TOPK_RANGE);
  int total[kDirectExperts];
  block_exclusive_scan_n<kDirectExperts>(cnt, total);  // cnt: prefix; orders the histogram
  // segment starts: fixed blocks of R*T rows (low-latency), else the
  // exclusive scan of the counts rounded up to expert_alignment
  if (!ll) {
    const int pe = (g.E + nth - 1) / nth;
    const int elo = min(g.E, tid * pe), ehi = min(g.E, elo + pe);
    int sum = 0;
    for (int i = elo; i < ehi; ++i) sum += (hist[i] + a.align - 1) / a.align * a.align;
    int all;
    int run = block_exclusive_scan(sum, &all);
    for (int i = elo; i < ehi; ++i) {
      starts[i] = run;
      run += (hist[i] + a.align - 1) / a.align * a.align;
    }
    if (tid == 0) starts[g.E] = all;
    __syncthreads();
  }
  int start_e[kDirectExperts];
#pragma unroll
  for (int j = 0; j < kDirectExperts; ++j)
    start_e[j] = e0 + j >= g.E ? 0 : (ll ? (e0 + j) * rt : starts[e0 + j]);
  // rows of these experts' entries, and the per-source prefixes of their
  // counts; (source boundary, token, k) tracked incrementally
  int next_src = TK > 0 ? (lo + TK - 1) / TK : 0;  // first source starting at or after lo
  int tok = g.K > 0 ? lo / g.K : 0, kk = lo - tok * g.K;
#pragma unroll
  for (int q = 0; q < kDirectPer; ++q) {
    const int i = lo + q;
    if (i >= hi) break;
    if (i == next_src * TK) {
#pragma unroll
      for (int j = 0; j < kDirectExperts; ++j) src_prefix[j][next_src] = cnt[j];
      ++next_src;
    }
    const int id = ids[q];
    const int j = id - e0;
    if (j >= 0 && j < kDirectExperts && id < g.E) {
      int pos = 0, st = 0;
#pragma unroll
      for (int jj = 0; jj < kDirectExperts; ++jj)
        if (jj == j) {
          pos = cnt[jj]++;
          st = start_e[jj];
        }
      const int row = ll ? (pos < rt ? st + pos : -1) : st + pos;
      if (!msg && row >= 0 && a.recv_src_idx && row < a.recv_cap) a.recv_src_idx[row] = tok;
      if (a.send_pos) a.send_pos[i] = msg ? -1 : row;
    } else if (first && (id < 0 || id >= g.E) && a.send_pos) {
      a.send_pos[i] = -1;  // masked or out-of-range entries
    }
    if (++kk == g.K) {
      kk = 0;
      ++tok;
    }
  }
  if (tid == 0)
#pragma unroll
    for (int j = 0; j < kDirectExperts; ++j) src_prefix[j][g.R] = total[j];
  if (M == 0)
    for (int s2 = tid; s2 < g.R; s2 += nth)
#pragma unroll
      for (int j = 0; j < kDirectExperts; ++j) src_prefix[j][s2] = 0;
  __syncthreads();
  const int ne = min(kDirectExperts, g.E - e0);
  for (int x = tid; x < g.R * ne; x += nth) {
    const int s2 = x / ne, j = x - s2 * ne;
    a.cnt_expert[(int64_t)s2 * g.E + e0 + j] = src_prefix[j][s2 + 1] - src_prefix[j][s2];
  }
  if (tid < ne) {
    a.recv_per_expert[e0 + tid] = src_prefix[tid][g.R];
    a.expert_start[e0 + tid] = ll ? (e0 + tid) * rt : starts[e0 + tid];
  }
  // alignment padding rows of these segments
  if (!ll && !msg && a.recv_src_idx && a.align > 1) {
    for (int j = 0; j < ne; ++j) {
      const int n = src_prefix[j][g.R], st = starts[e0 + j];
      const int end = st + (n + a.align - 1) / a.align * a.align;
      for (int r = st + n + tid; r < end; r += nth)
        if (r < a.recv_cap) a.recv_src_idx[r] = -1;
    }
  }
  if (!first) return;
  // block 0: rows per rank, row bases and the error word
  for (int d = tid; d <= g.R; d += nth) {
    const int base = ll ? d * g.L * rt : starts[d * g.L];
    a.row_base[d] = base;
    if (d < g.R) a.rows[d] = ll ? g.L * rt : starts[(d + 1) * g.L] - base;
  }
  int bits = 0;
  for (int i = tid; i < g.E; i += nth) {
    const int n = hist[i];
    if (ll && n > rt) bits |= EP_DEVERR_LL_OVERFLOW;
    const int used = ll ? min(n, rt) : n;
    const int64_t top = (ll ? (int64_t)i * rt : (int64_t)starts[i]) + used;
    if (!msg && a.recv_src_idx && used > 0 && top > a.recv_cap) bits |= EP_DEVERR_CAPACITY;
  }
  if (bits) atomicOr(err_bits, bits);
  __syncthreads();
  if (tid == 0) *a.err = *err_bits;
}

__device__ void direct_rank_block(const LayoutArgs& a, int d, int* src_prefix) {
  const Geometry& g = a.g;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int N = g.R * g.T;
  const int per = (N + nth - 1) / nth;  // <= kDirectPer
  const int lo = min(N, tid * per), hi = min(N, lo + per);
  const int e_lo = d * g.L, e_hi = e_lo + g.L;  // experts on rank d
  // bit q: token lo + q has an expert on rank d
  uint32_t flags = 0;
  for (int q = 0; q < hi - lo; ++q) {
    const int32_t* ids = a.topk + (int64_t)(lo + q) * g.K;
    int f = 0;
    for (int k0 = 0; k0 < g.K; k0 += 8) {  // eight loads in flight at a time
      int v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = k0 + j < g.K ? ids[k0 + j] : -1;
#pragma unroll
      for (int j = 0; j < 8; ++j) f |= v[j] >= e_lo && v[j] < e_hi;
    }
    flags |= (uint32_t)f << q;
  }
  const int cnt = __popc(flags);
  int total;
  int run = block_exclusive_scan(cnt, &total);
  const int run0 = run;
  int next_src = g.T > 0 ? (lo + g.T - 1) / g.T : 0;
  for (int q = 0; q < hi - lo; ++q) {
    if (lo + q == next_src * g.T) src_prefix[next_src++] = run;
    run += (flags >> q) & 1;
  }
  if (tid == 0) src_prefix[g.R] = total;
  if (N == 0)
    for (int s2 = tid; s2 < g.R; s2 += nth) src_prefix[s2] = 0;
  __syncthreads();
  run = run0;
  int src = g.T > 0 ? lo / g.T : 0, t = lo - src * g.T;
  for (int q = 0; q < hi - lo; ++q) {
    const int f = (flags >> q) & 1;
    const int64_t at = (int64_t)(lo + q) * g.R + d;
    a.in_rank[at] = (uint8_t)f;
    if (a.send_head) a.send_head[at] = f ? run - src_prefix[src] : -1;
    run += f;
    if (++t == g.T) {
      t = 0;
      ++src;
    }
  }
  for (int s2 = tid; s2 < g.R; s2 += nth) {
    a.cnt_rank[s2 * g.R + d] = src_prefix[s2 + 1] - src_prefix[s2];
    a.rpm[s2 * g.R + d] = src_prefix[s2 + 1];
  }
}

__global__ __launch_bounds__(kDirectThreads) void layout_direct(LayoutArgs a) {
  __shared__ int hist[2048];
  __shared__ int starts[2049];
  __shared__ int src_prefix[kDirectExperts][257];
  __shared__ int err_bits;
  const int eb = (a.g.E + kDirectExperts - 1) / kDirectExperts;
  if ((int)blockIdx.x < eb)
    direct_expert_block(a, blockIdx.x * kDirectExperts, hist, starts, src_prefix, &err_bits);
  else
    direct_rank_block(a, blockIdx.x - eb, src_prefix[0]);
}

hipError_t launch_layout_counts(const LayoutArgs& a, hipStream_t stream) {
  const Geometry& g = a.g;
  // LDS per wavefront: expert and rank counters plus one batch of rows;
  // at most 64 KiB per block, and blocks for every CU where there are
  // chunks enough (measured on MI355X: four waves per block are 1 us faster
  // than one or two at 1,024 chunks; one wave per block makes the
  // low-latency decode step, 128 chunks, 1% faster than four)
  const size_t per_wave = sizeof(int32_t) * (size_t)(g.E + g.R + g.tb * g.R);
  int waves = (int)(65536 / per_wave);
  if (waves > kLayoutWaves) waves = kLayoutWaves;
  if (waves > g.NC / kCountBlocks) waves = g.NC / kCountBlocks;
  if (waves < 1) waves = 1;
  const int nb = (g.NC + waves - 1) / waves;
  if (nb > 0)
    hipLaunchKernelGGL(layout_count, dim3(nb), dim3(64 * waves), per_wave * waves, stream, a);
  // up to 512 threads (measured on MI355X at 1024 chunks: two elements per
  // thread is 1 us faster than one element on each of 1024 threads, and
  // than four on each of 256)
  int scan_threads = (g.NC + kWave - 1) / kWave * kWave;
  if (scan_threads < 256) scan_threads = 256;
  if (scan_threads > 512) scan_threads = 512;
  hipLaunchKernelGGL(layout_scan, dim3(g.E + g.R), dim3(scan_threads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream) {
  const Geometry& g = a.g;
  if (g.direct && (int64_t)g.R * g.T * g.K <= (int64_t)kDirectPer * kDirectThreads) {
    const int eb = (g.E + kDirectExperts - 1) / kDirectExperts;
    hipLaunchKernelGGL(layout_direct, dim3(eb + g.R), dim3(kDirectThreads), 0, stream, a);
    return hipGetLastError();
  }
  hipError_t e = launch_layout_counts(a, stream);
  if (e != hipSuccess) return e;
  const int64_t work = (int64_t)g.R * g.T * (g.K > g.R ? g.K : g.R);
  // a thread per item, at most 1024 blocks: every block first scans the
  // segment starts, so past that more items per thread are cheaper than
  // more blocks (measured on MI355X: the 64-rank message layout is 3.7 us
  // faster with 1024 blocks of four items per thread than with 4096)
  int64_t fb = (work + 255) / 256;
  if (fb > 1024) fb = 1024;
  if (fb < 1) fb = 1;
  hipLaunchKernelGGL(layout_finalize, dim3((unsigned)fb), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ep
