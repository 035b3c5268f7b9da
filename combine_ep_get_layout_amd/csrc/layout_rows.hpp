// Slot arithmetic shared by the layout's finalize pass and the dispatch
// kernels that take the layout's last step themselves: block scan, segment
// starts, the row of a routed entry and the stream index of a sent token,
// from the scanned chunk histograms.
#pragma once

#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {

// Exclusive block scan of one int per thread (up to 1024 threads); returns
// the exclusive prefix, *total receives the block sum.
__device__ inline int block_exclusive_scan(int v, int* total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < kWave; o <<= 1) {
    const int n = __shfl_up(incl, o);
    if (lane >= o) incl += n;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  const int nw = blockDim.x >> 6;
  for (int w = 0; w < nw; ++w) {
    if (w < wave) before += wsum[w];
    all += wsum[w];
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Segment starts in LDS: start[e] for e in [0, E].  Every block of the
// finalize launch computes them itself from the per-expert receive counts
// (an exclusive scan of the counts rounded up to expert_alignment; fixed
// blocks of R*T rows in low-latency mode).
// Rank-major mode: partition bases in rbase[0..R] (exclusive scan of the
// rows each rank receives, the last row of the rank prefix matrix), and
// start[e] = base of e's rank.
__device__ void rank_bases(const LayoutArgs& a, int* start, int* rbase) {
  const Geometry& g = a.g;
  const int per = (g.R + blockDim.x - 1) / blockDim.x;
  const int lo = min(g.R, (int)threadIdx.x * per), hi = min(g.R, lo + per);
  int sum = 0;
  for (int d = lo; d < hi; ++d) sum += a.rpm[(g.R - 1) * g.R + d];
  int total;
  int run = block_exclusive_scan(sum, &total);
  for (int d = lo; d < hi; ++d) {
    rbase[d] = run;
    run += a.rpm[(g.R - 1) * g.R + d];
  }
  if (threadIdx.x == 0) rbase[g.R] = total;
  __syncthreads();
  for (int e = threadIdx.x; e < g.E; e += blockDim.x) start[e] = rbase[e / g.L];
  if (threadIdx.x == 0) start[g.E] = total;
  __syncthreads();
}

__device__ inline void segment_starts(const LayoutArgs& a, int* start) {
  const Geometry& g = a.g;
  if (a.mode == EP_MODE_LOW_LATENCY) {
    const int rt = g.R * g.T;
    for (int e = threadIdx.x; e <= g.E; e += blockDim.x) start[e] = e * rt;
    __syncthreads();
    return;
  }
  const int per = (g.E + blockDim.x - 1) / blockDim.x;
  const int lo = min(g.E, (int)threadIdx.x * per), hi = min(g.E, lo + per);
  int sum = 0;
  for (int e = lo; e < hi; ++e) {
    const int n = a.recv_per_expert[e];
    sum += (n + a.align - 1) / a.align * a.align;
  }
  int total;
  int run = block_exclusive_scan(sum, &total);
  for (int e = lo; e < hi; ++e) {
    start[e] = run;
    const int n = a.recv_per_expert[e];
    run += (n + a.align - 1) / a.align * a.align;
  }
  if (threadIdx.x == 0) start[g.E] = total;
  __syncthreads();
}

// Row of routed entry (token st = s*T + t, expert e, rank `local` among
// the chunk's entries of e; -1 = not routed): the segment start plus the
// entries of e in earlier (source, chunk)s plus `local`.  -1 for unrouted
// entries and for low-latency positions past the expert's R*T rows (which
// raise EP_DEVERR_LL_OVERFLOW).
__device__ inline int entry_row(const LayoutArgs& a, int start_e, const int32_t* hist_e,
                                int64_t st, int e, int local) {
  if (local < 0) return -1;
  const Geometry& g = a.g;
  const int s = (int)(st / g.T), t = (int)(st % g.T);
  const int pos = hist_e[(int64_t)e * g.NC + s * g.C + t / g.ct] + local;
  if (a.mode == EP_MODE_LOW_LATENCY && pos >= g.R * g.T) {
    set_err(a.err, EP_DEVERR_LL_OVERFLOW);
    return -1;
  }
  return start_e + pos;
}

// Index of token st in the (s, d) stream from its rank `v` among the
// chunk's tokens sent to d (-1 = not sent).
__device__ inline int stream_index(const LayoutArgs& a, const int32_t* hist_r, int64_t st, int d,
                                   int v) {
  if (v < 0) return -1;
  const Geometry& g = a.g;
  const int s = (int)(st / g.T), t = (int)(st % g.T);
  return v + hist_r[(int64_t)d * g.NC + s * g.C + t / g.ct];
}

}  // namespace ep
