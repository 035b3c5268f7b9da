// Dispatch scatter on gfx950: every routed (token, expert) entry receives
// the token's row, as bf16 or as FP8 E4M3 codes with per-128-channel
// scales.
//
// "DeepEP" deep dive (llm-infra-atlas, moe/06_deepep): sec. 1.1 (normal
// mode, contiguous per-expert layout, FP8 dispatch), sec. 1.2 (low-latency
// packed masked layout; fp32 or power-of-two scales, column-major), sec. 4.6
// (these kernels move bytes and do no matrix math: HBM is the roof).
//
// Work split: one block per token; the source row is read once, not K
// times, and stored to each of the token's K rows with 16-byte stores.
//  - bf16 up to hidden 16384: the row is staged in LDS and two wavefronts
//    each store half of every destination row (dispatch_copy_lds);
//  - wider bf16 rows, and FP8: one wavefront per piece of the row, held in
//    registers (quantised once if asked), the whole row in flight at once.
// (Measured on MI355X at hidden 7168: plain stores beat non-temporal ones
// for the bf16 scatter, and so they do for normal-mode FP8 codes; the
// low-latency FP8 codes go out non-temporal, see dispatch_fp8.  The kernels
// sit at the chip's write-dominated bandwidth.)
#include "ep_device.hpp"
#include "ep_internal.hpp"
#include "layout_rows.hpp"
#include "quant.hpp"

namespace ep {

// Row split: one block per token, one wavefront per row piece of NV
// 16-byte vectors per lane (the whole row in flight at once; each wave's
// store instructions write 64 x 16 contiguous bytes).  The wavefront count
// is rounded up to a multiple of four, one per SIMD of a compute unit.
// Measured on MI355X at hidden 7168 (whole library, alternating runs): the
// FP8 low-latency dispatch with eight waves, one idle, is 2% faster than
// with seven; the register bf16 copy (used above hidden 16384) with four
// waves of four vectors is 1.4% faster than eight waves of two and 1.7%
// faster than seven waves of two.  The FP8 normal-mode launcher overrides
// the split at 64 and 256 pairs (one wavefront, below).
struct RowSplit {
  int nv;     // vectors per lane
  int waves;  // wavefronts per block (row pieces, padded)
};

inline RowSplit row_split(int vectors, int prefer_nv) {
  RowSplit r;
  r.nv = prefer_nv;
  while ((vectors + kWave * r.nv - 1) / (kWave * r.nv) > 16) ++r.nv;
  r.waves = (vectors + kWave * r.nv - 1) / (kWave * r.nv);
  r.waves = (r.waves + 3) / 4 * 4;  // <= 16
  return r;
}

// Rank-major mode: the token's rows on its destination ranks.  Lanes k < K
// hold send_pos of entry k; bit k of the result is set when entry k is the
// first entry with that row (one row per destination rank).
__device__ __forceinline__ uint64_t first_of_rows(int myrow, int K) {
  bool dup = false;
  for (int k2 = 0; k2 < K; ++k2) {
    const int r2 = __builtin_amdgcn_readlane(myrow, k2);
    dup |= k2 < lane_id() && r2 == myrow;
  }
  return __ballot(lane_id() < K && myrow >= 0 && !dup);
}

// Rank-major per-row metadata.  Lane k (< K) writes entry k of the row as
// rank d sees it: the local id of expert e_k when it lives on d, else -1,
// and its weight, else 0.
struct RowMeta {
  const int32_t* topk;
  const float* w;
  int32_t* idx;  // [capacity][K] or NULL
  float* wts;    // [capacity][K] or NULL
  int L, E;
};

__device__ __forceinline__ void write_row_meta(const RowMeta& m, int K, int64_t row, int d,
                                               int myid, float myw) {
  const int lane = lane_id();
  if (lane >= K) return;
  const bool on = myid >= 0 && myid < m.E && myid / m.L == d;
  if (m.idx) m.idx[row * K + lane] = on ? myid - d * m.L : -1;
  if (m.wts) m.wts[row * K + lane] = on ? myw : 0.0f;
}

// Layout fused into dispatch ("DeepEP" deep dive, sec. 4.6: V2 moves the
// layout's last step into the dispatch kernel).  The block of token `tok`
// derives the token's K rows from the scanned chunk histograms (lanes
// k < K hold row k); the writer wave also stores the layout's per-token
// outputs (send_pos, recv_src_idx, send_head).  `start` = segment starts
// (LDS) in normal mode; low-latency blocks are fixed at e * R*T.
// Lanes k < K: entry k's expert id and its rank in its chunk (-1 elsewhere).
struct TokenEntries {
  int e, local;
};

__device__ __forceinline__ TokenEntries fused_token_entries(const LayoutArgs& a, int64_t tok) {
  TokenEntries t{-1, -1};
  if (lane_id() < a.g.K) {
    const int64_t i = tok * a.g.K + lane_id();
    t.e = a.topk[i];
    t.local = a.local_e[i];
  }
  return t;
}

__device__ __forceinline__ int fused_token_rows(const LayoutArgs& a, int64_t tok, bool writer,
                                                const int* start, TokenEntries te) {
  const Geometry& g = a.g;
  const int lane = lane_id();
  int row = -1;
  if (lane < g.K) {
    const int64_t i = tok * g.K + lane;
    const int e = te.e;
    const int local = te.local;
    if (writer && (e < -1 || e >= g.E)) set_err(a.err, EP_DEVERR_TOPK_RANGE);
    if (local >= 0) {
      const int start_e = a.mode == EP_MODE_LOW_LATENCY ? e * g.R * g.T : start[e];
      row = entry_row(a, start_e, a.hist_e, tok, e, local);
    }
    if (writer) {
      if (a.send_pos) a.send_pos[i] = row;
      if (row >= 0 && a.recv_src_idx) {
        if (row < a.recv_cap) a.recv_src_idx[row] = (int)tok;
        else set_err(a.err, EP_DEVERR_CAPACITY);
      }
    }
  }
  if (writer && a.send_head)
    for (int d = lane; d < g.R; d += kWave) {
      const int64_t hi = tok * g.R + d;
      a.send_head[hi] = stream_index(a, a.hist_r, tok, d, a.local_r[hi]);
    }
  return row;
}

// The same, loading the token's entries itself.
__device__ __forceinline__ int fused_token_rows(const LayoutArgs& a, int64_t tok, bool writer,
                                                const int* start) {
  return fused_token_rows(a, tok, writer, start, fused_token_entries(a, tok));
}

// The layout's per-expert and per-rank outputs, written by block b for
// expert b (and rank b), plus the alignment padding rows of expert b's
// segment.  Every block of a fused dispatch calls this first.
__device__ __forceinline__ void fused_publish(const LayoutArgs& a, const int* start) {
  const Geometry& g = a.g;
  const int b = blockIdx.x;
  const bool ll = a.mode == EP_MODE_LOW_LATENCY;
  const int rt = g.R * g.T;
  if (b < g.E && threadIdx.x == 0) a.expert_start[b] = ll ? b * rt : start[b];
  if (b <= g.R && threadIdx.x == 0) {
    const int base = ll ? b * g.L * rt : start[b * g.L];
    a.row_base[b] = base;
    if (b < g.R) a.rows[b] = ll ? g.L * rt : start[(b + 1) * g.L] - base;
  }
  if (!ll && b < g.E && a.recv_src_idx && a.align > 1) {
    const int first = start[b] + a.recv_per_expert[b];
    for (int r = first + (int)threadIdx.x; r < start[b + 1]; r += blockDim.x)
      if (r < a.recv_cap) a.recv_src_idx[r] = -1;
  }
}

template <int NV, bool RM, bool FU>
__global__ __launch_bounds__(1024) void dispatch_copy(const u32x4* __restrict__ x,
                                                      const int32_t* __restrict__ send_pos,
                                                      u32x4* __restrict__ recv, int V, int K,
                                                      int64_t cap, int32_t* err, RowMeta meta,
                                                      LayoutArgs la) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x;
  const int base = uniform(threadIdx.x >> 6) * kWave * NV;
  __shared__ int start[FU ? 2049 : 1];
  if (FU) {
    if (la.mode != EP_MODE_LOW_LATENCY) segment_starts(la, start);
    fused_publish(la, start);
    if (tok >= la.g.R * la.g.T) return;  // publishing-only block
  }
  const u32x4* src = x + (int64_t)tok * V;
  u32x4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = src[min(base + lane + kWave * i, V - 1)];  // in bounds
  const int myrow = FU ? fused_token_rows(la, tok, base == 0, start)
                       : (lane < K ? send_pos[(int64_t)tok * K + lane] : -1);
  // rank-major: each destination row once; the first wave writes its metadata
  const uint64_t keep = RM ? first_of_rows(myrow, K) : ~0ull;
  const bool meta_wave = RM && base == 0 && (meta.idx || meta.wts);
  const int myid = meta_wave && lane < K ? meta.topk[(int64_t)tok * K + lane] : -1;
  const float myw = meta_wave && meta.wts && lane < K ? meta.w[(int64_t)tok * K + lane] : 0.0f;
  for (int k = 0; k < K; ++k) {
    if (RM && !((keep >> k) & 1)) continue;
    const int row = __builtin_amdgcn_readlane(myrow, k);
    if (row < 0) continue;
    if (row >= cap) {
      if (lane == 0 && base == 0) set_err(err, EP_DEVERR_CAPACITY);
      continue;
    }
    if (meta_wave)
      write_row_meta(meta, K, row, __builtin_amdgcn_readlane(myid, k) / meta.L, myid, myw);
    u32x4* dst = recv + (int64_t)row * V;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = base + lane + kWave * i;
      if (j < V) dst[j] = v[i];
    }
  }
}

// LDS-staged copy (bf16, hidden up to 16384): one block of two wavefronts
// per token.  The block loads the token's row into LDS once, then wave w
// stores half w of the row (7 KiB contiguous at hidden 7168) to each of
// the token's K rows, reading it back from LDS (one LDS read per store: the
// stores leave at the pace of the reads, which measured 2% faster than
// issuing a wave's eight reads first).  Measured on MI355X at the
// prefill shape (8 x 4096 tokens, hidden 7168, top-8, Zipf routing): 2.6%
// faster than the register-resident split above (four waves, 4 KiB each).
// With four or eight waves, the same LDS-staged scheme is 3-5% slower than
// the register split. So is one wave per destination row. Register splits
// of two waves (7 KiB each) are 2% slower.
template <bool RM, bool FU>
__global__ __launch_bounds__(128) void dispatch_copy_lds(const u32x4* __restrict__ x,
                                                         const int32_t* __restrict__ send_pos,
                                                         u32x4* __restrict__ recv, int V, int K,
                                                         int64_t cap, int32_t* err, RowMeta meta,
                                                         LayoutArgs la) {
  extern __shared__ u32x4 row_lds[];  // V vectors
  __shared__ int start[FU ? 2049 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int tok = blockIdx.x;
  if (FU) {
    if (la.mode != EP_MODE_LOW_LATENCY) segment_starts(la, start);
    fused_publish(la, start);
    if (tok >= la.g.R * la.g.T) return;  // publishing-only block
  }
  const u32x4* src = x + (int64_t)tok * V;
  // as compiled, each thread keeps one load in flight, each waiting for the
  // previous one (measured on MI355X: loading a thread's vectors together
  // first is 1% slower at the prefill shape, 12% slower in rank-major mode)
  for (int j = threadIdx.x; j < V; j += blockDim.x) row_lds[j] = src[j];
  const int myrow = FU ? fused_token_rows(la, tok, wave == 0, start)
                       : (lane < K ? send_pos[(int64_t)tok * K + lane] : -1);
  // rank-major: each destination row once; wave 0 writes its metadata
  const uint64_t keep = RM ? first_of_rows(myrow, K) : ~0ull;
  const bool meta_wave = RM && wave == 0 && (meta.idx || meta.wts);
  const int myid = meta_wave && lane < K ? meta.topk[(int64_t)tok * K + lane] : -1;
  const float myw = meta_wave && meta.wts && lane < K ? meta.w[(int64_t)tok * K + lane] : 0.0f;
  __syncthreads();
  // halves split on a 128-byte line (8 vectors) of the row
  const int half = min(V, ((V + 1) / 2 + 7) & ~7);
  const int lo = wave * half, hi = min(V, lo + half);
  // the token's rows are stored in ascending address order (lane k < K
  // ranks its row among the token's, repeats by k; measured on MI355X at
  // the prefill routing: expert-major dispatch 763.6 -> 762.0 us over seven
  // interleaved pairs, rank-major 506.7 -> 503.8 us over four, every pair
  // faster)
  int rank = 0;
  for (int k2 = 0; k2 < K; ++k2) {
    const int r2 = __builtin_amdgcn_readlane(myrow, k2);
    rank += lane < K && (r2 < myrow || (r2 == myrow && k2 < lane));
  }
  for (int kk = 0; kk < K; ++kk) {
    const uint64_t sel = __ballot(lane < K && rank == kk);
    const int k = sel ? __builtin_ctzll(sel) : kk;
    if (RM && !((keep >> k) & 1)) continue;
    const int row = __builtin_amdgcn_readlane(myrow, k);
    if (row < 0) continue;
    if (row >= cap) {
      if (lane == 0 && wave == 0) set_err(err, EP_DEVERR_CAPACITY);
      continue;
    }
    if (meta_wave)
      write_row_meta(meta, K, row, __builtin_amdgcn_readlane(myid, k) / meta.L, myid, myw);
    u32x4* dst = recv + (int64_t)row * V;
    for (int j = lo + lane; j < hi; j += kWave) dst[j] = row_lds[j];
    // expert-major rows: each wave lets its stores of one row complete
    // before it starts the next (measured on MI355X at the prefill shape:
    // dispatch 766.6 -> 763.6 us over six interleaved runs; waiting after
    // every fourth store or every store took 792 and 804 us, and rank-major
    // rows, about five per token, were 1.3% slower with the per-row wait)
    // s_waitcnt immediate (gfx9 family): vmcnt [3:0] and [15:14] = 0,
    // expcnt [6:4] = 7 and lgkmcnt [11:8] = 15, i.e. only vmcnt(0)
    if (!RM) __builtin_amdgcn_s_waitcnt(0x0F70);
  }
}

// P = 16-channel pairs per row (H / 16); a group of 128 channels is 8
// pairs = 8 consecutive lanes, reduced with DPP.

template <int NP, int Q, bool LL, bool RM, bool FU>
__global__ __launch_bounds__(NP >= 3 ? 512 : 1024) void dispatch_fp8(const u32x4* __restrict__ x,
                                                     const int32_t* __restrict__ send_pos,
                                                     u32x4* __restrict__ codes,
                                                     void* __restrict__ scales, int P, int K,
                                                     int64_t cap, int G, int RT, int n_tok,
                                                     int32_t* err, RowMeta meta, LayoutArgs la,
                                                     bool tok_stage) {
  const int lane = threadIdx.x & 63;
  __shared__ int start[FU && !LL ? 2049 : 1];
  if (FU) {
    if (!LL) segment_starts(la, start);
    fused_publish(la, start);
  }
  // blocks past the token grid only publish (fused), never alias a token
  if ((int)blockIdx.x >= (LL ? xcd_blocks(n_tok) : n_tok)) return;
  // low-latency: die blockIdx.x % kXcds takes a contiguous run of tokens, so
  // consecutive slots of an expert (consecutive tokens) are stored from one
  // L2 and their 4-byte column-major scales merge into whole lines there
  const int tok = LL ? xcd_run(blockIdx.x, n_tok) : blockIdx.x;
  if (tok >= n_tok) return;
  const int base = uniform(threadIdx.x >> 6) * kWave * NP;
  // fused low-latency: the token's expert ids and chunk ranks are loaded
  // with the row, before the quantisation, so their latency overlaps it
  // (measured on MI355X: the decode step's layout + dispatch 2% faster;
  // at the training shape the early loads cost 1%, so normal mode loads
  // them after the quantisation)
  TokenEntries te{-1, -1};
  if (FU && LL) te = fused_token_entries(la, tok);
  const u32x4* src = x + (int64_t)tok * (2 * (int64_t)P);
  u32x4 lo[NP], hi[NP];
  load_pairs<NP>(src, base, P, lo, hi);
  u32x4 cv[NP];
  float scf[NP];
  uint32_t sce[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) quantise_pair<Q>(lo[i], hi[i], cv[i], scf[i], sce[i]);
  if (FU && !LL) te = fused_token_entries(la, tok);
  const int myrow = FU ? fused_token_rows(la, tok, base == 0, start, te)
                       : (lane < K ? send_pos[(int64_t)tok * K + lane] : -1);
  // rank-major: each destination row once; the first wave writes its metadata
  const uint64_t keep = RM ? first_of_rows(myrow, K) : ~0ull;
  const bool meta_wave = RM && base == 0 && (meta.idx || meta.wts);
  const int myid = meta_wave && lane < K ? meta.topk[(int64_t)tok * K + lane] : -1;
  const float myw = meta_wave && meta.wts && lane < K ? meta.w[(int64_t)tok * K + lane] : 0.0f;
  // with the row -> token map: the token's G scales go to the staging once
  // ([token][G], consecutive tokens in consecutive bytes); a second kernel
  // places them in every row's column entries
  const bool row_scales = !tok_stage;
  if (!row_scales) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int j = base + lane + kWave * i;
      if (j < P && (lane & 7) == 0) {
        const int64_t si = (int64_t)tok * G + (j >> 3);
        if (Q == EP_QUANT_FP8_F32) ((float*)scales)[si] = scf[i];
        else ((uint8_t*)scales)[si] = (uint8_t)sce[i];
      }
    }
  }
  for (int k = 0; k < K; ++k) {
    if (RM && !((keep >> k) & 1)) continue;
    const int row = __builtin_amdgcn_readlane(myrow, k);
    if (row < 0) continue;
    if (row >= cap) {
      if (lane == 0 && base == 0) set_err(err, EP_DEVERR_CAPACITY);
      continue;
    }
    if (meta_wave)
      write_row_meta(meta, K, row, __builtin_amdgcn_readlane(myid, k) / meta.L, myid, myw);
    u32x4* dst = codes + (int64_t)row * P;
    int64_t sbase, sstride;
    if (LL) {  // column-major per expert, written in place
      const int e = row / RT, pos = row - e * RT;
      sbase = (int64_t)e * G * RT + pos;
      sstride = RT;
    } else {  // row-major staging; scales_to_columns transposes it
      sbase = (int64_t)row * G;
      sstride = 1;
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int j = base + lane + kWave * i;
      if (j < P) {
        // low-latency codes: non-temporal stores (measured on MI355X at the
        // decode shape: dispatch and the combine after it each 1 us faster,
        // as no dirty lines are left to write back; non-temporal 4-byte
        // scale stores made the dispatch 22 us slower, since they no longer
        // merge into lines in L2).  Normal mode keeps plain stores (the
        // training shape was 3% slower with non-temporal ones).
        if (LL) __builtin_nontemporal_store(cv[i], dst + j);
        else dst[j] = cv[i];
        if (row_scales && (lane & 7) == 0) {
          const int64_t si = sbase + (int64_t)(j >> 3) * sstride;
          if (Q == EP_QUANT_FP8_F32)
            ((float*)scales)[si] = scf[i];
          else
            ((uint8_t*)scales)[si] = (uint8_t)sce[i];
        }
      }
    }
  }
}

// Normal-mode FP8 scales: the dispatch kernel stores each row's G scales
// contiguously in a staging buffer (row-major, coalesced); this kernel
// writes them column-major, scales[g * cap + row], a tile of consecutive
// rows per group per store, through LDS.  Rows past the filled part of their
// expert segment (alignment padding) are not written; with no padding
// (expert_alignment 1, or rank-major) every staged row is filled and the
// segment search is skipped.  A scattered per-row store of one byte per
// group would cost a memory transaction per byte instead.  The tile is
// read with 16-byte loads (tile_rows is a multiple of 16, so every tile
// starts 16-byte aligned).
template <int SB>
__global__ __launch_bounds__(256) void scales_to_columns(const uint8_t* __restrict__ stage,
                                                         uint8_t* __restrict__ scales, int G,
                                                         int64_t cap, int64_t limit,
                                                         const int32_t* row_base_end,
                                                         const int32_t* __restrict__ expert_start,
                                                         const int32_t* __restrict__ count,
                                                         int E, int tile_rows, int all_filled) {
  extern __shared__ uint32_t lds[];
  int* starts = (int*)lds;                  // E + 1
  int* filled = starts + E + 1;             // tile_rows
  uint32_t* tile = lds + ((E + 1 + tile_rows + 3) & ~3);  // tile_rows * G * SB bytes, 16-aligned
  const int64_t total = min((int64_t)*row_base_end, limit);  // rows that were staged
  const int64_t r0 = (int64_t)blockIdx.x * tile_rows;
  if (r0 >= total) return;
  const int nrows = (int)min((int64_t)tile_rows, total - r0);
  if (!all_filled) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) starts[e] = expert_start[e];
    if (threadIdx.x == 0) starts[E] = (int)total;
  }
  const int nbytes = nrows * G * SB;
  const uint8_t* src = stage + r0 * G * SB;
  uint8_t* t8 = (uint8_t*)tile;
  const int nvec = nbytes / 16;
  for (int i = threadIdx.x; i < nvec; i += blockDim.x)
    ((u32x4*)tile)[i] = ((const u32x4*)src)[i];
  for (int i = nvec * 16 + threadIdx.x; i < nbytes; i += blockDim.x) t8[i] = src[i];
  __syncthreads();
  for (int r = threadIdx.x; r < tile_rows; r += blockDim.x) {
    const int64_t row = r0 + r;
    int ok = 0;
    if (r < nrows && all_filled) {
      ok = 1;
    } else if (r < nrows) {
      int lo = 0, hi = E;  // last e with starts[e] <= row
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (starts[mid] <= row) lo = mid;
        else hi = mid;
      }
      ok = row - starts[lo] < count[lo];
    }
    filled[r] = ok;
  }
  __syncthreads();
  for (int it = threadIdx.x; it < G * tile_rows; it += blockDim.x) {
    const int g = it / tile_rows, r = it % tile_rows;
    if (r < nrows && filled[r]) {
      const int64_t di = (int64_t)g * cap + r0 + r;
      if (SB == 4) ((uint32_t*)scales)[di] = tile[r * G + g];
      else scales[di] = t8[r * G + g];
    }
  }
}

// Normal-mode and rank-major FP8 scales from the per-token staging: the
// dispatch kernel stored each token's G scales once, at stage[tok * G];
// this kernel reads each receive row's token from the layout's
// recv_src_idx (-1: alignment padding, never written; an index outside
// [0, n_tok) counts as padding), gathers a tile of rows' token scales into
// LDS with coalesced loads (consecutive threads read consecutive words of
// one token's scales) and writes the tile's part of every column
// scales[g * cap + row] as 16-byte vectors (16 / SB rows of one group
// each), entry by entry where a vector would cover a padding row or run
// past the filled rows, or where the columns are not 16-byte aligned
// (vec_ok = 0).  Against one staged copy per receive row, the staging
// shrinks K-fold and is written by consecutive tokens into whole lines.
// (Measured on MI355X at the FP8 training shape: 27 us; without LDS, four
// rows per thread gathered word by word and transposed in registers, 38 us.)
constexpr int kGatherLoads = 8;  // staged-scale words in flight per thread

template <int SB>
__global__ __launch_bounds__(256) void scales_from_tokens(const uint8_t* __restrict__ stage,
                                                          uint8_t* __restrict__ scales, int G,
                                                          int64_t cap, int64_t limit,
                                                          const int32_t* row_base_end,
                                                          const int32_t* __restrict__ row_token,
                                                          int n_tok, int tile_rows, int vec_ok) {
  extern __shared__ uint32_t lds[];
  int* tok = (int*)lds;                                // tile_rows
  uint8_t* tile = (uint8_t*)(lds + tile_rows);         // tile_rows * G * SB bytes
  const int64_t total = min((int64_t)*row_base_end, limit);
  const int64_t r0 = (int64_t)blockIdx.x * tile_rows;
  if (r0 >= total) return;
  const int nrows = (int)min((int64_t)tile_rows, total - r0);
  // Every load below is unconditional (indices clamped into the buffers,
  // values selected afterwards) and a thread issues kGatherLoads of them
  // before it stores any into LDS: a load under a branch, or a load whose
  // value is stored before the next is issued, waits for the one before.
  // (Measured on MI355X at the FP8 training shape, three interleaved runs
  // each: layout + dispatch 1.0438 -> 1.0390 ms against one gather load per
  // round trip, which compiled to a wait after every word.)
  for (int r = threadIdx.x; r < tile_rows; r += 2 * blockDim.x) {
    const int r2 = r + blockDim.x;
    const int t1 = row_token[r0 + min(r, nrows - 1)];
    const int t2 = row_token[r0 + min(r2, nrows - 1)];
    const int v1 = r < nrows && t1 < n_tok ? t1 : -1;
    const int v2 = r2 < nrows && t2 < n_tok ? t2 : -1;
    tok[r] = v1;
    // unconditional, so the second load is not sunk behind the first
    // store: past the tile the thread rewrites its own first entry
    tok[r2 < tile_rows ? r2 : r] = r2 < tile_rows ? v2 : v1;
  }
  __syncthreads();
  const int rb = G * SB;  // bytes of one token's scales
  if (rb % 4 == 0) {
    const int nw = rb / 4;
    const int n = nrows * nw;
    // entry i = (row r, word w) of the tile; one block-wide step of
    // blockDim.x entries advances (r, w) by (dr, dw)
    const int bd = blockDim.x;
    const int dr = bd / nw, dw = bd - dr * nw;
    int r = threadIdx.x / nw, w = threadIdx.x - r * nw;
    for (int i0 = threadIdx.x; i0 < n; i0 += kGatherLoads * bd) {
      int t[kGatherLoads], wq[kGatherLoads];
#pragma unroll
      for (int q = 0; q < kGatherLoads; ++q) {
        const int tv = tok[min(r, tile_rows - 1)];
        t[q] = i0 + q * bd < n ? tv : -1;
        wq[q] = w;
        w += dw;
        r += dr;
        const bool wrap = w >= nw;
        w = wrap ? w - nw : w;
        r = wrap ? r + 1 : r;
      }
      uint32_t v[kGatherLoads];
#pragma unroll
      for (int q = 0; q < kGatherLoads; ++q)
        v[q] = ((const uint32_t*)stage)[(int64_t)(t[q] >= 0 ? t[q] : 0) * nw + wq[q]];
      // stores are unconditional too (entries past the tile rewrite the
      // thread's first entry with its own value), so no load is sunk
      // behind a store
      const uint32_t first = t[0] >= 0 ? v[0] : 0u;
#pragma unroll
      for (int q = 0; q < kGatherLoads; ++q) {
        const int i = i0 + q * bd;
        ((uint32_t*)tile)[i < n ? i : i0] = i < n ? (t[q] >= 0 ? v[q] : 0u) : first;
      }
    }
  } else {
    for (int i = threadIdx.x; i < nrows * rb; i += blockDim.x) {
      const int r = i / rb, q = i - r * rb;
      const int t = tok[r];
      tile[i] = t >= 0 ? stage[(int64_t)t * rb + q] : (uint8_t)0;
    }
  }
  __syncthreads();
  constexpr int kPer = 16 / SB;  // rows per column vector
  const int nvec = tile_rows / kPer;
  // consecutive threads take consecutive groups of the same rows, so their
  // LDS reads fall in the same few words
  for (int it = threadIdx.x; it < G * nvec; it += blockDim.x) {
    const int g = it % G, rv = (it / G) * kPer;
    // rows past the filled ones hold tok = -1 too; one OR over the
    // vector's rows, with no branch between the LDS reads
    int neg = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) neg |= tok[rv + q];
    const bool full = vec_ok && rv + kPer <= nrows && neg >= 0;
    const int64_t di = (int64_t)g * cap + r0 + rv;
    if (full) {
      u32x4 v;
      if (SB == 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = ((const uint32_t*)tile)[(rv + q) * G + g];
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t word = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) word |= (uint32_t)tile[(rv + 4 * w + b) * rb + g] << (8 * b);
          v[w] = word;
        }
      }
      *(u32x4*)(scales + di * SB) = v;
    } else {
      for (int q = 0; q < kPer; ++q) {
        const int r = rv + q;
        if (r >= nrows || tok[r] < 0) continue;
        if (SB == 4) ((uint32_t*)scales)[di + q] = ((const uint32_t*)tile)[r * G + g];
        else scales[di + q] = tile[r * rb + g];
      }
    }
  }
}

inline RowMeta row_meta(const DispatchArgs& a) {
  RowMeta m;
  m.topk = a.topk;
  m.w = a.w;
  m.idx = a.recv_topk_idx;
  m.wts = a.recv_topk_weights;
  m.L = a.g.L;
  m.E = a.g.E;
  return m;
}

// A fused dispatch also needs one block per expert and per rank boundary
// to publish the layout's per-expert outputs.
inline int fused_blocks(const DispatchArgs& a, int blocks) {
  if (!a.fused) return blocks;
  int b = blocks;
  if (b < a.g.E) b = a.g.E;
  if (b < a.g.R + 1) b = a.g.R + 1;
  return b;
}

template <int NV, bool RM>
static void launch_copy_nv(const DispatchArgs& a, int V, int waves, hipStream_t st) {
  const int N = a.g.R * a.g.T;
  if (a.fused)
    hipLaunchKernelGGL((dispatch_copy<NV, false, true>), dim3(fused_blocks(a, N)),
                       dim3(kWave * waves), 0, st, (const u32x4*)a.x, a.send_pos,
                       (u32x4*)a.recv_x, V, a.g.K, a.cap, a.err, row_meta(a), a.la);
  else
    hipLaunchKernelGGL((dispatch_copy<NV, RM, false>), dim3(N), dim3(kWave * waves), 0, st,
                       (const u32x4*)a.x, a.send_pos, (u32x4*)a.recv_x, V, a.g.K, a.cap, a.err,
                       row_meta(a), a.la);
}

// LDS-staged bf16 copy up to hidden 16384 (32 KiB of LDS per block)
constexpr int kCopyLdsMaxVectors = 2048;

constexpr size_t kRankMajorLds = 20480;

template <bool RM>
static void launch_copy_lds(const DispatchArgs& a, int V, hipStream_t st) {
  const int N = a.g.R * a.g.T;
  // the row's LDS, which sets how many blocks share a compute unit (160 KiB
  // of LDS: 11 at hidden 7168).  Rank-major blocks ask for at least 20 KiB,
  // at most eight per compute unit (measured on MI355X at the prefill
  // routing, three interleaved runs each: rank-major dispatch 0.5055 ->
  // 0.5004 ms; the expert-major copy is 0.8% slower with ten blocks, 1.5%
  // with eight and 5.7% with six, so it keeps the row's size)
  size_t lds = sizeof(u32x4) * (size_t)V;
  if (RM && lds < kRankMajorLds) lds = kRankMajorLds;
  if (a.fused)
    hipLaunchKernelGGL((dispatch_copy_lds<false, true>), dim3(fused_blocks(a, N)), dim3(128), lds,
                       st, (const u32x4*)a.x, a.send_pos, (u32x4*)a.recv_x, V, a.g.K, a.cap, a.err,
                       row_meta(a), a.la);
  else
    hipLaunchKernelGGL((dispatch_copy_lds<RM, false>), dim3(N), dim3(128), lds, st,
                       (const u32x4*)a.x, a.send_pos, (u32x4*)a.recv_x, V, a.g.K, a.cap, a.err,
                       row_meta(a), a.la);
}

template <int NP, int Q, bool LL, bool RM>
static void launch_fp8_np(const DispatchArgs& a, int P, int waves, hipStream_t st) {
  const int N = a.g.R * a.g.T;
  // normal and rank-major modes: rows also index the staging buffer, so they
  // stay below both
  const int64_t cap = LL ? a.cap : (a.cap < a.stage_rows ? a.cap : a.stage_rows);
  const int blocks = LL ? xcd_blocks(N) : N;
  const bool tok_stage = !LL && a.row_token != nullptr;
  void* sc = LL ? a.recv_scales : a.stage;  // low-latency scales go in place
  if (a.fused && !RM)
    hipLaunchKernelGGL((dispatch_fp8<NP, Q, LL, false, true>), dim3(fused_blocks(a, blocks)),
                       dim3(kWave * waves), 0, st, (const u32x4*)a.x, a.send_pos,
                       (u32x4*)a.recv_x, sc, P, a.g.K, cap, a.g.G, a.g.R * a.g.T, N, a.err,
                       row_meta(a), a.la, tok_stage);
  else
    hipLaunchKernelGGL((dispatch_fp8<NP, Q, LL, RM, false>), dim3(blocks), dim3(kWave * waves),
                       0, st, (const u32x4*)a.x, a.send_pos, (u32x4*)a.recv_x, sc, P, a.g.K,
                       cap, a.g.G, a.g.R * a.g.T, N, a.err, row_meta(a), a.la, tok_stage);
  if (!LL) {
    // 256 rows per tile, fewer for wide rows (the tile lives in LDS), at
    // least 16 (16-byte aligned tiles)
    const int sb = Q == EP_QUANT_FP8_F32 ? 4 : 1;
    int tile_rows = 256;
    while (tile_rows > 16 && (size_t)tile_rows * a.g.G * sb > 32768) tile_rows >>= 1;
    if (tok_stage) {
      // the gather from the token staging takes 512-row tiles (measured on
      // MI355X at the training shape: 24 us against 27 us for 256 rows,
      // 28 us for 128 and 33 us for 1024, with one gather load per round
      // trip; with eight in flight, 256-row tiles or sixteen loads per
      // thread are 1-2 us slower over layout + dispatch)
      tile_rows = 512;
      while (tile_rows > 16 && (size_t)tile_rows * a.g.G * sb > 32768) tile_rows >>= 1;
      const size_t lds = sizeof(int) * (size_t)tile_rows + (size_t)tile_rows * a.g.G * sb;
      const int vec_ok = ((a.cap * sb) % 16 == 0 && ((uintptr_t)a.recv_scales % 16) == 0) ? 1 : 0;
      const int64_t tiles = (cap + tile_rows - 1) / tile_rows;
      if (tiles > 0) {
        if (Q == EP_QUANT_FP8_F32)
          hipLaunchKernelGGL(scales_from_tokens<4>, dim3((unsigned)tiles), dim3(256), lds, st,
                             (const uint8_t*)a.stage, (uint8_t*)a.recv_scales, a.g.G, a.cap, cap,
                             a.row_base + a.g.R, a.row_token, N, tile_rows, vec_ok);
        else
          hipLaunchKernelGGL(scales_from_tokens<1>, dim3((unsigned)tiles), dim3(256), lds, st,
                             (const uint8_t*)a.stage, (uint8_t*)a.recv_scales, a.g.G, a.cap, cap,
                             a.row_base + a.g.R, a.row_token, N, tile_rows, vec_ok);
      }
      return;
    }
    const size_t lds = sizeof(int) * ((a.g.E + 1 + tile_rows + 3) & ~3) +
                       (size_t)tile_rows * a.g.G * sb;
    const int all_filled = RM || a.align == 1 ? 1 : 0;
    const int64_t tiles = (cap + tile_rows - 1) / tile_rows;
    if (tiles > 0) {
      if (Q == EP_QUANT_FP8_F32)
        hipLaunchKernelGGL(scales_to_columns<4>, dim3((unsigned)tiles), dim3(256), lds, st,
                           (const uint8_t*)a.stage, (uint8_t*)a.recv_scales, a.g.G, a.cap, cap,
                           a.row_base + a.g.R, a.expert_start, a.recv_per_expert, a.g.E,
                           tile_rows, all_filled);
      else
        hipLaunchKernelGGL(scales_to_columns<1>, dim3((unsigned)tiles), dim3(256), lds, st,
                           (const uint8_t*)a.stage, (uint8_t*)a.recv_scales, a.g.G, a.cap, cap,
                           a.row_base + a.g.R, a.expert_start, a.recv_per_expert, a.g.E,
                           tile_rows, all_filled);
    }
  }
}

template <int Q, bool LL, bool RM>
static void launch_fp8_q(const DispatchArgs& a, hipStream_t st) {
  const int P = a.g.H / 16;
  RowSplit rs = row_split(P, 1);
  if (rs.nv >= 3) rs = RowSplit{4, ((P + kWave * 4 - 1) / (kWave * 4) + 3) / 4 * 4};  // <= 8 waves
  // Normal and rank-major modes, one wavefront per token where measured
  // faster on MI355X (training routing, interleaved runs):
  //  - up to 64 pairs (hidden 1024): one pair per lane, 24% faster than four
  //    wavefronts of which three are idle;
  //  - 256 pairs (hidden 4096): four pairs per lane, 0.6-1.2% faster than
  //    four wavefronts of one pair each.
  // At 128 and 192 pairs one wavefront was 2-5% slower, so those keep the
  // split above.
  if (!LL && (P <= kWave || P == kWave * 4)) rs = RowSplit{(P + kWave - 1) / kWave, 1};
  switch (rs.nv) {
    case 1: launch_fp8_np<1, Q, LL, RM>(a, P, rs.waves, st); break;
    case 2: launch_fp8_np<2, Q, LL, RM>(a, P, rs.waves, st); break;
    case 3: launch_fp8_np<3, Q, LL, RM>(a, P, rs.waves, st); break;
    default: launch_fp8_np<4, Q, LL, RM>(a, P, rs.waves, st); break;  // hidden <= 32768
  }
}

template <int Q>
static void launch_fp8_mode(const DispatchArgs& a, hipStream_t st) {
  if (a.mode == EP_MODE_LOW_LATENCY) launch_fp8_q<Q, true, false>(a, st);
  else if (a.rank_major) launch_fp8_q<Q, false, true>(a, st);
  else launch_fp8_q<Q, false, false>(a, st);
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t st) {
  const int64_t N = (int64_t)a.g.R * a.g.T;
  if (N == 0) return hipSuccess;
  if (a.quant == EP_QUANT_NONE) {
    const int V = a.g.H / 8;
    if (V <= kCopyLdsMaxVectors) {
      if (a.rank_major) launch_copy_lds<true>(a, V, st);
      else launch_copy_lds<false>(a, V, st);
    } else {
      const RowSplit rs = row_split(V, 4);  // hidden <= 32768: nv = 4, <= 16 waves
      if (a.rank_major) launch_copy_nv<4, true>(a, V, rs.waves, st);
      else launch_copy_nv<4, false>(a, V, rs.waves, st);
    }
  } else if (a.quant == EP_QUANT_FP8_F32) {
    launch_fp8_mode<EP_QUANT_FP8_F32>(a, st);
  } else {
    launch_fp8_mode<EP_QUANT_FP8_UE8M0>(a, st);
  }
  return hipGetLastError();
}

}  // namespace ep
