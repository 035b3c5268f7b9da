// Combine gather-reduce on gfx950: each token gathers the expert outputs of
// its K routed rows and takes their top-k weighted sum, fp32 accumulation in
// k order (fused multiply-add), rounded to bf16 nearest-even.
//
// "DeepEP" deep dive (llm-infra-atlas, moe/06_deepep), sec. 2.3: combine
// walks dispatch's address book backwards; sec. 5: combine is the inverse
// of dispatch; sec. 1.1: bf16 combine.
//
// Work split: one block per token (two in the pipelined form), one
// wavefront per piece of the output row.  The K row indices and weights are
// loaded once per wave (one lane each) and read as scalars; the receive rows
// stream in with 16-byte non-temporal loads.  How many row loads a
// wavefront keeps in flight (one, or eight before their multiply-adds) is
// chosen per shape by measurement (launch_combine, below).
#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {

// One block per token, one wavefront per row piece (NV vectors per lane);
// the K rows are read in groups with all loads of a group issued before its
// fused multiply-adds (8 rows per group for one vector per lane, fewer for
// wider pieces so the loads stay in registers; one row per group in the
// SERIAL form).

// Rank-major mode: a token's entries on one destination rank share a row;
// bit k is set for the first entry of each distinct row (lanes k < K hold
// the rows).
__device__ __forceinline__ uint64_t first_rows(int myrow, int K) {
  bool dup = false;
  for (int k2 = 0; k2 < K; ++k2) {
    const int r2 = __builtin_amdgcn_readlane(myrow, k2);
    dup |= k2 < lane_id() && r2 == myrow;
  }
  return __ballot(lane_id() < K && myrow >= 0 && !dup);
}

// Entries whose row is not read (masked, rank-major repeats, rows past y)
// still issue loads, of a stand-in row: the token's first row that is read
// anyway, whose lines the same wavefront fetches, so the stand-in costs no
// HBM bytes.  The loads stay unconditional because a branch around a load
// makes the compiler wait for every load issued before it, which would
// serialise a group's loads (measured on MI355X: the two-token pipeline at
// hidden 4096 was 18% slower with branches).  -1: the token reads no row.
__device__ __forceinline__ int stand_in_row(int myrow, uint64_t keep, int K, int64_t y_rows) {
  const int lane = lane_id();
  const uint64_t ok = __ballot(lane < K && myrow >= 0 && myrow < y_rows && ((keep >> lane) & 1));
  return ok ? __builtin_amdgcn_readlane(myrow, __builtin_ctzll(ok)) : -1;
}

// Row whose loads entry k issues: its own when it is read, else the stand-in.
__device__ __forceinline__ int read_row(int myrow, uint64_t keep, int k, int K, int64_t y_rows,
                                        int stand_in) {
  const int row = k < K ? __builtin_amdgcn_readlane(myrow, k) : -1;
  return row >= 0 && row < y_rows && ((keep >> k) & 1) ? row : stand_in;
}

// RM (rank-major): sum the token's distinct rows with weight 1 and skip the
// loads of repeated rows.  SERIAL: one row's loads (NV vectors per lane) in
// flight per wavefront, each row waiting for the previous one.
template <int NV, bool RM, bool SERIAL = false>
__global__ __launch_bounds__(1024) void combine_rows(const u32x4* __restrict__ y,
                                                     const int32_t* __restrict__ send_pos,
                                                     const float* __restrict__ w,
                                                     u32x4* __restrict__ out, int V, int K,
                                                     int64_t y_rows, int32_t* err) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x;
  const int base = uniform(threadIdx.x >> 6) * kWave * NV;
  const int myrow = lane < K ? send_pos[(int64_t)tok * K + lane] : -1;
  const float myw = RM ? 1.0f : (lane < K ? w[(int64_t)tok * K + lane] : 0.0f);
  const uint64_t keep = RM ? first_rows(myrow, K) : ~0ull;
  // nothing branches on the loaded rows before the loop (only y_rows, a
  // launch argument), so the loop's setup overlaps the index loads; a token
  // that reads no row at all loads row 0's lines as its stand-in
  const int stand_in = max(stand_in_row(myrow, keep, K, y_rows), 0);
  constexpr int kGroup = SERIAL ? 1 : (NV == 1 ? 8 : (NV == 2 ? 4 : 2));
  float acc[NV][8];
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[i][q] = 0.0f;
  for (int k0 = 0; y_rows > 0 && k0 < K; k0 += kGroup) {
    u32x4 v[kGroup][NV];
#pragma unroll
    for (int kk = 0; kk < kGroup; ++kk) {
      const int k = k0 + kk;
      if (RM) {
        // rank-major: a repeated row (about three of a token's eight at the
        // prefill routing) is not read at all; a stand-in load per repeat
        // made this combine 15% slower on MI355X
        const int row = read_row(myrow, keep, k, K, y_rows, -1);
        const u32x4* src = y + (int64_t)(row < 0 ? 0 : row) * V;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          if (row < 0) {
            v[kk][i] = u32x4{0u, 0u, 0u, 0u};
            continue;
          }
          v[kk][i] = __builtin_nontemporal_load(src + min(base + lane + kWave * i, V - 1));
        }
        continue;
      }
      const int row = read_row(myrow, keep, k, K, y_rows, stand_in);
      const u32x4* src = y + (int64_t)row * V;
#pragma unroll
      for (int i = 0; i < NV; ++i)
        v[kk][i] = __builtin_nontemporal_load(src + min(base + lane + kWave * i, V - 1));
    }
#pragma unroll
    for (int kk = 0; kk < kGroup; ++kk) {
      const int k = k0 + kk;
      if (k >= K) break;
      if (RM && !((keep >> k) & 1)) continue;
      const int row = __builtin_amdgcn_readlane(myrow, k);
      if (row < 0 || row >= y_rows) continue;
      const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myw), k));
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[i][2 * q] = __builtin_fmaf(wk, bf16_lo(v[kk][i][q]), acc[i][2 * q]);
          acc[i][2 * q + 1] = __builtin_fmaf(wk, bf16_hi(v[kk][i][q]), acc[i][2 * q + 1]);
        }
    }
  }
  const bool past = __ballot(lane < K && myrow >= y_rows) != 0;  // every lane takes part
  if (past && lane == 0 && base == 0) set_err(err, EP_DEVERR_CAPACITY);
  u32x4* dst = out + (int64_t)tok * V;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = base + lane + kWave * i;
    if (j < V) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = f32_to_bf16_rne(acc[i][2 * q]) | (f32_to_bf16_rne(acc[i][2 * q + 1]) << 16);
      __builtin_nontemporal_store(o, dst + j);
    }
  }
}

// Two tokens per block, for one vector per lane and K <= 8: the second
// token's row loads are issued before the first token's multiply-adds, so
// each wave keeps a full set of loads in flight while it computes.
constexpr int kPipeK = 8;
constexpr int kPipeTokens = 2;
constexpr int64_t kPipeMinTokens = 8192;

// Loads of one token's (up to kPipeK) rows, one vector per lane; entries
// whose row is not read load the stand-in row (a token that reads no row
// at all loads row 0's lines, its only HBM cost), so the previous token's
// loads stay in flight meanwhile.
template <bool RM>
__device__ __forceinline__ void load_rows8(const u32x4* __restrict__ y, int myrow, uint64_t keep,
                                           int K, int j, int V, int64_t y_rows,
                                           u32x4 (&v)[kPipeK]) {
  if (y_rows == 0) {  // nothing to read; every entry is skipped (uniform per launch)
#pragma unroll
    for (int k = 0; k < kPipeK; ++k) v[k] = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const int stand_in = RM ? -1 : max(stand_in_row(myrow, keep, K, y_rows), 0);
#pragma unroll
  for (int k = 0; k < kPipeK; ++k) {
    const int row = read_row(myrow, keep, k, K, y_rows, stand_in);
    if (RM && row < 0) {  // rank-major repeats are not read (as in combine_rows)
      v[k] = u32x4{0u, 0u, 0u, 0u};
      continue;
    }
    v[k] = __builtin_nontemporal_load(y + (int64_t)row * V + min(j, V - 1));
  }
}

// ST (hidden <= 4096): the block's output rows are staged in LDS and
// stored by all its wavefronts after both tokens are summed, instead of
// each wavefront storing its piece as soon as it is summed.  Measured on
// MI355X at the prefill routing: 3% faster at hidden 4096 and 0.7% at
// 2048, but 4-10% slower at 5120-7168, so wider rows store directly.
constexpr int kStageMaxVectors = 512;

template <bool RM, bool ST>
__global__ __launch_bounds__(1024) void combine_rows_pipe(const u32x4* __restrict__ y,
                                                          const int32_t* __restrict__ send_pos,
                                                          const float* __restrict__ w,
                                                          u32x4* __restrict__ out, int V, int K,
                                                          int n_tok, int64_t y_rows,
                                                          int32_t* err) {
  extern __shared__ u32x4 out_lds[];
  const int lane = threadIdx.x & 63;
  const int j = uniform(threadIdx.x >> 6) * kWave + lane;
  const int tok0 = blockIdx.x * kPipeTokens;
  int myrow = lane < K ? send_pos[(int64_t)tok0 * K + lane] : -1;
  uint64_t keep = RM ? first_rows(myrow, K) : ~0ull;
  u32x4 a[kPipeK];
  load_rows8<RM>(y, myrow, keep, K, j, V, y_rows, a);
  for (int r = 0; r < kPipeTokens; ++r) {
    const int tok = tok0 + r;
    if (tok >= n_tok) break;
    const float myw = RM ? 1.0f : (lane < K ? w[(int64_t)tok * K + lane] : 0.0f);
    u32x4 b[kPipeK];
    int nextrow = -1;
    uint64_t nextkeep = 0;
    const bool more = r + 1 < kPipeTokens && tok + 1 < n_tok;
    if (more) {
      nextrow = lane < K ? send_pos[(int64_t)(tok + 1) * K + lane] : -1;
      nextkeep = RM ? first_rows(nextrow, K) : ~0ull;
      load_rows8<RM>(y, nextrow, nextkeep, K, j, V, y_rows, b);
    }
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
    for (int k = 0; k < kPipeK; ++k) {
      if (k >= K) break;
      if (RM && !((keep >> k) & 1)) continue;
      const int row = __builtin_amdgcn_readlane(myrow, k);
      if (row < 0) continue;
      if (row >= y_rows) {
        if (lane == 0 && j < kWave) set_err(err, EP_DEVERR_CAPACITY);
        continue;
      }
      const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myw), k));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = __builtin_fmaf(wk, bf16_lo(a[k][q]), acc[2 * q]);
        acc[2 * q + 1] = __builtin_fmaf(wk, bf16_hi(a[k][q]), acc[2 * q + 1]);
      }
    }
    if (j < V) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = f32_to_bf16_rne(acc[2 * q]) | (f32_to_bf16_rne(acc[2 * q + 1]) << 16);
      if (ST) out_lds[r * V + j] = o;
      else __builtin_nontemporal_store(o, out + (int64_t)tok * V + j);
    }
    if (more) {
#pragma unroll
      for (int k = 0; k < kPipeK; ++k) a[k] = b[k];
      myrow = nextrow;
      keep = nextkeep;
    }
  }
  if (ST) {
    __syncthreads();
    const int nt = min(kPipeTokens, n_tok - tok0);
    for (int r = 0; r < nt; ++r)
      for (int jj = threadIdx.x; jj < V; jj += blockDim.x)
        __builtin_nontemporal_store(out_lds[r * V + jj], out + (int64_t)(tok0 + r) * V + jj);
  }
}

template <int NV, bool RM>
static void launch_nv(const CombineArgs& a, int V, int waves, hipStream_t st) {
  const int N = a.g.R * a.g.T;
  hipLaunchKernelGGL((combine_rows<NV, RM>), dim3(N), dim3(kWave * waves), 0, st,
                     (const u32x4*)a.y, a.send_pos, a.w, (u32x4*)a.out, V, a.g.K, a.y_rows,
                     a.err);
}

template <bool RM>
static void launch_rows(const CombineArgs& a, int nv, int V, int waves, hipStream_t st) {
  switch (nv) {
    case 1: launch_nv<1, RM>(a, V, waves, st); break;
    case 2: launch_nv<2, RM>(a, V, waves, st); break;
    case 3: launch_nv<3, RM>(a, V, waves, st); break;
    default: launch_nv<4, RM>(a, V, waves, st); break;  // hidden <= 32768: nv <= 4
  }
}

// Kernel choice by measurement on MI355X (prefill routing, 8 x 4096 tokens,
// top-8; interleaved runs per box):
//  - normal and low-latency modes at hidden 7168-8192 or up to 2048: one
//    token per block, one row load in flight per wavefront (combine_rows
//    SERIAL): at 7168 2.4% faster than the two-token pipeline, at 2048
//    4.9%; with fewer than 8,192 tokens at 7168-8192 the wavefronts take
//    four vectors per lane (the decode shape, 1,024 tokens: 8% faster than
//    eight loads in flight; at the prefill shape one vector per lane wins
//    by 9%);
//  - otherwise, from 8,192 tokens with top-k <= 8, the two-token pipeline
//    (outputs staged in LDS up to hidden 4096) -- best at 4096-6144 --
//    except rank-major rows wider than 4096, where one token per block with
//    eight row loads in flight is 4% faster;
//  - otherwise one token per block, eight row loads in flight.
constexpr int kSerialMinVectors = 896;  // hidden 7168
constexpr int kSerialMaxVectors = 256;  // hidden 2048

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  const int64_t N = (int64_t)a.g.R * a.g.T;
  if (N == 0) return hipSuccess;
  const int V = a.g.H / 8;
  int nv = 1;
  while ((V + kWave * nv - 1) / (kWave * nv) > 16) ++nv;
  const int waves = (V + kWave * nv - 1) / (kWave * nv);
  const u32x4* y = (const u32x4*)a.y;
  u32x4* out = (u32x4*)a.out;
  if (nv == 1 && !a.rank_major && (V >= kSerialMinVectors || V <= kSerialMaxVectors)) {
    if (V >= kSerialMinVectors && N < kPipeMinTokens) {
      // few tokens (decode): four vectors per lane, 5% faster than one at
      // 1,024 tokens
      const int w4 = (V + kWave * 4 - 1) / (kWave * 4);
      hipLaunchKernelGGL((combine_rows<4, false, true>), dim3((unsigned)N), dim3(kWave * w4), 0,
                         st, y, a.send_pos, a.w, out, V, a.g.K, a.y_rows, a.err);
    } else {
      hipLaunchKernelGGL((combine_rows<1, false, true>), dim3((unsigned)N), dim3(kWave * waves),
                         0, st, y, a.send_pos, a.w, out, V, a.g.K, a.y_rows, a.err);
    }
    return hipGetLastError();
  }
  // two tokens per block only when there are enough blocks to fill the chip
  const bool pipe = nv == 1 && a.g.K <= kPipeK && N >= kPipeMinTokens &&
                    !(a.rank_major && V > kStageMaxVectors);
  if (pipe) {
    const int n = (int)N;
    const dim3 grid((n + kPipeTokens - 1) / kPipeTokens), block(kWave * waves);
    const bool stage = V <= kStageMaxVectors;
    const size_t lds = stage ? sizeof(u32x4) * (size_t)kPipeTokens * V : 0;
    if (a.rank_major && stage)
      hipLaunchKernelGGL((combine_rows_pipe<true, true>), grid, block, lds, st, y, a.send_pos,
                         a.w, out, V, a.g.K, n, a.y_rows, a.err);
    else if (stage)
      hipLaunchKernelGGL((combine_rows_pipe<false, true>), grid, block, lds, st, y, a.send_pos,
                         a.w, out, V, a.g.K, n, a.y_rows, a.err);
    else
      hipLaunchKernelGGL((combine_rows_pipe<false, false>), grid, block, 0, st, y, a.send_pos,
                         a.w, out, V, a.g.K, n, a.y_rows, a.err);
    return hipGetLastError();
  }
  if (a.rank_major) launch_rows<true>(a, nv, V, waves, st);
  else launch_rows<false>(a, nv, V, waves, st);
  return hipGetLastError();
}

}  // namespace ep
