/*
 * ep_oracle.c -- plain, slow, single-threaded CPU oracle.  TEST
 * INFRASTRUCTURE ONLY: see ep_oracle.h for the sources it follows and for
 * who may call it.  Written for a reader checking it against the pages:
 * straight loops in the order the method states its steps, no blocking,
 * no fusion, no parallelism.
 *
 * Build: gcc -O2 -std=c99 -fPIC -shared -ffp-contract=off (no fast-math:
 * IEEE fp32 division and round-to-nearest-even are relied on).
 */
#include "ep_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ====================================================================== */
/* Scalar codecs                                                           */
/* ====================================================================== */

/* OCP 8-bit floating point, E4M3 variant without infinities ("E4M3FN"):
 * 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent field 0
 * holds subnormals m * 2^-9; S.1111.111 is NaN, so the largest finite
 * magnitude is 1.75 * 2^8 = 448.  Rounding is to nearest, ties to even.
 * Reading: magnitudes that round above 448 saturate to 448 (the scaled
 * inputs never exceed 448 by more than fp32 rounding slop, where plain
 * round-to-nearest already gives 448).  Sign is kept, so tiny negative
 * values encode as 0x80 (-0).  Inputs are finite. */
uint8_t orc_e4m3_encode(float v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  float a = fabsf(v);
  if (a > 448.0f) return sign | 0x7E;
  if (a < ldexpf(1.0f, -6)) {
    /* subnormal range: integer multiple of 2^-9, m = 8 is the smallest
     * normal (exponent field 1, mantissa 0), which is also code 8. */
    float m = rintf(ldexpf(a, 9)); /* exact scaling, then RNE to integer */
    return sign | (uint8_t)m;
  }
  int ex;
  float f = frexpf(a, &ex);          /* a = f * 2^ex, f in [0.5, 1) */
  float sig = 2.0f * f;              /* a = sig * 2^(ex-1), sig in [1, 2) */
  int e = ex - 1;
  float q = rintf((sig - 1.0f) * 8.0f); /* 3-bit mantissa, RNE (exact ops) */
  if (q == 8.0f) { q = 0.0f; e += 1; }
  int biased = e + 7;
  if (biased > 15 || (biased == 15 && q == 7.0f)) return sign | 0x7E;
  return sign | (uint8_t)((biased << 3) | (int)q);
}

float orc_e4m3_decode(uint8_t code) {
  float sgn = (code & 0x80) ? -1.0f : 1.0f;
  int ef = (code >> 3) & 0xF;
  int m = code & 0x7;
  if (ef == 15 && m == 7) return NAN;
  if (ef == 0) return sgn * ldexpf((float)m, -9);
  return sgn * ldexpf(1.0f + (float)m / 8.0f, ef - 7);
}

void orc_e4m3_encode_array(const float* v, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}

/* bfloat16 = the upper half of an IEEE binary32: 8 significant bits, the
 * binary32 exponent range.  Round a double to it once, nearest-even. */
uint16_t orc_bf16_from_double(double v) {
  uint32_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (a == 0.0) return (uint16_t)sign;
  double q;
  if (a < ldexp(1.0, -126)) {
    /* bf16 subnormals are multiples of 2^-133 */
    q = rint(ldexp(a, 133));
    q = ldexp(q, -133);
  } else {
    int ex;
    double f = frexp(a, &ex);           /* a = f * 2^ex, f in [0.5, 1) */
    double m = rint(ldexp(f, 8));       /* 8 significant bits, RNE      */
    q = ldexp(m, ex - 8);
  }
  if (q >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u); /* inf */
  float qf = (float)q; /* exact: q has at most 8 significant bits */
  uint32_t bits;
  memcpy(&bits, &qf, 4);
  return (uint16_t)(sign | (bits >> 16));
}

double orc_bf16_to_double(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

static float bf16_to_float(uint16_t b) { return (float)orc_bf16_to_double(b); }

/* Per-128-channel group scale with an fp32 scale: the group's largest
 * magnitude maps to 448, the largest E4M3 value.  Reading: amax is floored
 * at 1e-4 so an all-zero group does not divide by zero. */
float orc_fp8_scale_f32(float amax) {
  float a = amax > 1e-4f ? amax : 1e-4f;
  return a / 448.0f; /* IEEE fp32 division, nearest-even */
}

/* Power-of-two ("UE8M0") scale: the fp32 scale rounded UP to a power of two,
 * stored as its 8-bit biased exponent.  Rounding up keeps amax / scale <= 448. */
uint8_t orc_fp8_scale_ue8m0(float amax) {
  float r = orc_fp8_scale_f32(amax);
  int ex;
  float f = frexpf(r, &ex);   /* r = f * 2^ex, f in [0.5, 1) */
  /* r is a power of two exactly when f == 0.5: then r = 2^(ex-1) */
  int e = (f == 0.5f) ? ex - 1 : ex;
  return (uint8_t)(e + 127);
}

/* ====================================================================== */
/* Layout: counts, rank prefix matrix, receive offsets, slots              */
/* ====================================================================== */

static int topk_ok(const orc_problem* p, int32_t e) { return e >= -1 && e < p->E; }

static int64_t roundup64(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

int64_t orc_recv_rows(const orc_problem* p, const int32_t* topk) {
  const int R = p->R, T = p->T, E = p->E, K = p->K;
  if (p->mode == ORC_MODE_LL) return (int64_t)E * R * T;
  if (p->mode == ORC_MODE_RANK) { /* one row per (token, destination rank) */
    const int L = E / R;
    int64_t total = 0;
    uint8_t* hit = (uint8_t*)malloc((size_t)(R > 0 ? R : 1));
    for (int64_t tok = 0; tok < (int64_t)R * T; ++tok) {
      memset(hit, 0, (size_t)R);
      for (int k = 0; k < K; ++k) {
        int32_t e = topk[tok * K + k];
        if (e >= 0 && e < E && !hit[e / L]) { hit[e / L] = 1; ++total; }
      }
    }
    free(hit);
    return total;
  }
  if (p->mode != ORC_MODE_NORMAL) return 0;
  int64_t* n = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  for (int64_t i = 0; i < (int64_t)R * T * K; ++i) {
    int32_t e = topk[i];
    if (e >= 0 && e < E) n[e]++;
  }
  int64_t total = 0;
  for (int e = 0; e < E; ++e) total += roundup64(n[e], p->align);
  free(n);
  return total;
}

/*
 * [DEEP] sec. 2.1 / 2.3 / 3.2 / 4.3.
 *  - The expert e lives on rank e / L, L = E / R.
 *  - cnt_expert[s][e]: (token, k) entries of source s routed to e.
 *  - cnt_rank[s][r]: tokens of s with at least one expert on rank r
 *    (a token is sent once per destination rank; in_rank marks it).
 *  - rank_prefix[i][j] = sum over source ranks s <= i of cnt_rank[s][j]
 *    (inclusive, "ranks not above i").
 *  - Receive side, per expert: n[e] = sum_s cnt_expert[s][e]; normal mode
 *    rounds it up to expert_alignment and lays the L experts of rank d out
 *    back to back (segment offsets = prefix sum of the aligned counts);
 *    the R ranks' partitions are packed back to back (row_base).
 *    LL mode gives every expert a fixed R*T-row block.
 *  - Slots: walking source ranks, then tokens, then k in ascending order,
 *    each entry takes the next free row of its expert's segment, so each
 *    segment is ordered by (source rank, token, k).
 *  - send_head[s][t][d]: index of token t among the tokens s sends to
 *    rank d (in token order), -1 when t is not sent to d.
 *  - recv_src_idx[row] = s * T + t for every filled row, -1 elsewhere.
 *  - Rank-major mode ([DEEP] sec. 2.3, the V1 receive buffer): rank d
 *    receives each token with an expert on d once; its partition is ordered
 *    by source rank (segment of s starts at rank_prefix[s-1][d], the
 *    exclusive prefix) and then by the token's index in the (s, d) stream
 *    (send_head); partitions are packed back to back.  send_pos[s][t][k]
 *    is the row of token t on the rank of expert k (the same row for every
 *    k on that rank).
 * Entries equal to -1 mean "no expert" and are skipped (reading: the
 * pages never state the index type or a masked value; int32 with -1 as
 * masked is the plain reading).  Out-of-range entries set an error bit and
 * are skipped.  In LL mode a position past the R*T rows of its block sets
 * an error bit and gets send_pos -1.
 */
int orc_layout(const orc_problem* p, const int32_t* topk, int32_t* cnt_rank,
               int32_t* cnt_expert, uint8_t* in_rank, int32_t* rank_prefix,
               int32_t* recv_per_expert, int32_t* expert_start, int32_t* rows,
               int32_t* row_base, int32_t* send_pos, int32_t* send_head,
               int32_t* recv_src_idx, int64_t recv_cap) {
  const int R = p->R, T = p->T, E = p->E, K = p->K;
  const int L = E / R;
  int err = 0;

  memset(cnt_rank, 0, sizeof(int32_t) * R * R);
  memset(cnt_expert, 0, sizeof(int32_t) * R * E);
  memset(in_rank, 0, (size_t)R * T * R);

  /* counts */
  for (int s = 0; s < R; ++s)
    for (int t = 0; t < T; ++t)
      for (int k = 0; k < K; ++k) {
        int32_t e = topk[((int64_t)s * T + t) * K + k];
        if (!topk_ok(p, e)) { err |= ORC_ERR_TOPK_RANGE; continue; }
        if (e < 0) continue;
        cnt_expert[s * E + e] += 1;
        int r = e / L;
        uint8_t* flag = &in_rank[((int64_t)s * T + t) * R + r];
        if (!*flag) {
          *flag = 1;
          cnt_rank[s * R + r] += 1;
        }
      }

  /* rank prefix matrix (inclusive over source ranks) */
  for (int j = 0; j < R; ++j) {
    int32_t acc = 0;
    for (int i = 0; i < R; ++i) {
      acc += cnt_rank[i * R + j];
      rank_prefix[i * R + j] = acc;
    }
  }

  /* receive counts per expert */
  for (int e = 0; e < E; ++e) {
    int32_t n = 0;
    for (int s = 0; s < R; ++s) n += cnt_expert[s * E + e];
    recv_per_expert[e] = n;
  }

  /* segment starts */
  if (p->mode == ORC_MODE_RANK) {
    int32_t base = 0;
    for (int d = 0; d < R; ++d) {
      row_base[d] = base;
      rows[d] = rank_prefix[(R - 1) * R + d];
      for (int l = 0; l < L; ++l) expert_start[d * L + l] = base;
      base += rows[d];
    }
    row_base[R] = base;
  } else if (p->mode == ORC_MODE_LL) {
    for (int e = 0; e < E; ++e) expert_start[e] = e * R * T;
    for (int d = 0; d < R; ++d) {
      rows[d] = L * R * T;
      row_base[d] = d * L * R * T;
    }
    row_base[R] = E * R * T;
  } else {
    int32_t base = 0;
    for (int d = 0; d < R; ++d) {
      row_base[d] = base;
      int32_t off = 0;
      for (int l = 0; l < L; ++l) {
        int e = d * L + l;
        expert_start[e] = base + off;
        off += (int32_t)roundup64(recv_per_expert[e], p->align);
      }
      rows[d] = off;
      base += off;
    }
    row_base[R] = base;
  }

  int64_t nrows = (p->mode == ORC_MODE_LL) ? (int64_t)E * R * T : row_base[R];
  if (recv_src_idx != NULL) {
    if (p->mode != ORC_MODE_MSG && recv_cap < nrows) err |= ORC_ERR_CAPACITY;
    for (int64_t i = 0; i < recv_cap; ++i) recv_src_idx[i] = -1;
  }

  if (p->mode == ORC_MODE_RANK) {
    /* rank-level slots: the stream index of the token, after the tokens of
     * earlier sources */
    int32_t* head = (int32_t*)malloc(sizeof(int32_t) * (R > 0 ? R : 1));
    for (int s = 0; s < R; ++s) {
      for (int d = 0; d < R; ++d) head[d] = 0;
      for (int t = 0; t < T; ++t) {
        for (int d = 0; d < R; ++d) {
          int64_t hi = ((int64_t)s * T + t) * R + d;
          int32_t v = in_rank[hi] ? head[d]++ : -1;
          if (send_head != NULL) send_head[hi] = v;
          if (v < 0) continue;
          int32_t row = row_base[d] + (rank_prefix[s * R + d] - cnt_rank[s * R + d]) + v;
          if (recv_src_idx != NULL && row < recv_cap) recv_src_idx[row] = s * T + t;
        }
        for (int k = 0; k < K; ++k) {
          int64_t i = ((int64_t)s * T + t) * K + k;
          int32_t e = topk[i], row = -1;
          if (e >= 0 && e < E) {
            int d = e / L;
            row = row_base[d] + (rank_prefix[s * R + d] - cnt_rank[s * R + d]) +
                  (head[d] - 1); /* this token was the last one counted on d */
          }
          if (send_pos != NULL) send_pos[i] = row;
        }
      }
    }
    free(head);
    return err;
  }

  /* expert-level slots: one running counter per expert across all sources */
  int32_t* next = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int s = 0; s < R; ++s)
    for (int t = 0; t < T; ++t)
      for (int k = 0; k < K; ++k) {
        int64_t i = ((int64_t)s * T + t) * K + k;
        int32_t e = topk[i];
        int32_t row = -1;
        if (e >= 0 && e < E) {
          int32_t pos = next[e]++;
          if (p->mode == ORC_MODE_LL && pos >= R * T) {
            err |= ORC_ERR_LL_OVERFLOW;
          } else {
            row = expert_start[e] + pos;
          }
        }
        if (send_pos != NULL) send_pos[i] = (p->mode == ORC_MODE_MSG) ? -1 : row;
        if (recv_src_idx != NULL && row >= 0 && p->mode != ORC_MODE_MSG && row < recv_cap)
          recv_src_idx[row] = s * T + t;
      }
  free(next);

  /* rank-level slots: token order within each (source, destination) stream */
  if (send_head != NULL) {
    for (int s = 0; s < R; ++s)
      for (int d = 0; d < R; ++d) {
        int32_t c = 0;
        for (int t = 0; t < T; ++t) {
          int64_t i = ((int64_t)s * T + t) * R + d;
          send_head[i] = in_rank[i] ? c++ : -1;
        }
      }
  }
  return err;
}

/* ====================================================================== */
/* Dispatch                                                                */
/* ====================================================================== */

static int64_t scale_index(const orc_problem* p, int64_t row, int g, int64_t cap) {
  const int64_t RT = (int64_t)p->R * p->T;
  const int G = p->H / 128;
  if (p->mode == ORC_MODE_LL) {
    int64_t e = row / RT, pos = row % RT;
    return (e * G + g) * RT + pos;
  }
  return (int64_t)g * cap + row;
}

/* Quantise one token: per 128-channel group, amax -> scale -> codes.
 * [DEEP] sec. 1.1 (FP8 dispatch, bf16 combine) and sec. 1.2 (scale options:
 * fp32 scale, or power-of-two scale; column-major scale tensor). */
static void quantise_token(const orc_problem* p, const uint16_t* xrow, uint8_t* codes,
                           float* sc_f32, uint8_t* sc_e8) {
  const int H = p->H, G = H / 128;
  for (int g = 0; g < G; ++g) {
    float amax = 0.0f;
    for (int c = g * 128; c < (g + 1) * 128; ++c) {
      float v = fabsf(bf16_to_float(xrow[c]));
      if (v > amax) amax = v;
    }
    if (p->quant == ORC_Q_FP8_F32) {
      float sc = orc_fp8_scale_f32(amax);
      sc_f32[g] = sc;
      for (int c = g * 128; c < (g + 1) * 128; ++c)
        codes[c] = orc_e4m3_encode(bf16_to_float(xrow[c]) / sc);
    } else {
      uint8_t ex = orc_fp8_scale_ue8m0(amax);
      sc_e8[g] = ex;
      for (int c = g * 128; c < (g + 1) * 128; ++c)
        codes[c] = orc_e4m3_encode(ldexpf(bf16_to_float(xrow[c]), 127 - (int)ex));
    }
  }
}

/* Rank-major receive metadata (see the header). */
int orc_rank_topk(const orc_problem* p, const int32_t* topk, const float* w,
                  const int32_t* send_pos, int64_t cap, int32_t* recv_topk_idx,
                  float* recv_topk_weights) {
  const int R = p->R, T = p->T, E = p->E, K = p->K, L = E / R;
  int err = 0;
  for (int64_t tok = 0; tok < (int64_t)R * T; ++tok)
    for (int k = 0; k < K; ++k) {
      int32_t row = send_pos[tok * K + k];
      if (row < 0) continue;
      if (row >= cap) { err |= ORC_ERR_CAPACITY; continue; }
      int d = topk[tok * K + k] / L;
      for (int k2 = 0; k2 < K; ++k2) {
        int32_t e = topk[tok * K + k2];
        int on_d = e >= 0 && e < E && e / L == d;
        recv_topk_idx[(int64_t)row * K + k2] = on_d ? e - d * L : -1;
        recv_topk_weights[(int64_t)row * K + k2] = on_d ? w[tok * K + k2] : 0.0f;
      }
    }
  return err;
}

/* Every routed (token, expert) entry copies the token to its slot row:
 * recv[send_pos[s][t][k]] = x[s][t] (bf16), or the token's FP8 codes plus
 * one scale per 128-channel group. */
int orc_dispatch(const orc_problem* p, const uint16_t* x, const int32_t* topk,
                 const int32_t* send_pos, void* recv, void* scales, int64_t cap) {
  const int R = p->R, T = p->T, H = p->H, K = p->K, G = H / 128;
  int err = 0;
  uint8_t* codes = (uint8_t*)malloc((size_t)H);
  float* sf = (float*)malloc(sizeof(float) * (G > 0 ? G : 1));
  uint8_t* se = (uint8_t*)malloc((size_t)(G > 0 ? G : 1));
  for (int s = 0; s < R; ++s)
    for (int t = 0; t < T; ++t) {
      const uint16_t* xrow = x + ((int64_t)s * T + t) * H;
      if (p->quant != ORC_Q_NONE) quantise_token(p, xrow, codes, sf, se);
      for (int k = 0; k < K; ++k) {
        int64_t i = ((int64_t)s * T + t) * K + k;
        (void)topk;
        int32_t row = send_pos[i];
        if (row < 0) continue;
        if (p->mode == ORC_MODE_RANK) { /* one row per destination rank */
          int seen = 0;
          for (int k2 = 0; k2 < k; ++k2) seen |= send_pos[i - k + k2] == row;
          if (seen) continue;
        }
        if (row >= cap) { err |= ORC_ERR_CAPACITY; continue; }
        if (p->quant == ORC_Q_NONE) {
          memcpy((uint16_t*)recv + (int64_t)row * H, xrow, sizeof(uint16_t) * H);
        } else {
          memcpy((uint8_t*)recv + (int64_t)row * H, codes, (size_t)H);
          for (int g = 0; g < G; ++g) {
            int64_t si = scale_index(p, row, g, cap);
            if (p->quant == ORC_Q_FP8_F32) ((float*)scales)[si] = sf[g];
            else ((uint8_t*)scales)[si] = se[g];
          }
        }
      }
    }
  free(codes);
  free(sf);
  free(se);
  return err;
}

/* The expert used for end-to-end checks is the identity: it returns its
 * input rows, dequantised to bf16: y = bf16(decode(code) * scale), the
 * product formed exactly in fp64 and rounded once. */
void orc_dequant_rows(const orc_problem* p, const uint8_t* codes, const void* scales,
                      int64_t cap, const int32_t* row_list, int64_t nrows, uint16_t* y) {
  const int H = p->H, G = H / 128;
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t row = row_list[i];
    for (int g = 0; g < G; ++g) {
      int64_t si = scale_index(p, row, g, cap);
      double sc = (p->quant == ORC_Q_FP8_F32)
                      ? (double)((const float*)scales)[si]
                      : ldexp(1.0, (int)((const uint8_t*)scales)[si] - 127);
      for (int c = g * 128; c < (g + 1) * 128; ++c) {
        double v = (double)orc_e4m3_decode(codes[row * H + c]) * sc;
        y[i * H + c] = orc_bf16_from_double(v);
      }
    }
  }
}

/* ====================================================================== */
/* Combine                                                                 */
/* ====================================================================== */

/* Inverse of dispatch ([DEEP] sec. 2.3, the handle walked backwards; sec. 5
 * combine is the inverse path): each token gathers the expert outputs of
 * its routed rows and takes their top-k weighted sum.  The oracle forms
 * the exact sum in fp64 (k ascending) and rounds once to bf16; a token
 * with no routed entry gets 0. */
int orc_combine(const orc_problem* p, const uint16_t* y, int64_t y_rows, const float* w,
                const int32_t* send_pos, const int64_t* token_list, int64_t ntok,
                uint16_t* out) {
  const int R = p->R, T = p->T, H = p->H, K = p->K;
  int err = 0;
  int64_t count = token_list ? ntok : (int64_t)R * T;
  double* acc = (double*)malloc(sizeof(double) * H);
  for (int64_t j = 0; j < count; ++j) {
    int64_t tok = token_list ? token_list[j] : j; /* tok = s * T + t */
    for (int c = 0; c < H; ++c) acc[c] = 0.0;
    for (int k = 0; k < K; ++k) {
      int32_t row = send_pos[tok * K + k];
      if (row < 0) continue;
      double wk;
      if (p->mode == ORC_MODE_RANK) {
        /* rank-major: the token's rows on its destination ranks, each once,
         * unweighted (the expert stage on rank d already applied the
         * weights of d's experts) */
        int seen = 0;
        for (int k2 = 0; k2 < k; ++k2) seen |= send_pos[tok * K + k2] == row;
        if (seen) continue;
        wk = 1.0;
      } else {
        wk = (double)w[tok * K + k];
      }
      if (row >= y_rows) { err |= ORC_ERR_CAPACITY; continue; }
      const uint16_t* yrow = y + (int64_t)row * H;
      for (int c = 0; c < H; ++c) acc[c] += wk * orc_bf16_to_double(yrow[c]);
    }
    for (int c = 0; c < H; ++c) out[j * H + c] = orc_bf16_from_double(acc[c]);
  }
  free(acc);
  return err;
}

/* ====================================================================== */
/* Messages + write descriptors                                            */
/* ====================================================================== */

/* Body of one (source, destination) message carrying n tokens, in order:
 *   [0] payload rows  n*H e4m3 codes (or n*H bf16 when unquantised)
 *   [1] scales        n*G (fp32, or one exponent byte each; none for bf16)
 *   [2] top-k weights n*K fp32
 *   [3] top-k ids     n*K int32 (global expert ids as routed)
 *   [4] source token  n   int32 (token index within the source rank)
 * Each section is zero-padded to a 16-byte multiple so every section and
 * the whole body stay 16-byte aligned ([EAAS]: payload packed 16-byte
 * aligned).  Reading: the pages pack hidden state, weights, then scales,
 * with the expert ids in the header; here the ids travel in the body
 * because a 16-byte header cannot carry n tokens' ids, and the scales
 * follow their codes. */
int64_t orc_msg_body_bytes(const orc_problem* p, int64_t n, int64_t sec_off[6]) {
  const int64_t H = p->H, G = p->H / 128, K = p->K;
  int64_t len[5];
  len[0] = n * H * (p->quant == ORC_Q_NONE ? 2 : 1);
  len[1] = n * G * (p->quant == ORC_Q_FP8_F32 ? 4 : (p->quant == ORC_Q_FP8_UE8M0 ? 1 : 0));
  len[2] = n * K * 4;
  len[3] = n * K * 4;
  len[4] = n * 4;
  int64_t off = 0;
  for (int i = 0; i < 5; ++i) {
    if (sec_off) sec_off[i] = off;
    off += roundup64(len[i], 16);
  }
  if (sec_off) sec_off[5] = off;
  return off;
}

static void put_be32(uint8_t* b, uint32_t v) {
  b[0] = (uint8_t)(v >> 24); b[1] = (uint8_t)(v >> 16);
  b[2] = (uint8_t)(v >> 8);  b[3] = (uint8_t)v;
}
static void put_be64(uint8_t* b, uint64_t v) {
  put_be32(b, (uint32_t)(v >> 32));
  put_be32(b + 4, (uint32_t)v);
}
static void put_le32(uint8_t* b, uint32_t v) {
  b[0] = (uint8_t)v; b[1] = (uint8_t)(v >> 8);
  b[2] = (uint8_t)(v >> 16); b[3] = (uint8_t)(v >> 24);
}

/* One 64-byte write descriptor: control, remote-address and data segments
 * of 16 bytes each plus 16 bytes of zero padding, multi-byte fields
 * big-endian ([IBGDA] sec. 3, [GIC] WQE anatomy).  The opcode (0x08) and
 * the completion-update flag (0x08) are this format's own constants; keys
 * name (rank, region index). */
static void write_desc(uint8_t* d, uint32_t wqe_idx, uint32_t qpn, uint64_t raddr,
                       uint32_t rkey, uint32_t len, uint32_t lkey, uint64_t laddr) {
  memset(d, 0, 64);
  put_be32(d + 0, (wqe_idx << 8) | 0x08u);
  put_be32(d + 4, (qpn << 8) | 3u);
  d[11] = 0x08;
  put_be64(d + 16, raddr);
  put_be32(d + 24, rkey);
  put_be32(d + 32, len);
  put_be32(d + 36, lkey);
  put_be64(d + 40, laddr);
}

/*
 * [EAAS] packing kernel then the three puts; [IBGDA] sec. 1 chunking.
 *  - Only (s, d) pairs with n = cnt_rank[s][d] > 0 get a message.
 *  - Message region: 16-byte header {s, d, n, body_bytes} (u32, little
 *    endian), body, 16-byte completion flag {epoch, 0, 0, 0}.  Reading:
 *    the pages name the header and the flag but give no fields.
 *  - Tokens of message (s, d): the tokens t of s with in_rank[s][t][d], in
 *    ascending t.  Each carries its codes, scales, all K weights, all K
 *    expert ids and t.
 *  - Source s's send arena holds its messages for d ascending; destination
 *    d's receive arena holds the messages from s ascending; each rank's
 *    arena starts at a multiple of region_bytes.
 *  - Descriptors, message by message (s, then d): the payload put (body),
 *    the header put, the flag put ([EAAS]: payload, head, completion flag;
 *    the flag goes last so a receiver that sees it sees the rest,
 *    [GIC] Ordering).  Each put is cut into chunks that cross no multiple
 *    of region_bytes on either side: chunk = min(remaining, bytes to the
 *    next local boundary, bytes to the next remote boundary).  Addresses
 *    are offsets from the start of the rank's own arena.  qpn = s*R + d,
 *    the work-queue index counts from 0 within each message.
 */
int orc_messages(const orc_problem* p, const uint16_t* x, const int32_t* topk,
                 const float* w, uint8_t* send_arena, int64_t send_cap, int64_t* table,
                 int64_t* arena_base, uint8_t* desc, int64_t desc_cap, int64_t* num_desc) {
  const int R = p->R, T = p->T, H = p->H, K = p->K, G = H / 128;
  const int64_t RB = p->region_bytes;
  int err = 0;

  /* counts and token membership, from the layout */
  orc_problem q = *p;
  q.mode = ORC_MODE_MSG;
  int32_t* cnt_rank = (int32_t*)malloc(sizeof(int32_t) * R * R);
  int32_t* cnt_expert = (int32_t*)malloc(sizeof(int32_t) * R * p->E);
  uint8_t* in_rank = (uint8_t*)malloc((size_t)R * T * R);
  int32_t* rpm = (int32_t*)malloc(sizeof(int32_t) * R * R);
  int32_t* rpe = (int32_t*)malloc(sizeof(int32_t) * p->E);
  int32_t* est = (int32_t*)malloc(sizeof(int32_t) * p->E);
  int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * R);
  int32_t* rbase = (int32_t*)malloc(sizeof(int32_t) * (R + 1));
  err |= orc_layout(&q, topk, cnt_rank, cnt_expert, in_rank, rpm, rpe, est, rows, rbase,
                    NULL, NULL, NULL, 0);

  /* region sizes and arena offsets */
  int64_t* region = (int64_t*)calloc((size_t)R * R, sizeof(int64_t));
  for (int s = 0; s < R; ++s)
    for (int d = 0; d < R; ++d) {
      int64_t n = cnt_rank[s * R + d];
      region[s * R + d] = n > 0 ? 16 + orc_msg_body_bytes(p, n, NULL) + 16 : 0;
    }
  int64_t* send_base = arena_base;
  int64_t* recv_base = arena_base + (R + 1);
  send_base[0] = 0;
  for (int s = 0; s < R; ++s) {
    int64_t tot = 0;
    for (int d = 0; d < R; ++d) tot += region[s * R + d];
    send_base[s + 1] = send_base[s] + roundup64(tot, RB);
  }
  recv_base[0] = 0;
  for (int d = 0; d < R; ++d) {
    int64_t tot = 0;
    for (int s = 0; s < R; ++s) tot += region[s * R + d];
    recv_base[d + 1] = recv_base[d] + roundup64(tot, RB);
  }
  if (send_base[R] > send_cap) err |= ORC_ERR_CAPACITY;

  int64_t desc_count = 0;
  uint8_t* codes = (uint8_t*)malloc((size_t)H);
  float* sf = (float*)malloc(sizeof(float) * (G > 0 ? G : 1));
  uint8_t* se = (uint8_t*)malloc((size_t)(G > 0 ? G : 1));
  for (int s = 0; s < R; ++s) {
    int64_t soff = send_base[s];
    for (int d = 0; d < R; ++d) {
      int64_t* row = table + ((int64_t)s * R + d) * 8;
      int64_t n = cnt_rank[s * R + d];
      int64_t roff = recv_base[d];
      for (int s2 = 0; s2 < s; ++s2) roff += region[s2 * R + d];
      if (n == 0) {
        row[0] = -1; row[1] = -1; row[2] = 0; row[3] = 0;
        row[4] = 0; row[5] = desc_count; row[6] = 0; row[7] = 0;
        continue;
      }
      int64_t sec[6];
      int64_t body = orc_msg_body_bytes(p, n, sec);
      row[0] = soff; row[1] = roff; row[2] = region[s * R + d]; row[3] = n;
      row[4] = body; row[5] = desc_count; row[7] = 0;

      int fits = (soff + region[s * R + d] <= send_cap);
      if (fits) {
        uint8_t* m = send_arena + soff;
        memset(m, 0, (size_t)region[s * R + d]);
        put_le32(m + 0, (uint32_t)s);
        put_le32(m + 4, (uint32_t)d);
        put_le32(m + 8, (uint32_t)n);
        put_le32(m + 12, (uint32_t)body);
        uint8_t* b = m + 16;
        int64_t j = 0; /* index of the token within the message */
        for (int t = 0; t < T; ++t) {
          if (!in_rank[((int64_t)s * T + t) * R + d]) continue;
          const uint16_t* xrow = x + ((int64_t)s * T + t) * H;
          if (p->quant == ORC_Q_NONE) {
            memcpy(b + sec[0] + j * H * 2, xrow, (size_t)H * 2);
          } else {
            quantise_token(p, xrow, codes, sf, se);
            memcpy(b + sec[0] + j * H, codes, (size_t)H);
            if (p->quant == ORC_Q_FP8_F32) memcpy(b + sec[1] + j * G * 4, sf, (size_t)G * 4);
            else memcpy(b + sec[1] + j * G, se, (size_t)G);
          }
          memcpy(b + sec[2] + j * K * 4, w + ((int64_t)s * T + t) * K, (size_t)K * 4);
          memcpy(b + sec[3] + j * K * 4, topk + ((int64_t)s * T + t) * K, (size_t)K * 4);
          put_le32(b + sec[4] + j * 4, (uint32_t)t);
          ++j;
        }
        put_le32(m + 16 + body, p->epoch);
      }

      /* descriptors: payload, header, flag */
      int64_t put_off[3] = {16, 0, 16 + body};
      int64_t put_len[3] = {body, 16, 16};
      uint32_t wqe = 0;
      for (int u = 0; u < 3; ++u) {
        int64_t la = soff - send_base[s] + put_off[u];
        int64_t ra = roff - recv_base[d] + put_off[u];
        int64_t rem = put_len[u];
        while (rem > 0) {
          int64_t c = rem;
          if (RB - la % RB < c) c = RB - la % RB;
          if (RB - ra % RB < c) c = RB - ra % RB;
          if (desc_count < desc_cap) {
            /* a key keeps the region index in its low 16 bits; a piece in
             * region 65536 or later of either arena cannot be named, so its
             * keys are all ones (rank 0xFFFF: no such rank) and the capacity
             * bit is raised */
            uint32_t rkey = (uint32_t)((d << 16) | (ra / RB));
            uint32_t lkey = (uint32_t)((s << 16) | (la / RB));
            if (la / RB > 0xFFFF || ra / RB > 0xFFFF) {
              rkey = lkey = 0xFFFFFFFFu;
              err |= ORC_ERR_CAPACITY;
            }
            write_desc(desc + desc_count * 64, wqe, (uint32_t)(s * R + d), (uint64_t)ra, rkey,
                       (uint32_t)c, lkey, (uint64_t)la);
          } else {
            err |= ORC_ERR_CAPACITY;
          }
          ++desc_count; ++wqe;
          la += c; ra += c; rem -= c;
        }
      }
      row[6] = wqe;
      soff += region[s * R + d];
    }
  }
  *num_desc = desc_count;
  free(codes); free(sf); free(se); free(region);
  free(cnt_rank); free(cnt_expert); free(in_rank); free(rpm); free(rpe); free(est);
  free(rows); free(rbase);
  return err;
}

/* ---- message delivery (loopback) and receive -------------------------- */

static uint32_t get_be32(const uint8_t* b) {
  return ((uint32_t)b[0] << 24) | ((uint32_t)b[1] << 16) | ((uint32_t)b[2] << 8) | b[3];
}
static uint64_t get_be64(const uint8_t* b) {
  return ((uint64_t)get_be32(b) << 32) | get_be32(b + 4);
}
static uint32_t get_le32(const uint8_t* b) {
  return (uint32_t)b[0] | ((uint32_t)b[1] << 8) | ((uint32_t)b[2] << 16) | ((uint32_t)b[3] << 24);
}

/* [IBGDA] sec. 1 and [GIC] WQE anatomy: a write descriptor names the local
 * (lkey, laddr) and remote (rkey, raddr) addresses and the length; the
 * loopback "wire" copies the bytes.  Field offsets are this library's own
 * descriptor format (see orc_messages). */
int orc_messages_execute(const orc_problem* p, const uint8_t* send_arena, int64_t send_cap,
                         const int64_t* arena_base, const uint8_t* desc, int64_t num_desc,
                         uint8_t* recv_arena, int64_t recv_cap) {
  const int R = p->R;
  const int64_t* send_base = arena_base;
  const int64_t* recv_base = arena_base + (R + 1);
  int err = 0;
  for (int64_t i = 0; i < num_desc; ++i) {
    const uint8_t* dsc = desc + i * 64;
    const uint64_t raddr = get_be64(dsc + 16);
    const uint32_t rkey = get_be32(dsc + 24);
    const uint32_t len = get_be32(dsc + 32);
    const uint32_t lkey = get_be32(dsc + 36);
    const uint64_t laddr = get_be64(dsc + 40);
    const uint32_t s = lkey >> 16, d = rkey >> 16;
    if (s >= (uint32_t)R || d >= (uint32_t)R) {
      err |= ORC_ERR_MESSAGE;
      continue;
    }
    const int64_t src = send_base[s] + (int64_t)laddr, dst = recv_base[d] + (int64_t)raddr;
    if (src + len > send_base[s + 1] || src + len > send_cap || dst + len > recv_base[d + 1] ||
        dst + len > recv_cap) {
      err |= ORC_ERR_CAPACITY;
      continue;
    }
    memcpy(recv_arena + dst, send_arena + src, len);
  }
  return err;
}

/* [EAAS] (the receiver reads a loaded server's message once its completion
 * flag has arrived) and [DEEP] sec. 1.2 (low-latency packed layout, one
 * block of R*T rows per expert, recv_count).  Slots follow the stable
 * (source, token, k) order pinned for low-latency dispatch; the receiver
 * learns the per-source expert counts from the count exchange of [DEEP]
 * sec. 2.1 (cnt_expert), and everything else from the message bytes. */
int orc_messages_unpack(const orc_problem* p, const uint8_t* recv_arena, int64_t recv_cap,
                        const int64_t* table, const int32_t* cnt_expert, void* recv,
                        void* scales, int32_t* recv_count, int32_t* recv_src_idx) {
  const int R = p->R, T = p->T, H = p->H, E = p->E, K = p->K, L = E / R, G = H / 128;
  const int64_t RT = (int64_t)R * T;
  const int cb = p->quant == ORC_Q_NONE ? 2 : 1;
  const int sb = p->quant == ORC_Q_FP8_F32 ? 4 : (p->quant == ORC_Q_FP8_UE8M0 ? 1 : 0);
  int err = 0;
  for (int e = 0; e < E; ++e) {
    int64_t n = 0;
    for (int s = 0; s < R; ++s) n += cnt_expert[(int64_t)s * E + e];
    recv_count[e] = (int32_t)n;
  }
  int64_t* run = (int64_t*)malloc(sizeof(int64_t) * (L > 0 ? L : 1));
  for (int d = 0; d < R; ++d) {
    for (int s = 0; s < R; ++s) {
      const int64_t* row = table + ((int64_t)s * R + d) * 8;
      const int64_t n = row[3];
      if (n <= 0) continue;
      const int64_t off = row[1], region = row[2], body = row[4];
      if (off < 0 || off + region > recv_cap) {
        err |= ORC_ERR_CAPACITY;
        continue;
      }
      const uint8_t* m = recv_arena + off;
      int ok = get_le32(m) == (uint32_t)s && get_le32(m + 4) == (uint32_t)d &&
               get_le32(m + 8) == (uint32_t)n && get_le32(m + 12) == (uint32_t)body &&
               get_le32(m + 16 + body) == p->epoch && get_le32(m + 20 + body) == 0 &&
               get_le32(m + 24 + body) == 0 && get_le32(m + 28 + body) == 0;
      if (!ok) {
        err |= ORC_ERR_MESSAGE;
        continue;
      }
      int64_t sec[6];
      orc_msg_body_bytes(p, n, sec);
      const uint8_t* b = m + 16;
      /* slots of earlier sources, per local expert */
      for (int l = 0; l < L; ++l) {
        int64_t base = 0;
        for (int s2 = 0; s2 < s; ++s2) base += cnt_expert[(int64_t)s2 * E + d * L + l];
        run[l] = base;
      }
      for (int64_t j = 0; j < n; ++j) {
        const uint32_t t = get_le32(b + sec[4] + j * 4);
        for (int k = 0; k < K; ++k) {
          const int32_t e = (int32_t)get_le32(b + sec[3] + (j * K + k) * 4);
          if (e < 0 || e >= E || e / L != d) continue;
          const int64_t pos = run[e - d * L]++;
          if (pos >= RT) {
            err |= ORC_ERR_LL_OVERFLOW;
            continue;
          }
          if (t >= (uint32_t)T) {
            err |= ORC_ERR_MESSAGE;
            continue;
          }
          const int64_t r = (int64_t)e * RT + pos;
          memcpy((uint8_t*)recv + r * H * cb, b + sec[0] + j * H * cb, (size_t)H * cb);
          for (int g = 0; g < G && sb > 0; ++g)
            memcpy((uint8_t*)scales + (((int64_t)e * G + g) * RT + pos) * sb,
                   b + sec[1] + (j * G + g) * sb, (size_t)sb);
          recv_src_idx[r] = (int32_t)((int64_t)s * T + t);
        }
      }
    }
  }
  free(run);
  return err;
}
