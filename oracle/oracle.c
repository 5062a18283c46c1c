/*
 * Plain, sequential CPU oracle for the MoE dispatch / combine layout
 * transformation.  TEST INFRASTRUCTURE ONLY (see oracle.h): it is compiled
 * with gcc, without fast-math or FP contraction, and is deliberately
 * straightforward rather than fast.  Every loop follows the definition it
 * cites; nothing is blocked, fused or reordered.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16                                                                      */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float v) {
  uint32_t b;
  memcpy(&b, &v, sizeof b);
  return b;
}

static float bits_f32(uint32_t b) {
  float v;
  memcpy(&v, &b, sizeof v);
  return v;
}

/* [P3] "Combine: reverse routing plus reduction": keep the upper 16 bits of
 * the fp32 pattern after adding 0x7FFF plus the lowest kept bit, which rounds
 * to nearest with ties to an even kept pattern.  The page states the
 * procedure for finite numbers; for NaN (where the page is silent) the sign
 * and upper payload are kept and the quiet bit is set. */
uint16_t oracle_bf16_round(float v) {
  uint32_t bits = f32_bits(v);
  if (isnan(v)) return (uint16_t)((bits >> 16) | 0x0040u);
  uint32_t lsb = (bits >> 16) & 1u;
  uint32_t rounded = bits + 0x7FFFu + lsb;
  return (uint16_t)(rounded >> 16);
}

/* A bf16 pattern is the upper half of an fp32 pattern. */
float oracle_bf16_to_float(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* ------------------------------------------------------------------------ */
/* FP8 E4M3 (OCP 8-bit floating point, "FN" variant)                         */
/* ------------------------------------------------------------------------ */

/* Code layout: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 encodes subnormals m * 2^-9; field 15 with mantissa 7 is
 * NaN (there is no infinity), so the largest finite magnitude is
 * 1.75 * 2^8 = 448 (code 0x7E). */
double oracle_e4m3_value(uint8_t code) {
  int sign = code >> 7;
  int efield = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if ((code & 0x7F) == 0x7F) return NAN;
  if (efield == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp(1.0 + m / 8.0, efield - 7);
  return sign ? -mag : mag;
}

/* Round to the nearest finite E4M3 value, ties to the even code.  The 127
 * non-negative finite codes 0x00..0x7E are increasing in value, so the two
 * candidates bracketing |v| are found by bisection over the codes.  Values
 * above 448 take the largest code (saturation); zero results keep the sign of
 * v.  Distances are computed in double: for |v| >= 2^-10 both operands and
 * their difference are exact there (the fp32 input carries at most 24
 * significant bits and the codes are multiples of 2^-9 below 2^9), and below
 * 2^-10 the nearer code is 0 without any tie. */
uint8_t oracle_e4m3_encode(float v) {
  if (isnan(v)) return 0x7F;
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs((double)v);
  if (a >= oracle_e4m3_value(0x7E)) return sign | 0x7E;
  int lo = 0, hi = 0x7E; /* invariant: value(lo) <= a < value(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (oracle_e4m3_value((uint8_t)mid) <= a)
      lo = mid;
    else
      hi = mid;
  }
  double dlo = a - oracle_e4m3_value((uint8_t)lo);
  double dhi = oracle_e4m3_value((uint8_t)hi) - a;
  int code;
  if (dlo < dhi)
    code = lo;
  else if (dhi < dlo)
    code = hi;
  else
    code = (lo % 2 == 0) ? lo : hi;
  return sign | (uint8_t)code;
}

void oracle_bf16_round_array(int64_t n, const float *in, uint16_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_round(in[i]);
}

void oracle_e4m3_encode_array(int64_t n, const float *in, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(in[i]);
}

void oracle_e4m3_value_array(int64_t n, const uint8_t *in, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_value(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Validation                                                                */
/* ------------------------------------------------------------------------ */

static int check_sizes(int32_t T, int32_t k, int32_t E, int32_t R, int32_t A) {
  if (T < 0 || k < 1 || E < 1 || R < 1 || A < 1) return ORACLE_BAD_ARG;
  if (E % R != 0 || k > E) return ORACLE_BAD_ARG;
  return ORACLE_OK;
}

/* [P3] "Dispatch: layout, move, and epilogue": -1 marks an unused selection.
 * [P3] "A runnable routing ledger": an expert outside the range or repeated
 * within one token is rejected. */
static int check_routes(int32_t T, int32_t k, int32_t E, const int32_t *idx) {
  for (int64_t t = 0; t < T; ++t) {
    for (int j = 0; j < k; ++j) {
      int32_t e = idx[t * k + j];
      if (e < -1 || e >= E) return ORACLE_BAD_ROUTE;
      if (e < 0) continue;
      for (int jj = 0; jj < j; ++jj)
        if (idx[t * k + jj] == e) return ORACLE_BAD_ROUTE;
    }
  }
  return ORACLE_OK;
}

/* [P3] "A runnable routing ledger": the gate of a used selection must be a
 * finite number; an unused selection's gate is never read.  (The ledger
 * also rejects negative gates; here a gate is any finite number, since
 * combine is linear in it and the pages' interfaces take float weights.) */
static int check_gates(int32_t T, int32_t k, const int32_t *idx, const float *w) {
  if (w == NULL) return ORACLE_OK;
  for (int64_t t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j)
      if (idx[t * k + j] >= 0 && !isfinite(w[t * k + j])) return ORACLE_BAD_ARG;
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Layout                                                                    */
/* ------------------------------------------------------------------------ */

/* [P2] "6.1 Layout Metadata" and "7.1 Does Sort Exist?": count, then prefix
 * sum.  [P3] "Why expert parallelism needs a communication layer": a token
 * travels to a destination rank once however many of its experts live there,
 * so the per-rank count is of distinct tokens.  [P3] "Dispatch: layout, move,
 * and epilogue": expert segments start at aligned offsets (the start of
 * expert e+1 is the start of e plus its count rounded up to A). */
int oracle_layout(int32_t T, int32_t k, int32_t E, int32_t R, int32_t A,
                  const int32_t *topk_idx, int32_t *num_tokens_per_rank,
                  int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank,
                  int32_t *expert_offsets, int32_t *rank_offsets) {
  int rc = check_sizes(T, k, E, R, A);
  if (rc) return rc;
  rc = check_routes(T, k, E, topk_idx);
  if (rc) return rc;
  const int32_t experts_per_rank = E / R;

  /* counts per expert */
  for (int e = 0; e < E; ++e) num_tokens_per_expert[e] = 0;
  for (int64_t t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int32_t e = topk_idx[t * k + j];
      if (e >= 0) num_tokens_per_expert[e] += 1;
    }

  /* token -> rank membership, and distinct tokens per rank */
  for (int64_t t = 0; t < T; ++t) {
    for (int r = 0; r < R; ++r) is_token_in_rank[t * R + r] = 0;
    for (int j = 0; j < k; ++j) {
      int32_t e = topk_idx[t * k + j];
      if (e >= 0) is_token_in_rank[t * R + e / experts_per_rank] = 1;
    }
  }
  for (int r = 0; r < R; ++r) {
    int32_t n = 0;
    for (int64_t t = 0; t < T; ++t) n += is_token_in_rank[t * R + r];
    num_tokens_per_rank[r] = n;
  }

  /* aligned exclusive prefix sum over experts */
  expert_offsets[0] = 0;
  for (int e = 0; e < E; ++e) {
    int64_t padded = ((int64_t)num_tokens_per_expert[e] + A - 1) / A * A;
    expert_offsets[e + 1] = (int32_t)(expert_offsets[e] + padded);
  }
  /* rank r's partition is the span of its experts' segments */
  for (int r = 0; r <= R; ++r) rank_offsets[r] = expert_offsets[r * experts_per_rank];
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Dispatch                                                                  */
/* ------------------------------------------------------------------------ */

/* [P3] "Precision: FP8 on the wire, BF16 for the reduction": one fp32 scale
 * per 128 values.  The scale is amax / 448 rounded to fp32, each value is
 * divided by it in fp32 and rounded to the nearest E4M3 code.  An all-zero
 * block (where the pages say nothing) gets scale 0 and zero codes. */
static void quantize_row_e4m3(int32_t H, const uint16_t *xrow, uint8_t *q,
                              float *scales) {
  for (int32_t b = 0; b < H / 128; ++b) {
    float amax = 0.0f;
    for (int c = 0; c < 128; ++c) {
      float v = fabsf(oracle_bf16_to_float(xrow[b * 128 + c]));
      if (v > amax) amax = v;
    }
    float scale = amax / 448.0f;
    scales[b] = scale;
    for (int c = 0; c < 128; ++c) {
      if (scale > 0.0f) {
        float v = oracle_bf16_to_float(xrow[b * 128 + c]) / scale;
        q[b * 128 + c] = oracle_e4m3_encode(v);
      } else {
        q[b * 128 + c] = 0x00;
      }
    }
  }
}

/* [P2] "6.1 Layout Metadata": the destination of a row is prefix[expert]++,
 * i.e. a stable counting sort.  Walking tokens in order and slots in order
 * puts each expert's rows in ascending token order, the order [P3]
 * "EPHandle" names for the deterministic mode.  [P2] "6.2 Identity Metadata"
 * and [P3] "A four-token routing ledger": each expert row keeps its source
 * (token, top-k slot) and its gate weight.  Rank r's receive partition is
 * the span of its experts' segments ([P2] 1.1: token-major to
 * destination-major to expert-major).  Alignment padding rows carry no
 * source (-1), weight 0 and zero payload. */
int oracle_dispatch(int32_t T, int32_t H, int32_t k, int32_t E, int32_t R,
                    int32_t A, int32_t fp8, const uint16_t *x,
                    const int32_t *topk_idx, const float *topk_weights,
                    int64_t capacity, void *recv_x, float *recv_scales,
                    float *recv_weights, int32_t *tok_slot_row,
                    int32_t *row_src) {
  int rc = check_sizes(T, k, E, R, A);
  if (rc) return rc;
  if (H < 1 || capacity < 0) return ORACLE_BAD_ARG;
  if (fp8 && (H % 128 != 0 || recv_scales == NULL)) return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < (int64_t)T * H; ++i)
    if (!isfinite(oracle_bf16_to_float(x[i]))) return ORACLE_BAD_ARG;
  rc = check_routes(T, k, E, topk_idx);
  if (rc) return rc;
  rc = check_gates(T, k, topk_idx, topk_weights);
  if (rc) return rc;

  int32_t *cnt = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  int32_t *off = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t *rank_cnt = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
  int32_t *rank_off = (int32_t *)malloc(sizeof(int32_t) * (size_t)(R + 1));
  uint8_t *in_rank = (uint8_t *)malloc((size_t)T * (size_t)R + 1);
  int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  rc = oracle_layout(T, k, E, R, A, topk_idx, rank_cnt, cnt, in_rank, off, rank_off);
  if (rc == ORACLE_OK && off[E] > capacity) rc = ORACLE_NO_CAPACITY;
  if (rc != ORACLE_OK) {
    free(cnt); free(off); free(rank_cnt); free(rank_off); free(in_rank); free(fill);
    return rc;
  }

  const int32_t nblk = H / 128;
  uint8_t *qrow = fp8 ? (uint8_t *)malloc((size_t)H) : NULL;
  float *srow = fp8 ? (float *)malloc(sizeof(float) * (size_t)nblk) : NULL;

  for (int64_t t = 0; t < T; ++t) {
    const uint16_t *xrow = x + t * H;
    if (fp8) quantize_row_e4m3(H, xrow, qrow, srow);
    for (int j = 0; j < k; ++j) {
      int32_t e = topk_idx[t * k + j];
      if (e < 0) {
        tok_slot_row[t * k + j] = -1;
        continue;
      }
      int64_t p = off[e] + fill[e];
      fill[e] += 1;
      tok_slot_row[t * k + j] = (int32_t)p;
      row_src[p] = (int32_t)(t * k + j);
      if (recv_weights && topk_weights) recv_weights[p] = topk_weights[t * k + j];
      if (fp8) {
        memcpy((uint8_t *)recv_x + p * H, qrow, (size_t)H);
        memcpy(recv_scales + p * nblk, srow, sizeof(float) * (size_t)nblk);
      } else {
        memcpy((uint16_t *)recv_x + p * H, xrow, sizeof(uint16_t) * (size_t)H);
      }
    }
  }

  /* alignment padding */
  for (int e = 0; e < E; ++e) {
    for (int64_t p = (int64_t)off[e] + cnt[e]; p < off[e + 1]; ++p) {
      row_src[p] = -1;
      if (recv_weights && topk_weights) recv_weights[p] = 0.0f;
      if (fp8) {
        memset((uint8_t *)recv_x + p * H, 0, (size_t)H);
        for (int b = 0; b < nblk; ++b) recv_scales[p * nblk + b] = 0.0f;
      } else {
        memset((uint16_t *)recv_x + p * H, 0, sizeof(uint16_t) * (size_t)H);
      }
    }
  }

  free(qrow); free(srow);
  free(cnt); free(off); free(rank_cnt); free(rank_off); free(in_rank); free(fill);
  return ORACLE_OK;
}

/* [P3] "Dispatch: layout, move, and epilogue" (pre-quantised input): the
 * same stable placement as oracle_dispatch, with the token's codes and
 * scales copied unchanged. */
int oracle_dispatch_fp8_input(int32_t T, int32_t H, int32_t k, int32_t E, int32_t R,
                              int32_t A, const uint8_t *x_codes, const float *x_scales,
                              const int32_t *topk_idx, const float *topk_weights,
                              int64_t capacity, uint8_t *recv_codes, float *recv_scales,
                              float *recv_weights, int32_t *tok_slot_row, int32_t *row_src) {
  int rc = check_sizes(T, k, E, R, A);
  if (rc) return rc;
  if (H < 128 || H % 128 != 0 || capacity < 0) return ORACLE_BAD_ARG;
  rc = check_routes(T, k, E, topk_idx);
  if (rc) return rc;
  rc = check_gates(T, k, topk_idx, topk_weights);
  if (rc) return rc;
  int32_t *cnt = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  int32_t *off = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t *rank_cnt = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
  int32_t *rank_off = (int32_t *)malloc(sizeof(int32_t) * (size_t)(R + 1));
  uint8_t *in_rank = (uint8_t *)malloc((size_t)T * (size_t)R + 1);
  int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  rc = oracle_layout(T, k, E, R, A, topk_idx, rank_cnt, cnt, in_rank, off, rank_off);
  if (rc == ORACLE_OK && off[E] > capacity) rc = ORACLE_NO_CAPACITY;
  if (rc == ORACLE_OK) {
    const int32_t nblk = H / 128;
    for (int64_t t = 0; t < T; ++t) {
      for (int j = 0; j < k; ++j) {
        int32_t e = topk_idx[t * k + j];
        if (e < 0) {
          tok_slot_row[t * k + j] = -1;
          continue;
        }
        int64_t p = off[e] + fill[e];
        fill[e] += 1;
        tok_slot_row[t * k + j] = (int32_t)p;
        row_src[p] = (int32_t)(t * k + j);
        if (recv_weights && topk_weights) recv_weights[p] = topk_weights[t * k + j];
        memcpy(recv_codes + p * H, x_codes + t * H, (size_t)H);
        memcpy(recv_scales + p * nblk, x_scales + t * nblk, sizeof(float) * (size_t)nblk);
      }
    }
    for (int e = 0; e < E; ++e) {
      for (int64_t p = (int64_t)off[e] + cnt[e]; p < off[e + 1]; ++p) {
        row_src[p] = -1;
        if (recv_weights && topk_weights) recv_weights[p] = 0.0f;
        memset(recv_codes + p * H, 0, (size_t)H);
        for (int b = 0; b < nblk; ++b) recv_scales[p * nblk + b] = 0.0f;
      }
    }
  }
  free(cnt); free(off); free(rank_cnt); free(rank_off); free(in_rank); free(fill);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Combine                                                                   */
/* ------------------------------------------------------------------------ */

/* [P2] 1.2: combine brings expert-major rows back to token-major and
 * recovers the router's weighted sum, e.g. 0.73 x Expert2(T0) + 0.27 x
 * Expert7(T0).  [P3] "Combine: reverse routing plus reduction": the gate is
 * applied exactly once, contributions are accumulated in fp32 and cast to
 * bf16 once at the end (an intermediate bf16 subtotal can lose a small term
 * to cancellation).  The terms are taken in slot order j = 0..k-1, each as
 * one fused multiply-add; an unused slot contributes nothing and the
 * remaining gates are not renormalised ([P3] "A runnable routing ledger"). */
int oracle_combine(int32_t T, int32_t H, int32_t k, int64_t capacity,
                   const uint16_t *y, const int32_t *tok_slot_row,
                   const float *topk_weights, uint16_t *out, float *acc_out) {
  if (T < 0 || H < 1 || k < 1 || capacity < 0) return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < (int64_t)T * k; ++i)
    if (tok_slot_row[i] < -1 || tok_slot_row[i] >= capacity) return ORACLE_BAD_ARG;

  for (int64_t t = 0; t < T; ++t) {
    for (int64_t c = 0; c < H; ++c) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) {
        int64_t p = tok_slot_row[t * k + j];
        if (p < 0) continue;
        float yv = oracle_bf16_to_float(y[p * H + c]);
        if (topk_weights)
          acc = fmaf(topk_weights[t * k + j], yv, acc);
        else
          acc = acc + yv;
      }
      out[t * H + c] = oracle_bf16_round(acc);
      if (acc_out) acc_out[t * H + c] = acc;
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Non-expanded (rank-deduplicated) path                                      */
/* ------------------------------------------------------------------------ */

int oracle_dispatch_ranked(int32_t T, int32_t H, int32_t k, int32_t E, int32_t R,
                           int32_t fp8, const uint16_t *x, const int32_t *topk_idx,
                           const float *topk_weights, int64_t capacity,
                           int32_t *rank_token_offsets, void *recv_x, float *recv_scales,
                           int32_t *recv_topk_idx, float *recv_topk_weights,
                           int32_t *recv_src, int32_t *tok_rank_row) {
  int rc = check_sizes(T, k, E, R, 1);
  if (rc) return rc;
  if (H < 1 || capacity < 0) return ORACLE_BAD_ARG;
  if (fp8 && (H % 128 != 0 || recv_scales == NULL)) return ORACLE_BAD_ARG;
  rc = check_routes(T, k, E, topk_idx);
  if (rc) return rc;
  for (int64_t i = 0; i < (int64_t)T * H; ++i)
    if (!isfinite(oracle_bf16_to_float(x[i]))) return ORACLE_BAD_ARG;
  rc = check_gates(T, k, topk_idx, topk_weights);
  if (rc) return rc;
  const int32_t epr = E / R;
  const int32_t nblk = H / 128;

  /* distinct tokens per rank, then rank partition starts */
  rank_token_offsets[0] = 0;
  for (int r = 0; r < R; ++r) {
    int32_t n = 0;
    for (int64_t t = 0; t < T; ++t) {
      int in = 0;
      for (int j = 0; j < k; ++j) {
        int32_t e = topk_idx[t * k + j];
        if (e >= 0 && e / epr == r) in = 1;
      }
      n += in;
    }
    rank_token_offsets[r + 1] = rank_token_offsets[r] + n;
  }
  if (rank_token_offsets[R] > capacity) return ORACLE_NO_CAPACITY;

  uint8_t *qrow = fp8 ? (uint8_t *)malloc((size_t)H) : NULL;
  float *srow = fp8 ? (float *)malloc(sizeof(float) * (size_t)(nblk > 0 ? nblk : 1)) : NULL;
  int32_t *fill = (int32_t *)calloc((size_t)R, sizeof(int32_t));
  for (int64_t t = 0; t < T; ++t) {
    if (fp8) quantize_row_e4m3(H, x + t * H, qrow, srow);
    for (int r = 0; r < R; ++r) {
      int in = 0;
      for (int j = 0; j < k; ++j) {
        int32_t e = topk_idx[t * k + j];
        if (e >= 0 && e / epr == r) in = 1;
      }
      if (!in) {
        tok_rank_row[t * R + r] = -1;
        continue;
      }
      int64_t q = rank_token_offsets[r] + fill[r];
      fill[r] += 1;
      tok_rank_row[t * R + r] = (int32_t)q;
      recv_src[q] = (int32_t)t;
      for (int j = 0; j < k; ++j) {
        int32_t e = topk_idx[t * k + j];
        int local = e >= 0 && e / epr == r;
        recv_topk_idx[q * k + j] = local ? e - r * epr : -1;
        if (recv_topk_weights)
          recv_topk_weights[q * k + j] = (local && topk_weights) ? topk_weights[t * k + j] : 0.0f;
      }
      if (fp8) {
        memcpy((uint8_t *)recv_x + q * H, qrow, (size_t)H);
        memcpy(recv_scales + q * nblk, srow, sizeof(float) * (size_t)nblk);
      } else {
        memcpy((uint16_t *)recv_x + q * H, x + t * H, sizeof(uint16_t) * (size_t)H);
      }
    }
  }
  free(qrow); free(srow); free(fill);
  return ORACLE_OK;
}

int oracle_expand(int32_t T, int32_t H, int32_t k, int32_t E, int32_t R, int32_t A,
                  int32_t fp8, const int32_t *rank_token_offsets, const void *ne_x,
                  const float *ne_scales, const int32_t *recv_topk_idx,
                  const float *recv_topk_weights, const int32_t *recv_src,
                  int64_t capacity, void *recv_x, float *recv_scales, float *recv_weights,
                  int32_t *tok_slot_row, int32_t *row_src) {
  int rc = check_sizes(T, k, E, R, A);
  if (rc) return rc;
  if (H < 1 || capacity < 0 || (fp8 && H % 128 != 0)) return ORACLE_BAD_ARG;
  const int32_t epr = E / R;
  const int32_t nblk = H / 128;
  const int64_t rows = rank_token_offsets[R];
  for (int64_t q = 0; q < rows; ++q)
    for (int j = 0; j < k; ++j)
      if (recv_topk_idx[q * k + j] < -1 || recv_topk_idx[q * k + j] >= epr) return ORACLE_BAD_ROUTE;

  /* count each expert's rows from the received slices, then aligned starts */
  int32_t *cnt = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  int32_t *off = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  for (int r = 0; r < R; ++r)
    for (int64_t q = rank_token_offsets[r]; q < rank_token_offsets[r + 1]; ++q)
      for (int j = 0; j < k; ++j)
        if (recv_topk_idx[q * k + j] >= 0) cnt[r * epr + recv_topk_idx[q * k + j]] += 1;
  off[0] = 0;
  for (int e = 0; e < E; ++e) off[e + 1] = off[e] + (cnt[e] + A - 1) / A * A;
  if (off[E] > capacity) {
    free(cnt); free(off); free(fill);
    return ORACLE_NO_CAPACITY;
  }
  for (int64_t i = 0; i < (int64_t)T * k; ++i) tok_slot_row[i] = -1;

  /* rows of a rank arrive in ascending source order, so filling each expert
   * segment while walking the rank's rows keeps the segment sorted */
  for (int r = 0; r < R; ++r) {
    for (int64_t q = rank_token_offsets[r]; q < rank_token_offsets[r + 1]; ++q) {
      int64_t t = recv_src[q];
      for (int j = 0; j < k; ++j) {
        int32_t le = recv_topk_idx[q * k + j];
        if (le < 0) continue;
        int32_t e = r * epr + le;
        int64_t p = off[e] + fill[e];
        fill[e] += 1;
        tok_slot_row[t * k + j] = (int32_t)p;
        row_src[p] = (int32_t)(t * k + j);
        if (recv_weights && recv_topk_weights) recv_weights[p] = recv_topk_weights[q * k + j];
        if (fp8) {
          memcpy((uint8_t *)recv_x + p * H, (const uint8_t *)ne_x + q * H, (size_t)H);
          memcpy(recv_scales + p * nblk, ne_scales + q * nblk, sizeof(float) * (size_t)nblk);
        } else {
          memcpy((uint16_t *)recv_x + p * H, (const uint16_t *)ne_x + q * H,
                 sizeof(uint16_t) * (size_t)H);
        }
      }
    }
  }
  for (int e = 0; e < E; ++e) {
    for (int64_t p = (int64_t)off[e] + cnt[e]; p < off[e + 1]; ++p) {
      row_src[p] = -1;
      if (recv_weights && recv_topk_weights) recv_weights[p] = 0.0f;
      if (fp8) {
        memset((uint8_t *)recv_x + p * H, 0, (size_t)H);
        for (int b = 0; b < nblk; ++b) recv_scales[p * nblk + b] = 0.0f;
      } else {
        memset((uint16_t *)recv_x + p * H, 0, sizeof(uint16_t) * (size_t)H);
      }
    }
  }
  free(cnt); free(off); free(fill);
  return ORACLE_OK;
}

int oracle_combine_ranked(int32_t T, int32_t H, int32_t k, int32_t R, int64_t rows,
                          int64_t capacity, int32_t weighted, const uint16_t *y,
                          const int32_t *tok_slot_row, const int32_t *recv_topk_idx,
                          const float *recv_topk_weights, const int32_t *recv_src,
                          const int32_t *tok_rank_row, float *partials, uint16_t *out,
                          float *acc_out) {
  if (T < 0 || H < 1 || k < 1 || R < 1 || rows < 0 || capacity < 0) return ORACLE_BAD_ARG;
  float *part = partials ? partials : (float *)malloc(sizeof(float) * (size_t)(rows * H + 1));
  /* stage 1: per (token, rank) row, the rank's experts' weighted rows */
  for (int64_t q = 0; q < rows; ++q) {
    int64_t t = recv_src[q];
    for (int64_t c = 0; c < H; ++c) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) {
        if (recv_topk_idx[q * k + j] < 0) continue;
        int64_t p = tok_slot_row[t * k + j];
        if (p < 0 || p >= capacity) continue;
        float yv = oracle_bf16_to_float(y[p * H + c]);
        if (weighted)
          acc = fmaf(recv_topk_weights[q * k + j], yv, acc);
        else
          acc = acc + yv;
      }
      part[q * H + c] = acc;
    }
  }
  /* stage 2: per token, the partials of its ranks in rank order */
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t c = 0; c < H; ++c) {
      float acc = 0.0f;
      for (int r = 0; r < R; ++r) {
        int64_t q = tok_rank_row[t * R + r];
        if (q < 0) continue;
        acc = acc + part[q * H + c];
      }
      out[t * H + c] = oracle_bf16_round(acc);
      if (acc_out) acc_out[t * H + c] = acc;
    }
  }
  if (!partials) free(part);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Backward                                                                  */
/* ------------------------------------------------------------------------ */

/* [P3] "Combine: reverse routing plus reduction", backward duality: the
 * transpose of copying a token's row into each of its expert rows is
 * summing the gradients of those rows back into the token. */
int oracle_dispatch_backward(int32_t T, int32_t H, int32_t k, int64_t capacity,
                             const uint16_t *grad_recv, const int32_t *tok_slot_row,
                             uint16_t *grad_x, float *acc_out) {
  if (T < 0 || H < 1 || k < 1 || capacity < 0) return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < (int64_t)T * k; ++i)
    if (tok_slot_row[i] < -1 || tok_slot_row[i] >= capacity) return ORACLE_BAD_ARG;
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t c = 0; c < H; ++c) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) {
        int64_t p = tok_slot_row[t * k + j];
        if (p < 0) continue;
        acc = acc + oracle_bf16_to_float(grad_recv[p * H + c]);
      }
      grad_x[t * H + c] = oracle_bf16_round(acc);
      if (acc_out) acc_out[t * H + c] = acc;
    }
  }
  return ORACLE_OK;
}

/* Backward of out[t] = sum_j w[t,j] * y[p_j]: the gradient reaching expert
 * row p_j is w[t,j] * grad_out[t] (the gate applied once, as in the forward
 * pass), and the gradient of the gate is the dot product of the expert row
 * with grad_out[t] ([P3] "Combine: reverse routing plus reduction": the
 * autograd wrapper must still produce gate gradients). */
int oracle_combine_backward(int32_t T, int32_t H, int32_t k, int64_t capacity,
                            int64_t rows_used, const uint16_t *grad_out,
                            const int32_t *tok_slot_row, const float *topk_weights,
                            const uint16_t *expert_out, uint16_t *grad_expert_out,
                            double *grad_w, double *grad_w_abs) {
  if (T < 0 || H < 1 || k < 1 || capacity < 0 || rows_used < 0 || rows_used > capacity)
    return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < (int64_t)T * k; ++i)
    if (tok_slot_row[i] < -1 || tok_slot_row[i] >= rows_used) return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < rows_used * H; ++i) grad_expert_out[i] = 0;
  for (int64_t t = 0; t < T; ++t) {
    for (int j = 0; j < k; ++j) {
      int64_t p = tok_slot_row[t * k + j];
      double dot = 0.0, mag = 0.0;
      if (p >= 0) {
        float w = topk_weights ? topk_weights[t * k + j] : 1.0f;
        for (int64_t c = 0; c < H; ++c) {
          float g = oracle_bf16_to_float(grad_out[t * H + c]);
          grad_expert_out[p * H + c] = oracle_bf16_round(w * g);
          if (expert_out) {
            double term = (double)oracle_bf16_to_float(expert_out[p * H + c]) * (double)g;
            dot += term;
            mag += fabs(term);
          }
        }
      }
      if (grad_w) grad_w[t * k + j] = dot;
      if (grad_w_abs) grad_w_abs[t * k + j] = mag;
    }
  }
  return ORACLE_OK;
}
