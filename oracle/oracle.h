/*
 * Plain, sequential CPU oracle for the MoE expert-parallel dispatch / combine
 * layout transformation.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code: only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant with
 * the HIP implementation.
 *
 * Sources (the pages are cited by title and section):
 *   [P2]  "GPU microarchitecture: DeepEP first principles" (backyes.github.io),
 *         sections 1.1-1.2 (dispatch / combine as layout transformation),
 *         "6.1 Layout Metadata", "6.2 Identity Metadata", "7.1 Does Sort Exist?".
 *   [P3]  "Deep Dive - DeepEP" (leetllm.com), sections "Why expert parallelism
 *         needs a communication layer", "Dispatch: layout, move, and epilogue",
 *         "Combine: reverse routing plus reduction", "Precision: FP8 on the
 *         wire, BF16 for the reduction", "A runnable routing ledger".
 *
 * Conventions: T tokens, H hidden, k top-k, E experts, R logical ranks
 * (E % R == 0, E/R experts per rank, expert e lives on rank e / (E/R)),
 * A expert alignment.  topk_idx is int32 [T,k] row-major, -1 = unused slot.
 * Hidden rows are bf16 bit patterns (uint16).  All functions return
 * ORACLE_OK or one of the error codes below and write nothing on error.
 */
#ifndef EP_ORACLE_H
#define EP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1      /* sizes / dtype / non-finite hidden values or gates */
#define ORACLE_BAD_ROUTE 2    /* expert id outside [-1, E) or repeated in a row */
#define ORACLE_NO_CAPACITY 3  /* receive buffer has fewer rows than needed */

/* bf16 <-> fp32 (round to nearest even, the bit procedure of [P3] "Combine"). */
uint16_t oracle_bf16_round(float v);
float oracle_bf16_to_float(uint16_t b);

/* OCP FP8 E4M3 "FN" code <-> value.  Decode returns NaN for 0x7F / 0xFF.
 * Encode is round-to-nearest, ties to the even code, saturating at 448,
 * sign kept on zero results. */
double oracle_e4m3_value(uint8_t code);
uint8_t oracle_e4m3_encode(float v);

/* Element-wise array forms of the conversions above. */
void oracle_bf16_round_array(int64_t n, const float *in, uint16_t *out);
void oracle_e4m3_encode_array(int64_t n, const float *in, uint8_t *out);
void oracle_e4m3_value_array(int64_t n, const uint8_t *in, double *out);

/* Layout: per-expert counts, per-rank distinct-token counts, token-in-rank
 * mask [T,R] (0/1 bytes), aligned expert offsets [E+1], rank offsets [R+1]. */
int oracle_layout(int32_t T, int32_t k, int32_t E, int32_t R, int32_t A,
                  const int32_t *topk_idx,
                  int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                  uint8_t *is_token_in_rank, int32_t *expert_offsets,
                  int32_t *rank_offsets);

/* Dispatch: stable counting-sort placement of every valid (t, j) selection
 * into expert-major receive rows, plus the handle.
 *   fp8 == 0: recv_x is bf16 [capacity, H]; recv_scales unused (may be NULL).
 *   fp8 != 0: recv_x is e4m3 bytes [capacity, H]; recv_scales fp32
 *             [capacity, H/128]; requires H % 128 == 0.
 * topk_weights and recv_weights may be NULL (then no weights are copied).
 * A hidden value, or the gate of a used selection, that is an infinity or
 * NaN is rejected (ORACLE_BAD_ARG); unused selections' gates are not read.
 * Rows [0, expert_offsets[E]) are written; rows past it are left untouched. */
int oracle_dispatch(int32_t T, int32_t H, int32_t k, int32_t E, int32_t R,
                    int32_t A, int32_t fp8, const uint16_t *x,
                    const int32_t *topk_idx, const float *topk_weights,
                    int64_t capacity, void *recv_x, float *recv_scales,
                    float *recv_weights, int32_t *tok_slot_row,
                    int32_t *row_src);

/* Combine: out[t,c] = bf16(sum over valid j, in slot order j = 0..k-1, of
 * w[t,j] * y[tok_slot_row[t,j], c]) accumulated in fp32 with one fused
 * multiply-add per term.  topk_weights == NULL means y is already weighted
 * and the terms are plain fp32 additions.  acc_out (nullable) receives the
 * fp32 accumulator before the bf16 rounding. */
int oracle_combine(int32_t T, int32_t H, int32_t k, int64_t capacity,
                   const uint16_t *y, const int32_t *tok_slot_row,
                   const float *topk_weights, uint16_t *out, float *acc_out);

/* Dispatch of rows that arrive already quantised ([P3] "Dispatch: layout,
 * move, and epilogue": hidden states are BF16, or FP8 values plus scale
 * factors).  The E4M3 codes x_codes [T,H] and the fp32 scales
 * x_scales [T, H/128] are copied bit for bit to every receive row of the
 * token, at the rows oracle_dispatch would use.  Padding rows get zero
 * codes and zero scales. */
int oracle_dispatch_fp8_input(int32_t T, int32_t H, int32_t k, int32_t E, int32_t R,
                              int32_t A, const uint8_t *x_codes, const float *x_scales,
                              const int32_t *topk_idx, const float *topk_weights,
                              int64_t capacity, uint8_t *recv_codes, float *recv_scales,
                              float *recv_weights, int32_t *tok_slot_row, int32_t *row_src);

/* Non-expanded (rank-deduplicated) dispatch ([P3] "Why expert parallelism
 * needs a communication layer": a token crosses to a destination rank once
 * however many of its experts live there; "Dispatch: layout, move, and
 * epilogue": in non-expanded mode a received row is a source token with its
 * top-k metadata).  Rank r's rows are [rank_token_offsets[r],
 * rank_token_offsets[r+1]), one per token with an expert on r, in ascending
 * token order.  Row q carries the token's payload (bf16, or E4M3 codes and
 * scales as oracle_dispatch computes them), recv_src[q] = t, and the token's
 * top-k slice for this rank: recv_topk_idx[q,j] = e - r*E/R (local expert)
 * when slot j's expert e lives on r, else -1; recv_topk_weights[q,j] = w[t,j]
 * there, else 0.  tok_rank_row[t,r] = q, or -1.  Row count = the sum of
 * num_tokens_per_rank; capacity must hold it. */
int oracle_dispatch_ranked(int32_t T, int32_t H, int32_t k, int32_t E, int32_t R,
                           int32_t fp8, const uint16_t *x, const int32_t *topk_idx,
                           const float *topk_weights, int64_t capacity,
                           int32_t *rank_token_offsets, void *recv_x, float *recv_scales,
                           int32_t *recv_topk_idx, float *recv_topk_weights,
                           int32_t *recv_src, int32_t *tok_rank_row);

/* Receiver-side expand of non-expanded rows into the expert-major layout
 * ([P3] "Dispatch: layout, move, and epilogue": the copy epilogue expands
 * rows into the receive layout the expert GEMM uses).  Uses only what the
 * receiver holds: the rows, recv_src, the local top-k slice and the rank
 * partition bounds.  Experts' segments start at aligned offsets (alignment
 * A) and fill in ascending source token order, so the result is the
 * expanded dispatch of the same route: recv_x [capacity, H] (row_bytes per
 * row: 2H for bf16, H for E4M3 plus H/128 scales), row_src = t*k + j,
 * recv_weights, tok_slot_row [T,k], padding zeroed. */
int oracle_expand(int32_t T, int32_t H, int32_t k, int32_t E, int32_t R, int32_t A,
                  int32_t fp8, const int32_t *rank_token_offsets, const void *ne_x,
                  const float *ne_scales, const int32_t *recv_topk_idx,
                  const float *recv_topk_weights, const int32_t *recv_src,
                  int64_t capacity, void *recv_x, float *recv_scales, float *recv_weights,
                  int32_t *tok_slot_row, int32_t *row_src);

/* Combine through per-rank partial sums ([P3] "Combine: reverse routing
 * plus reduction": staging partial sums per rank sends fewer rows; kept in
 * fp32 here because a bf16 subtotal can lose a small term to cancellation).
 * Stage 1, per non-expanded row q of token t on rank r:
 *   partial[q,c] = fp32 sum over slots j in order with recv_topk_idx[q,j] >= 0
 *                  of w * y[tok_slot_row[t,j], c]   (one fused multiply-add each,
 *                  from +0; w = recv_topk_weights[q,j], or a plain add when
 *                  weighted == 0)
 * Stage 2: out[t,c] = bf16(fp32 sum over r = 0..R-1 with tok_rank_row[t,r] >= 0
 *                  of partial[tok_rank_row[t,r], c], from +0).
 * partials (nullable) receives stage 1 [rows, H]; acc_out stage 2's fp32. */
int oracle_combine_ranked(int32_t T, int32_t H, int32_t k, int32_t R, int64_t rows,
                          int64_t capacity, int32_t weighted, const uint16_t *y,
                          const int32_t *tok_slot_row, const int32_t *recv_topk_idx,
                          const float *recv_topk_weights, const int32_t *recv_src,
                          const int32_t *tok_rank_row, float *partials, uint16_t *out,
                          float *acc_out);

/* Backward of dispatch ([P3] "Combine: reverse routing plus reduction",
 * backward duality: for the unweighted route, copying a row forward becomes
 * summing its gradients backward):
 *   grad_x[t,c] = bf16(sum over valid j, in slot order, of
 *                      grad_recv[tok_slot_row[t,j], c])
 * accumulated in fp32 from +0.  acc_out (nullable) gets the fp32 sums. */
int oracle_dispatch_backward(int32_t T, int32_t H, int32_t k, int64_t capacity,
                             const uint16_t *grad_recv, const int32_t *tok_slot_row,
                             uint16_t *grad_x, float *acc_out);

/* Backward of combine.  For each valid (t, j) with row p = tok_slot_row[t,j]:
 *   grad_expert_out[p,c] = bf16(fp32(w[t,j] * grad_out[t,c]))   (w = 1 when
 *                          topk_weights is NULL: a copy of grad_out[t])
 *   grad_w[t,j]          = sum_c expert_out[p,c] * grad_out[t,c], exact
 *                          (fp64; each product of two bf16 values is exact)
 *   grad_w_abs[t,j]      = sum_c |expert_out[p,c] * grad_out[t,c]|
 * Rows [0, rows_used) that no selection references (alignment padding) get
 * zero gradients; rows at or past rows_used are left untouched.  Unused
 * slots get grad_w = 0.  expert_out, grad_w and grad_w_abs may be NULL
 * together (no gate gradient). */
int oracle_combine_backward(int32_t T, int32_t H, int32_t k, int64_t capacity,
                            int64_t rows_used, const uint16_t *grad_out,
                            const int32_t *tok_slot_row, const float *topk_weights,
                            const uint16_t *expert_out, uint16_t *grad_expert_out,
                            double *grad_w, double *grad_w_abs);

#ifdef __cplusplus
}
#endif

#endif /* EP_ORACLE_H */
