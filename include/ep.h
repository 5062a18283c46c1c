/*
 * ep.h - C ABI of libep.so: MoE expert-parallel dispatch / combine layout
 * transformation on one AMD Instinct MI355X (gfx950).
 *
 * The expert-parallel group is emulated on one GPU as R logical ranks, each a
 * partition of one receive buffer in HBM, so the hop between ranks is an
 * in-HBM copy.  Three calls make up the path:
 *
 *   ep_get_dispatch_layout  counts and prefix offsets per expert and rank
 *   ep_dispatch             token-major rows -> rank partitions -> expert
 *                           segments (bf16 copy, or FP8 E4M3 + fp32 scales),
 *                           plus the source-index handle
 *   ep_combine              expert-major rows -> token-major, gate applied
 *                           once, fixed-order fp32 sum, bf16 result
 *
 * Further calls on the same data: ep_layout_dispatch (the first two in one
 * call, one launch for batches of at most 256 tokens), ep_dispatch_fp8_input
 * (pre-quantised rows), ep_dispatch_backward and ep_combine_backward, and
 * the non-expanded path ep_dispatch_ranked -> ep_expand ->
 * ep_combine_ranked.  A measurement aid is declared apart, in ep_probe.h.
 *
 * Pages cited: "GPU microarchitecture: DeepEP first principles"
 * (backyes.github.io) and "Deep Dive - DeepEP" (leetllm.com), by section.
 *
 * Conventions for every call
 *   - Sizes: T tokens, H hidden, k top-k, E experts, R logical ranks with
 *     E % R == 0 (expert e lives on rank e / (E/R)), A expert alignment.
 *   - Pointers named *_host are host memory; every other pointer is device
 *     memory owned by the caller.  The library allocates nothing, keeps no
 *     state between calls and may be called from several threads on
 *     different streams at once, as long as their buffers do not overlap.
 *   - Every call enqueues work on `stream` and returns without waiting,
 *     except where a *_host output is requested (then it synchronises that
 *     stream).  Waiting on the stream orders later work after the results;
 *     it is a stream dependency, not a host barrier ("Deep Dive - DeepEP",
 *     "EventOverlap: a stream contract").
 *   - Errors never cross the ABI as exceptions.  Bad sizes, pointers or
 *     dtypes are rejected synchronously with EP_ERR_INVALID_ARG before any
 *     work is enqueued ("Deep Dive - DeepEP", "Combine: reverse routing plus
 *     reduction": fail at the contract boundary, not after a silent
 *     reinterpretation).  Problems only the GPU can see (a bad route, too
 *     few receive rows, a workspace that does not belong to this
 *     configuration and route, an inf or NaN among the hidden values or the gates of
 *     valid selections) are OR-ed as bits into the caller's device status
 *     word and surface through ep_read_status.  HIP launch failures return
 *     EP_ERR_HIP.  ep_last_error_string() describes the last failure of the
 *     calling thread.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ep_status {
  EP_OK = 0,
  EP_ERR_INVALID_ARG = 1,   /* sizes, pointers, dtype, alignment (synchronous) */
  EP_ERR_INVALID_ROUTE = 2, /* expert id outside [-1, E) or repeated in a token */
  EP_ERR_CAPACITY = 3,      /* receive buffer has fewer rows than the layout needs */
  EP_ERR_WORKSPACE = 4,     /* workspace not written by a layout of this config
                               and this route */
  EP_ERR_HIP = 5,           /* a HIP runtime call failed */
  EP_ERR_NONFINITE = 6      /* a hidden value or a valid selection's gate is inf or NaN */
} ep_status_t;

/* Bits the kernels OR into the device status word. */
#define EP_STATUS_BIT_ROUTE 0x1
#define EP_STATUS_BIT_CAPACITY 0x2
#define EP_STATUS_BIT_WORKSPACE 0x4
#define EP_STATUS_BIT_NONFINITE 0x8

typedef enum ep_dtype {
  EP_DTYPE_BF16 = 0,     /* rows are bf16, copied bit for bit */
  EP_DTYPE_FP8_E4M3 = 1  /* OCP E4M3 ("FN", max 448) codes + one fp32 scale per 128 values */
} ep_dtype_t;

/* Limits of this implementation (checked; EP_ERR_INVALID_ARG beyond them). */
#define EP_MAX_EXPERTS 1024
#define EP_MAX_TOPK 32
#define EP_MAX_RANKS 64
#define EP_LAYOUT_DISPATCH_MAX_TOKENS 256 /* ep_layout_dispatch's one-launch bound */

typedef struct ep_config {
  int32_t num_tokens;       /* T >= 0 */
  int32_t hidden;           /* H >= 8, H % 8 == 0 (H % 128 == 0 for FP8);
                               T * ceil(H / 512) <= 2^26 - 4: one 64-lane
                               wave per (token, 512-column chunk), and a
                               launch holds fewer than 2^32 lanes */
  int32_t num_topk;         /* 1 <= k <= min(E, EP_MAX_TOPK) */
  int32_t num_experts;      /* 1 <= E <= EP_MAX_EXPERTS */
  int32_t num_ranks;        /* 1 <= R <= EP_MAX_RANKS, E % R == 0 */
  int32_t expert_alignment; /* A >= 1; T*k + E*(A-1) < 2^31 */
} ep_config_t;

/*
 * The handle ep_dispatch returns and ep_combine consumes: route and
 * reverse-slot metadata, never gate values ("Deep Dive - DeepEP", sections
 * "A four-token routing ledger" and "EPHandle: route metadata with a
 * lifetime").  It is a plain host struct that borrows the caller's device
 * arrays; it stays valid while they live and only for the route it was
 * built from.
 */
typedef struct ep_handle {
  ep_config_t config;
  int64_t capacity;              /* rows of the receive / expert-output buffers */
  const int32_t *tok_slot_row;   /* [T, k]: receive row of selection (t, j), -1 if unused */
  const int32_t *row_src;        /* [capacity]: t*k + j of the row's source, -1 for padding */
  const int32_t *expert_offsets; /* [E + 1]: aligned start of each expert segment */
} ep_handle_t;

/*
 * Handle of the non-expanded (rank-deduplicated) dispatch: what the source
 * keeps to expand and to combine through per-rank partial sums.  A plain
 * host struct borrowing the caller's device arrays, valid for one route.
 */
typedef struct ep_ranked_handle {
  ep_config_t config;
  int64_t capacity;                  /* expanded rows (expert-major buffers) */
  int64_t ranked_capacity;           /* non-expanded rows;
                                        ranked_capacity * ceil(H / 512) <= 2^26 - 4 */
  const int32_t *rank_token_offsets; /* [R + 1]: rank r's rows are [off[r], off[r+1]) */
  const int32_t *tok_rank_row;       /* [T, R]: non-expanded row of (t, r), -1 if none */
  const int32_t *tok_slot_row;       /* [T, k]: expanded row of (t, j), -1 if unused */
  const int32_t *ne_topk_idx;        /* [ranked_capacity, k]: local expert of slot j or -1 */
  const float *ne_topk_weights;      /* [ranked_capacity, k]: gate of slot j there, else 0 */
  const int32_t *ne_src;             /* [ranked_capacity]: source token of the row */
} ep_ranked_handle_t;

/* Static description of a status code (never NULL). */
const char *ep_status_string(ep_status_t status);

/* Message for the last failing call on this thread ("" if none).  The
 * message says which check failed, so that a rejected call is diagnosed at
 * the boundary ("Deep Dive - DeepEP", "Combine: reverse routing plus
 * reduction").  ep_last_error is the same function under a shorter name. */
const char *ep_last_error_string(void);
const char *ep_last_error(void);

/* Host only.  Bytes of device workspace that ep_get_dispatch_layout fills
 * and ep_dispatch reads for this configuration: a planning number the caller
 * allocates once and reuses, as a buffer size hint is ("Deep Dive - DeepEP",
 * "V2's single interface: ElasticBuffer": reusing a buffer avoids
 * allocation; size it for the worst case rather than growing it). */
ep_status_t ep_layout_workspace_bytes(const ep_config_t *cfg, size_t *bytes_host);

/*
 * Prepares a workspace for its first layout (the one-time set-up of a
 * reusable buffer, "Deep Dive - DeepEP", "V2's single interface:
 * ElasticBuffer"): clears its header (the marker that a layout completed
 * and the counter the layout's workgroups use to elect the one that
 * finishes the prefix sums).  Call once per allocation
 * (a zero-filled allocation needs no call); every layout leaves the header
 * ready for the next one.  Enqueued on `stream` as a small kernel (no
 * memset), so it may be captured in a graph.  workspace must be 256-byte
 * aligned with at least 256 bytes.
 */
ep_status_t ep_workspace_init(void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Host only.  Receive rows that always suffice without reading counts back:
 * T*k + E*(A-1) (every slot valid, every expert segment padded).  This is
 * the worst-case envelope a caller sizes its receive buffers by ("Deep Dive
 * - DeepEP", "V2's single interface: ElasticBuffer"); a caller that skips
 * the CPU-synchronised count must size by it and read only the valid
 * ranges ("Current boundary: V2.5 changes the integration contract"). */
ep_status_t ep_recv_capacity_rows(const ep_config_t *cfg, int64_t *rows_host);

/*
 * Layout: "count, prefix sum" of the counting sort ("GPU microarchitecture:
 * DeepEP first principles", sections "6.1 Layout Metadata" and "7.1 Does
 * Sort Exist?"), with per-rank counts of distinct tokens (a token goes to a
 * rank once however many of its experts live there: "Deep Dive - DeepEP",
 * "Why expert parallelism needs a communication layer") and aligned expert
 * segment starts ("Deep Dive - DeepEP", "Dispatch: layout, move, and
 * epilogue").
 *
 *   topk_idx             [T, k] int32, row-major; -1 = unused selection
 *   num_tokens_per_rank  [R] int32 out: distinct tokens with an expert on rank r
 *   num_tokens_per_expert[E] int32 out: selections of expert e
 *   is_token_in_rank     [T, R] uint8 out: 1 if token t has an expert on rank r
 *   expert_offsets       [E + 1] int32 out: offsets[0] = 0, offsets[e+1] =
 *                        offsets[e] + ceil(count[e] / A) * A.  The valid rows of
 *                        expert e are [offsets[e], offsets[e] + count[e]).
 *   rank_offsets         [R + 1] int32 out: rank r's receive partition is
 *                        rows [rank_offsets[r], rank_offsets[r+1])
 *   workspace            device scratch of ep_layout_workspace_bytes() bytes,
 *                        256-byte aligned, prepared once by ep_workspace_init
 *                        (or zero-filled), read later by ep_dispatch (keep it
 *                        until then).  Two layouts must not use one workspace
 *                        at the same time (e.g. on two streams).
 *   status               device int32 the kernels OR EP_STATUS_BIT_* into;
 *                        the caller zeroes it before a new route
 *   num_recv_rows_host   optional: if not NULL, the call synchronises the
 *                        stream and stores offsets[E] (rows used) here, and
 *                        returns the device status (the CPU-sync variant)
 */
ep_status_t ep_get_dispatch_layout(const ep_config_t *cfg, const int32_t *topk_idx,
                                   int32_t *num_tokens_per_rank,
                                   int32_t *num_tokens_per_expert,
                                   uint8_t *is_token_in_rank, int32_t *expert_offsets,
                                   int32_t *rank_offsets, void *workspace,
                                   size_t workspace_bytes, int32_t *status,
                                   int32_t *num_recv_rows_host, hipStream_t stream);

/*
 * Dispatch: token-major -> destination-major -> expert-major in one pass
 * ("GPU microarchitecture: DeepEP first principles", section 1.1).  Each
 * valid selection (t, j) with expert e gets the receive row
 *     expert_offsets[e] + #{t' < t : token t' also selected e}
 * (the stable placement dst = prefix[expert]++ of section "6.1 Layout
 * Metadata"; rows of a segment are in ascending token order, the order the
 * deterministic mode of "Deep Dive - DeepEP", "EPHandle", sorts by).
 *
 *   recv_dtype    EP_DTYPE_BF16: recv_x is bf16 [capacity, H], a bit copy of x.
 *                 EP_DTYPE_FP8_E4M3: recv_x is uint8 [capacity, H] and
 *                 recv_scales fp32 [capacity, H/128]; per token and 128-value
 *                 block, scale = amax/448 (fp32, round to nearest even) and
 *                 code = E4M3(x / scale) rounded to nearest even, with scale 0
 *                 and zero codes for an all-zero block ("Deep Dive - DeepEP",
 *                 "Precision: FP8 on the wire, BF16 for the reduction").
 *   x             [T, H] bf16 hidden states.  An inf or NaN sets
 *                 EP_STATUS_BIT_NONFINITE ("Deep Dive - DeepEP", "A runnable
 *                 routing ledger": a row that is not finite is rejected); the
 *                 rows of every other token are still exact, and the FP8
 *                 codes and scale of a block holding it are meaningless.
 *   topk_idx      [T, k] int32, the same array given to the layout
 *   topk_weights  [T, k] fp32 gates or NULL; an inf or NaN gate of a valid
 *                 selection sets EP_STATUS_BIT_NONFINITE (the ledger rejects
 *                 it too); unused selections' gates are never read
 *   expert_offsets[E + 1] from ep_get_dispatch_layout
 *   workspace     the workspace that layout filled for this route.  The
 *                 layout records each selection's expert, so a route that
 *                 differs from the layout's is seen per selection: such a
 *                 selection gets no row and EP_STATUS_BIT_WORKSPACE is set
 *   capacity      rows of recv_x / recv_scales / recv_weights / row_src; a
 *                 selection whose row would be >= capacity is dropped and
 *                 EP_STATUS_BIT_CAPACITY is set (ep_recv_capacity_rows() or
 *                 the synchronised row count always suffices)
 *   zero_padding  non-zero: alignment padding rows get zero payload and zero
 *                 scales (do_zero_padding, "Deep Dive - DeepEP", "Dispatch:
 *                 layout, move, and epilogue": clearing the gaps is the
 *                 caller's choice); zero: their payload and scales are left
 *                 as they were.  Either way padding rows get row_src -1 and
 *                 gate 0, so they never enter a combined row.
 *   recv_weights  [capacity] fp32 out or NULL: the gate of each row
 *   tok_slot_row  [T, k] int32 out: row of (t, j), -1 if unused
 *   row_src       [capacity] int32 out: t*k + j of each row, -1 for padding
 *   handle_host   optional: filled with the handle for ep_combine
 * Rows in [offsets[e] + count[e], offsets[e+1]) are alignment padding: zero
 * weight, row_src -1, and zero payload and scale when zero_padding is set.
 * Rows at or past expert_offsets[E] are not written.
 */
ep_status_t ep_dispatch(const ep_config_t *cfg, ep_dtype_t recv_dtype, const uint16_t *x,
                        const int32_t *topk_idx, const float *topk_weights,
                        const int32_t *expert_offsets, const void *workspace,
                        size_t workspace_bytes, int64_t capacity, int32_t zero_padding,
                        void *recv_x, float *recv_scales, float *recv_weights,
                        int32_t *tok_slot_row, int32_t *row_src, int32_t *status,
                        ep_handle_t *handle_host, hipStream_t stream);

/*
 * Layout and dispatch in one call (count, prefix sum and scatter: "GPU
 * microarchitecture: DeepEP first principles", "6.1 Layout Metadata"; "Deep
 * Dive - DeepEP", "Dispatch: layout, move, and epilogue").  It writes
 * exactly what ep_get_dispatch_layout followed by ep_dispatch writes, bit
 * for bit: every layout output, the workspace (so combine, the non-expanded
 * path and backward work after it unchanged), the receive rows and the
 * handle.  The arguments are those two calls' arguments; there is no
 * synchronising row count.
 *   - At most EP_LAYOUT_DISPATCH_MAX_TOKENS tokens: one launch, which saves
 *     the small-batch path a launch and a round trip through the workspace.
 *   - More tokens: the two calls' launches, one after the other.
 *
 * Returns EP_ERR_INVALID_ARG (nothing enqueued) for any argument the two
 * calls reject.
 */
ep_status_t ep_layout_dispatch(const ep_config_t *cfg, ep_dtype_t recv_dtype, const uint16_t *x,
                               const int32_t *topk_idx, const float *topk_weights,
                               int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                               uint8_t *is_token_in_rank, int32_t *expert_offsets,
                               int32_t *rank_offsets, void *workspace, size_t workspace_bytes,
                               int64_t capacity, int32_t zero_padding, void *recv_x,
                               float *recv_scales, float *recv_weights, int32_t *tok_slot_row,
                               int32_t *row_src, int32_t *status, ep_handle_t *handle_host,
                               hipStream_t stream);

/*
 * Layout and dispatch with no workspace argument and no allocation, for
 * callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, and harnesses that forbid allocation.
 *
 * It is ep_layout_dispatch without the workspace arguments: it writes what
 * ep_get_dispatch_layout followed by ep_dispatch writes to the caller's
 * arrays, bit for bit.  The layout's workspace is a
 * library-owned device array of EP_NOALLOC_SCRATCH_BYTES, one per GPU, kept
 * until the process ends: a configuration whose workspace
 * (ep_layout_workspace_bytes) is larger is rejected with EP_ERR_INVALID_ARG
 * and nothing enqueued.  The first call on a GPU takes the array's address
 * on that GPU and enqueues a clear of its header on `stream`.  Every call on
 * one GPU shares that array, so calls that overlap on one GPU (several
 * streams or threads at once) race and give wrong results; the caller
 * orders them.  The workspace is not visible to the caller, so the
 * non-expanded calls (which read it) need ep_get_dispatch_layout instead;
 * combine and both backward calls take this call's handle as usual.
 */
#define EP_NOALLOC_SCRATCH_BYTES (2 * 1024 * 1024)

ep_status_t ep_layout_dispatch_noalloc(const ep_config_t *cfg, ep_dtype_t recv_dtype,
                                       const uint16_t *x, const int32_t *topk_idx,
                                       const float *topk_weights, int32_t *num_tokens_per_rank,
                                       int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank,
                                       int32_t *expert_offsets, int32_t *rank_offsets,
                                       int64_t capacity, int32_t zero_padding, void *recv_x,
                                       float *recv_scales, float *recv_weights,
                                       int32_t *tok_slot_row, int32_t *row_src, int32_t *status,
                                       ep_handle_t *handle_host, hipStream_t stream);

/*
 * Dispatch of rows that arrive already quantised ("Deep Dive - DeepEP",
 * "Dispatch: layout, move, and epilogue": hidden states are BF16 or FP8
 * values plus scale factors; "Precision: FP8 on the wire, BF16 for the
 * reduction": one fp32 scale per 128 values).  Same placement, handle and
 * padding as ep_dispatch with EP_DTYPE_FP8_E4M3, but the token's codes and
 * scales are copied unchanged instead of being computed from bf16.
 *
 *   x_codes   [T, H] uint8 E4M3 codes (any byte value travels unchanged)
 *   x_scales  [T, H/128] fp32
 *   recv_x    [capacity, H] uint8 out; recv_scales [capacity, H/128] fp32 out
 *   other arguments as for ep_dispatch (H % 128 == 0 required)
 */
ep_status_t ep_dispatch_fp8_input(const ep_config_t *cfg, const uint8_t *x_codes,
                                  const float *x_scales, const int32_t *topk_idx,
                                  const float *topk_weights, const int32_t *expert_offsets,
                                  const void *workspace, size_t workspace_bytes,
                                  int64_t capacity, int32_t zero_padding, uint8_t *recv_x, float *recv_scales,
                                  float *recv_weights, int32_t *tok_slot_row, int32_t *row_src,
                                  int32_t *status, ep_handle_t *handle_host,
                                  hipStream_t stream);

/*
 * Combine: expert-major rows back to token-major ("GPU microarchitecture:
 * DeepEP first principles", section 1.2), each gate applied exactly once
 * ("Deep Dive - DeepEP", "Combine: reverse routing plus reduction"):
 *     out[t, c] = bf16( sum_{j = 0..k-1, row_j >= 0} w[t, j] * y[row_j, c] )
 * with row_j = tok_slot_row[t, j], accumulated in fp32 in slot order j = 0, 1,
 * ..., one fused multiply-add per term starting from +0, then rounded once to
 * bf16 (nearest even).  Unused slots contribute nothing and their gates are
 * never read; remaining gates are not renormalised.
 *
 *   handle        from ep_dispatch (config, capacity, tok_slot_row)
 *   expert_out    [capacity, H] bf16 expert outputs, row p = expert output of
 *                 receive row p
 *   topk_weights  [T, k] fp32 gates, or NULL when the caller already
 *                 weighted the rows (then the terms are plain fp32 adds)
 *   out           [T, H] bf16 out
 */
ep_status_t ep_combine(const ep_handle_t *handle, const uint16_t *expert_out,
                       const float *topk_weights, uint16_t *out, hipStream_t stream);

/*
 * Backward of dispatch: the transpose of the unweighted dispatch ("Deep
 * Dive - DeepEP", "Combine: reverse routing plus reduction": for the
 * unweighted route, copying a row forward becomes summing its gradients
 * backward).  For each token t and channel c,
 *     grad_x[t, c] = bf16( sum_{j = 0..k-1, row_j >= 0} grad_recv_x[row_j, c] )
 * accumulated in fp32 in slot order from +0 and rounded once (the same
 * arithmetic as ep_combine with NULL weights).  A gate multiplied in by the
 * caller before combine belongs to the caller's own backward.
 *
 *   handle       from ep_dispatch
 *   grad_recv_x  [capacity, H] bf16: gradient w.r.t. the receive rows
 *   grad_x       [T, H] bf16 out: gradient w.r.t. x
 */
ep_status_t ep_dispatch_backward(const ep_handle_t *handle, const uint16_t *grad_recv_x,
                                 uint16_t *grad_x, hipStream_t stream);

/*
 * Backward of combine ("Deep Dive - DeepEP", "Combine: reverse routing plus
 * reduction": backward duality, plus the gate gradient).  For each valid
 * selection (t, j) with row p = tok_slot_row[t, j]:
 *     grad_expert_out[p, c] = bf16( fp32(w[t, j] * grad_out[t, c]) )
 *     grad_weights[t, j]    = sum_c expert_out[p, c] * grad_out[t, c]
 * The row gradient applies the gate once (w = 1 when topk_weights is NULL,
 * which makes it a copy of grad_out[t]).  The gate gradient is an fp32 sum
 * in a fixed order (deterministic); its error against the exact sum is at
 * most H * 2^-24 / (1 - H * 2^-24) * sum_c |expert_out[p,c] * grad_out[t,c]|.
 * Unused slots get grad_weights 0.  Alignment padding rows of
 * grad_expert_out are zero-filled; rows at or past expert_offsets[E] are
 * not written.
 *
 *   handle           from ep_dispatch (with A > 1 it must carry row_src and
 *                    expert_offsets)
 *   grad_out         [T, H] bf16: gradient w.r.t. the combined rows
 *   topk_weights     [T, k] fp32 gates used in the forward combine, or NULL
 *   expert_out       [capacity, H] bf16 forward expert outputs (needed only
 *                    for grad_weights)
 *   grad_expert_out  [capacity, H] bf16 out
 *   grad_weights     [T, k] fp32 out, or NULL to skip the gate gradient
 * Rejects (EP_ERR_INVALID_ARG) T >= 2^24: one 256-lane workgroup per token.
 */
ep_status_t ep_combine_backward(const ep_handle_t *handle, const uint16_t *grad_out,
                                const float *topk_weights, const uint16_t *expert_out,
                                uint16_t *grad_expert_out, float *grad_weights,
                                hipStream_t stream);

/* Host only.  Non-expanded rows that always suffice: T * min(k, R), the
 * worst case of one row per (token, destination rank) ("Deep Dive -
 * DeepEP", "V2's single interface: ElasticBuffer" for sizing by the
 * envelope; "Why expert parallelism needs a communication layer" for one
 * row per destination rank). */
ep_status_t ep_ranked_capacity_rows(const ep_config_t *cfg, int64_t *rows_host);

/*
 * Non-expanded dispatch ("Deep Dive - DeepEP", "Why expert parallelism
 * needs a communication layer": a token crosses to a destination rank once
 * however many of its experts live there; "Dispatch: layout, move, and
 * epilogue": in non-expanded mode a received row is a source token with its
 * top-k metadata).  Rank r's rows are [rank_token_offsets[r],
 * rank_token_offsets[r+1]), one per token with an expert on r, in ascending
 * token order; the row count is the sum of num_tokens_per_rank.  Row q
 * carries the token's payload (bf16, or E4M3 codes + scales exactly as
 * ep_dispatch computes them), ne_src[q] = t and the token's top-k slice for
 * the rank: ne_topk_idx[q, j] = e - r*E/R when slot j's expert e lives on
 * r, else -1; ne_topk_weights[q, j] = w[t, j] there, else 0.  It also
 * writes tok_rank_row and the expanded handle tok_slot_row (the rows
 * ep_expand will fill, as ep_dispatch would place them).
 *
 *   workspace / expert_offsets  from ep_get_dispatch_layout of this route
 *   capacity         rows of the expanded buffers (for tok_slot_row)
 *   ranked_capacity  rows of ne_x / ne_scales / ne_topk_* / ne_src;
 *                    ranked_capacity * ceil(H / 512) <= 2^26 - 4
 *   ne_x             [ranked_capacity, H] bf16 or uint8 (E4M3) out
 *   ne_scales        [ranked_capacity, H/128] fp32 out (FP8 only)
 *   ne_topk_idx      [ranked_capacity, k] int32 out
 *   ne_topk_weights  [ranked_capacity, k] fp32 out, or NULL
 *   ne_src           [ranked_capacity] int32 out
 *   rank_token_offsets [R + 1] int32 out
 *   tok_rank_row     [T, R] int32 out;  tok_slot_row [T, k] int32 out
 */
ep_status_t ep_dispatch_ranked(const ep_config_t *cfg, ep_dtype_t recv_dtype, const uint16_t *x,
                               const int32_t *topk_idx, const float *topk_weights,
                               const int32_t *expert_offsets, const void *workspace,
                               size_t workspace_bytes, int64_t capacity, int64_t ranked_capacity,
                               void *ne_x, float *ne_scales, int32_t *ne_topk_idx,
                               float *ne_topk_weights, int32_t *ne_src,
                               int32_t *rank_token_offsets, int32_t *tok_rank_row,
                               int32_t *tok_slot_row, int32_t *status,
                               ep_ranked_handle_t *handle_host, hipStream_t stream);

/*
 * Receiver-side expand of non-expanded rows into the expert-major layout
 * ("Deep Dive - DeepEP", "Dispatch: layout, move, and epilogue": the copy
 * epilogue expands rows into the layout the expert GEMM reads).  Each
 * received row is copied to the expert row of each of its local slots;
 * the result (recv_x, recv_scales, recv_weights, row_src, padding) is
 * identical to ep_dispatch of the same route with the same zero_padding.
 * workspace / expert_offsets are the layout's.  recv_weights may be NULL.
 * handle_host (optional) receives the expanded handle for ep_combine.
 */
ep_status_t ep_expand(const ep_ranked_handle_t *ranked, ep_dtype_t recv_dtype, const void *ne_x,
                      const float *ne_scales, const int32_t *expert_offsets,
                      const void *workspace, size_t workspace_bytes, int32_t zero_padding,
                      void *recv_x, float *recv_scales, float *recv_weights, int32_t *row_src,
                      int32_t *status, ep_handle_t *handle_host, hipStream_t stream);

/*
 * Combine through per-rank partial sums ("Deep Dive - DeepEP", "Combine:
 * reverse routing plus reduction": staging per rank sends fewer rows; the
 * partials are kept in fp32 because a bf16 subtotal can lose a small term to
 * cancellation).  Stage 1, per non-expanded row q of token t on rank r:
 *     partials[q, c] = fp32 sum, slot order j = 0.., over slots local to r, of
 *                      ne_topk_weights[q, j] * expert_out[tok_slot_row[t, j], c]
 *                      (one fused multiply-add each from +0; plain adds when
 *                      weighted == 0)
 * Stage 2: out[t, c] = bf16( fp32 sum over r = 0..R-1 with a row on r of
 *                      partials[tok_rank_row[t, r], c], from +0 ).
 * The result differs from ep_combine only by fp32 re-association (grouped
 * by rank).
 *
 *   expert_out  [capacity, H] bf16
 *   partials    [ranked_capacity, H] fp32 scratch/out
 *   out         [T, H] bf16 out
 * Rejects (EP_ERR_INVALID_ARG), as every call taking a ranked handle does,
 * ranked_capacity * ceil(H / 512) > 2^26 - 4.
 */
ep_status_t ep_combine_ranked(const ep_ranked_handle_t *ranked, const uint16_t *expert_out,
                              int32_t weighted, float *partials, uint16_t *out,
                              hipStream_t stream);

/* Synchronises `stream`, reads the device status word and returns the
 * first error it holds (route, then capacity, then workspace, then
 * non-finite input) or EP_OK.  It is the host-synchronising read of what
 * the kernels found, as the CPU-synchronised dispatch mode is ("Deep Dive -
 * DeepEP", "Dispatch: layout, move, and epilogue": exact host-side results
 * need the CPU-synchronised path), and it surfaces failures at the
 * boundary ("Combine: reverse routing plus reduction"). */
ep_status_t ep_read_status(const int32_t *status, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
