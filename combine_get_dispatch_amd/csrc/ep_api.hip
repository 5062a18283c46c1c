// Host side of the libep.so C ABI: argument validation, workspace sizing,
// kernel launches and status read-back.  Declarations and contracts are in
// include/ep.h.  Every check below runs before any HIP call, so a rejected
// call enqueues nothing and touches no device state.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "ep.h"
#include "ep_internal.h"

namespace {

thread_local char g_last_error[512] = "";

ep_status_t fail(ep_status_t st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

ep_status_t hip_fail(hipError_t err, const char *what) {
  return fail(EP_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

// Work items one launch holds.  The item kernels run one 64-lane wave per
// work item (a token or non-expanded row and a 512-column chunk at most), in
// workgroups of at most four waves, and a launch holds fewer than 2^32 work
// items of one lane each: ceil(items / 4) * 256 <= 2^32 - 1.
constexpr int64_t kMaxLaunchItems = (int64_t{1} << 26) - 4;
// Tokens combine backward holds: one 256-lane workgroup per token.
constexpr int64_t kMaxBackwardTokens = (int64_t{1} << 24) - 1;

ep_status_t check_config(const ep_config_t *c) {
  if (c == nullptr) return fail(EP_ERR_INVALID_ARG, "config is NULL");
  if (c->num_tokens < 0) return fail(EP_ERR_INVALID_ARG, "num_tokens %d < 0", c->num_tokens);
  if (c->hidden < 8 || c->hidden % 8 != 0)
    return fail(EP_ERR_INVALID_ARG, "hidden %d must be a positive multiple of 8", c->hidden);
  if (c->num_experts < 1 || c->num_experts > EP_MAX_EXPERTS)
    return fail(EP_ERR_INVALID_ARG, "num_experts %d outside [1, %d]", c->num_experts,
                EP_MAX_EXPERTS);
  if (c->num_topk < 1 || c->num_topk > EP_MAX_TOPK || c->num_topk > c->num_experts)
    return fail(EP_ERR_INVALID_ARG, "num_topk %d outside [1, min(num_experts, %d)]",
                c->num_topk, EP_MAX_TOPK);
  if (c->num_ranks < 1 || c->num_ranks > EP_MAX_RANKS || c->num_experts % c->num_ranks != 0)
    return fail(EP_ERR_INVALID_ARG,
                "num_ranks %d must be in [1, %d] and divide num_experts %d", c->num_ranks,
                EP_MAX_RANKS, c->num_experts);
  if (c->expert_alignment < 1)
    return fail(EP_ERR_INVALID_ARG, "expert_alignment %d < 1", c->expert_alignment);
  const int64_t rows = (int64_t)c->num_tokens * c->num_topk +
                       (int64_t)c->num_experts * (c->expert_alignment - 1);
  if (rows >= INT32_MAX)
    return fail(EP_ERR_INVALID_ARG, "T*k + E*(A-1) = %lld does not fit int32 row indices",
                (long long)rows);
  const int64_t chunks = (c->hidden + ep::kCombineCols - 1) / ep::kCombineCols;
  if ((int64_t)c->num_tokens * chunks > kMaxLaunchItems)
    return fail(EP_ERR_INVALID_ARG,
                "num_tokens x hidden too large: %lld (token, 512-column) items, at most %lld "
                "fit one launch",
                (long long)((int64_t)c->num_tokens * chunks), (long long)kMaxLaunchItems);
  return EP_OK;
}

ep::Dims dims_of(const ep_config_t *c) {
  return ep::Dims{c->num_tokens, c->hidden, c->num_topk,
                  c->num_experts, c->num_ranks, c->expert_alignment};
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// recv_dtype is a known type; FP8 rows need hidden % 128 == 0.
ep_status_t check_dtype(const ep_config_t *c, ep_dtype_t recv_dtype, bool *fp8) {
  if (recv_dtype != EP_DTYPE_BF16 && recv_dtype != EP_DTYPE_FP8_E4M3)
    return fail(EP_ERR_INVALID_ARG, "unknown recv_dtype %d", (int)recv_dtype);
  *fp8 = recv_dtype == EP_DTYPE_FP8_E4M3;
  if (*fp8 && c->hidden % 128 != 0)
    return fail(EP_ERR_INVALID_ARG, "FP8 rows need hidden %% 128 == 0 (hidden %d)", c->hidden);
  return EP_OK;
}

// A row count that int32 row indices can address.
ep_status_t check_rows(const char *what, int64_t rows) {
  if (rows < 0 || rows >= INT32_MAX)
    return fail(EP_ERR_INVALID_ARG, "%s %lld outside [0, 2^31 - 1)", what, (long long)rows);
  return EP_OK;
}

// Non-expanded rows whose (row, 512-column chunk) items fit one launch.
ep_status_t check_ranked_items(int64_t ranked_capacity, int32_t hidden) {
  const int64_t chunks = (hidden + ep::kCombineCols - 1) / ep::kCombineCols;
  if (ranked_capacity * chunks > kMaxLaunchItems)
    return fail(EP_ERR_INVALID_ARG,
                "ranked_capacity %lld x hidden %d too large: at most %lld (row, 512-column) "
                "items fit one launch",
                (long long)ranked_capacity, hidden, (long long)kMaxLaunchItems);
  return EP_OK;
}

// The workspace holds this configuration's layout sections and is 256-byte
// aligned.
ep_status_t check_workspace(const ep_config_t *c, const void *workspace, size_t workspace_bytes) {
  const size_t need =
      ep::workspace_layout(c->num_tokens, c->num_topk, c->num_experts, c->num_ranks).total;
  if (workspace_bytes < need)
    return fail(EP_ERR_INVALID_ARG, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(EP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return EP_OK;
}

#define EP_TRY(expr)                  \
  do {                                \
    const ep_status_t st_ = (expr);   \
    if (st_ != EP_OK) return st_;     \
  } while (0)

}  // namespace

namespace ep {
// Lets the probe entry point (hbm_probe.hip) report through ep_last_error().
ep_status_t set_error(ep_status_t st, const char *message) { return fail(st, "%s", message); }
}  // namespace ep

extern "C" {

const char *ep_status_string(ep_status_t status) {
  switch (status) {
    case EP_OK: return "ok";
    case EP_ERR_INVALID_ARG: return "invalid argument";
    case EP_ERR_INVALID_ROUTE: return "invalid route (expert id out of range or repeated)";
    case EP_ERR_CAPACITY: return "receive buffer too small";
    case EP_ERR_WORKSPACE: return "workspace not written by a layout of this configuration and route";
    case EP_ERR_HIP: return "HIP runtime error";
    case EP_ERR_NONFINITE: return "a hidden value or a valid selection's gate is inf or NaN";
  }
  return "unknown status";
}

const char *ep_last_error_string(void) { return g_last_error; }

const char *ep_last_error(void) { return g_last_error; }

ep_status_t ep_layout_workspace_bytes(const ep_config_t *cfg, size_t *bytes_host) {
  EP_TRY(check_config(cfg));
  if (bytes_host == nullptr) return fail(EP_ERR_INVALID_ARG, "bytes_host is NULL");
  *bytes_host = ep::workspace_layout(cfg->num_tokens, cfg->num_topk, cfg->num_experts,
                                     cfg->num_ranks)
                    .total;
  return EP_OK;
}

ep_status_t ep_recv_capacity_rows(const ep_config_t *cfg, int64_t *rows_host) {
  EP_TRY(check_config(cfg));
  if (rows_host == nullptr) return fail(EP_ERR_INVALID_ARG, "rows_host is NULL");
  *rows_host = (int64_t)cfg->num_tokens * cfg->num_topk +
               (int64_t)cfg->num_experts * (cfg->expert_alignment - 1);
  return EP_OK;
}

ep_status_t ep_workspace_init(void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (workspace == nullptr) return fail(EP_ERR_INVALID_ARG, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(EP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < 256)
    return fail(EP_ERR_INVALID_ARG, "workspace has %zu bytes, needs at least 256",
                workspace_bytes);
  hipError_t err = ep::launch_workspace_init(static_cast<char *>(workspace), stream);
  if (err != hipSuccess) return hip_fail(err, "workspace init launch");
  return EP_OK;
}

ep_status_t ep_read_status(const int32_t *status, hipStream_t stream) {
  if (status == nullptr) return fail(EP_ERR_INVALID_ARG, "status is NULL");
  int32_t host = 0;
  hipError_t err = hipMemcpyAsync(&host, status, sizeof host, hipMemcpyDeviceToHost, stream);
  if (err != hipSuccess) return hip_fail(err, "reading the status word");
  err = hipStreamSynchronize(stream);
  if (err != hipSuccess) return hip_fail(err, "synchronising the stream");
  if (host & EP_STATUS_BIT_ROUTE)
    return fail(EP_ERR_INVALID_ROUTE, "an expert id is outside [-1, E) or repeated in a token");
  if (host & EP_STATUS_BIT_CAPACITY)
    return fail(EP_ERR_CAPACITY, "a selection did not fit in the receive rows");
  if (host & EP_STATUS_BIT_WORKSPACE)
    return fail(EP_ERR_WORKSPACE, "dispatch workspace does not match its configuration or route");
  if (host & EP_STATUS_BIT_NONFINITE)
    return fail(EP_ERR_NONFINITE,
                "a hidden value or the gate of a valid selection is an infinity or NaN");
  return EP_OK;
}

ep_status_t ep_get_dispatch_layout(const ep_config_t *cfg, const int32_t *topk_idx,
                                   int32_t *num_tokens_per_rank,
                                   int32_t *num_tokens_per_expert,
                                   uint8_t *is_token_in_rank, int32_t *expert_offsets,
                                   int32_t *rank_offsets, void *workspace,
                                   size_t workspace_bytes, int32_t *status,
                                   int32_t *num_recv_rows_host, hipStream_t stream) {
  EP_TRY(check_config(cfg));
  const bool empty = cfg->num_tokens == 0;
  if ((!empty && (topk_idx == nullptr || is_token_in_rank == nullptr)) ||
      num_tokens_per_rank == nullptr || num_tokens_per_expert == nullptr ||
      expert_offsets == nullptr || rank_offsets == nullptr || workspace == nullptr ||
      status == nullptr)
    return fail(EP_ERR_INVALID_ARG, "a required pointer is NULL");
  EP_TRY(check_workspace(cfg, workspace, workspace_bytes));
  hipError_t err = ep::launch_layout(dims_of(cfg), topk_idx, num_tokens_per_rank,
                                     num_tokens_per_expert, is_token_in_rank, expert_offsets,
                                     rank_offsets, static_cast<char *>(workspace), status,
                                     stream);
  if (err != hipSuccess) return hip_fail(err, "layout launch");
  if (num_recv_rows_host != nullptr) {
    err = hipMemcpyAsync(num_recv_rows_host, expert_offsets + cfg->num_experts, sizeof(int32_t),
                         hipMemcpyDeviceToHost, stream);
    if (err != hipSuccess) return hip_fail(err, "reading the row count");
    return ep_read_status(status, stream);
  }
  return EP_OK;
}

ep_status_t ep_dispatch(const ep_config_t *cfg, ep_dtype_t recv_dtype, const uint16_t *x,
                        const int32_t *topk_idx, const float *topk_weights,
                        const int32_t *expert_offsets, const void *workspace,
                        size_t workspace_bytes, int64_t capacity, int32_t zero_padding,
                        void *recv_x, float *recv_scales, float *recv_weights,
                        int32_t *tok_slot_row, int32_t *row_src, int32_t *status,
                        ep_handle_t *handle_host, hipStream_t stream) {
  EP_TRY(check_config(cfg));
  bool fp8 = false;
  EP_TRY(check_dtype(cfg, recv_dtype, &fp8));
  EP_TRY(check_rows("capacity", capacity));
  const bool empty = cfg->num_tokens == 0;
  if ((!empty && (x == nullptr || topk_idx == nullptr || tok_slot_row == nullptr)) ||
      expert_offsets == nullptr || workspace == nullptr || status == nullptr ||
      (capacity > 0 && (recv_x == nullptr || row_src == nullptr)) ||
      (fp8 && capacity > 0 && recv_scales == nullptr))
    return fail(EP_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(x) || !aligned16(recv_x))
    return fail(EP_ERR_INVALID_ARG, "x and recv_x must be 16-byte aligned");
  EP_TRY(check_workspace(cfg, workspace, workspace_bytes));
  hipError_t err = ep::launch_dispatch(dims_of(cfg), fp8, zero_padding != 0, x, topk_idx,
                                       topk_weights, expert_offsets,
                                       static_cast<const char *>(workspace),
                                       capacity, recv_x, recv_scales, recv_weights, tok_slot_row,
                                       row_src, status, stream);
  if (err != hipSuccess) return hip_fail(err, "dispatch launch");
  if (handle_host != nullptr) {
    handle_host->config = *cfg;
    handle_host->capacity = capacity;
    handle_host->tok_slot_row = tok_slot_row;
    handle_host->row_src = row_src;
    handle_host->expert_offsets = expert_offsets;
  }
  return EP_OK;
}

ep_status_t ep_layout_dispatch(const ep_config_t *cfg, ep_dtype_t recv_dtype, const uint16_t *x,
                               const int32_t *topk_idx, const float *topk_weights,
                               int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                               uint8_t *is_token_in_rank, int32_t *expert_offsets,
                               int32_t *rank_offsets, void *workspace, size_t workspace_bytes,
                               int64_t capacity, int32_t zero_padding, void *recv_x,
                               float *recv_scales,
                               float *recv_weights, int32_t *tok_slot_row, int32_t *row_src,
                               int32_t *status, ep_handle_t *handle_host, hipStream_t stream) {
  EP_TRY(check_config(cfg));
  bool fp8 = false;
  EP_TRY(check_dtype(cfg, recv_dtype, &fp8));
  EP_TRY(check_rows("capacity", capacity));
  const bool empty = cfg->num_tokens == 0;
  if ((!empty && (x == nullptr || topk_idx == nullptr || is_token_in_rank == nullptr ||
                  tok_slot_row == nullptr)) ||
      num_tokens_per_rank == nullptr || num_tokens_per_expert == nullptr ||
      expert_offsets == nullptr || rank_offsets == nullptr || workspace == nullptr ||
      status == nullptr || (capacity > 0 && (recv_x == nullptr || row_src == nullptr)) ||
      (fp8 && capacity > 0 && recv_scales == nullptr))
    return fail(EP_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(x) || !aligned16(recv_x))
    return fail(EP_ERR_INVALID_ARG, "x and recv_x must be 16-byte aligned");
  EP_TRY(check_workspace(cfg, workspace, workspace_bytes));
  hipError_t err = ep::launch_layout_dispatch(
      dims_of(cfg), fp8, zero_padding != 0, x, topk_idx, topk_weights, num_tokens_per_rank,
      num_tokens_per_expert, is_token_in_rank, expert_offsets, rank_offsets,
      static_cast<char *>(workspace), capacity, recv_x, recv_scales, recv_weights, tok_slot_row,
      row_src, status, stream);
  if (err != hipSuccess) return hip_fail(err, "layout-dispatch launch");
  if (handle_host != nullptr) {
    handle_host->config = *cfg;
    handle_host->capacity = capacity;
    handle_host->tok_slot_row = tok_slot_row;
    handle_host->row_src = row_src;
    handle_host->expert_offsets = expert_offsets;
  }
  return EP_OK;
}

ep_status_t ep_dispatch_fp8_input(const ep_config_t *cfg, const uint8_t *x_codes,
                                  const float *x_scales, const int32_t *topk_idx,
                                  const float *topk_weights, const int32_t *expert_offsets,
                                  const void *workspace, size_t workspace_bytes,
                                  int64_t capacity, int32_t zero_padding, uint8_t *recv_x,
                                  float *recv_scales,
                                  float *recv_weights, int32_t *tok_slot_row, int32_t *row_src,
                                  int32_t *status, ep_handle_t *handle_host,
                                  hipStream_t stream) {
  EP_TRY(check_config(cfg));
  bool fp8 = false;
  EP_TRY(check_dtype(cfg, EP_DTYPE_FP8_E4M3, &fp8));
  EP_TRY(check_rows("capacity", capacity));
  const bool empty = cfg->num_tokens == 0;
  if ((!empty && (x_codes == nullptr || x_scales == nullptr || topk_idx == nullptr ||
                  tok_slot_row == nullptr)) ||
      expert_offsets == nullptr || workspace == nullptr || status == nullptr ||
      (capacity > 0 && (recv_x == nullptr || recv_scales == nullptr || row_src == nullptr)))
    return fail(EP_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(x_codes) || !aligned16(recv_x))
    return fail(EP_ERR_INVALID_ARG, "x_codes and recv_x must be 16-byte aligned");
  EP_TRY(check_workspace(cfg, workspace, workspace_bytes));
  hipError_t err = ep::launch_dispatch_fp8_input(
      dims_of(cfg), zero_padding != 0, x_codes, x_scales, topk_idx, topk_weights, expert_offsets,
      static_cast<const char *>(workspace), capacity, recv_x, recv_scales, recv_weights,
      tok_slot_row, row_src, status, stream);
  if (err != hipSuccess) return hip_fail(err, "dispatch launch");
  if (handle_host != nullptr) {
    handle_host->config = *cfg;
    handle_host->capacity = capacity;
    handle_host->tok_slot_row = tok_slot_row;
    handle_host->row_src = row_src;
    handle_host->expert_offsets = expert_offsets;
  }
  return EP_OK;
}

ep_status_t ep_combine(const ep_handle_t *handle, const uint16_t *expert_out,
                       const float *topk_weights, uint16_t *out, hipStream_t stream) {
  if (handle == nullptr) return fail(EP_ERR_INVALID_ARG, "handle is NULL");
  EP_TRY(check_config(&handle->config));
  EP_TRY(check_rows("handle capacity", handle->capacity));
  if (handle->config.num_tokens > 0 &&
      (handle->tok_slot_row == nullptr || out == nullptr ||
       (handle->capacity > 0 && expert_out == nullptr)))
    return fail(EP_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(expert_out) || !aligned16(out))
    return fail(EP_ERR_INVALID_ARG, "expert_out and out must be 16-byte aligned");
  hipError_t err = ep::launch_combine(dims_of(&handle->config), handle->capacity, expert_out,
                                      handle->tok_slot_row, topk_weights, out, stream);
  if (err != hipSuccess) return hip_fail(err, "combine launch");
  return EP_OK;
}

ep_status_t ep_dispatch_backward(const ep_handle_t *handle, const uint16_t *grad_recv_x,
                                 uint16_t *grad_x, hipStream_t stream) {
  if (handle == nullptr) return fail(EP_ERR_INVALID_ARG, "handle is NULL");
  EP_TRY(check_config(&handle->config));
  EP_TRY(check_rows("handle capacity", handle->capacity));
  if (handle->config.num_tokens > 0 &&
      (handle->tok_slot_row == nullptr || grad_x == nullptr ||
       (handle->capacity > 0 && grad_recv_x == nullptr)))
    return fail(EP_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(grad_recv_x) || !aligned16(grad_x))
    return fail(EP_ERR_INVALID_ARG, "grad_recv_x and grad_x must be 16-byte aligned");
  hipError_t err = ep::launch_combine(dims_of(&handle->config), handle->capacity, grad_recv_x,
                                      handle->tok_slot_row, nullptr, grad_x, stream);
  if (err != hipSuccess) return hip_fail(err, "dispatch backward launch");
  return EP_OK;
}

ep_status_t ep_combine_backward(const ep_handle_t *handle, const uint16_t *grad_out,
                                const float *topk_weights, const uint16_t *expert_out,
                                uint16_t *grad_expert_out, float *grad_weights,
                                hipStream_t stream) {
  if (handle == nullptr) return fail(EP_ERR_INVALID_ARG, "handle is NULL");
  EP_TRY(check_config(&handle->config));
  EP_TRY(check_rows("handle capacity", handle->capacity));
  if (handle->config.num_tokens > kMaxBackwardTokens)
    return fail(EP_ERR_INVALID_ARG,
                "num_tokens %d too large for combine backward (one workgroup per token, at "
                "most %lld)",
                handle->config.num_tokens, (long long)kMaxBackwardTokens);
  const bool empty = handle->config.num_tokens == 0;
  if ((!empty && (handle->tok_slot_row == nullptr || grad_out == nullptr)) ||
      (handle->capacity > 0 && grad_expert_out == nullptr) ||
      (grad_weights != nullptr && !empty && expert_out == nullptr))
    return fail(EP_ERR_INVALID_ARG, "a required pointer is NULL");
  if (handle->config.expert_alignment > 1 &&
      (handle->row_src == nullptr || handle->expert_offsets == nullptr))
    return fail(EP_ERR_INVALID_ARG,
                "with expert_alignment > 1 the handle needs row_src and expert_offsets");
  if (!aligned16(grad_out) || !aligned16(expert_out) || !aligned16(grad_expert_out))
    return fail(EP_ERR_INVALID_ARG, "grad_out, expert_out and grad_expert_out must be 16-byte aligned");
  hipError_t err = ep::launch_combine_backward(
      dims_of(&handle->config), handle->capacity, grad_out, handle->tok_slot_row, topk_weights,
      expert_out, grad_expert_out, grad_weights, handle->expert_offsets, handle->row_src, stream);
  if (err != hipSuccess) return hip_fail(err, "combine backward launch");
  return EP_OK;
}

ep_status_t ep_ranked_capacity_rows(const ep_config_t *cfg, int64_t *rows_host) {
  EP_TRY(check_config(cfg));
  if (rows_host == nullptr) return fail(EP_ERR_INVALID_ARG, "rows_host is NULL");
  const int64_t per = cfg->num_topk < cfg->num_ranks ? cfg->num_topk : cfg->num_ranks;
  *rows_host = (int64_t)cfg->num_tokens * per;
  return EP_OK;
}

ep_status_t ep_dispatch_ranked(const ep_config_t *cfg, ep_dtype_t recv_dtype, const uint16_t *x,
                               const int32_t *topk_idx, const float *topk_weights,
                               const int32_t *expert_offsets, const void *workspace,
                               size_t workspace_bytes, int64_t capacity, int64_t ranked_capacity,
                               void *ne_x, float *ne_scales, int32_t *ne_topk_idx,
                               float *ne_topk_weights, int32_t *ne_src,
                               int32_t *rank_token_offsets, int32_t *tok_rank_row,
                               int32_t *tok_slot_row, int32_t *status,
                               ep_ranked_handle_t *handle_host, hipStream_t stream) {
  EP_TRY(check_config(cfg));
  bool fp8 = false;
  EP_TRY(check_dtype(cfg, recv_dtype, &fp8));
  EP_TRY(check_rows("capacity", capacity));
  EP_TRY(check_rows("ranked_capacity", ranked_capacity));
  EP_TRY(check_ranked_items(ranked_capacity, cfg->hidden));
  const bool empty = cfg->num_tokens == 0;
  if ((!empty && (x == nullptr || topk_idx == nullptr || tok_rank_row == nullptr ||
                  tok_slot_row == nullptr)) ||
      expert_offsets == nullptr || workspace == nullptr || status == nullptr ||
      rank_token_offsets == nullptr ||
      (ranked_capacity > 0 && (ne_x == nullptr || ne_topk_idx == nullptr || ne_src == nullptr ||
                               (fp8 && ne_scales == nullptr))))
    return fail(EP_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(x) || !aligned16(ne_x))
    return fail(EP_ERR_INVALID_ARG, "x and ne_x must be 16-byte aligned");
  EP_TRY(check_workspace(cfg, workspace, workspace_bytes));
  hipError_t err = ep::launch_dispatch_ranked(
      dims_of(cfg), fp8, x, topk_idx, topk_weights, expert_offsets,
      static_cast<const char *>(workspace), capacity, ranked_capacity, ne_x, ne_scales,
      ne_topk_idx, ne_topk_weights, ne_src, rank_token_offsets, tok_rank_row, tok_slot_row,
      status, stream);
  if (err != hipSuccess) return hip_fail(err, "ranked dispatch launch");
  if (handle_host != nullptr) {
    handle_host->config = *cfg;
    handle_host->capacity = capacity;
    handle_host->ranked_capacity = ranked_capacity;
    handle_host->rank_token_offsets = rank_token_offsets;
    handle_host->tok_rank_row = tok_rank_row;
    handle_host->tok_slot_row = tok_slot_row;
    handle_host->ne_topk_idx = ne_topk_idx;
    handle_host->ne_topk_weights = ne_topk_weights;
    handle_host->ne_src = ne_src;
  }
  return EP_OK;
}

static ep_status_t check_ranked(const ep_ranked_handle_t *h) {
  if (h == nullptr) return fail(EP_ERR_INVALID_ARG, "ranked handle is NULL");
  EP_TRY(check_config(&h->config));
  EP_TRY(check_rows("handle capacity", h->capacity));
  EP_TRY(check_rows("handle ranked_capacity", h->ranked_capacity));
  EP_TRY(check_ranked_items(h->ranked_capacity, h->config.hidden));
  if (h->rank_token_offsets == nullptr ||
      (h->config.num_tokens > 0 && (h->tok_rank_row == nullptr || h->tok_slot_row == nullptr)) ||
      (h->ranked_capacity > 0 && (h->ne_topk_idx == nullptr || h->ne_src == nullptr)))
    return fail(EP_ERR_INVALID_ARG, "ranked handle has a NULL array");
  return EP_OK;
}

ep_status_t ep_expand(const ep_ranked_handle_t *ranked, ep_dtype_t recv_dtype, const void *ne_x,
                      const float *ne_scales, const int32_t *expert_offsets,
                      const void *workspace, size_t workspace_bytes, int32_t zero_padding,
                      void *recv_x, float *recv_scales, float *recv_weights, int32_t *row_src,
                      int32_t *status, ep_handle_t *handle_host, hipStream_t stream) {
  EP_TRY(check_ranked(ranked));
  const ep_config_t *cfg = &ranked->config;
  bool fp8 = false;
  EP_TRY(check_dtype(cfg, recv_dtype, &fp8));
  if (expert_offsets == nullptr || workspace == nullptr || status == nullptr ||
      (ranked->ranked_capacity > 0 && (ne_x == nullptr || (fp8 && ne_scales == nullptr))) ||
      (ranked->capacity > 0 && (recv_x == nullptr || row_src == nullptr ||
                                (fp8 && recv_scales == nullptr))))
    return fail(EP_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(ne_x) || !aligned16(recv_x))
    return fail(EP_ERR_INVALID_ARG, "ne_x and recv_x must be 16-byte aligned");
  EP_TRY(check_workspace(cfg, workspace, workspace_bytes));
  hipError_t err = ep::launch_expand(
      dims_of(cfg), fp8, zero_padding != 0, ranked->ranked_capacity, ne_x, ne_scales,
      ranked->ne_topk_idx, ranked->ne_topk_weights, ranked->ne_src, ranked->rank_token_offsets,
      expert_offsets, static_cast<const char *>(workspace), ranked->capacity, recv_x, recv_scales,
      recv_weights, row_src, status, stream);
  if (err != hipSuccess) return hip_fail(err, "expand launch");
  if (handle_host != nullptr) {
    handle_host->config = *cfg;
    handle_host->capacity = ranked->capacity;
    handle_host->tok_slot_row = ranked->tok_slot_row;
    handle_host->row_src = row_src;
    handle_host->expert_offsets = expert_offsets;
  }
  return EP_OK;
}

ep_status_t ep_combine_ranked(const ep_ranked_handle_t *ranked, const uint16_t *expert_out,
                              int32_t weighted, float *partials, uint16_t *out,
                              hipStream_t stream) {
  EP_TRY(check_ranked(ranked));
  if (weighted && ranked->ranked_capacity > 0 && ranked->ne_topk_weights == nullptr)
    return fail(EP_ERR_INVALID_ARG, "weighted combine needs ne_topk_weights in the handle");
  if ((ranked->config.num_tokens > 0 && out == nullptr) ||
      (ranked->ranked_capacity > 0 && partials == nullptr) ||
      (ranked->capacity > 0 && expert_out == nullptr))
    return fail(EP_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(expert_out) || !aligned16(out) || !aligned16(partials))
    return fail(EP_ERR_INVALID_ARG, "expert_out, partials and out must be 16-byte aligned");
  hipError_t err = ep::launch_combine_ranked(
      dims_of(&ranked->config), ranked->capacity, ranked->ranked_capacity, expert_out,
      ranked->tok_slot_row, ranked->ne_topk_idx, weighted ? ranked->ne_topk_weights : nullptr,
      ranked->ne_src, ranked->rank_token_offsets, ranked->tok_rank_row, partials, out, stream);
  if (err != hipSuccess) return hip_fail(err, "ranked combine launch");
  return EP_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Layout and dispatch without a caller workspace, for callers that cannot
// allocate: the layout's workspace is the file-scope device array below,
// one copy per GPU, reached through its address on that GPU.
// ---------------------------------------------------------------------------

namespace {

static __device__ __align__(256) unsigned char scratch[EP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current GPU.  Taken once per
// GPU (with that GPU current), when its header is also cleared: the
// layout's ticket must start at zero, and every layout leaves it at zero.
ep_status_t scratch_on_current_device(hipStream_t stream, char **out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_fail(err, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(EP_ERR_HIP, "device %d is beyond the %d this library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return hip_fail(err, "hipGetSymbolAddress(scratch)");
    err = ep::launch_workspace_init(static_cast<char *>(ptr), stream);
    if (err != hipSuccess) return hip_fail(err, "scratch header init launch");
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<char *>(g_scratch_ptr[dev]);
  return EP_OK;
}

}  // namespace

extern "C" ep_status_t ep_layout_dispatch_noalloc(
    const ep_config_t *cfg, ep_dtype_t recv_dtype, const uint16_t *x, const int32_t *topk_idx,
    const float *topk_weights, int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
    uint8_t *is_token_in_rank, int32_t *expert_offsets, int32_t *rank_offsets, int64_t capacity,
    int32_t zero_padding, void *recv_x, float *recv_scales, float *recv_weights,
    int32_t *tok_slot_row, int32_t *row_src, int32_t *status, ep_handle_t *handle_host,
    hipStream_t stream) {
  EP_TRY(check_config(cfg));
  bool fp8 = false;
  EP_TRY(check_dtype(cfg, recv_dtype, &fp8));
  EP_TRY(check_rows("capacity", capacity));
  const size_t need =
      ep::workspace_layout(cfg->num_tokens, cfg->num_topk, cfg->num_experts, cfg->num_ranks)
          .total;
  if (need > (size_t)EP_NOALLOC_SCRATCH_BYTES)
    return fail(EP_ERR_INVALID_ARG,
                "ep_layout_dispatch_noalloc: this configuration's layout workspace needs %zu "
                "bytes, more than the library's %d-byte scratch",
                need, EP_NOALLOC_SCRATCH_BYTES);
  const bool empty = cfg->num_tokens == 0;
  if ((!empty && (x == nullptr || topk_idx == nullptr || is_token_in_rank == nullptr ||
                  tok_slot_row == nullptr)) ||
      num_tokens_per_rank == nullptr || num_tokens_per_expert == nullptr ||
      expert_offsets == nullptr || rank_offsets == nullptr || status == nullptr ||
      (capacity > 0 && (recv_x == nullptr || row_src == nullptr)) ||
      (fp8 && capacity > 0 && recv_scales == nullptr))
    return fail(EP_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(x) || !aligned16(recv_x))
    return fail(EP_ERR_INVALID_ARG, "x and recv_x must be 16-byte aligned");
  char *ws = nullptr;
  EP_TRY(scratch_on_current_device(stream, &ws));
  const hipError_t err = ep::launch_layout_dispatch(
      dims_of(cfg), fp8, zero_padding != 0, x, topk_idx, topk_weights, num_tokens_per_rank,
      num_tokens_per_expert, is_token_in_rank, expert_offsets, rank_offsets, ws, capacity, recv_x,
      recv_scales, recv_weights, tok_slot_row, row_src, status, stream);
  if (err != hipSuccess) return hip_fail(err, "layout-dispatch launch");
  if (handle_host != nullptr) {
    handle_host->config = *cfg;
    handle_host->capacity = capacity;
    handle_host->tok_slot_row = tok_slot_row;
    handle_host->row_src = row_src;
    handle_host->expert_offsets = expert_offsets;
  }
  return EP_OK;
}
