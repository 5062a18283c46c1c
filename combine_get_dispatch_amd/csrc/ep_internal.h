// Internal declarations shared by the host API (ep_api.hip) and the kernels
// (ep_kernels.hip) of libep.so.  Not installed; callers use include/ep.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

// A layout tile is one 256-thread workgroup with one token per lane, so a
// tile holds four wave64s' worth of tokens.
constexpr int kTileTokens = 256;
constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
// Waves MI355X holds at once: 256 compute units x 4 SIMDs x 8 waves.
constexpr int64_t kChipWaves = 256 * 4 * 8;

// Columns one dispatch wave moves per work item: 64 lanes x 16 values.
constexpr int kChunkCols = 1024;
// Columns one combine wave reduces per work item: 64 lanes x 8 bf16.
constexpr int kCombineCols = 512;

// Workspace header (int32 words): [0] magic once a layout has completed,
// [1..5] T, k, E, R, A of that layout, [6] tiles, [8] layout ticket.
constexpr int32_t kWorkspaceMagic = 0x45504C59;  // "EPLY"
constexpr int kHeaderInts = 16;
constexpr int kHeaderTicket = 8;

// A tile row of the workspace: the tile's count per expert, padded with
// zeros to a multiple of 4, then its token count per rank, padded likewise,
// so that every 16-byte quad of the row holds expert columns only or rank
// columns only.  After the layout's scan the same rows hold the tile bases
// (the counts of the earlier tiles).
__host__ __device__ constexpr int32_t tile_row_experts(int32_t E) { return (E + 3) & ~3; }
__host__ __device__ constexpr int32_t tile_row_ints(int32_t E, int32_t R) {
  return ((E + 3) & ~3) + ((R + 3) & ~3);
}

// How the scanning workgroup of a layout splits the tile rows: the tiles
// are cut into S slices of `per` consecutive tiles, and thread (q, s) =
// (tid % C4, tid / C4) owns column quad q of the tiles of slice s.  S is
// as small as slices of at most 8 tiles allow (every slice costs the
// column totals one more LDS read), and at most what the threads cover.
// With more quads than threads (E + R above 1024) there is one slice and a
// thread owns quads tid and tid + 256.
struct TileGrid {
  int32_t C4, S, per;
};

__host__ __device__ inline TileGrid tile_grid(int32_t E, int32_t R, int32_t ntiles) {
  TileGrid g;
  g.C4 = tile_row_ints(E, R) / 4;
  g.S = g.C4 <= kBlock ? kBlock / g.C4 : 1;
  const int32_t want = ntiles > 0 ? (ntiles + 7) / 8 : 1;
  if (g.S > want) g.S = want;
  g.per = (ntiles + g.S - 1) / g.S;
  return g;
}

// A selection's word in the workspace's slot table: its expert id in the
// high half and its stable rank inside its tile (below 256) in the low half,
// or -1 for a selection the layout did not count.  The expert lets every
// later reader check that it was given the layout's own route.
constexpr int kSlotExpertShift = 16;
constexpr int32_t kSlotRankMask = 0xFFFF;

// Byte offsets of the workspace sections for one configuration.
struct WorkspaceLayout {
  int32_t ntiles;
  size_t tile_cnt;       // int32 [ntiles, tile_row_ints(E, R)]: tile rows (above)
  size_t tile_rank_cnt;  // the rank columns of the tile rows (same rows, past the experts)
  size_t cnt;            // int32 [E]: unaligned count per expert
  size_t slot_rank;      // int32 [T, k]: (e, rank of (t, j) inside its tile's run of e)
  size_t rank_ballot;    // u64 [ntiles, 4 waves, R]: which lanes' tokens have an expert on r
  size_t rank_tok_off;   // int32 [R + 1]: starts of the ranks' token partitions
  size_t total;
};

WorkspaceLayout workspace_layout(int32_t T, int32_t k, int32_t E, int32_t R);

struct Dims {
  int32_t T, H, k, E, R, A;
};

// last: the layout is the call's last kernel (for kernel timing).
hipError_t launch_layout(const Dims &d, const int32_t *topk_idx, int32_t *num_tokens_per_rank,
                         int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank,
                         int32_t *expert_offsets, int32_t *rank_offsets, char *ws,
                         int32_t *status, hipStream_t stream, bool last = true);

hipError_t launch_workspace_init(char *ws, hipStream_t stream);

// The next hot-path kernel this thread launches records start and stop.
void time_next_kernel(hipEvent_t start, hipEvent_t stop);

// Dynamic LDS bytes of a layout workgroup with E experts.
size_t layout_lds_bytes(int32_t E);

// Layout and dispatch: one launch up to kTileTokens tokens, else the layout
// launch and the dispatch launch.
hipError_t launch_layout_dispatch(const Dims &d, bool fp8, bool zero_padding,
                                  const uint16_t *x, const int32_t *topk_idx,
                                  const float *topk_weights,
                                  int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                                  uint8_t *is_token_in_rank, int32_t *expert_offsets,
                                  int32_t *rank_offsets, char *ws, int64_t capacity, void *recv_x,
                                  float *recv_scales, float *recv_weights, int32_t *tok_slot_row,
                                  int32_t *row_src, int32_t *status, hipStream_t stream);

hipError_t launch_dispatch(const Dims &d, bool fp8, bool zero_padding, const uint16_t *x,
                           const int32_t *topk_idx, const float *topk_weights,
                           const int32_t *expert_offsets, const char *ws, int64_t capacity,
                           void *recv_x, float *recv_scales, float *recv_weights,
                           int32_t *tok_slot_row, int32_t *row_src, int32_t *status,
                           hipStream_t stream);

hipError_t launch_dispatch_fp8_input(const Dims &d, bool zero_padding, const uint8_t *x_codes,
                                     const float *x_scales, const int32_t *topk_idx,
                                     const float *topk_weights, const int32_t *expert_offsets,
                                     const char *ws,
                                     int64_t capacity, uint8_t *recv_x, float *recv_scales,
                                     float *recv_weights, int32_t *tok_slot_row,
                                     int32_t *row_src, int32_t *status, hipStream_t stream);

hipError_t launch_combine(const Dims &d, int64_t capacity, const uint16_t *expert_out,
                          const int32_t *tok_slot_row, const float *topk_weights,
                          uint16_t *out, hipStream_t stream);

hipError_t launch_combine_backward(const Dims &d, int64_t capacity, const uint16_t *grad_out,
                                   const int32_t *tok_slot_row, const float *topk_weights,
                                   const uint16_t *expert_out, uint16_t *grad_expert_out,
                                   float *grad_weights, const int32_t *expert_offsets,
                                   const int32_t *row_src, hipStream_t stream);

hipError_t launch_dispatch_ranked(const Dims &d, bool fp8, const uint16_t *x,
                                  const int32_t *topk_idx, const float *topk_weights,
                                  const int32_t *expert_offsets, const char *ws, int64_t capacity,
                                  int64_t ranked_capacity, void *ne_x, float *ne_scales,
                                  int32_t *ne_topk_idx, float *ne_topk_weights, int32_t *ne_src,
                                  int32_t *rank_token_offsets, int32_t *tok_rank_row,
                                  int32_t *tok_slot_row, int32_t *status, hipStream_t stream);

hipError_t launch_expand(const Dims &d, bool fp8, bool zero_padding, int64_t ranked_capacity,
                         const void *ne_x, const float *ne_scales, const int32_t *ne_topk_idx,
                         const float *ne_topk_weights, const int32_t *ne_src,
                         const int32_t *rank_token_offsets, const int32_t *expert_offsets,
                         const char *ws, int64_t capacity, void *recv_x, float *recv_scales,
                         float *recv_weights, int32_t *row_src, int32_t *status,
                         hipStream_t stream);

hipError_t launch_combine_ranked(const Dims &d, int64_t capacity, int64_t ranked_capacity,
                                 const uint16_t *y, const int32_t *tok_slot_row,
                                 const int32_t *ne_topk_idx, const float *ne_topk_weights,
                                 const int32_t *ne_src, const int32_t *rank_token_offsets,
                                 const int32_t *tok_rank_row, float *partials, uint16_t *out,
                                 hipStream_t stream);

}  // namespace ep
