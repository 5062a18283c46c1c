// HIP kernels of libep.so for gfx950 (CDNA4, wave64).
//
// Pages cited: "GPU microarchitecture: DeepEP first principles"
// (backyes.github.io) and "Deep Dive - DeepEP" (leetllm.com), by section.
//
// The path is pure data movement (no dense contraction, so no MFMA):
//   layout_kernel         one workgroup per 256-token tile: per-wave expert
//                         bitmasks in LDS (64-bit OR per selection), their
//                         popcounts give the tile histogram and each
//                         selection's stable rank inside the tile; ballots
//                         give distinct tokens per rank.  The last
//                         workgroup to finish (or the only one) scans: per
//                         expert over tiles (tile bases), then over experts
//                         (segment starts).
//   dispatch_kernel       one wave per (token, 1024-column chunk): reads the
//                         x chunk once with 16-byte loads, optionally
//                         quantises it to E4M3 in registers, and stores it to
//                         each of the token's receive rows.
//   combine_kernel        one one-wave workgroup per (token, 512-column
//                         chunk): k gathered 16-byte loads per lane, fp32
//                         FMAs in slot order, one bf16 rounding, one
//                         16-byte store.
//   layout_dispatch_kernel  layout and dispatch in one launch for at most
//                         256 tokens: every workgroup recounts the batch in
//                         LDS; workgroup 0 writes the layout outputs and the
//                         others move the rows.
// Also: the non-expanded path (dispatch_ranked_kernel, expand_kernel, the
// two ranked combine stages), the backward of combine, and the alignment
// padding fills.  Output positions never depend on atomics or scheduling,
// so every result is deterministic.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep.h"
#include "ep_internal.h"

namespace ep {

namespace {

__device__ __forceinline__ void flag(int32_t *status, int32_t bit) { atomicOr(status, bit); }

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int32_t lane_value(int32_t v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}

__device__ __forceinline__ float lane_value_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Streaming (non-temporal) 16-byte accesses for data touched exactly once per
// pass: the receive rows written by dispatch, the expert outputs read and the
// rows written by combine.  Written lines drain to HBM during the kernel that
// wrote them instead of being evicted during the next one.  (x is read with
// plain loads: streaming loads measured slower for it.)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream(const void *p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_stream(void *p, uint4 v) {
  const u32x4 q = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(q, static_cast<u32x4 *>(p));
}

// bf16 bits -> fp32 (exact), for the low and high halves of a 32-bit word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16 with v_cvt_pk_bf16_f32 (gfx950): round to nearest
// even, and a NaN keeps its sign and upper payload with the quiet bit set.
// These are the results of the integer procedure of "Deep Dive - DeepEP",
// "Combine: reverse routing plus reduction" (add 0x7FFF plus the lowest kept
// bit, keep the upper half), which the oracle implements; the parity tests
// compare every combined element with it.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS):
// shifts of 1, 2, 4 and 8 lanes inside each row of 16, then the last lane
// of row 0 added to row 1 (and of row 2 to row 3), then the last lane of
// row 1 to rows 2 and 3.  Lanes whose source falls outside the row add 0.
// Integer sums, so the result does not depend on the order of the adds.
__device__ __forceinline__ int32_t wave_inclusive_sum(int32_t v) {
  constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr + 1, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr + 2, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr + 4, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr + 8, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowBcast15, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowBcast31, 0xc, 0xf, false);
  return v;
}

// Workspace header check shared by the dispatch kernels: the workspace must
// have been written by a layout of exactly this configuration.  The six
// words come in two wide loads and are compared without short-circuit, so
// that the check costs one round trip instead of one per word.
__device__ __forceinline__ bool workspace_ok(const int32_t *__restrict__ hdr, const Dims &d) {
  const int4 a = *reinterpret_cast<const int4 *>(hdr);
  const int2 b = *reinterpret_cast<const int2 *>(hdr + 4);
  const int ok = (a.x == kWorkspaceMagic) & (a.y == d.T) & (a.z == d.k) & (a.w == d.E) &
                 (b.x == d.R) & (b.y == d.A);
  return ok != 0;
}

}  // namespace

// ---------------------------------------------------------------------------
// Layout (count, then prefix sum: "GPU microarchitecture: DeepEP first
// principles", "7.1 Does Sort Exist?"), in one launch.  Every workgroup
// counts one 256-token tile.  With several tiles, the last workgroup to
// finish (it draws the last ticket from a device-scope counter, a
// release-acquire read-modify-write) scans all tile histograms; a single
// workgroup scans its own counts straight from LDS.  The ticket lives in the
// workspace header; it starts at zero (ep_workspace_init) and the scanning
// workgroup resets it, so consecutive layouts on one stream can reuse the
// workspace.  The phases below are shared with layout_dispatch_kernel.
// ---------------------------------------------------------------------------

// The layout's LDS: [kWavesPerBlock][E] expert bitmasks; [kWavesPerBlock][E]
// counts of each expert in the earlier waves of the tile; [E + 1] words
// holding the tile's (later the batch's) count per expert, then the aligned
// offsets; per-rank token counts and per-wave scan totals.
struct LayoutLds {
  unsigned long long *masks;
  int32_t *prefix;
  int32_t *counts;
  int32_t *rank_cnt;
  int32_t *wave_total;
};

__device__ __forceinline__ LayoutLds layout_lds(unsigned long long *dyn, int E,
                                                int32_t *rank_cnt, int32_t *wave_total) {
  LayoutLds L;
  L.masks = dyn;
  L.prefix = reinterpret_cast<int32_t *>(dyn + kWavesPerBlock * E);
  L.counts = L.prefix + kWavesPerBlock * E;
  L.rank_cnt = rank_cnt;
  L.wave_total = wave_total;
  return L;
}

// The token's expert ids (-1 past k or for a token outside the batch),
// loaded together.
template <int K>
__device__ __forceinline__ void load_ids(const Dims &d, int64_t t, bool live,
                                         const int32_t *__restrict__ topk_idx, int32_t (&ex)[K]) {
#pragma unroll
  for (int j = 0; j < K; ++j) ex[j] = (live && j < d.k) ? topk_idx[t * d.k + j] : -1;
}

// Count phase of one tile, thread tid = token tile * 256 + tid.  Takes the
// token's k expert ids in ex (from load_ids; ids outside [-1, E) become -1), marks them
// in the wave's LDS bitmask of each expert, counts distinct tokens per rank
// and leaves per expert its count in the earlier waves (prefix) and in the
// tile (counts).  A repeated or out-of-range id sets the route bit when
// status is given; the per-wave rank ballots go to rank_ballot when given.
template <int K>
__device__ __forceinline__ void count_tile(const Dims &d, int tile, int experts_per_rank,
                                           const LayoutLds &L, int32_t (&ex)[K],
                                           unsigned long long &rmask,
                                           unsigned long long *__restrict__ rank_ballot,
                                           int32_t *__restrict__ status) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int E = d.E, R = d.R;
  const unsigned long long me = 1ull << lane;
  // rank of expert e = e / experts_per_rank as (e * magic) >> 21: exact for
  // e < 1024 and experts_per_rank <= 1024, since e * experts_per_rank < 2^21
  // (the identity also keeps e * magic below 2^32).
  static_assert(EP_MAX_EXPERTS <= 1024, "the rank division below needs E <= 1024");
  const uint32_t rank_magic = ((1u << 21) + (uint32_t)experts_per_rank - 1u) /
                              (uint32_t)experts_per_rank;

  for (int i = tid; i < kWavesPerBlock * E; i += kBlock) L.masks[i] = 0ull;
  for (int i = tid; i < R; i += kBlock) L.rank_cnt[i] = 0;
  __syncthreads();

  // Mark this token in its wave's bitmask of every expert it selected;
  // reject ids outside [-1, E).  Branch-free: a masked or rejected slot ORs
  // 0 into some in-range word (one per lane, so that these no-op atomics do
  // not queue on one address).  Slots past k (uniform) are skipped.
  bool bad = false;
  rmask = 0ull;
  const uint32_t spread = min((uint32_t)lane, (uint32_t)E - 1u);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if (j >= d.k) break;
    const int32_t e = ex[j];
    const bool valid = (uint32_t)e < (uint32_t)E;
    bad |= e < -1 || e >= E;
    ex[j] = valid ? e : -1;
    const uint32_t ev = valid ? (uint32_t)e : spread;
    atomicOr(&L.masks[wave * E + ev], valid ? me : 0ull);
    rmask |= valid ? 1ull << ((ev * rank_magic) >> 21) : 0ull;
  }
  // A repeated expert within the token is checked where the route status
  // is reported (the layout, and the fused kernel's lead workgroup).  A
  // repeat sets one bit twice, so the counts stay in bounds either way.
  if (status != nullptr) {
#pragma unroll
    for (int j = 1; j < K; ++j)
#pragma unroll
      for (int jj = 0; jj < j; ++jj) bad |= ex[j] >= 0 && ex[jj] == ex[j];
    if (bad) flag(status, EP_STATUS_BIT_ROUTE);
  }

  // Distinct tokens per rank in this tile: lane r keeps the wave's ballot
  // for rank r.  The ballots also go to the workspace: the non-expanded
  // dispatch places a token among a rank's tokens from these words.
  unsigned long long mine = 0ull;
  for (int r = 0; r < R; ++r) {
    const unsigned long long b = __ballot((rmask >> r) & 1ull);
    if (lane == r) mine = b;
  }
  if (lane < R) {
    if (rank_ballot != nullptr)
      rank_ballot[((int64_t)tile * kWavesPerBlock + wave) * R + lane] = mine;
    if (mine) atomicAdd(&L.rank_cnt[lane], (int32_t)__popcll(mine));
  }
  __syncthreads();

  // Per expert: its count in the earlier waves (for the stable ranks) and
  // in the tile.
  for (int e = tid; e < E; e += kBlock) {
    int32_t run = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
      L.prefix[w * E + e] = run;
      run += __popcll(L.masks[w * E + e]);
    }
    L.counts[e] = run;
  }
}

// Stable rank of selection e of token (wave, lane) inside its tile: tokens
// of earlier waves that chose e, plus lanes below this one in its own wave
// that chose e.
__device__ __forceinline__ int32_t tile_rank(const LayoutLds &L, int E, int wave, int lane,
                                             int32_t e) {
  return __popcll(L.masks[wave * E + e] & ((1ull << lane) - 1ull)) + L.prefix[wave * E + e];
}

// Per-token outputs: the rank mask (one byte per rank) and each selection's
// slot word (its expert and its stable in-tile rank, kSlotExpertShift).  Every LDS read is issued before the first
// result is used, and each row is written with the widest stores its size
// and alignment allow (one store per lane covers many slots, where one per
// slot would make every store instruction touch a cache line per few lanes).
template <int K>
__device__ __forceinline__ void token_outputs(const Dims &d, int64_t t, const LayoutLds &L,
                                              const int32_t (&ex)[K], unsigned long long rmask,
                                              uint8_t *__restrict__ is_token_in_rank,
                                              int32_t *__restrict__ slot_rank) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int R = d.R, k = d.k;
  unsigned long long m[K];
  int32_t pre[K], rank[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int32_t e = ex[j] >= 0 ? ex[j] : 0;
    m[j] = L.masks[wave * d.E + e];
    pre[j] = L.prefix[wave * d.E + e];
  }
#pragma unroll
  for (int j = 0; j < K; ++j)
    rank[j] = ex[j] >= 0 ? ex[j] << kSlotExpertShift |
                               (__popcll(m[j] & ((1ull << lane) - 1ull)) + pre[j])
                         : -1;

  // Four mask bits b0..b3 to the bytes b0, b1, b2, b3 of a word: the
  // multiplier's shifted copies (0, 7, 14, 21) do not overlap.
  auto bytes4 = [](unsigned long long bits) {
    return ((uint32_t)bits & 0xFu) * 0x204081u & 0x01010101u;
  };
  uint8_t *dst = is_token_in_rank + t * R;
  const uintptr_t base = reinterpret_cast<uintptr_t>(is_token_in_rank);
  if ((R & 15) == 0 && (base & 15) == 0) {
    for (int r = 0; r < R; r += 16)
      *reinterpret_cast<uint4 *>(dst + r) =
          make_uint4(bytes4(rmask >> r), bytes4(rmask >> (r + 4)), bytes4(rmask >> (r + 8)),
                     bytes4(rmask >> (r + 12)));
  } else if ((R & 7) == 0 && (base & 7) == 0) {
    for (int r = 0; r < R; r += 8)
      *reinterpret_cast<uint2 *>(dst + r) =
          make_uint2(bytes4(rmask >> r), bytes4(rmask >> (r + 4)));
  } else if ((R & 3) == 0 && (base & 3) == 0) {
    for (int r = 0; r < R; r += 4) *reinterpret_cast<uint32_t *>(dst + r) = bytes4(rmask >> r);
  } else {
    for (int r = 0; r < R; ++r) dst[r] = (uint8_t)((rmask >> r) & 1ull);
  }

  // The workspace row t * k is 16-byte aligned when k % 4 == 0, 8-byte
  // aligned when k is even.
  int32_t *row = slot_rank + t * k;
  if ((k & 3) == 0) {
#pragma unroll
    for (int j = 0; j + 3 < K; j += 4)
      if (j < k)
        *reinterpret_cast<int4 *>(row + j) =
            make_int4(rank[j], rank[j + 1], rank[j + 2], rank[j + 3]);
  } else if ((k & 1) == 0) {
#pragma unroll
    for (int j = 0; j + 1 < K; j += 2)
      if (j < k) *reinterpret_cast<int2 *>(row + j) = make_int2(rank[j], rank[j + 1]);
  } else {
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (j < k) row[j] = rank[j];
  }
}

// Scan phase, by a whole workgroup, once L.counts holds the batch's count
// per expert and thread r < R holds rank r's token count in rank_sum.
// Leaves the aligned segment starts in L.counts[0..E] and, with write set,
// stores the counts, offsets and rank partitions.  With kLate every global
// store comes after the last barrier: for a caller with no store pending,
// a store issued earlier could make the compiler's wait for a later load
// result (loads and stores share one counter on this chip) also wait for
// that store.  Without kLate the stores go out as soon as each value is
// known, which suits a caller whose own stores are pending anyway.
template <bool kLate>
__device__ __forceinline__ void scan_counts(const Dims &d, int experts_per_rank,
                                            const LayoutLds &L, int32_t rank_sum, bool write,
                                            int32_t *__restrict__ cnt_ws,
                                            int32_t *__restrict__ num_tokens_per_expert,
                                            int32_t *__restrict__ num_tokens_per_rank,
                                            int32_t *__restrict__ rank_tok_off,
                                            int32_t *__restrict__ expert_offsets,
                                            int32_t *__restrict__ rank_offsets) {
  constexpr int kMaxG = EP_MAX_EXPERTS / kBlock;  // experts per thread, at most
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int E = d.E, R = d.R;
  // Counts of experts tid, tid + 256, ... (kept for the stores below), and
  // their aligned sizes in LDS.
  int32_t cnt[kMaxG];
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    const int e = tid + i * kBlock;
    cnt[i] = 0;
    if (e < E) {
      cnt[i] = L.counts[e];
      if (!kLate && write) {
        cnt_ws[e] = cnt[i];
        num_tokens_per_expert[e] = cnt[i];
      }
      L.counts[e] = d.A == 1 ? cnt[i] : (cnt[i] + d.A - 1) / d.A * d.A;
    }
  }
  // The first wave (R <= 64 lanes) scans the rank counts into the starts of
  // the ranks' token partitions (the non-expanded layout).
  int32_t rank_start = 0, rank_total = 0;
  if (write && wave == 0) {
    const int32_t v = lane < R ? rank_sum : 0;
    const int32_t inc = wave_inclusive_sum(v);
    rank_start = inc - v;
    rank_total = inc;
    if (!kLate) {
      if (lane < R) {
        num_tokens_per_rank[lane] = rank_sum;
        rank_tok_off[lane] = rank_start;
      }
      if (lane == R - 1) rank_tok_off[R] = rank_total;
    }
  }
  __syncthreads();

  // Exclusive scan of the aligned counts over experts: each thread owns a
  // run of G consecutive experts; runs are scanned across the wave with
  // shuffles and across the four waves through LDS.
  const int G = (E + kBlock - 1) / kBlock;
  const int e0 = tid * G;
  int32_t local = 0;
  for (int i = 0; i < G; ++i)
    if (e0 + i < E) local += L.counts[e0 + i];
  const int32_t incl = wave_inclusive_sum(local);
  if (lane == kWave - 1) L.wave_total[wave] = incl;
  __syncthreads();
  int32_t base = incl - local;
  for (int w = 0; w < wave; ++w) base += L.wave_total[w];
  int32_t total = 0;
  for (int w = 0; w < kWavesPerBlock; ++w) total += L.wave_total[w];
  int32_t off[kMaxG];
#pragma unroll
  for (int i = 0; i < kMaxG; ++i) {
    off[i] = base;
    if (i < G && e0 + i < E) {
      const int32_t a = L.counts[e0 + i];
      L.counts[e0 + i] = base;
      if (!kLate && write) expert_offsets[e0 + i] = base;
      base += a;
    }
  }
  if (tid == 0) {
    L.counts[E] = total;
    if (!kLate && write) expert_offsets[E] = total;
  }
  __syncthreads();
  if (!write) return;
  if (kLate) {
    if (tid == 0) expert_offsets[E] = total;
#pragma unroll
    for (int i = 0; i < kMaxG; ++i) {
      const int e = tid + i * kBlock;
      if (e < E) {
        cnt_ws[e] = cnt[i];
        num_tokens_per_expert[e] = cnt[i];
      }
      if (i < G && e0 + i < E) expert_offsets[e0 + i] = off[i];
    }
    if (tid < R) {
      num_tokens_per_rank[tid] = rank_sum;
      rank_tok_off[tid] = rank_start;
    }
    if (tid == R - 1) rank_tok_off[R] = rank_total;
  }
  if (tid <= R) rank_offsets[tid] = L.counts[tid * experts_per_rank];
}

// Scan phase for at most 256 experts (one per thread): thread tid holds
// expert tid's count in the batch in cnt and, for tid < R, rank tid's token
// count in rank_sum.  One barrier (the four waves' totals), then every
// store (none unless write).  Rank r's row range starts at the aligned
// offset of its first expert, e = r * (E / R), and the thread that owns that
// expert writes it.  With kKeep the aligned offsets are also left in
// L.counts[0..E), visible to the whole workgroup on return.
template <bool kKeep = false>
__device__ __forceinline__ void scan_small(const Dims &d, int experts_per_rank,
                                           const LayoutLds &L, int32_t cnt, int32_t rank_sum,
                                           bool write, int32_t *__restrict__ cnt_ws,
                                           int32_t *__restrict__ num_tokens_per_expert,
                                           int32_t *__restrict__ num_tokens_per_rank,
                                           int32_t *__restrict__ rank_tok_off,
                                           int32_t *__restrict__ expert_offsets,
                                           int32_t *__restrict__ rank_offsets) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int E = d.E, R = d.R;
  const int32_t size = tid < E ? (d.A == 1 ? cnt : (cnt + d.A - 1) / d.A * d.A) : 0;
  const int32_t incl = wave_inclusive_sum(size);
  if (lane == kWave - 1) L.wave_total[wave] = incl;
  int32_t rank_start = 0, rank_total = 0;
  if (wave == 0) {
    const int32_t v = lane < R ? rank_sum : 0;
    rank_total = wave_inclusive_sum(v);
    rank_start = rank_total - v;
  }
  __syncthreads();
  int32_t base = incl - size, total = 0;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) {
    const int32_t wt = L.wave_total[w];
    base += w < wave ? wt : 0;
    total += wt;
  }
  if (kKeep) {
    if (tid < E) L.counts[tid] = base;
    __syncthreads();
  }
  if (!write) return;
  if (tid < E) {
    cnt_ws[tid] = cnt;
    num_tokens_per_expert[tid] = cnt;
    expert_offsets[tid] = base;
    if (tid % experts_per_rank == 0) rank_offsets[tid / experts_per_rank] = base;
  }
  if (tid == 0) {
    expert_offsets[E] = total;
    rank_offsets[R] = total;
  }
  if (tid < R) {
    num_tokens_per_rank[tid] = rank_sum;
    rank_tok_off[tid] = rank_start;
  }
  if (tid == R - 1) rank_tok_off[R] = rank_total;
}

// Marks the workspace as written by a layout of this configuration.
__device__ __forceinline__ void write_header(int32_t *__restrict__ header, const Dims &d,
                                             int32_t ntiles) {
  header[1] = d.T;
  header[2] = d.k;
  header[3] = d.E;
  header[4] = d.R;
  header[5] = d.A;
  header[6] = ntiles;
  header[0] = kWorkspaceMagic;
}

// Word 3 of a raw buffer resource on this chip family (32-bit data format,
// no swizzle): loads past num_records return zero.
constexpr int32_t kBufferWord3 = 0x00020000;
// Cache-policy operand of a buffer load: the non-temporal (streaming) hint.
constexpr int kBufferNt = 2;
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resource over n bytes from p.  A load at an offset at or past n
// returns zeros (the hardware's range check) without touching memory, so a
// lane with nothing to load is given offset n and the load is still issued:
// it has no branch of its own, and the waits after it can count it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void *p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)n,
                                           kBufferWord3);
}

__device__ __forceinline__ int4 add4(int4 a, int4 b) {
  return make_int4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// Zero tile bases: the row of a batch's only tile.
__device__ __forceinline__ void zero_tile_row(const Dims &d, int32_t *__restrict__ rows) {
  const int C4 = tile_row_ints(d.E, d.R) / 4;
  for (int q = threadIdx.x; q < C4; q += kBlock)
    reinterpret_cast<int4 *>(rows)[q] = make_int4(0, 0, 0, 0);
}

// Quad q of this tile's row, from its counts in LDS (zeros in the padding).
// Both LDS arrays are 16-byte aligned, so a whole quad is one LDS read.
__device__ __forceinline__ int4 tile_row_quad(const Dims &d, const LayoutLds &L, int q) {
  const int Ep = tile_row_experts(d.E);
  const bool expert = 4 * q < Ep;
  const int32_t *src = expert ? L.counts : L.rank_cnt;
  const int c = expert ? 4 * q : 4 * q - Ep;
  const int n = expert ? d.E : d.R;
  if (c + 4 <= n) return *reinterpret_cast<const int4 *>(src + c);
  return make_int4(c < n ? src[c] : 0, c + 1 < n ? src[c + 1] : 0, c + 2 < n ? src[c + 2] : 0,
                   c + 3 < n ? src[c + 3] : 0);
}

// Quad q of tile row tt, or zero when tt is not below te.  The load itself
// is unconditional (from a row clamped into [0, te - 1], row 0 if te <= 0),
// so that a run of these issues every load before the first result is
// used: a load in a branch of its own gets its result copied, and so
// waited for, inside that branch.
__device__ __forceinline__ int4 row_quad_or_zero(const int4 *__restrict__ rows, int C4, int q,
                                                 int tt, int te) {
  const int4 v = rows[(int64_t)max(0, min(tt, te - 1)) * C4 + q];
  return tt < te ? v : make_int4(0, 0, 0, 0);
}

// Sum of quad q over tiles [tb, te), eight rows in flight at a time.
__device__ __forceinline__ int4 sum_quad(const int4 *__restrict__ rows, int C4, int q, int tb,
                                         int te) {
  int4 acc = make_int4(0, 0, 0, 0);
  for (int t0 = tb; t0 < te; t0 += 8) {
    int4 c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = row_quad_or_zero(rows, C4, q, t0 + i, te);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = add4(acc, c[i]);
  }
  return acc;
}

// Quad q of tiles [tb, te) replaced in place by its running sum from run
// (the exclusive prefix over the tiles), eight rows at a time: every load
// of a batch is issued before its stores.
__device__ __forceinline__ void quad_bases(int4 *__restrict__ rows, int C4, int q, int tb, int te,
                                           int4 run) {
  for (int t0 = tb; t0 < te; t0 += 8) {
    int4 c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = row_quad_or_zero(rows, C4, q, t0 + i, te);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (t0 + i < te) rows[(int64_t)(t0 + i) * C4 + q] = run;
      run = add4(run, c[i]);
    }
  }
}

// K is a compile-time bound on k (k <= K) so that a token's expert ids stay
// in registers between the marking pass and the ranking pass.  kRegs selects
// the scanner's read-back: 0 for the per-expert columns (at most 16 tiles of
// at most 256 experts), otherwise the number of tile-row quads a scanning
// thread holds in registers (the tiles of its slice; a slice longer than
// that is read twice).
template <int K, int kRegs>
__global__ __launch_bounds__(kBlock) void layout_kernel(
    const int32_t *__restrict__ topk_idx, Dims d, int32_t ntiles, int32_t experts_per_rank,
    int32_t *__restrict__ tile_rows, int32_t *__restrict__ slot_rank,
    uint8_t *__restrict__ is_token_in_rank, int32_t *__restrict__ cnt_ws,
    int32_t *__restrict__ num_tokens_per_expert, int32_t *__restrict__ num_tokens_per_rank,
    int32_t *__restrict__ expert_offsets, int32_t *__restrict__ rank_offsets,
    int32_t *__restrict__ header, unsigned long long *__restrict__ rank_ballot_ws,
    int32_t *__restrict__ rank_tok_off, int32_t *__restrict__ status) {
  extern __shared__ __align__(16) unsigned long long dyn_lds[];
  __shared__ __align__(16) int32_t rank_cnt[EP_MAX_RANKS];
  __shared__ int32_t wave_total[kWavesPerBlock];
  __shared__ int4 slice_total[kBlock + EP_MAX_RANKS / 4];
  __shared__ int is_last;
  const LayoutLds L = layout_lds(dyn_lds, d.E, rank_cnt, wave_total);
  const int tid = threadIdx.x;
  const int tile = blockIdx.x;
  const int E = d.E, R = d.R;
  const bool many = gridDim.x > 1;
  const bool has_tile = tile < ntiles;
  const int64_t t = (int64_t)tile * kTileTokens + tid;
  const bool live = has_tile && t < d.T;
  unsigned long long rmask = 0ull;
  int32_t ex[K];
  int4 *rows4 = reinterpret_cast<int4 *>(tile_rows);
  const TileGrid g = tile_grid(E, R, ntiles);

  if (has_tile) {
    load_ids<K>(d, t, live, topk_idx, ex);
    count_tile<K>(d, tile, experts_per_rank, L, ex, rmask, rank_ballot_ws, status);
  } else {
    // An empty batch: one workgroup writes zero counts and offsets.
    for (int e = tid; e < E; e += kBlock) L.counts[e] = 0;
    for (int i = tid; i < R; i += kBlock) L.rank_cnt[i] = 0;
  }
  __syncthreads();

  // With several tiles the first wave publishes the tile's row of counts
  // for the scan and draws a ticket; the workgroup that draws the last one
  // scans.  The publishing wave issues a device-scope release fence after
  // all of its row stores and before its (relaxed) ticket increment; the
  // thread that draws the last ticket issues a device-scope acquire fence
  // after its increment, before the barrier that tells the rest of its
  // workgroup.  The increments form one modification order, so each
  // publisher's release fence synchronises with that acquire fence, and
  // every tile's counts happen before the scan.  One wave stores the whole
  // row, so the release covers stores of its own instruction stream only,
  // and it is issued once per workgroup.
  if (many) {
    if (tid < kWave) {
      for (int q = tid; q < g.C4; q += kWave)
        rows4[(int64_t)tile * g.C4 + q] = tile_row_quad(d, L, q);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      if (tid == 0) {
        const bool last = __hip_atomic_fetch_add(&header[kHeaderTicket], 1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT) ==
                          (int)gridDim.x - 1;
        if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        is_last = last;
      }
    }
    __syncthreads();
  }
  const bool scans = !many || is_last;

  // The scanner reads the tile rows back in one of two ways.  Up to
  // kColumnTiles tiles of at most 256 experts (the kRegs = 0 kernel),
  // thread e holds its expert's
  // column (and thread r < R its rank's) in registers, one word per tile:
  // the totals need no exchange between threads.  Otherwise it reads them
  // by column quads, 16 bytes per load: thread (q, s) takes quad q of the
  // tiles of slice s (see TileGrid), and holds them in registers when the
  // slice fits.  Each wave issues its own acquire fence before its loads, so
  // that none of them can be served from a cached copy older than the
  // scanner's acquire.
  constexpr int kColumnTiles = 16;
  const int Ep = tile_row_experts(E), C = 4 * g.C4;
  constexpr bool kColumns = kRegs == 0;
  const bool by_column = kColumns && many;
  int32_t col[kColumnTiles], rcol[kColumnTiles];
#pragma unroll
  for (int b = 0; b < kColumnTiles; ++b) col[b] = rcol[b] = 0;
  const bool wide = g.C4 > kBlock;
  const int q0 = wide ? tid : tid % g.C4;
  const int s = wide ? 0 : tid / g.C4;
  const bool owner = s < g.S;
  const int tb = s * g.per;
  const int te = min(ntiles, tb + g.per);
  const bool in_regs = !kColumns && !wide && g.per <= kRegs;
  constexpr int kQuads = kColumns ? 1 : kRegs;
  int4 v[kQuads];
#pragma unroll
  for (int i = 0; i < kQuads; ++i) v[i] = make_int4(0, 0, 0, 0);
  if (many && scans) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (by_column) {
      if (tid < E) {
#pragma unroll
        for (int b = 0; b < kColumnTiles; ++b) {
          if (b < ntiles) {
            col[b] = tile_rows[(int64_t)b * C + tid];
            if (tid < R) rcol[b] = tile_rows[(int64_t)b * C + Ep + tid];
          }
        }
      }
    } else if (in_regs) {
      // Buffer loads, whose hardware range check returns zeros for an
      // offset at or past the end: a row outside the thread's slice is
      // given that offset, so every load is issued unconditionally and none
      // waits inside a branch of its own.  Here ntiles <= 24 * 256, so the
      // rows' bytes fit the 32-bit range.
      const uint32_t nbytes = (uint32_t)ntiles * (uint32_t)g.C4 * 16u;
      const __amdgpu_buffer_rsrc_t rsrc =
          __builtin_amdgcn_make_buffer_rsrc(tile_rows, (short)0, (int)nbytes, kBufferWord3);
#pragma unroll
      for (int i = 0; i < kQuads; ++i) {
        const int tt = tb + i;
        const uint32_t off =
            owner && tt < te ? ((uint32_t)tt * (uint32_t)g.C4 + (uint32_t)q0) * 16u : nbytes;
        const i32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off, 0, 0);
        v[i] = make_int4(w.x, w.y, w.z, w.w);
      }
    }
  }

  // The other workgroups write their per-token outputs after the ticket:
  // stores issued before the publishing wave's release would be written
  // back by it too, and delay the ticket.
  if (!scans) {
    if (live) token_outputs<K>(d, t, L, ex, rmask, is_token_in_rank, slot_rank);
    return;
  }

  // Column totals: each owner sums its quads over its slice, the slice
  // totals meet in LDS, and thread e < E (r < R) adds up column e (rank
  // column r) over the slices.  A single workgroup already holds its counts.
  int32_t rank_sum = 0, batch_cnt = 0;
  int4 base = make_int4(0, 0, 0, 0);
  if (by_column) {
#pragma unroll
    for (int b = 0; b < kColumnTiles; ++b) {
      batch_cnt += col[b];
      rank_sum += rcol[b];
    }
    scan_small(d, experts_per_rank, L, batch_cnt, rank_sum, true, cnt_ws,
               num_tokens_per_expert, num_tokens_per_rank, rank_tok_off, expert_offsets,
               rank_offsets);
  } else if (!kColumns && many) {
    if (owner) {
      int4 tot = make_int4(0, 0, 0, 0);
      if (in_regs) {
#pragma unroll
        for (int i = 0; i < kQuads; ++i) tot = add4(tot, v[i]);
      } else {
        tot = sum_quad(rows4, g.C4, q0, tb, te);
        if (wide && q0 + kBlock < g.C4)
          slice_total[q0 + kBlock] = sum_quad(rows4, g.C4, q0 + kBlock, tb, te);
      }
      slice_total[s * g.C4 + q0] = tot;
    }
    __syncthreads();
    if (owner)
      for (int ss = 0; ss < s; ++ss) base = add4(base, slice_total[ss * g.C4 + q0]);
    const int32_t *st = reinterpret_cast<const int32_t *>(slice_total);
    if (E <= kBlock) {
      if (tid < E)
        for (int ss = 0; ss < g.S; ++ss) batch_cnt += st[ss * C + tid];
      if (tid < R)
        for (int ss = 0; ss < g.S; ++ss) rank_sum += st[ss * C + Ep + tid];
      scan_small(d, experts_per_rank, L, batch_cnt, rank_sum, true, cnt_ws,
                 num_tokens_per_expert, num_tokens_per_rank, rank_tok_off, expert_offsets,
                 rank_offsets);
    } else {
      for (int e = tid; e < E; e += kBlock) {
        int32_t sum = 0;
        for (int ss = 0; ss < g.S; ++ss) sum += st[ss * C + e];
        L.counts[e] = sum;
      }
      if (tid < R)
        for (int ss = 0; ss < g.S; ++ss) rank_sum += st[ss * C + Ep + tid];
      scan_counts<false>(d, experts_per_rank, L, rank_sum, true, cnt_ws, num_tokens_per_expert,
                         num_tokens_per_rank, rank_tok_off, expert_offsets, rank_offsets);
    }
  } else {
    if (ntiles > 0) zero_tile_row(d, tile_rows);
    if (tid < E) batch_cnt = L.counts[tid];
    if (tid < R) rank_sum = L.rank_cnt[tid];
    if (E <= kBlock)
      scan_small(d, experts_per_rank, L, batch_cnt, rank_sum, true, cnt_ws,
                 num_tokens_per_expert, num_tokens_per_rank, rank_tok_off, expert_offsets,
                 rank_offsets);
    else
      scan_counts<false>(d, experts_per_rank, L, rank_sum, true, cnt_ws, num_tokens_per_expert,
                         num_tokens_per_rank, rank_tok_off, expert_offsets, rank_offsets);
  }

  // Every store of the scanner comes after its scan (loads and stores share
  // one wait counter on this chip, so an earlier store could hold up the
  // scan's loads): its own per-token outputs, then the tile bases, written
  // over the counts as each quad's running sum over the tiles from its
  // slice's base.
  if (live) token_outputs<K>(d, t, L, ex, rmask, is_token_in_rank, slot_rank);
  if (by_column) {
    if (tid < E) {
      int32_t run = 0, rank_run = 0;
#pragma unroll
      for (int b = 0; b < kColumnTiles; ++b) {
        if (b < ntiles) {
          tile_rows[(int64_t)b * C + tid] = run;
          if (tid < R) tile_rows[(int64_t)b * C + Ep + tid] = rank_run;
        }
        run += col[b];
        rank_run += rcol[b];
      }
    }
  } else if (!kColumns && many && owner) {
    if (in_regs) {
      int4 run = base;
#pragma unroll
      for (int i = 0; i < kQuads; ++i)
        if (tb + i < te) {
          rows4[(int64_t)(tb + i) * g.C4 + q0] = run;
          run = add4(run, v[i]);
        }
    } else {
      quad_bases(rows4, g.C4, q0, tb, te, base);
      if (wide && q0 + kBlock < g.C4)
        quad_bases(rows4, g.C4, q0 + kBlock, tb, te, make_int4(0, 0, 0, 0));
    }
  }
  if (tid == 0) {
    write_header(header, d, ntiles);
    if (many) atomicExch(&header[kHeaderTicket], 0);
  }
}

// Zeroes the workspace header (magic and ticket) once, before first use.
__global__ void workspace_init_kernel(int32_t *__restrict__ header) {
  if (threadIdx.x < kHeaderInts) header[threadIdx.x] = 0;
}

// ---------------------------------------------------------------------------
// Dispatch ("GPU microarchitecture: DeepEP first principles", 1.1 and 6.1;
// "Deep Dive - DeepEP", "Dispatch: layout, move, and epilogue")
// ---------------------------------------------------------------------------

// A selection's inputs to its receive row, for lanes below k: its expert id,
// the layout's slot word and (for the handle) its gate, loaded together by
// buffer loads over the token's k entries (zeros on the other lanes, and for
// the gate when it is not wanted).
struct SlotIn {
  int32_t e, w;
  float gate;
};

__device__ __forceinline__ SlotIn load_slot(const Dims &d, int64_t t, int lane, bool want_gate,
                                            const int32_t *__restrict__ topk_idx,
                                            const float *__restrict__ topk_weights,
                                            const int32_t *__restrict__ slot_rank) {
  const uint32_t n = (uint32_t)d.k * 4u;
  const uint32_t off = lane < d.k ? (uint32_t)lane * 4u : n;
  const int64_t s0 = t * d.k;
  const bool g = want_gate && topk_weights != nullptr;
  const void *gp = g ? static_cast<const void *>(topk_weights + s0)
                     : static_cast<const void *>(topk_idx + s0);
  SlotIn in;
  in.e = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(buffer_over(topk_idx + s0, n), (int)off,
                                                       0, 0);
  in.w = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(buffer_over(slot_rank + s0, n), (int)off,
                                                       0, 0);
  in.gate = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(buffer_over(gp, g ? n : 0u), (int)off, 0, 0));
  return in;
}

// The checks on a selection's inputs, as values of the whole wave (not
// branches, so that the loads of `in` are not moved into a branch, where
// their wait would also wait for every load issued before them).  act: a
// lane below k of a workspace that passed its header check (ok).  The
// layout's slot word must name the same expert (or both must leave the slot
// out): otherwise the route is not the layout's (mismatch).  use: a valid
// selection with a matching slot word, which gets a row.  A valid
// selection's gate must be finite ("Deep Dive - DeepEP", "A runnable
// routing ledger").
struct SlotCheck {
  bool act, use, mismatch, nonfinite;
};

__device__ __forceinline__ SlotCheck check_slot(const Dims &d, int lane, const SlotIn &in, bool ok,
                                                bool gates) {
  SlotCheck c;
  c.act = ok && lane < d.k;
  const bool valid = c.act && in.e >= 0 && in.e < d.E;
  const bool slotted = c.act && in.w >= 0;
  c.mismatch = valid != slotted || (valid && (in.w >> kSlotExpertShift) != in.e);
  c.use = valid && !c.mismatch;
  c.nonfinite = gates && valid && !__builtin_isfinite(in.gate);
  return c;
}

// The handle of selection (t, lane): its row, and for a row the source
// selection and (with gates) the gate.
__device__ __forceinline__ void write_handle_entry(const Dims &d, int64_t t, int lane,
                                                   int32_t row, float gate, bool gates,
                                                   float *__restrict__ recv_weights,
                                                   int32_t *__restrict__ tok_slot_row,
                                                   int32_t *__restrict__ row_src) {
  const int64_t s = t * d.k + lane;
  tok_slot_row[s] = row;
  if (row >= 0) {
    row_src[row] = (int32_t)s;
    if (gates && recv_weights != nullptr) recv_weights[row] = gate;
  }
}

// A selection's receive row is the expert's segment start, plus the
// selections of e in earlier tiles (the tile base), plus its rank inside
// the tile: the stable counting-sort position.  The first two come by
// buffer loads, issued whatever the lane (zeros, and no memory access, for
// a selection check_slot did not accept), so that they have no branch of
// their own; the caller adds them up as late as it can.
struct RowBase {
  int32_t start, base;
};

__device__ __forceinline__ RowBase load_row_base(const Dims &d, int64_t t, int32_t e, bool use,
                                                 const int32_t *__restrict__ expert_offsets,
                                                 const int32_t *__restrict__ tile_base) {
  const uint32_t nb = (uint32_t)d.E * 4u;
  const int eo = (int)(use ? (uint32_t)e * 4u : nb);
  const int32_t *trow = tile_base + (t / kTileTokens) * tile_row_ints(d.E, d.R);
  RowBase b;
  b.start = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(buffer_over(expert_offsets, nb), eo, 0, 0);
  b.base = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(buffer_over(trow, nb), eo, 0, 0);
  return b;
}

// The row from its base and the slot word's in-tile rank: -1 for a
// selection not accepted or past the capacity (fits false).
__device__ __forceinline__ int32_t row_from_base(const RowBase &b, int32_t w, bool use,
                                                 int64_t capacity, bool &fits) {
  const int64_t r = (int64_t)b.start + b.base + (w & kSlotRankMask);
  fits = r >= 0 && r < capacity;
  return use && fits ? (int32_t)r : -1;
}

// A selection's status bits, raised after its stores.
__device__ __forceinline__ void report_slot(const SlotCheck &c, bool fits, int32_t *status) {
  if (c.use && !fits) flag(status, EP_STATUS_BIT_CAPACITY);
  if (c.mismatch) flag(status, EP_STATUS_BIT_WORKSPACE);
  if (c.nonfinite) flag(status, EP_STATUS_BIT_NONFINITE);
}

// Largest magnitude of the 16 bf16 values of v0 and v1, as bf16 bits with
// the sign cleared.  For finite values the integer order of these bits is
// the order of the magnitudes, and an infinity (0x7F80) or a NaN (above it)
// sorts above every finite value: one compare of the result with 0x7F80
// tells whether all 16 values are finite.  Packed 16-bit maxima, two values
// per instruction.
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2_t magnitudes(uint32_t w) {
  return __builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu);
}

__device__ __forceinline__ uint32_t absmax_bits16(const uint4 v0, const uint4 v1) {
  u16x2_t m = __builtin_elementwise_max(magnitudes(v0.x), magnitudes(v0.y));
  m = __builtin_elementwise_max(m, magnitudes(v0.z));
  m = __builtin_elementwise_max(m, magnitudes(v0.w));
  m = __builtin_elementwise_max(m, magnitudes(v1.x));
  m = __builtin_elementwise_max(m, magnitudes(v1.y));
  m = __builtin_elementwise_max(m, magnitudes(v1.z));
  m = __builtin_elementwise_max(m, magnitudes(v1.w));
  return m.x > m.y ? m.x : m.y;
}

constexpr uint32_t kBf16Inf = 0x7F80u;  // magnitude bits of an infinity

// A hidden value that is an infinity or NaN is an error at the boundary
// ("Deep Dive - DeepEP", "A runnable routing ledger": a row that is not
// finite is rejected): the wave reports it once in the status word.
__device__ __forceinline__ void report_nonfinite(bool bad, int lane, int32_t *status) {
  if (__ballot(bad) != 0ull && lane == 0) flag(status, EP_STATUS_BIT_NONFINITE);
}

// FP8 rows: per token and 128-value block, amax over the block, scale =
// amax / 448 and codes = E4M3(x / scale), both rounded to nearest even
// ("Deep Dive - DeepEP", "Precision: FP8 on the wire, BF16 for the
// reduction").  An all-zero block gets scale 0 and zero codes.

// Eight bf16 values divided by s (correctly rounded fp32 division) and
// converted to E4M3 with round to nearest even, packed little-endian.
__device__ __forceinline__ uint2 quantize8(const uint4 v, float s) {
  int lo = 0, hi = 0;
  if (s > 0.0f) {
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(v.x) / s, bf16_hi(v.x) / s, lo, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(v.y) / s, bf16_hi(v.y) / s, lo, true);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(v.z) / s, bf16_hi(v.z) / s, hi, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(v.w) / s, bf16_hi(v.w) / s, hi, true);
  }
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// The 16 values a lane owns (v0 then v1) as E4M3 codes, with the scale of
// their 128-value block: the amax is taken over the block's 8 lanes, which
// must all call this together.  finite is false when the block holds an
// infinity or NaN (its scale and codes are then meaningless).
__device__ __forceinline__ uint4 quantize16(const uint4 v0, const uint4 v1, float &scale,
                                            bool &finite) {
  uint32_t mbits = absmax_bits16(v0, v1);
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) mbits = max(mbits, (uint32_t)__shfl_xor((int)mbits, m));
  finite = mbits < kBf16Inf;
  scale = __uint_as_float(mbits << 16) / 448.0f;
  const uint2 q0 = quantize8(v0, scale);
  const uint2 q1 = quantize8(v1, scale);
  return make_uint4(q0.x, q0.y, q1.x, q1.y);
}

// One dispatch work item's slice of x (token t, 1024-column chunk): 16 bf16
// values per lane in two 16-byte loads.  bf16 rows take columns
// c + lane * 8 and c + 512 + lane * 8; FP8 rows take the 16 consecutive
// columns c + lane * 16, so that 8 lanes hold one 128-value block.
struct XSlice {
  uint4 v[2];
};

template <bool kFp8>
__device__ __forceinline__ int slice_col(int chunk, int lane, int u) {
  return kFp8 ? chunk * kChunkCols + lane * 16 + u * 8
              : chunk * kChunkCols + u * (kWave * 8) + lane * 8;
}

template <bool kFp8>
__device__ __forceinline__ XSlice load_x_slice(const uint16_t *__restrict__ x, int64_t t,
                                               int64_t H, int chunk, int lane,
                                               bool live = true) {
  // Buffer loads over the token's row: a part past its end reads zeros, and
  // so does every part when live is false (an empty buffer).
  const uint32_t n = live ? (uint32_t)H * 2u : 0u;
  const __amdgpu_buffer_rsrc_t rsrc = buffer_over(x + (live ? t : 0) * H, n);
  XSlice xs;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    // FP8 needs H % 128 == 0, so the 8 lanes of a block are all in range or
    // all out; bf16 guards each 8-column part.
    const int col = slice_col<kFp8>(chunk, lane, u);
    const bool in = kFp8 ? slice_col<kFp8>(chunk, lane, 0) < H : col < H;
    const uint32_t off = in ? (uint32_t)col * 2u : n;
    const i32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off, 0, 0);
    xs.v[u] = make_uint4((uint32_t)w.x, (uint32_t)w.y, (uint32_t)w.z, (uint32_t)w.w);
  }
  return xs;
}

// The slice as stored: E4M3 codes in v[0] plus the block's scale, or the
// bf16 bits as loaded.  finite is false when one of its hidden values is an
// infinity or NaN.
struct XOut {
  uint4 v[2];
  float scale;
  bool finite;
};

template <bool kFp8>
__device__ __forceinline__ XOut encode_slice(const XSlice &xs) {
  XOut o;
  if (kFp8) {
    o.v[0] = quantize16(xs.v[0], xs.v[1], o.scale, o.finite);
    o.v[1] = o.v[0];
  } else {
    // lanes past the row's end hold zeros, which are finite
    o.v[0] = xs.v[0];
    o.v[1] = xs.v[1];
    o.scale = 0.0f;
    o.finite = absmax_bits16(xs.v[0], xs.v[1]) < kBf16Inf;
  }
  return o;
}

// Stores the encoded slice to each of the token's receive rows (lane j
// holds the row of slot j, -1 for none): bf16 bits, or E4M3 codes plus one
// scale per 128-value block.  One 16-byte non-temporal store per lane per
// row part.
template <bool kFp8>
__device__ __forceinline__ void store_slice(const XOut &o, int32_t row, int k, int64_t H,
                                            int chunk, int lane, void *__restrict__ recv_x,
                                            float *__restrict__ recv_scales) {
  if (kFp8) {
    const int col = slice_col<true>(chunk, lane, 0);
    const bool in = col < H;
    const int64_t nblk = H / 128;
    for (int j = 0; j < k; ++j) {
      const int32_t r = lane_value(row, j);
      if (r < 0 || !in) continue;
      store_stream(static_cast<uint8_t *>(recv_x) + (int64_t)r * H + col, o.v[0]);
      if ((lane & 7) == 0) recv_scales[(int64_t)r * nblk + col / 128] = o.scale;
    }
  } else {
    for (int j = 0; j < k; ++j) {
      const int32_t r = lane_value(row, j);
      if (r < 0) continue;
      uint16_t *dst = static_cast<uint16_t *>(recv_x) + (int64_t)r * H;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int col = slice_col<false>(chunk, lane, u);
        if (col < H) store_stream(dst + col, o.v[u]);
      }
    }
  }
}

// Encodes and stores the slice, reporting a non-finite hidden value.
template <bool kFp8>
__device__ __forceinline__ void store_x_slice(const XSlice &xs, int32_t row, int k, int64_t H,
                                              int chunk, int lane, void *__restrict__ recv_x,
                                              float *__restrict__ recv_scales,
                                              int32_t *__restrict__ status) {
  const XOut o = encode_slice<kFp8>(xs);
  report_nonfinite(!o.finite, lane, status);
  store_slice<kFp8>(o, row, k, H, chunk, lane, recv_x, recv_scales);
}

// One wave per (token, 1024-column chunk): the selection rows, then the x
// slice to each of them (bf16 bit copy, or fused FP8 quantisation).
//
// Every load is issued before the first wait, in one straight line: the
// selection's id, slot word and gate first, then the x slice, then (once the
// ids are in) the segment start and tile base, by buffer loads whose lanes
// without a row read zeros.  Loads return in issue order, so the wait for
// the ids does not include x, the second link of the row chain overlaps the
// x loads, and the FP8 encoding overlaps that link.  The status bits are
// raised after the stores.  The loads before the header check stay in
// bounds whatever the header says (the host has checked that the workspace
// holds this configuration's arrays), and a failed check gives every
// selection no row.
template <bool kFp8>
__global__ __launch_bounds__(kBlock) void dispatch_kernel(
    Dims d, int32_t nchunks, const uint16_t *__restrict__ x, const int32_t *__restrict__ topk_idx,
    const float *__restrict__ topk_weights, const int32_t *__restrict__ expert_offsets,
    const int32_t *__restrict__ header, const int32_t *__restrict__ tile_base,
    const int32_t *__restrict__ slot_rank, int64_t capacity, void *__restrict__ recv_x,
    float *__restrict__ recv_scales, float *__restrict__ recv_weights,
    int32_t *__restrict__ tok_slot_row, int32_t *__restrict__ row_src,
    int32_t *__restrict__ status) {
  const int lane = threadIdx.x & (kWave - 1);
  const int item = uniform(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave);
  if (item >= d.T * nchunks) return;
  const int64_t t = item / nchunks;
  const int chunk = item - (int)t * nchunks;
  const bool gates = chunk == 0 && topk_weights != nullptr;
  const SlotIn in = load_slot(d, t, lane, gates, topk_idx, topk_weights, slot_rank);
  const XSlice xs = load_x_slice<kFp8>(x, t, d.H, chunk, lane);
  const bool ok = workspace_ok(header, d);
  const SlotCheck c = check_slot(d, lane, in, ok, gates);
  const RowBase b = load_row_base(d, t, in.e, c.use, expert_offsets, tile_base);
  const XOut o = encode_slice<kFp8>(xs);
  bool fits;
  const int32_t row = row_from_base(b, in.w, c.use, capacity, fits);
  store_slice<kFp8>(o, row, d.k, d.H, chunk, lane, recv_x, recv_scales);
  if (chunk == 0 && c.act)
    write_handle_entry(d, t, lane, row, in.gate, gates, recv_weights, tok_slot_row, row_src);
  if (!ok && lane == 0) flag(status, EP_STATUS_BIT_WORKSPACE);
  report_slot(c, fits, status);
  report_nonfinite(ok && !o.finite, lane, status);
}

// Layout and dispatch in one launch, for a batch of at most one tile (256
// tokens): count, prefix sum and scatter in a single pass ("GPU
// microarchitecture: DeepEP first principles", 6.1).  Every workgroup counts
// and scans the whole batch in LDS.  Workgroup 0 then writes every layout
// output and the workspace, so later calls (combine, the non-expanded path,
// backward) see exactly what ep_get_dispatch_layout and ep_dispatch leave;
// each other workgroup moves its four work items (token, 1024-column chunk)
// to the rows the scan gives.  The x slice and the token's expert ids are loaded
// first, so their loads overlap the count.
template <int K, bool kFp8>
__global__ __launch_bounds__(kBlock) void layout_dispatch_kernel(
    const int32_t *__restrict__ topk_idx, Dims d, int32_t ntiles, int32_t experts_per_rank,
    int32_t nchunks, const uint16_t *__restrict__ x, const float *__restrict__ topk_weights,
    int32_t *__restrict__ tile_cnt, int32_t *__restrict__ slot_rank,
    uint8_t *__restrict__ is_token_in_rank,
    int32_t *__restrict__ cnt_ws, int32_t *__restrict__ num_tokens_per_expert,
    int32_t *__restrict__ num_tokens_per_rank, int32_t *__restrict__ expert_offsets,
    int32_t *__restrict__ rank_offsets, int32_t *__restrict__ header,
    unsigned long long *__restrict__ rank_ballot_ws, int32_t *__restrict__ rank_tok_off,
    int64_t capacity, void *__restrict__ recv_x, float *__restrict__ recv_scales,
    float *__restrict__ recv_weights, int32_t *__restrict__ tok_slot_row,
    int32_t *__restrict__ row_src, int32_t *__restrict__ status) {
  extern __shared__ __align__(16) unsigned long long dyn_lds[];
  __shared__ __align__(16) int32_t rank_cnt[EP_MAX_RANKS];
  __shared__ int32_t wave_total[kWavesPerBlock];
  const LayoutLds L = layout_lds(dyn_lds, d.E, rank_cnt, wave_total);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const bool lead = blockIdx.x == 0;
  const int64_t t = tid;  // the batch is tile 0: thread = token
  const bool live = ntiles > 0 && t < d.T;

  // This wave's work item, its x slice and its token's expert ids.
  // Workgroup 0 moves no rows: its layout writes then delay no dispatch work.
  const int64_t item =
      lead ? 0 : ((int64_t)blockIdx.x - 1) * kWavesPerBlock + uniform(tid / kWave);
  const bool has_item = !lead && item < (int64_t)d.T * nchunks;
  const int64_t ti = has_item ? item / nchunks : 0;
  const int chunk = has_item ? (int)(item - ti * nchunks) : 0;
  // The count waits on the batch's ids, so they are loaded first; then the
  // x slice, the item token's ids and (for the handle) its gate, by buffer
  // loads issued whatever the wave (an empty buffer when it has no item), so
  // that the count's wait for the ids counts the later loads and leaves
  // them in flight (loads return in issue order; in a branch they made the
  // compiler wait for all of them).  The gate is loaded here too: a
  // load issued after the handle's stores would make the wave wait for those
  // stores before its row stores.
  int32_t ex[K];
  load_ids<K>(d, t, live, topk_idx, ex);
  const XSlice xs = load_x_slice<kFp8>(x, ti, d.H, chunk, lane, has_item);
  const uint32_t nki = has_item ? (uint32_t)d.k * 4u : 0u;
  const int koff = (int)(lane < d.k ? (uint32_t)lane * 4u : nki);
  const int32_t eid_l = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
      buffer_over(topk_idx + ti * d.k, nki), koff, 0, 0);
  const bool gates = has_item && chunk == 0 && topk_weights != nullptr;
  const float gate = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(
                 buffer_over(gates ? static_cast<const void *>(topk_weights + ti * d.k)
                                   : static_cast<const void *>(topk_idx),
                             gates ? nki : 0u),
                 koff, 0, 0));
  const int32_t eid = has_item && lane < d.k ? eid_l : -1;

  // Every workgroup counts, also for an empty batch (no live token: zero
  // counts, and no ballots, for which the workspace then has no room).  A
  // branch around the count would leave the id loads pending on one path,
  // and the compiler would then wait for all stores issued before the
  // first later use of those registers.
  unsigned long long rmask = 0ull;
  count_tile<K>(d, 0, experts_per_rank, L, ex, rmask,
                lead && ntiles > 0 ? rank_ballot_ws : nullptr, lead ? status : nullptr);
  __syncthreads();
  if (lead && live) token_outputs<K>(d, t, L, ex, rmask, is_token_in_rank, slot_rank);
  if (d.E <= kBlock)
    scan_small<true>(d, experts_per_rank, L, tid < d.E ? L.counts[tid] : 0,
                     tid < d.R ? L.rank_cnt[tid] : 0, lead, cnt_ws, num_tokens_per_expert,
                     num_tokens_per_rank, rank_tok_off, expert_offsets, rank_offsets);
  else
    scan_counts<true>(d, experts_per_rank, L, tid < d.R ? L.rank_cnt[tid] : 0, lead, cnt_ws,
                      num_tokens_per_expert, num_tokens_per_rank, rank_tok_off, expert_offsets,
                      rank_offsets);
  if (lead) {
    // One tile: its bases are zero.
    if (ntiles > 0) zero_tile_row(d, tile_cnt);
    if (tid == 0) write_header(header, d, ntiles);
  }
  if (!has_item) return;

  // Receive rows of the token's selections: segment start plus the stable
  // rank inside the batch, as the dispatch kernels give them.
  int32_t row = -1;
  if (lane < d.k) {
    if (eid >= 0 && eid < d.E) {
      const int64_t r = (int64_t)L.counts[eid] +
                        tile_rank(L, d.E, (int)(ti / kWave), (int)(ti % kWave), eid);
      if (r < capacity)
        row = (int32_t)r;
      else
        flag(status, EP_STATUS_BIT_CAPACITY);
    }
    if (chunk == 0) {
      const int64_t sidx = ti * d.k + lane;
      if (eid >= 0 && eid < d.E && !__builtin_isfinite(gate))
        flag(status, EP_STATUS_BIT_NONFINITE);
      tok_slot_row[sidx] = row;
      if (row >= 0) {
        row_src[row] = (int32_t)sidx;
        if (recv_weights != nullptr && topk_weights != nullptr) recv_weights[row] = gate;
      }
    }
  }
  store_x_slice<kFp8>(xs, row, d.k, d.H, chunk, lane, recv_x, recv_scales, status);
}

// Pre-quantised rows ("Deep Dive - DeepEP", "Dispatch: layout, move, and
// epilogue": hidden states may arrive as FP8 values plus scale factors):
// the token's E4M3 codes and per-128 scales are copied unchanged to each of
// its receive rows.  Each lane moves 16 code bytes (a block is 8 lanes).
__global__ __launch_bounds__(kBlock) void dispatch_fp8_input_kernel(
    Dims d, int32_t nchunks, const uint8_t *__restrict__ x_codes,
    const float *__restrict__ x_scales, const int32_t *__restrict__ topk_idx,
    const float *__restrict__ topk_weights, const int32_t *__restrict__ expert_offsets,
    const int32_t *__restrict__ header, const int32_t *__restrict__ tile_base,
    const int32_t *__restrict__ slot_rank, int64_t capacity, uint8_t *__restrict__ recv_x,
    float *__restrict__ recv_scales, float *__restrict__ recv_weights,
    int32_t *__restrict__ tok_slot_row, int32_t *__restrict__ row_src,
    int32_t *__restrict__ status) {
  const int lane = threadIdx.x & (kWave - 1);
  const int item = uniform(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave);
  if (item >= d.T * nchunks) return;
  const int64_t t = item / nchunks;
  const int chunk = item - (int)t * nchunks;
  // The loads in one straight line: the codes and the block scale (buffer
  // loads: zeros past the row's end, and the scale only on a block's first
  // lane), the ids and slot words, then the segment start and tile base.
  // (Codes first measured a little faster here than ids first; with no
  // encoding to overlap, the second link has nothing to hide behind.)  The
  // codes are used only in the store loop, and the compiler would otherwise
  // place their loads there, after the row chain: their pointers are made
  // opaque (so that the loads cannot be taken for reads of constant memory,
  // which may be placed anywhere), and an empty asm statement that clobbers
  // memory and takes the ids and slot words follows the loads, so that what
  // is computed from the ids stays after them.
  asm volatile("" : "+s"(x_codes), "+s"(x_scales));
  const bool gates = chunk == 0 && topk_weights != nullptr;
  const int64_t H = d.H;
  const int64_t nblk = H / 128;
  const int col = chunk * kChunkCols + lane * 16;
  const bool live = col < H;
  const uint32_t nq = (uint32_t)H;
  const uint32_t ns = (uint32_t)nblk * 4u;
  const i32x4_t qw = __builtin_amdgcn_raw_buffer_load_b128(buffer_over(x_codes + t * H, nq),
                                                           (int)(live ? (uint32_t)col : nq), 0, 0);
  const float scale = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(
                 buffer_over(x_scales + t * nblk, ns),
                 (int)(live && (lane & 7) == 0 ? (uint32_t)(col / 128) * 4u : ns), 0, 0));
  SlotIn in = load_slot(d, t, lane, gates, topk_idx, topk_weights, slot_rank);
  const bool ok = workspace_ok(header, d);
  asm volatile("" : "+v"(in.e), "+v"(in.w)::"memory");
  const SlotCheck c = check_slot(d, lane, in, ok, gates);
  const RowBase b = load_row_base(d, t, in.e, c.use, expert_offsets, tile_base);
  const uint4 q = make_uint4((uint32_t)qw.x, (uint32_t)qw.y, (uint32_t)qw.z, (uint32_t)qw.w);
  bool fits;
  const int32_t row = row_from_base(b, in.w, c.use, capacity, fits);
  for (int j = 0; j < d.k; ++j) {
    const int32_t r = lane_value(row, j);
    if (r < 0 || !live) continue;
    store_stream(recv_x + (int64_t)r * H + col, q);
    if ((lane & 7) == 0) recv_scales[(int64_t)r * nblk + col / 128] = scale;
  }
  if (chunk == 0 && c.act)
    write_handle_entry(d, t, lane, row, in.gate, gates, recv_weights, tok_slot_row, row_src);
  if (!ok && lane == 0) flag(status, EP_STATUS_BIT_WORKSPACE);
  report_slot(c, fits, status);
}

// Alignment padding rows of expert e: no source, zero gate and, with
// zero_padding, zero payload and zero scales ("Deep Dive - DeepEP",
// "Dispatch: layout, move, and epilogue": padding is not a token, and
// clearing its payload is the caller's choice).  Expert e's rows are split
// over kPadSplit workgroups (blockIdx.y strides the rows), so that the fill
// keeps the chip busy.  The workspace must hold a layout of this
// configuration (else nothing is written and the workspace bit is set), and
// the rows written stay inside [expert_offsets[e], expert_offsets[e+1]) and
// below capacity whatever the counts hold.
constexpr int kPadSplit = 8;

__global__ __launch_bounds__(kBlock) void pad_fill_kernel(
    Dims d, bool fp8, bool zero_payload, const int32_t *__restrict__ header,
    const int32_t *__restrict__ expert_offsets, const int32_t *__restrict__ cnt, int64_t capacity,
    void *__restrict__ recv_x, float *__restrict__ recv_scales, float *__restrict__ recv_weights,
    int32_t *__restrict__ row_src, int32_t *__restrict__ status) {
  if (!workspace_ok(header, d)) {
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
      flag(status, EP_STATUS_BIT_WORKSPACE);
    return;
  }
  const int e = blockIdx.x;
  const int64_t start = expert_offsets[e];
  int64_t last = expert_offsets[e + 1];
  if (last > capacity) last = capacity;
  const int32_t c = cnt[e];
  if (start < 0 || c < 0) return;
  const int64_t first = start + c;
  const int64_t row_bytes = fp8 ? (int64_t)d.H : (int64_t)d.H * 2;
  const int64_t nblk = d.H / 128;
  for (int64_t r = first + blockIdx.y; r < last; r += gridDim.y) {
    if (zero_payload) {
      uint4 *dst = reinterpret_cast<uint4 *>(static_cast<char *>(recv_x) + r * row_bytes);
      for (int64_t i = threadIdx.x; i < row_bytes / 16; i += kBlock)
        dst[i] = make_uint4(0, 0, 0, 0);
      if (fp8)
        for (int64_t i = threadIdx.x; i < nblk; i += kBlock) recv_scales[r * nblk + i] = 0.0f;
    }
    if (threadIdx.x == 0) {
      row_src[r] = -1;
      if (recv_weights != nullptr) recv_weights[r] = 0.0f;
    }
  }
}

// ---------------------------------------------------------------------------
// Combine ("GPU microarchitecture: DeepEP first principles", 1.2; "Deep Dive
// - DeepEP", "Combine: reverse routing plus reduction")
// ---------------------------------------------------------------------------

// The fixed-order gather-reduce of one token's (or one non-expanded row's)
// slots over its 8 columns at col: acc = sum over slots j in order of
// g_j * y[row_j] (an FMA each from +0), or of y[row_j] unweighted, over the
// slots with a row only.  Lane j below k holds slot j's row (-1 for none)
// and gate.  The slots with a row are taken in slot order, KB at a time:
// the batch's KB 16-byte loads per lane are all issued before its FMAs.
// They are buffer loads over each slot's row (an empty buffer for a batch
// entry past the last slot, a lane past the row's end given an offset past
// it), issued whatever the entry and the lane and all consumed by the FMAs,
// with a select keeping the sum as it was for an entry with no slot; so the
// compiler's waits count them exactly (plain loads under a branch per slot
// had it wait for each gather before issuing the next).  combine_kernel
// takes KB = 1 while the chip is full of waves: one row load in flight per
// wave then measured faster than several (more rows' pages open at once in
// the memory queues).  Its last kChipWaves work items take KB = 8 (every
// row of the token in flight together): they run while the chip empties,
// where a wave's latency is the launch's tail, and a grid the chip holds
// at once (a decode-sized batch) is all tail.
template <bool kWeighted, int KB>
__device__ __forceinline__ void gather_rows(const uint16_t *__restrict__ y, int64_t H,
                                            int32_t row, float gate, int col, float acc[8]) {
  const uint32_t nrow = (uint32_t)H * 2u;
  const int off = (int)(col < H ? (uint32_t)col * 2u : nrow);
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  unsigned long long left = __ballot(row >= 0);
  while (left != 0ull) {
    i32x4_t v[KB];
    int32_t rj[KB];
    int sj[KB];
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
      sj[jj] = left != 0ull ? (int)__builtin_ctzll(left) : -1;
      left &= left - 1ull;
      rj[jj] = sj[jj] >= 0 ? lane_value(row, sj[jj]) : -1;
      const uint16_t *src = y + (int64_t)(rj[jj] >= 0 ? rj[jj] : 0) * H;
      v[jj] = __builtin_amdgcn_raw_buffer_load_b128(buffer_over(src, rj[jj] >= 0 ? nrow : 0u),
                                                    off, 0, kBufferNt);
    }
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
      const bool use = rj[jj] >= 0;
      const float g = kWeighted ? lane_value_f(gate, sj[jj] & (kWave - 1)) : 1.0f;
      const uint32_t w4[4] = {(uint32_t)v[jj].x, (uint32_t)v[jj].y, (uint32_t)v[jj].z,
                              (uint32_t)v[jj].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = bf16_lo(w4[i]), hi = bf16_hi(w4[i]);
        const float a0 = kWeighted ? __builtin_fmaf(g, lo, acc[2 * i]) : acc[2 * i] + lo;
        const float a1 = kWeighted ? __builtin_fmaf(g, hi, acc[2 * i + 1]) : acc[2 * i + 1] + hi;
        acc[2 * i] = use ? a0 : acc[2 * i];
        acc[2 * i + 1] = use ? a1 : acc[2 * i + 1];
      }
    }
  }
}

// One one-wave workgroup per (token, 512-column chunk).  A workgroup's
// slot on its compute unit is given back only when all of its waves have
// ended, and a wave's length varies with its gathers' latency, so a single
// wave per workgroup keeps more gathers in flight: 86.7 against 87.6 us at
// Prefill, 358.0 against 360.3 us at Large (events, two passes).
template <bool kWeighted>
__global__ __launch_bounds__(kWave) void combine_kernel(
    Dims d, int32_t nchunks, int64_t capacity, const uint16_t *__restrict__ y,
    const int32_t *__restrict__ tok_slot_row, const float *__restrict__ topk_weights,
    uint16_t *__restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int item = (int)blockIdx.x;
  if (item >= d.T * nchunks) return;
  const int64_t t = item / nchunks;
  const int chunk = item - (int)t * nchunks;

  // The token's rows and gates, loaded together (lanes below k).
  const uint32_t nk = (uint32_t)d.k * 4u;
  const int koff = (int)(lane < d.k ? (uint32_t)lane * 4u : nk);
  const int32_t r = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
      buffer_over(tok_slot_row + t * d.k, nk), koff, 0, 0);
  const float gate =
      kWeighted ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                buffer_over(topk_weights + t * d.k, nk), koff,
                                                0, 0))
                : 1.0f;
  const int32_t row = lane < d.k && r >= 0 && r < capacity ? r : -1;

  const int64_t H = d.H;
  const int col = chunk * kCombineCols + lane * 8;
  float acc[8];
  if (item >= d.T * nchunks - kChipWaves)
    gather_rows<kWeighted, 8>(y, H, row, gate, col, acc);
  else
    gather_rows<kWeighted, 1>(y, H, row, gate, col, acc);
  if (col < H) {
    uint4 o;
    o.x = pack_bf16(acc[0], acc[1]);
    o.y = pack_bf16(acc[2], acc[3]);
    o.z = pack_bf16(acc[4], acc[5]);
    o.w = pack_bf16(acc[6], acc[7]);
    store_stream(out + t * H + col, o);
  }
}

// ---------------------------------------------------------------------------
// Non-expanded (rank-deduplicated) path ("Deep Dive - DeepEP", "Why expert
// parallelism needs a communication layer": a token crosses to a rank once
// however many of its experts live there; "Dispatch: layout, move, and
// epilogue": a non-expanded row is a source token with its top-k metadata,
// and the copy epilogue expands rows into the expert GEMM layout).
// ---------------------------------------------------------------------------

// One payload chunk of a token (16 values per lane): bf16 bits, or E4M3
// codes plus the block scale (held by lanes 0, 8, 16, ...).
struct Payload16 {
  uint4 lo, hi;  // bf16: 16 values; FP8: lo = 16 codes
  float scale;
};

// Lanes own 16 values; with H % 16 == 8 (bf16 rows) the last lane of a row
// owns only its lower 8, so the upper half is guarded separately (FP8 rows
// have H % 128 == 0).
__device__ __forceinline__ Payload16 load_payload(const uint16_t *__restrict__ x, int64_t t,
                                                  int64_t H, int col, bool in) {
  Payload16 p;
  p.lo = make_uint4(0, 0, 0, 0);
  p.hi = p.lo;
  p.scale = 0.0f;
  if (in) {
    p.lo = *reinterpret_cast<const uint4 *>(x + t * H + col);
    if (col + 8 < H) p.hi = *reinterpret_cast<const uint4 *>(x + t * H + col + 8);
  }
  return p;
}

// FP8 rows: the loaded bf16 values become codes and the block scale (all
// lanes of the wave together); bf16 rows are left as loaded.
template <bool kFp8>
__device__ __forceinline__ void encode_payload(Payload16 &p, int lane, int32_t *status) {
  bool finite = true;
  if (kFp8)
    p.lo = quantize16(p.lo, p.hi, p.scale, finite);
  else
    finite = absmax_bits16(p.lo, p.hi) < kBf16Inf;
  report_nonfinite(!finite, lane, status);
}

template <bool kFp8>
__device__ __forceinline__ void store_payload(void *__restrict__ rows, float *__restrict__ scales,
                                              int64_t r, int64_t H, int col, int lane,
                                              const Payload16 &p) {
  if (kFp8) {
    store_stream(static_cast<uint8_t *>(rows) + r * H + col, p.lo);
    if ((lane & 7) == 0) scales[r * (H / 128) + col / 128] = p.scale;
  } else {
    uint16_t *dst = static_cast<uint16_t *>(rows) + r * H + col;
    store_stream(dst, p.lo);
    if (col + 8 < H) store_stream(dst + 8, p.hi);
  }
}

// Row of token t on rank r (lanes r < R), -1 if the token has no expert on
// r: the rank's partition start, plus earlier tiles' tokens on r, plus the
// tokens on r before t in its tile (earlier waves' ballots, then lanes below
// in its own wave's ballot).
__device__ __forceinline__ int32_t rank_row(const Dims &d, int64_t t, int lane,
                                            const unsigned long long *__restrict__ rank_ballot,
                                            const int32_t *__restrict__ rank_tok_off,
                                            const int32_t *__restrict__ tile_rank_base,
                                            int64_t ranked_capacity, int32_t *__restrict__ status) {
  int32_t row = -1;
  if (lane < d.R) {
    const int64_t tile = t / kTileTokens;
    const int w = (int)(t % kTileTokens) / kWave;
    const int tl = (int)(t % kWave);
    const unsigned long long *b = rank_ballot + tile * kWavesPerBlock * d.R + lane;
    const unsigned long long mine = b[(int64_t)w * d.R];
    if ((mine >> tl) & 1ull) {
      int32_t pos = __popcll(mine & ((1ull << tl) - 1ull));
      for (int ww = 0; ww < w; ++ww) pos += __popcll(b[(int64_t)ww * d.R]);
      const int64_t r = (int64_t)rank_tok_off[lane] +
                        tile_rank_base[tile * tile_row_ints(d.E, d.R) + lane] + pos;
      if (r < ranked_capacity)
        row = (int32_t)r;
      else
        flag(status, EP_STATUS_BIT_CAPACITY);
    }
  }
  return row;
}

template <bool kFp8>
__global__ __launch_bounds__(kBlock) void dispatch_ranked_kernel(
    Dims d, int32_t nchunks, const uint16_t *__restrict__ x, const int32_t *__restrict__ topk_idx,
    const float *__restrict__ topk_weights, const int32_t *__restrict__ expert_offsets,
    const int32_t *__restrict__ header, const int32_t *__restrict__ tile_base,
    const int32_t *__restrict__ slot_rank, const int32_t *__restrict__ tile_rank_base,
    const unsigned long long *__restrict__ rank_ballot, const int32_t *__restrict__ rank_tok_off,
    int64_t capacity, int64_t ranked_capacity, void *__restrict__ ne_x,
    float *__restrict__ ne_scales, int32_t *__restrict__ ne_topk_idx,
    float *__restrict__ ne_topk_weights, int32_t *__restrict__ ne_src,
    int32_t *__restrict__ rank_token_offsets, int32_t *__restrict__ tok_rank_row,
    int32_t *__restrict__ tok_slot_row, int32_t *__restrict__ status) {
  const int lane = threadIdx.x & (kWave - 1);
  const int item = uniform(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave);
  if (item == 0) {
    if (!workspace_ok(header, d)) {
      if (lane == 0) flag(status, EP_STATUS_BIT_WORKSPACE);
    } else {
      for (int i = lane; i <= d.R; i += kWave) rank_token_offsets[i] = rank_tok_off[i];
    }
  }
  if (item >= d.T * nchunks) return;
  const int64_t t = item / nchunks;
  const int chunk = item - (int)t * nchunks;
  // The payload's loads go first: they overlap the reads that give the
  // token's rank rows.  FP8 encoding waits until those are issued.  The
  // first chunk's wave also loads the token's ids, gates and in-tile ranks
  // here, so that they arrive with the rank rows: its metadata then takes
  // one more round trip (the expanded rows' segment starts), not three.
  const int64_t H = d.H;
  const int col = chunk * kChunkCols + lane * 16;
  const bool in = col < H;
  Payload16 p = load_payload(x, t, H, col, in);
  int32_t ej = -1, srank = -1;
  float gj = 0.0f;
  if (chunk == 0 && lane < d.k) {
    ej = topk_idx[t * d.k + lane];
    srank = slot_rank[t * d.k + lane];
    if (topk_weights != nullptr) gj = topk_weights[t * d.k + lane];
  }
  if (!workspace_ok(header, d)) return;
  const int32_t row = rank_row(d, t, lane, rank_ballot, rank_tok_off, tile_rank_base,
                               ranked_capacity, status);
  if (chunk == 0) {
    const int epr = d.E / d.R;
    // The expanded handle (rows the receiver's expand will fill), as the
    // dispatch kernels give them: segment start + earlier tiles + in-tile
    // rank, with the same check of the layout's slot word.
    int32_t srow = -1;
    if (lane < d.k) {
      const bool valid = ej >= 0 && ej < d.E;
      if (valid != (srank >= 0) || (valid && (srank >> kSlotExpertShift) != ej)) {
        flag(status, EP_STATUS_BIT_WORKSPACE);
      } else if (valid) {
        const int64_t r = (int64_t)expert_offsets[ej] +
                          tile_base[(t / kTileTokens) * tile_row_ints(d.E, d.R) + ej] +
                          (srank & kSlotRankMask);
        if (r >= 0 && r < capacity)
          srow = (int32_t)r;
        else
          flag(status, EP_STATUS_BIT_CAPACITY);
      }
    }
    if (lane < d.R) {
      tok_rank_row[t * d.R + lane] = row;
      if (row >= 0) ne_src[row] = (int32_t)t;
    }
    // The token's top-k slice for each of its ranks: pairs (r, j) over
    // lanes.  Every lane runs every round so the shuffles' source lanes are
    // always active.
    for (int base = 0; base < d.R * d.k; base += kWave) {
      const int pr = base + lane;
      const int r = min(pr / d.k, d.R - 1);
      const int j = pr - (pr / d.k) * d.k;
      const int32_t rr = __shfl(row, r);
      const int32_t e = __shfl(ej, j);
      const float g = __shfl(gj, j);
      if (pr >= d.R * d.k || rr < 0) continue;
      const bool local = e >= 0 && e < d.E && e / epr == r;
      ne_topk_idx[(int64_t)rr * d.k + j] = local ? e - r * epr : -1;
      // each valid slot is local to exactly one rank, so its gate is
      // checked once
      const float gate = (local && topk_weights != nullptr) ? g : 0.0f;
      if (!__builtin_isfinite(gate)) flag(status, EP_STATUS_BIT_NONFINITE);
      if (ne_topk_weights != nullptr) ne_topk_weights[(int64_t)rr * d.k + j] = gate;
    }
    if (lane < d.k) tok_slot_row[t * d.k + lane] = srow;
  }

  encode_payload<kFp8>(p, lane, status);
  for (int r = 0; r < d.R; ++r) {
    const int32_t rr = lane_value(row, r);
    if (rr < 0 || !in) continue;
    store_payload<kFp8>(ne_x, ne_scales, rr, H, col, lane, p);
  }
}

// Receiver-side expand: non-expanded row q (rank r, token t) goes to the
// expert-major row of each of its local slots.  One wave per (received row,
// batch of kExpandBatch 1024-column chunks: the whole row up to H = 8192);
// the first batch's wave also writes the rows' sources and gates.  The
// loads take three round trips: the row count and the workspace header (a
// row past the count has nothing to load); then the batch's payload with
// everything that depends on q alone (the partition starts that give r, the
// source token, the local ids and gates); then everything that depends on t
// and the expert (the slot words, segment starts and tile bases).  Buffer
// loads give lanes with nothing to load zeros, so no load has a branch of
// its own.
constexpr int kExpandBatch = 8;

template <bool kFp8>
__global__ __launch_bounds__(kBlock) void expand_kernel(
    Dims d, int32_t nchunks, int64_t ranked_capacity, const void *__restrict__ ne_x,
    const float *__restrict__ ne_scales, const int32_t *__restrict__ ne_topk_idx,
    const float *__restrict__ ne_topk_weights, const int32_t *__restrict__ ne_src,
    const int32_t *__restrict__ rank_token_offsets, const int32_t *__restrict__ expert_offsets,
    const int32_t *__restrict__ header, const int32_t *__restrict__ tile_base,
    const int32_t *__restrict__ slot_rank, int64_t capacity, void *__restrict__ recv_x,
    float *__restrict__ recv_scales, float *__restrict__ recv_weights,
    int32_t *__restrict__ row_src, int32_t *__restrict__ status) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nbatches = (nchunks + kExpandBatch - 1) / kExpandBatch;
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + uniform(threadIdx.x / kWave);
  const int64_t q = item / nbatches;
  const int batch = (int)(item - q * nbatches);
  if (q >= ranked_capacity) return;
  const int64_t rows = rank_token_offsets[d.R];
  const bool ok = workspace_ok(header, d);
  if (q >= rows || !ok) {
    if (q < rows && lane == 0) flag(status, EP_STATUS_BIT_WORKSPACE);
    return;
  }
  const int64_t H = d.H;
  asm volatile("" : "+s"(ne_x), "+s"(ne_scales));

  // The row's rank: how many partition starts 1..R are at or below q.
  const uint32_t nro = (uint32_t)(d.R + 1) * 4u;
  int32_t start_l = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
      buffer_over(rank_token_offsets, nro),
      (int)(lane >= 1 && lane <= d.R ? (uint32_t)lane * 4u : nro), 0, 0);
  int64_t t = ne_src[q];
  const uint32_t nk = (uint32_t)d.k * 4u;
  const int koff = (int)(lane < d.k ? (uint32_t)lane * 4u : nk);
  int32_t le = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
      buffer_over(ne_topk_idx + q * d.k, nk), koff, 0, 0);
  const bool gates = batch == 0 && recv_weights != nullptr && ne_topk_weights != nullptr;
  const float gate = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(
                 buffer_over(gates ? static_cast<const void *>(ne_topk_weights + q * d.k)
                                   : static_cast<const void *>(ne_topk_idx + q * d.k),
                             gates ? nk : 0u),
                 koff, 0, 0));

  // Then the batch's payload.  It is used only in the store loop, and the
  // compiler would otherwise place its loads there, after the chain below.
  // Its pointers are made opaque (so that the loads cannot be taken for
  // reads of constant memory, which may be placed anywhere), and an empty
  // asm statement that clobbers memory and takes the values loaded above
  // follows them: the payload's loads stay before the wait for those
  // values, and what is computed from them stays after it.
  Payload16 pl[kExpandBatch];
  const int c0 = batch * kExpandBatch;
  if (kFp8) {
    const uint32_t nq = (uint32_t)H;
    const uint32_t ns = (uint32_t)(H / 128) * 4u;
    const __amdgpu_buffer_rsrc_t codes =
        buffer_over(static_cast<const uint8_t *>(ne_x) + q * H, nq);
    const __amdgpu_buffer_rsrc_t scales = buffer_over(ne_scales + q * (H / 128), ns);
#pragma unroll
    for (int b = 0; b < kExpandBatch; ++b) {
      const int col = (c0 + b) * kChunkCols + lane * 16;
      const bool live = c0 + b < nchunks && col < H;
      const i32x4_t w =
          __builtin_amdgcn_raw_buffer_load_b128(codes, (int)(live ? (uint32_t)col : nq), 0, 0);
      pl[b].lo = make_uint4((uint32_t)w.x, (uint32_t)w.y, (uint32_t)w.z, (uint32_t)w.w);
      pl[b].hi = pl[b].lo;
      pl[b].scale = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(
                     scales, (int)(live && (lane & 7) == 0 ? (uint32_t)(col / 128) * 4u : ns),
                     0, 0));
    }
  } else {
    // With H % 16 == 8 the last lane's upper half lies past the row's end
    // and reads zeros.
    const uint32_t nx = (uint32_t)H * 2u;
    const __amdgpu_buffer_rsrc_t src = buffer_over(static_cast<const uint16_t *>(ne_x) + q * H, nx);
#pragma unroll
    for (int b = 0; b < kExpandBatch; ++b) {
      const int col = (c0 + b) * kChunkCols + lane * 16;
      const bool live = c0 + b < nchunks && col < H;
      const uint32_t off = live ? (uint32_t)col * 2u : nx;
      const i32x4_t lo = __builtin_amdgcn_raw_buffer_load_b128(src, (int)off, 0, 0);
      const i32x4_t hi = __builtin_amdgcn_raw_buffer_load_b128(src, (int)(live ? off + 16u : nx), 0, 0);
      pl[b].lo = make_uint4((uint32_t)lo.x, (uint32_t)lo.y, (uint32_t)lo.z, (uint32_t)lo.w);
      pl[b].hi = make_uint4((uint32_t)hi.x, (uint32_t)hi.y, (uint32_t)hi.z, (uint32_t)hi.w);
      pl[b].scale = 0.0f;
    }
  }
  asm volatile("" : "+v"(start_l), "+v"(le), "+s"(t)::"memory");

  const int r = uniform((int)__popcll(__ballot(lane >= 1 && lane <= d.R && start_l <= q)));
  const bool route_ok = r < d.R && t >= 0 && t < d.T;
  const int epr = d.E / d.R;
  const bool local = route_ok && lane < d.k && le >= 0 && le < epr;
  const int32_t e = r * epr + le;
  const int64_t ts = route_ok ? t : 0;  // the loads' token, in range
  const int32_t w = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
      buffer_over(slot_rank + ts * d.k, nk), (int)(local ? (uint32_t)lane * 4u : nk), 0, 0);
  const RowBase base = load_row_base(d, ts, e, local, expert_offsets, tile_base);
  const bool same = local && w >= 0 && (w >> kSlotExpertShift) == e;
  bool fits;
  const int32_t row = row_from_base(base, w, same, capacity, fits);

  for (int j = 0; j < d.k; ++j) {
    const int32_t rr = lane_value(row, j);
    if (rr < 0) continue;
#pragma unroll
    for (int b = 0; b < kExpandBatch; ++b) {
      const int col = (c0 + b) * kChunkCols + lane * 16;
      if (c0 + b < nchunks && col < H)
        store_payload<kFp8>(recv_x, recv_scales, rr, H, col, lane, pl[b]);
    }
  }
  if (batch == 0 && row >= 0) {
    row_src[row] = (int32_t)(t * d.k + lane);
    if (gates) recv_weights[row] = gate;
  }
  if (!route_ok && lane == 0) flag(status, EP_STATUS_BIT_ROUTE);
  if (batch == 0 && local && !same) flag(status, EP_STATUS_BIT_WORKSPACE);
  if (batch == 0 && same && !fits) flag(status, EP_STATUS_BIT_CAPACITY);
}

// Ranked combine, stage 1: per non-expanded row, the fp32 sum of its local
// slots' (weighted) expert rows in slot order.
template <bool kWeighted, int KB>
__global__ __launch_bounds__(kBlock) void combine_ranked_partial_kernel(
    Dims d, int32_t nchunks, int64_t capacity, int64_t ranked_capacity,
    const uint16_t *__restrict__ y, const int32_t *__restrict__ tok_slot_row,
    const int32_t *__restrict__ ne_topk_idx, const float *__restrict__ ne_topk_weights,
    const int32_t *__restrict__ ne_src, const int32_t *__restrict__ rank_token_offsets,
    float *__restrict__ partials) {
  const int lane = threadIdx.x & (kWave - 1);
  const int item = uniform(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave);
  const int64_t q = item / nchunks;
  const int chunk = item - (int)q * nchunks;
  if (q >= ranked_capacity) return;
  // The row count first: the grid covers the capacity, and the rows past the
  // count (a third to a half of them) should cost no more than that.  Then
  // the row's source token, local ids and gates in one round trip, the
  // expanded rows of the local slots in a second (buffer loads: zeros for
  // lanes with nothing to load), then the gathers.  The empty asm statement
  // taking the ids and gates keeps their loads before the source check,
  // which the compiler would otherwise move first.
  const int64_t rows = rank_token_offsets[d.R];
  if (q >= rows) return;
  const int64_t t = ne_src[q];
  const uint32_t nk = (uint32_t)d.k * 4u;
  const int koff = (int)(lane < d.k ? (uint32_t)lane * 4u : nk);
  int32_t le = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
      buffer_over(ne_topk_idx + q * d.k, nk), koff, 0, 0);
  float gate =
      kWeighted ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                buffer_over(ne_topk_weights + q * d.k, nk), koff,
                                                0, 0))
                : 1.0f;
  asm volatile("" : "+v"(le), "+v"(gate));
  const bool live = t >= 0 && t < d.T;
  const bool local = live && lane < d.k && le >= 0;
  const int32_t p = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
      buffer_over(tok_slot_row + (live ? t : 0) * d.k, nk),
      (int)(local ? (uint32_t)lane * 4u : nk), 0, 0);
  const int32_t row = local && p >= 0 && p < capacity ? p : -1;
  if (!live) return;
  const int64_t H = d.H;
  const int col = chunk * kCombineCols + lane * 8;
  float acc[8];
  gather_rows<kWeighted, KB>(y, H, row, gate, col, acc);
  if (col < H) {
    // Plain (not streaming) stores: the partials are read again by stage 2
    // right away.  Measured over a whole non-expanded step, they save more
    // here than the deferred write-back of their lines costs later.
    float *dst = partials + q * H + col;
    *reinterpret_cast<uint4 *>(dst) = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                                                 __float_as_uint(acc[2]), __float_as_uint(acc[3]));
    *reinterpret_cast<uint4 *>(dst + 4) =
        make_uint4(__float_as_uint(acc[4]), __float_as_uint(acc[5]), __float_as_uint(acc[6]),
                   __float_as_uint(acc[7]));
  }
}

// Ranked combine, stage 2: per token, the fp32 sum of its ranks' partials in
// rank order, rounded once to bf16.  Lane r below R holds the token's row on
// rank r (-1 for none); the ranks with a row are taken in rank order, KB at
// a time, with the loads of gather_rows: buffer loads (two 16-byte parts per
// lane of a row's 8 fp32 columns) issued whatever the entry, all consumed
// through a select, so the waits count them exactly.
template <int KB>
__device__ __forceinline__ void sum_partials(const float *__restrict__ partials, int64_t H,
                                             int32_t q, int col, float acc[8]) {
  const uint32_t nrow = (uint32_t)H * 4u;
  const uint32_t off = col < H ? (uint32_t)col * 4u : nrow;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  unsigned long long left = __ballot(q >= 0);
  while (left != 0ull) {
    i32x4_t a[KB], b[KB];
    int32_t qj[KB];
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
      const int s = left != 0ull ? (int)__builtin_ctzll(left) : -1;
      left &= left - 1ull;
      qj[jj] = s >= 0 ? lane_value(q, s) : -1;
      const __amdgpu_buffer_rsrc_t rsrc =
          buffer_over(partials + (int64_t)(qj[jj] >= 0 ? qj[jj] : 0) * H, qj[jj] >= 0 ? nrow : 0u);
      a[jj] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off, 0, kBufferNt);
      b[jj] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(off + 16u), 0, kBufferNt);
    }
#pragma unroll
    for (int jj = 0; jj < KB; ++jj) {
      const bool use = qj[jj] >= 0;
      const float v[8] = {__int_as_float(a[jj].x), __int_as_float(a[jj].y),
                          __int_as_float(a[jj].z), __int_as_float(a[jj].w),
                          __int_as_float(b[jj].x), __int_as_float(b[jj].y),
                          __int_as_float(b[jj].z), __int_as_float(b[jj].w)};
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = use ? acc[i] + v[i] : acc[i];
    }
  }
}

// One wave per (token, 512-column chunk); the launch's last kChipWaves work
// items take every rank's row at once, the others one at a time, as in
// combine_kernel.
__global__ __launch_bounds__(kBlock) void combine_ranked_sum_kernel(
    Dims d, int32_t nchunks, int64_t ranked_capacity, const float *__restrict__ partials,
    const int32_t *__restrict__ tok_rank_row, uint16_t *__restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int item = uniform(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave);
  if (item >= d.T * nchunks) return;
  const int64_t t = item / nchunks;
  const int chunk = item - (int)t * nchunks;
  const uint32_t nr = (uint32_t)d.R * 4u;
  const int32_t v = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
      buffer_over(tok_rank_row + t * d.R, nr), (int)(lane < d.R ? (uint32_t)lane * 4u : nr), 0,
      0);
  const int32_t q = lane < d.R && v >= 0 && v < ranked_capacity ? v : -1;
  const int64_t H = d.H;
  const int col = chunk * kCombineCols + lane * 8;
  float acc[8];
  if (item >= d.T * nchunks - kChipWaves)
    sum_partials<8>(partials, H, q, col, acc);
  else
    sum_partials<1>(partials, H, q, col, acc);
  if (col < H) {
    uint4 o;
    o.x = pack_bf16(acc[0], acc[1]);
    o.y = pack_bf16(acc[2], acc[3]);
    o.z = pack_bf16(acc[4], acc[5]);
    o.w = pack_bf16(acc[6], acc[7]);
    store_stream(out + t * H + col, o);
  }
}

// ---------------------------------------------------------------------------
// Backward of combine ("Deep Dive - DeepEP", "Combine: reverse routing plus
// reduction": backward duality, and the gate gradient the autograd wrapper
// still owes).  One 4-wave workgroup per token; wave w takes the 512-column
// chunks w, w + 4, ...:
//   grad_expert_out[row_j, c] = bf16(w[t,j] * grad_out[t,c])
//   grad_w[t,j]               = sum_c expert_out[row_j, c] * grad_out[t,c]
// Each lane accumulates its columns' products in fp32 in a fixed order, an
// xor butterfly adds the wave's 64 lane sums, and the four wave sums are
// added in wave order: every run gives the same bits.
// ---------------------------------------------------------------------------

template <int K>
__global__ __launch_bounds__(kBlock) void combine_backward_kernel(
    Dims d, int64_t capacity, const uint16_t *__restrict__ grad_out,
    const int32_t *__restrict__ tok_slot_row, const float *__restrict__ topk_weights,
    const uint16_t *__restrict__ expert_out, uint16_t *__restrict__ grad_expert_out,
    float *__restrict__ grad_weights) {
  __shared__ float wave_dot[kWavesPerBlock][K];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t t = blockIdx.x;
  const int64_t H = d.H;
  const bool want_gate = grad_weights != nullptr;

  int32_t row = -1;
  float gate = 1.0f;
  if (lane < d.k) {
    const int32_t r = tok_slot_row[t * d.k + lane];
    if (r >= 0 && r < capacity) row = r;
    if (topk_weights != nullptr) gate = topk_weights[t * d.k + lane];
  }
  int32_t rows[K];
  float gates[K];
  float dot[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    rows[j] = j < d.k ? lane_value(row, j) : -1;
    gates[j] = j < d.k ? lane_value_f(gate, j) : 0.0f;
    dot[j] = 0.0f;
  }

  for (int64_t col = (int64_t)wave * kCombineCols + lane * 8; col < H;
       col += (int64_t)kWavesPerBlock * kCombineCols) {
    const uint4 gv = *reinterpret_cast<const uint4 *>(grad_out + t * H + col);
    const float g[8] = {bf16_lo(gv.x), bf16_hi(gv.x), bf16_lo(gv.y), bf16_hi(gv.y),
                        bf16_lo(gv.z), bf16_hi(gv.z), bf16_lo(gv.w), bf16_hi(gv.w)};
    uint4 yv[K];
    if (want_gate) {
#pragma unroll
      for (int j = 0; j < K; ++j)
        if (rows[j] >= 0) yv[j] = load_stream(expert_out + (int64_t)rows[j] * H + col);
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (rows[j] < 0) continue;
      uint4 o;
      o.x = pack_bf16(gates[j] * g[0], gates[j] * g[1]);
      o.y = pack_bf16(gates[j] * g[2], gates[j] * g[3]);
      o.z = pack_bf16(gates[j] * g[4], gates[j] * g[5]);
      o.w = pack_bf16(gates[j] * g[6], gates[j] * g[7]);
      store_stream(grad_expert_out + (int64_t)rows[j] * H + col, o);
      if (want_gate) {
        const uint32_t w4[4] = {yv[j].x, yv[j].y, yv[j].z, yv[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dot[j] = __builtin_fmaf(bf16_lo(w4[i]), g[2 * i], dot[j]);
          dot[j] = __builtin_fmaf(bf16_hi(w4[i]), g[2 * i + 1], dot[j]);
        }
      }
    }
  }

  if (want_gate) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      float v = dot[j];
#pragma unroll
      for (int m = kWave / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m);
      if (lane == 0) wave_dot[wave][j] = v;
    }
    __syncthreads();
    if (threadIdx.x < d.k) {
      const int j = threadIdx.x;
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w) v += wave_dot[w][j];
      const int32_t r = tok_slot_row[t * d.k + j];
      grad_weights[t * d.k + j] = (r >= 0 && r < capacity) ? v : 0.0f;
    }
  }
}

// Alignment padding rows of a gradient w.r.t. the receive buffer get zeros
// (one workgroup per expert; padding rows are those without a source).
__global__ __launch_bounds__(kBlock) void zero_padding_rows_kernel(
    Dims d, const int32_t *__restrict__ expert_offsets, const int32_t *__restrict__ row_src,
    int64_t capacity, uint16_t *__restrict__ rows_out) {
  const int e = blockIdx.x;
  int64_t last = expert_offsets[e + 1];
  if (last > capacity) last = capacity;
  const int64_t H = d.H;
  const int64_t first = expert_offsets[e] > 0 ? expert_offsets[e] : 0;
  for (int64_t r = first; r < last; ++r) {
    if (row_src[r] >= 0) continue;
    uint4 *dst = reinterpret_cast<uint4 *>(rows_out + r * H);
    for (int64_t i = threadIdx.x; i < H / 8; i += kBlock) dst[i] = make_uint4(0, 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Kernel timing requested by ep_time_next_kernel: the first kernel of the
// thread's next layout / dispatch / combine call records the start event
// when it begins, and that call's last kernel records the stop event when
// it ends (both launched through hipExtLaunchKernelGGL).
namespace {
thread_local hipEvent_t t_time_start = nullptr, t_time_stop = nullptr;
}  // namespace

void time_next_kernel(hipEvent_t start, hipEvent_t stop) {
  t_time_start = start;
  t_time_stop = stop;
}

// A launch of one of those calls' kernels; `last` marks the call's last one.
template <typename F, typename... Args>
static void launch_kernel(bool last, F kernel, dim3 grid, dim3 block, uint32_t lds,
                          hipStream_t stream, Args... args) {
  const hipEvent_t start = t_time_start, stop = last ? t_time_stop : nullptr;
  t_time_start = nullptr;
  if (last) t_time_stop = nullptr;
  if (start != nullptr || stop != nullptr)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, start, stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
}

WorkspaceLayout workspace_layout(int32_t T, int32_t k, int32_t E, int32_t R) {
  WorkspaceLayout w;
  w.ntiles = (T + kTileTokens - 1) / kTileTokens;
  size_t off = align256(sizeof(int32_t) * kHeaderInts);
  w.tile_cnt = off;
  w.tile_rank_cnt = off + sizeof(int32_t) * (size_t)tile_row_experts(E);
  off += align256(sizeof(int32_t) * (size_t)w.ntiles * tile_row_ints(E, R));
  w.cnt = off;
  off += align256(sizeof(int32_t) * (size_t)E);
  w.slot_rank = off;
  off += align256(sizeof(int32_t) * (size_t)T * k);
  w.rank_ballot = off;
  off += align256(sizeof(unsigned long long) * (size_t)w.ntiles * kWavesPerBlock * R);
  w.rank_tok_off = off;
  off += align256(sizeof(int32_t) * ((size_t)R + 1));
  w.total = off;
  return w;
}

hipError_t launch_layout(const Dims &d, const int32_t *topk_idx, int32_t *num_tokens_per_rank,
                         int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank,
                         int32_t *expert_offsets, int32_t *rank_offsets, char *ws,
                         int32_t *status, hipStream_t stream, bool last) {
  const WorkspaceLayout w = workspace_layout(d.T, d.k, d.E, d.R);
  const size_t lds = layout_lds_bytes(d.E);
  auto pick = [&](auto k8, auto k16, auto k32) { return d.k <= 8 ? k8 : (d.k <= 16 ? k16 : k32); };
  // Up to 16 tiles of at most 256 experts: the per-expert column read-back.
  // Otherwise slices of up to 8 tiles per scanning thread take the smaller
  // quad kernel, up to 24 the one that holds 24 quads, and longer slices are
  // read twice.
  const TileGrid g = tile_grid(d.E, d.R, w.ntiles);
  auto kernel = w.ntiles <= 16 && d.E <= kBlock
                    ? pick(layout_kernel<8, 0>, layout_kernel<16, 0>, layout_kernel<32, 0>)
                : g.C4 <= kBlock && g.per > 8 && g.per <= 24
                    ? pick(layout_kernel<8, 24>, layout_kernel<16, 24>, layout_kernel<32, 24>)
                    : pick(layout_kernel<8, 8>, layout_kernel<16, 8>, layout_kernel<32, 8>);
  // An empty batch still needs one workgroup to write zero counts and offsets.
  const unsigned grid = w.ntiles > 0 ? (unsigned)w.ntiles : 1u;
  launch_kernel(last, kernel, dim3(grid), dim3(kBlock), (uint32_t)lds, stream, topk_idx, d,
                w.ntiles, d.E / d.R, reinterpret_cast<int32_t *>(ws + w.tile_cnt),
                reinterpret_cast<int32_t *>(ws + w.slot_rank), is_token_in_rank,
                reinterpret_cast<int32_t *>(ws + w.cnt), num_tokens_per_expert,
                num_tokens_per_rank, expert_offsets, rank_offsets, reinterpret_cast<int32_t *>(ws),
                reinterpret_cast<unsigned long long *>(ws + w.rank_ballot),
                reinterpret_cast<int32_t *>(ws + w.rank_tok_off), status);
  return hipGetLastError();
}

hipError_t launch_workspace_init(char *ws, hipStream_t stream) {
  hipLaunchKernelGGL(workspace_init_kernel, dim3(1), dim3(kWave), 0, stream,
                     reinterpret_cast<int32_t *>(ws));
  return hipGetLastError();
}

hipError_t launch_dispatch(const Dims &d, bool fp8, bool zero_padding, const uint16_t *x,
                           const int32_t *topk_idx, const float *topk_weights,
                           const int32_t *expert_offsets, const char *ws, int64_t capacity,
                           void *recv_x, float *recv_scales, float *recv_weights,
                           int32_t *tok_slot_row, int32_t *row_src, int32_t *status,
                           hipStream_t stream) {
  const WorkspaceLayout w = workspace_layout(d.T, d.k, d.E, d.R);
  const int32_t *header = reinterpret_cast<const int32_t *>(ws);
  const int32_t *tile_base = reinterpret_cast<const int32_t *>(ws + w.tile_cnt);
  const int32_t *slot_rank = reinterpret_cast<const int32_t *>(ws + w.slot_rank);
  const int32_t nchunks = (d.H + kChunkCols - 1) / kChunkCols;
  if (d.T > 0) {
    const int64_t items = (int64_t)d.T * nchunks;
    const dim3 grid((unsigned)((items + kWavesPerBlock - 1) / kWavesPerBlock));
    auto kernel = fp8 ? dispatch_kernel<true> : dispatch_kernel<false>;
    launch_kernel(d.A == 1, kernel, grid, dim3(kBlock), 0u, stream, d, nchunks, x, topk_idx,
                  topk_weights, expert_offsets, header, tile_base, slot_rank, capacity, recv_x,
                  recv_scales, recv_weights, tok_slot_row, row_src, status);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (d.A > 1) {
    launch_kernel(true, pad_fill_kernel, dim3(d.E, kPadSplit), dim3(kBlock), 0u, stream, d, fp8,
                  zero_padding, reinterpret_cast<const int32_t *>(ws), expert_offsets,
                  reinterpret_cast<const int32_t *>(ws + w.cnt), capacity, recv_x, recv_scales,
                  topk_weights != nullptr ? recv_weights : nullptr, row_src, status);
    return hipGetLastError();
  }
  return hipSuccess;
}

size_t layout_lds_bytes(int32_t E) {
  return sizeof(unsigned long long) * kWavesPerBlock * (size_t)E +
         sizeof(int32_t) * kWavesPerBlock * (size_t)E + sizeof(int32_t) * ((size_t)E + 1);
}

hipError_t launch_layout_dispatch(const Dims &d, bool fp8, bool zero_padding,
                                  const uint16_t *x, const int32_t *topk_idx,
                                  const float *topk_weights,
                                  int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                                  uint8_t *is_token_in_rank, int32_t *expert_offsets,
                                  int32_t *rank_offsets, char *ws, int64_t capacity, void *recv_x,
                                  float *recv_scales, float *recv_weights, int32_t *tok_slot_row,
                                  int32_t *row_src, int32_t *status, hipStream_t stream) {
  if (d.T > kTileTokens) {
    // Several tiles: the layout launch, then the dispatch launch.
    hipError_t err = launch_layout(d, topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                                   is_token_in_rank, expert_offsets, rank_offsets, ws, status,
                                   stream, false);
    if (err != hipSuccess) return err;
    return launch_dispatch(d, fp8, zero_padding, x, topk_idx, topk_weights, expert_offsets, ws,
                           capacity, recv_x, recv_scales, recv_weights, tok_slot_row, row_src,
                           status, stream);
  }
  const WorkspaceLayout w = workspace_layout(d.T, d.k, d.E, d.R);
  const int32_t nchunks = (d.H + kChunkCols - 1) / kChunkCols;
  const int64_t items = (int64_t)d.T * nchunks;
  // one workgroup for the layout outputs, then one wave per work item
  const unsigned grid = 1u + (unsigned)((items + kWavesPerBlock - 1) / kWavesPerBlock);
  auto pick = [&](auto k8, auto k16, auto k32) { return d.k <= 8 ? k8 : (d.k <= 16 ? k16 : k32); };
  auto kernel = fp8 ? pick(layout_dispatch_kernel<8, true>, layout_dispatch_kernel<16, true>,
                           layout_dispatch_kernel<32, true>)
                    : pick(layout_dispatch_kernel<8, false>, layout_dispatch_kernel<16, false>,
                           layout_dispatch_kernel<32, false>);
  launch_kernel(d.A == 1, kernel, dim3(grid), dim3(kBlock), (uint32_t)layout_lds_bytes(d.E),
                stream, topk_idx, d, w.ntiles, d.E / d.R, nchunks, x, topk_weights,
                reinterpret_cast<int32_t *>(ws + w.tile_cnt),
                reinterpret_cast<int32_t *>(ws + w.slot_rank), is_token_in_rank,
                reinterpret_cast<int32_t *>(ws + w.cnt), num_tokens_per_expert,
                num_tokens_per_rank, expert_offsets, rank_offsets, reinterpret_cast<int32_t *>(ws),
                reinterpret_cast<unsigned long long *>(ws + w.rank_ballot),
                reinterpret_cast<int32_t *>(ws + w.rank_tok_off), capacity, recv_x, recv_scales,
                recv_weights, tok_slot_row, row_src, status);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (d.A > 1) {
    launch_kernel(true, pad_fill_kernel, dim3(d.E, kPadSplit), dim3(kBlock), 0u, stream, d, fp8,
                  zero_padding, reinterpret_cast<const int32_t *>(ws), expert_offsets,
                  reinterpret_cast<const int32_t *>(ws + w.cnt), capacity, recv_x, recv_scales,
                  topk_weights != nullptr ? recv_weights : nullptr, row_src, status);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_dispatch_fp8_input(const Dims &d, bool zero_padding, const uint8_t *x_codes,
                                     const float *x_scales, const int32_t *topk_idx,
                                     const float *topk_weights, const int32_t *expert_offsets,
                                     const char *ws,
                                     int64_t capacity, uint8_t *recv_x, float *recv_scales,
                                     float *recv_weights, int32_t *tok_slot_row,
                                     int32_t *row_src, int32_t *status, hipStream_t stream) {
  const WorkspaceLayout w = workspace_layout(d.T, d.k, d.E, d.R);
  const int32_t *header = reinterpret_cast<const int32_t *>(ws);
  const int32_t *tile_base = reinterpret_cast<const int32_t *>(ws + w.tile_cnt);
  const int32_t *slot_rank = reinterpret_cast<const int32_t *>(ws + w.slot_rank);
  const int32_t nchunks = (d.H + kChunkCols - 1) / kChunkCols;
  if (d.T > 0) {
    const int64_t items = (int64_t)d.T * nchunks;
    const dim3 grid((unsigned)((items + kWavesPerBlock - 1) / kWavesPerBlock));
    launch_kernel(d.A == 1, dispatch_fp8_input_kernel, grid, dim3(kBlock), 0u, stream, d,
                  nchunks, x_codes, x_scales, topk_idx, topk_weights, expert_offsets, header,
                  tile_base, slot_rank, capacity, recv_x, recv_scales, recv_weights,
                  tok_slot_row, row_src, status);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (d.A > 1) {
    launch_kernel(true, pad_fill_kernel, dim3(d.E, kPadSplit), dim3(kBlock), 0u, stream, d, true,
                  zero_padding, reinterpret_cast<const int32_t *>(ws), expert_offsets,
                  reinterpret_cast<const int32_t *>(ws + w.cnt), capacity,
                  static_cast<void *>(recv_x), recv_scales,
                  topk_weights != nullptr ? recv_weights : nullptr, row_src, status);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_combine(const Dims &d, int64_t capacity, const uint16_t *expert_out,
                          const int32_t *tok_slot_row, const float *topk_weights,
                          uint16_t *out, hipStream_t stream) {
  if (d.T == 0) return hipSuccess;
  const int32_t nchunks = (d.H + kCombineCols - 1) / kCombineCols;
  const int64_t items = (int64_t)d.T * nchunks;
  auto kernel = topk_weights != nullptr ? combine_kernel<true> : combine_kernel<false>;
  launch_kernel(true, kernel, dim3((unsigned)items), dim3(kWave), 0u, stream, d, nchunks,
                capacity, expert_out, tok_slot_row, topk_weights, out);
  return hipGetLastError();
}

}  // namespace ep

namespace ep {

hipError_t launch_combine_backward(const Dims &d, int64_t capacity, const uint16_t *grad_out,
                                   const int32_t *tok_slot_row, const float *topk_weights,
                                   const uint16_t *expert_out, uint16_t *grad_expert_out,
                                   float *grad_weights, const int32_t *expert_offsets,
                                   const int32_t *row_src, hipStream_t stream) {
  if (d.T > 0) {
    const dim3 grid((unsigned)d.T);
    auto kernel = d.k <= 8 ? combine_backward_kernel<8>
                           : (d.k <= 16 ? combine_backward_kernel<16> : combine_backward_kernel<32>);
    hipLaunchKernelGGL(kernel, grid, dim3(kBlock), 0, stream, d, capacity, grad_out, tok_slot_row,
                       topk_weights, expert_out, grad_expert_out, grad_weights);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (d.A > 1) {
    hipLaunchKernelGGL(zero_padding_rows_kernel, dim3(d.E), dim3(kBlock), 0, stream, d,
                       expert_offsets, row_src, capacity, grad_expert_out);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace ep

namespace ep {

hipError_t launch_dispatch_ranked(const Dims &d, bool fp8, const uint16_t *x,
                                  const int32_t *topk_idx, const float *topk_weights,
                                  const int32_t *expert_offsets, const char *ws, int64_t capacity,
                                  int64_t ranked_capacity, void *ne_x, float *ne_scales,
                                  int32_t *ne_topk_idx, float *ne_topk_weights, int32_t *ne_src,
                                  int32_t *rank_token_offsets, int32_t *tok_rank_row,
                                  int32_t *tok_slot_row, int32_t *status, hipStream_t stream) {
  const WorkspaceLayout w = workspace_layout(d.T, d.k, d.E, d.R);
  const int32_t nchunks = (d.H + kChunkCols - 1) / kChunkCols;
  const int64_t items = d.T > 0 ? (int64_t)d.T * nchunks : 1;  // item 0 also copies offsets
  const dim3 grid((unsigned)((items + kWavesPerBlock - 1) / kWavesPerBlock));
  auto kernel = fp8 ? dispatch_ranked_kernel<true> : dispatch_ranked_kernel<false>;
  hipLaunchKernelGGL(kernel, grid, dim3(kBlock), 0, stream, d, nchunks, x, topk_idx, topk_weights,
                     expert_offsets, reinterpret_cast<const int32_t *>(ws),
                     reinterpret_cast<const int32_t *>(ws + w.tile_cnt),
                     reinterpret_cast<const int32_t *>(ws + w.slot_rank),
                     reinterpret_cast<const int32_t *>(ws + w.tile_rank_cnt),
                     reinterpret_cast<const unsigned long long *>(ws + w.rank_ballot),
                     reinterpret_cast<const int32_t *>(ws + w.rank_tok_off), capacity,
                     ranked_capacity, ne_x, ne_scales, ne_topk_idx, ne_topk_weights, ne_src,
                     rank_token_offsets, tok_rank_row, tok_slot_row, status);
  return hipGetLastError();
}

hipError_t launch_expand(const Dims &d, bool fp8, bool zero_padding, int64_t ranked_capacity,
                         const void *ne_x, const float *ne_scales, const int32_t *ne_topk_idx,
                         const float *ne_topk_weights, const int32_t *ne_src,
                         const int32_t *rank_token_offsets, const int32_t *expert_offsets,
                         const char *ws, int64_t capacity, void *recv_x, float *recv_scales,
                         float *recv_weights, int32_t *row_src, int32_t *status,
                         hipStream_t stream) {
  const WorkspaceLayout w = workspace_layout(d.T, d.k, d.E, d.R);
  const int32_t nchunks = (d.H + kChunkCols - 1) / kChunkCols;
  if (ranked_capacity > 0) {
    const int64_t items = ranked_capacity * ((nchunks + kExpandBatch - 1) / kExpandBatch);
    const dim3 grid((unsigned)((items + kWavesPerBlock - 1) / kWavesPerBlock));
    auto kernel = fp8 ? expand_kernel<true> : expand_kernel<false>;
    hipLaunchKernelGGL(kernel, grid, dim3(kBlock), 0, stream, d, nchunks, ranked_capacity, ne_x,
                       ne_scales, ne_topk_idx, ne_topk_weights, ne_src, rank_token_offsets,
                       expert_offsets, reinterpret_cast<const int32_t *>(ws),
                       reinterpret_cast<const int32_t *>(ws + w.tile_cnt),
                       reinterpret_cast<const int32_t *>(ws + w.slot_rank), capacity, recv_x,
                       recv_scales, recv_weights, row_src, status);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (d.A > 1) {
    hipLaunchKernelGGL(pad_fill_kernel, dim3(d.E, kPadSplit), dim3(kBlock), 0, stream, d, fp8,
                       zero_padding, reinterpret_cast<const int32_t *>(ws), expert_offsets,
                       reinterpret_cast<const int32_t *>(ws + w.cnt), capacity, recv_x,
                       recv_scales, ne_topk_weights != nullptr ? recv_weights : nullptr, row_src,
                       status);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_combine_ranked(const Dims &d, int64_t capacity, int64_t ranked_capacity,
                                 const uint16_t *y, const int32_t *tok_slot_row,
                                 const int32_t *ne_topk_idx, const float *ne_topk_weights,
                                 const int32_t *ne_src, const int32_t *rank_token_offsets,
                                 const int32_t *tok_rank_row, float *partials, uint16_t *out,
                                 hipStream_t stream) {
  const int32_t nchunks = (d.H + kCombineCols - 1) / kCombineCols;
  if (ranked_capacity > 0) {
    const int64_t items = ranked_capacity * nchunks;
    const dim3 grid((unsigned)((items + kWavesPerBlock - 1) / kWavesPerBlock));
    // KB = 8 only for a grid the chip holds at once: a non-expanded row has
    // few local slots (1.5 to 2 of 8 in the workloads), so a wide batch is
    // mostly empty entries, and as the tail of a large grid (as combine_kernel
    // takes it) it measured slower (Large 1083 -> 1093 us).  One kernel
    // holding both widths also measured slower than either alone.
    const bool wide = items <= kChipWaves;
    auto kernel = ne_topk_weights != nullptr
                      ? (wide ? combine_ranked_partial_kernel<true, 8>
                              : combine_ranked_partial_kernel<true, 1>)
                      : (wide ? combine_ranked_partial_kernel<false, 8>
                              : combine_ranked_partial_kernel<false, 1>);
    hipLaunchKernelGGL(kernel, grid, dim3(kBlock), 0, stream, d, nchunks, capacity,
                       ranked_capacity, y, tok_slot_row, ne_topk_idx, ne_topk_weights, ne_src,
                       rank_token_offsets, partials);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (d.T > 0) {
    const int64_t items = (int64_t)d.T * nchunks;
    const dim3 grid((unsigned)((items + kWavesPerBlock - 1) / kWavesPerBlock));
    hipLaunchKernelGGL(combine_ranked_sum_kernel, grid, dim3(kBlock), 0, stream, d, nchunks,
                       ranked_capacity, partials, tok_rank_row, out);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace ep
