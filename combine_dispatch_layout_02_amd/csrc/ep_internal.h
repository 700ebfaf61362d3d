// ep_internal.h -- launcher interface between the C ABI (ep_abi.hip) and the
// kernels.  Not installed; callers use include/ep.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ep {

// Workspace layout (bytes from the workspace base; every region 256-aligned).
//   ctrl        : u32[64]            [0] error flags
//   tile_count  : i32[tiles][E+R+N]  per tile: expert pair counts (then, after
//                                    the scan, the exclusive prefix of expert e
//                                    over earlier tiles), rank and node token
//                                    counts
//   local_rank  : i32[T * k]         plan word of a pair: (expert << kPlanLrBits)
//                                    | rank of the pair among the same-expert
//                                    pairs of its tile that precede it; -1:
//                                    masked.  A copy that reuses the plan
//                                    checks the expert against topk_idx.
//   plan_offset : i32[E + 1]         expert segment starts
//   rank_mask   : u64[tiles][R][TW]  (token, rank) rows only: per tile, rank
//                                    and 64-token wave of the tile (TW =
//                                    ceil(tile_tokens / 64) waves), bit i set
//                                    when the wave's token i reaches the rank
//   plan_rank_offset : i32[R + 1]    (token, rank) region starts
//   tile_pairs  : int2[E][tiles]     per expert e and tile u: {pairs of u with
//                                    an expert below e, pairs of u with e}
//                                    (layout + dispatch in one call,
//                                    multi-tile batches)
//   rank_pairs  : int2[R][tiles]     the same per rank for (token, rank) rows:
//                                    {tokens of u reaching ranks below r,
//                                    tokens of u reaching r}
// A tile holds tile_tokens whole tokens (tile_tokens * k <= count_threads
// pairs, one thread per pair).
constexpr int kWsRegions = 8;   // ctrl, tile_count, local_rank, plan_offset, rank_mask,
                                // plan_rank_offset, tile_pairs, rank_pairs (in this order)
struct WsLayout {
    size_t ctrl, tile_count, local_rank, plan_offset, rank_mask, plan_rank_offset, tile_pairs, rank_pairs,
        total;
    size_t region_bytes[kWsRegions];   // bytes each region needs (its offset above, 256-aligned)
    int tiles;           // ceil(T / tile_tokens)
    int tile_tokens;
    int tile_waves;      // ceil(tile_tokens * k / 64): waves that own pair masks
    int count_threads;   // tile_waves * 64
    int tile_token_waves;   // ceil(tile_tokens / 64): words per (tile, rank) of rank_mask
};

constexpr int kCtrlWords = 64;
constexpr uint32_t kErrBadExpert = 0x1u;
constexpr uint32_t kErrBadSlot = 0x2u;   // internal consistency check of the plan
constexpr uint32_t kErrRankOverflow = 0x4u;
constexpr uint32_t kErrStalePlan = 0x8u;   // topk_idx differs from the planned one
constexpr int kPlanLrBits = 16;            // local ranks < pairs per tile <= 2^16; experts < 2^15

struct Shape {
    int64_t T;
    int H, E, R, N, k;
    int x_fmt, y_fmt;
    int M;   // rank_capacity: 0 compacted layout, > 0 RANK_MAJOR
    int rank_rows;   // 1: the layout also plans (token, rank) receive rows
    int64_t rows() const { return M > 0 ? (int64_t)R * M : T * k; }   // receive rows (pairs)
    int64_t rank_rows_cap() const { return T * (k < R ? k : R); }      // (token, rank) rows
};

WsLayout ws_layout(const Shape &s);

// Dynamic LDS bytes per workgroup of the launches that take it (the same
// functions the launchers use): the count kernel; the single-launch layout +
// dispatch forms (threads per block through *threads); the totals block of
// the copies that scan the tile counts.
size_t plan_count_lds(const Shape &s, const WsLayout &L);
size_t fused_dispatch_lds(const Shape &s, int *threads);
size_t fused_ranks_lds(const Shape &s, int *threads);
size_t scan_copy_lds(const Shape &s);

// Kernel launchers; every one enqueues on `stream` and returns the launch status.
hipError_t launch_ws_init(uint32_t *ws, size_t words, hipStream_t stream);

// Layout counts (outputs may be null) and the dispatch plan in the workspace.
// count_only: the count launch alone, which also writes tile_pairs (for
// launch_dispatch_scan_copy) or, with rank rows, rank_pairs (for
// launch_dispatch_ranks_scan); multi-tile batches.
hipError_t launch_plan(const Shape &s, const WsLayout &L, const int64_t *topk_idx,
                       int32_t *per_rank, int32_t *per_expert, uint8_t *in_rank,
                       int32_t *per_node, int64_t *algo, char *ws, hipStream_t stream,
                       bool count_only = false);

hipError_t launch_dispatch_copy(const Shape &s, const WsLayout &L, const void *x,
                                const float *x_scales, const int64_t *topk_idx,
                                const float *topk_w, void *recv_x, float *recv_x_scales,
                                int32_t *recv_src_idx, float *recv_topk_w, int32_t *token_slot,
                                int32_t *expert_offset, char *ws, hipStream_t stream);

// Layout + dispatch of a multi-tile batch in two launches: the count launch
// (launch_plan with count_only) and the copy, which rebuilds the segment
// starts and prefixes over tiles from the tile counts (each wave for its own
// slots) while one extra block writes the layout totals (outputs may be null)
// and the handle's segment starts.  scan_in_copy_fits tells whether a shape
// qualifies (compacted layout, no rank rows, 2 ... kScanCopyMaxTiles tiles).
constexpr int kScanCopyMaxTiles = 256;
bool scan_in_copy_fits(const Shape &s, const WsLayout &L);
hipError_t launch_dispatch_scan_copy(const Shape &s, const WsLayout &L, const void *x,
                                     const float *x_scales, const int64_t *topk_idx,
                                     const float *topk_w, void *recv_x, float *recv_x_scales,
                                     int32_t *recv_src_idx, float *recv_topk_w, int32_t *token_slot,
                                     int32_t *expert_offset, int32_t *per_rank, int32_t *per_expert,
                                     int32_t *per_node, int64_t *algo, char *ws, hipStream_t stream);

// Cached dispatch: rows placed by a previous dispatch's handle (token_slot
// [T][k], or token_rank_slot [T][R] for (token, rank) rows).
hipError_t launch_dispatch_cached(const Shape &s, const void *x, const float *x_scales,
                                  const int32_t *token_slot, void *recv_x, float *recv_x_scales,
                                  hipStream_t stream);
hipError_t launch_dispatch_ranks_cached(const Shape &s, const void *x, const float *x_scales,
                                        const int32_t *token_rank_slot, void *recv_x,
                                        float *recv_x_scales, hipStream_t stream);

// Single-launch layout + dispatch (compacted layout, T * k <= 2048 pairs):
// fused_dispatch_fits tells whether a shape qualifies.  Layout outputs may be
// null (all together); the workspace plan is neither read nor written.
bool fused_dispatch_fits(const Shape &s);
hipError_t launch_dispatch_fused(const Shape &s, const void *x, const float *x_scales,
                                 const int64_t *topk_idx, const float *topk_w, void *recv_x,
                                 float *recv_x_scales, int32_t *recv_src_idx, float *recv_topk_w,
                                 int32_t *token_slot, int32_t *expert_offset, int32_t *per_rank,
                                 int32_t *per_expert, uint8_t *in_rank, int32_t *per_node,
                                 int64_t *algo, uint32_t *ctrl, hipStream_t stream);

// Tokens [0, n) whose receive rows the dispatch stores plain (they stay in
// the memory-side cache for the combine); the others are stored non-temporal.
int64_t cached_tokens(const Shape &s);

hipError_t launch_combine(const Shape &s, const void *expert_out, const uint8_t *expert_scales,
                          const int32_t *token_slot, const float *topk_w, void *y,
                          hipStream_t stream);

// (token, rank) receive layout
hipError_t launch_dispatch_ranks(const Shape &s, const WsLayout &L, const void *x,
                                 const float *x_scales, const int64_t *topk_idx,
                                 const float *topk_w, void *recv_x, float *recv_x_scales,
                                 int32_t *recv_src_idx, int32_t *recv_topk_idx, float *recv_topk_w,
                                 int32_t *token_rank_slot, int32_t *rank_offset, const char *ws,
                                 hipStream_t stream);

// Layout + (token, rank) dispatch of a multi-tile batch in two launches:
// launch_plan with count_only, then this copy, which rebuilds each region
// start and prefix over tiles from rank_pairs while one extra block writes
// the layout totals and the handle's region starts.  ranks_scan_fits: rank
// rows, 2 ... kScanCopyMaxTiles tiles.
bool ranks_scan_fits(const Shape &s, const WsLayout &L);
hipError_t launch_dispatch_ranks_scan(const Shape &s, const WsLayout &L, const void *x,
                                      const float *x_scales, const int64_t *topk_idx, const float *topk_w,
                                      void *recv_x, float *recv_x_scales, int32_t *recv_src_idx,
                                      int32_t *recv_topk_idx, float *recv_topk_w, int32_t *token_rank_slot,
                                      int32_t *rank_offset, int32_t *per_rank, int32_t *per_expert,
                                      int32_t *per_node, int64_t *algo, char *ws, hipStream_t stream);

// Single-launch layout + (token, rank) dispatch (T * k <= 2048 pairs, rank
// rows); the workspace plan is neither read nor written.
bool fused_ranks_fits(const Shape &s);
hipError_t launch_dispatch_ranks_fused(const Shape &s, const void *x, const float *x_scales,
                                       const int64_t *topk_idx, const float *topk_w, int32_t *per_rank,
                                       int32_t *per_expert, uint8_t *in_rank, int32_t *per_node,
                                       int64_t *algo, void *recv_x, float *recv_x_scales,
                                       int32_t *recv_src_idx, int32_t *recv_topk_idx, float *recv_topk_w,
                                       int32_t *token_rank_slot, int32_t *rank_offset, uint32_t *ctrl,
                                       hipStream_t stream);

hipError_t launch_expert_reduce_ranks(const Shape &s, const void *recv_x, const float *recv_scales,
                                      const int32_t *rank_offset, const int32_t *recv_topk_idx,
                                      const float *recv_topk_w, const float *factor,
                                      uint16_t *partial, hipStream_t stream);

hipError_t launch_combine_ranks(const Shape &s, const uint16_t *partial,
                                const int32_t *token_rank_slot, void *y, hipStream_t stream);

hipError_t launch_quant_fp8(int64_t rows, int H, const uint16_t *x, uint8_t *q, float *scales,
                            hipStream_t stream);

hipError_t launch_expert_scale_bf16(const Shape &s, const int32_t *expert_offset,
                                    const float *factor, const uint16_t *recv, uint16_t *out,
                                    hipStream_t stream);

hipError_t launch_expert_requant_mxfp8(const Shape &s, const int32_t *expert_offset,
                                       const float *factor, const uint8_t *recv_q,
                                       const float *recv_scales, uint8_t *out_q,
                                       uint8_t *out_e8m0, hipStream_t stream);

hipError_t launch_expert_requant_nvfp4(const Shape &s, const int32_t *expert_offset,
                                       const float *factor, const uint16_t *recv, uint8_t *out_q,
                                       uint16_t *out_scales, hipStream_t stream);

hipError_t launch_calib_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);

// Streaming kernels (stream.hip): kind 0 read, 1 write, 2 copy; nt selects
// non-temporal loads / stores.  Whole chunks of `chunk` bytes, `waves` waves.
hipError_t launch_stream(int kind, bool nt, const void *src, void *dst, size_t bytes, size_t chunk, int waves,
                         hipStream_t stream);

// Waves per token for the row kernels: the smallest power of two that gives
// `target` waves in all, never so many that a wave has fewer than 64 row
// vectors.
int waves_per_token(int64_t T, int64_t row_vectors, int64_t target);

}  // namespace ep
