/*
 * ep.h -- C ABI of the MI355X (gfx950) MoE expert-parallel dispatch / combine
 * library (libep_hip.so).
 *
 * One GPU's share of the exchange at its real shape: one source's T tokens are
 * routed to E experts spread over R virtual ranks grouped into N virtual
 * nodes.  Every destination is a contiguous region of ONE receive allocation:
 * expert segments lie back to back in expert order, a virtual rank's region
 * is the union of its experts' segments, a virtual node's region the union of
 * its ranks' regions.
 *
 * Sources (web pages; sections named, no line numbers):
 *   [MORI]  "MORI-EP Benchmark": "Bandwidth Computation" (RDMA bandwidth, Algo
 *           BW vs Physical BW, NVL / XGMI bandwidth), "Why DeepEP and Mori RDMA
 *           token counts are equivalent" (Steps 1-3), "Combine", and the
 *           reference script print_bw_values.py (rank layout, fp8 factor).
 *   [MEB]   "MoE-EP Benchmark" README, "Environment reference"
 *           (MEGA_COMBINE_DTYPE: mxfp8 = 32 e4m3 + e8m0 scale).
 *   [PR860] MSCCL++ pull request 860: get_dispatch_layout / dispatch /
 *           combine(handle) surface (PR body, "Scope"); combine consumes the
 *           receiver-side layout returned by dispatch (internode combine
 *           fix commit); TOKEN_MAJOR compacted prefix offsets (RANK_MAJOR
 *           commit); one copy per dispatched token per expert (LL combine
 *           byte commit); capacity-sized buffers instead of a CPU wait for
 *           exact receive counts (DeepEP V2 graph-capture comment); DeepEP's
 *           expanded receive layout, one row per (token, source rank) (the
 *           high-throughput path; BW accounting commit); cached_notify and
 *           the previous handle (cached dispatch).
 *
 * Conventions for every call:
 *   - Data pointers are DEVICE pointers owned by the caller, except where a
 *     parameter says "host".  The library never allocates device memory,
 *     never synchronizes (except ep_check), and enqueues work only on
 *     `stream` (a hipStream_t; NULL = the null stream).
 *   - Calls return EP_OK (0) or a negative ep_status; argument errors are
 *     detected on the host before anything is enqueued.  No exception
 *     crosses the ABI.
 *   - topk_idx is [T, k] int64 row-major; a negative id marks a masked slot
 *     and is skipped everywhere ([MORI] script pads -1 entries); an id >= E
 *     is invalid: it is treated as masked and raises EP_ERRFLAG_BAD_EXPERT in
 *     the workspace's error word (read back with ep_check).
 *   - bf16 values are raw 16-bit patterns; e4m3 (OCP "fn") and e8m0 are bytes.
 *   - Calls that share one workspace must be ordered (same stream, or
 *     explicit events); two concurrent calls on one workspace race.
 *   - Plain C: the header needs only <stddef.h> and <stdint.h>; streams are
 *     passed as void *.
 */
#ifndef EP_HIP_H
#define EP_HIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EP_ABI_VERSION 8

/* Status codes. */
enum ep_status {
    EP_OK = 0,
    EP_EINVAL = -1,      /* shape or argument out of the supported range */
    EP_EALIGN = -2,      /* a row buffer is not 16-byte aligned */
    EP_EWORKSPACE = -3,  /* workspace missing or smaller than ep_workspace_bytes */
    EP_EHIP = -4,        /* a HIP runtime call or kernel launch failed */
    EP_EDEVICE = -5      /* a kernel flagged bad input (ep_check) */
};

/* Bits of the device error word. */
#define EP_ERRFLAG_BAD_EXPERT 0x1u
#define EP_ERRFLAG_BAD_SLOT   0x2u   /* internal: a computed slot fell outside the receive rows (skipped) */
#define EP_ERRFLAG_RANK_OVERFLOW 0x4u /* RANK_MAJOR: a rank received more pairs than rank_capacity (dropped) */
#define EP_ERRFLAG_STALE_PLAN 0x8u    /* a dispatch reusing the layout call's plan met a topk_idx that differs
                                         from the planned one (the pairs / tokens concerned get no rows) */

/* Payload formats. */
enum ep_format {
    EP_FMT_BF16 = 0,         /* 2 bytes per element */
    EP_FMT_FP8_S128 = 1,     /* e4m3 bytes + one fp32 scale per 128 elements ([MORI] script's fp8 factor) */
    EP_FMT_MXFP8 = 2,        /* e4m3 bytes + one e8m0 byte per 32 elements ([MEB]) */
    EP_FMT_NVFP4 = 3         /* e2m1 nibbles (2 per byte, even element low) + one bf16 scale
                                per 16 elements ([MEB] "16e2m1xbf16") */
};

/* Problem shape.  Supported range (else EP_EINVAL):
 *   0 <= num_tokens, num_tokens * num_topk < 2^31;
 *   1 <= num_topk <= 32;
 *   1 <= num_experts <= 4096, num_experts % num_ranks == 0;
 *   1 <= num_ranks <= 64, 1 <= num_nodes <= num_ranks, num_ranks % num_nodes == 0;
 *   hidden >= 8, hidden % 8 == 0 (16-byte bf16 row vectors);
 *   fp8 / mxfp8 / nvfp4 formats: hidden % 128 == 0;
 *   x_format in {BF16, FP8_S128}; y_format in {BF16, MXFP8, NVFP4};
 *   rank_capacity >= 0, num_ranks * rank_capacity < 2^31;
 *   rank_rows in {0, 1}; with 1, num_tokens * num_ranks < 2^31.
 * Receive rows ("rows" below): T*k for the compacted layout (rank_capacity
 * 0), num_ranks * rank_capacity for the RANK_MAJOR layout.  The (token,
 * rank) layout (rank_rows 1, the ep_*_ranks calls) has T * min(k, R) rows. */
typedef struct ep_shape {
    int64_t num_tokens;   /* T: tokens of this source */
    int32_t hidden;       /* H: elements per token row */
    int32_t num_experts;  /* E */
    int32_t num_ranks;    /* R: virtual ranks; expert e lives on rank e / (E/R) */
    int32_t num_nodes;    /* N: virtual nodes; expert e lives on node e / (E/N) */
    int32_t num_topk;     /* k */
    int32_t x_format;     /* format of dispatched rows: EP_FMT_BF16 | EP_FMT_FP8_S128 */
    int32_t y_format;     /* format of the rows combine reads: EP_FMT_BF16 | EP_FMT_MXFP8 | EP_FMT_NVFP4 */
    int32_t rank_capacity;/* 0: compacted (token-major) receive layout; M > 0: RANK_MAJOR,
                             rank r owns receive rows [r*M, (r+1)*M) ([PR860] RANK_MAJOR
                             commit: a fixed [num_ranks, max_tokens_per_rank, hidden]
                             slot instead of the compacted prefix offset) */
    int32_t rank_rows;    /* 1: ep_dispatch_layout also plans the (token, rank) receive
                             rows the ep_*_ranks calls use; 0: it does not */
} ep_shape;

/* Version of this ABI (EP_ABI_VERSION). */
int ep_abi_version(void);

/* Human-readable text of a status code (static storage). */
const char *ep_strerror(int status);

/* Host-only check of a shape against the supported range. */
int ep_validate_shape(const ep_shape *shape);

/* Host-only: bytes of device workspace ep_dispatch_layout / ep_dispatch need
 * for this shape (written to *bytes).  The workspace holds the error word,
 * per-tile expert / rank / node counts, each pair's rank inside its tile and
 * the expert segment starts (the dispatch plan). */
int ep_workspace_bytes(const ep_shape *shape, size_t *bytes);

/* Zero a workspace (a fill kernel on `stream`, no memset node): clears the
 * error word.  Call once after allocation. */
int ep_workspace_init(void *ws, size_t ws_bytes, void *stream);

/*
 * Layout pass ([MORI] "Why ... equivalent" Steps 1-3, "Algo BW vs Physical
 * BW"; [PR860] get_dispatch_layout).  For each token: the set of ranks and
 * the set of nodes its valid experts live on (rank = e / (E/R), node =
 * e / (E/N)), duplicates collapsed.  Outputs (device, written in full):
 *   num_tokens_per_rank   [R] int32: tokens whose rank set contains r
 *   num_tokens_per_expert [E] int32: valid (t, j) pairs routed to e
 *   is_token_in_rank      [T, R] uint8 (0/1) row-major
 *   num_tokens_per_node   [N] int32: tokens whose node set contains n
 *   rdma_algo_token_count [1] int64: deduplicated (token, node) pairs, local
 *                         node included (= sum of num_tokens_per_node)
 * The physical count algo * (N-1)/N and the exact per-source count are host
 * arithmetic (ep_accounting).  Deterministic: integer counts only.
 * The call also leaves the dispatch plan of this topk_idx (expert segment
 * starts, per-tile prefixes, ranks inside tiles) in the workspace, where
 * ep_dispatch_from_layout uses it.
 */
int ep_dispatch_layout(const ep_shape *shape, const int64_t *topk_idx,
                       int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                       uint8_t *is_token_in_rank, int32_t *num_tokens_per_node,
                       int64_t *rdma_algo_token_count,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * Dispatch: slot assignment plus the row permutation ([PR860] TOKEN_MAJOR
 * compacted prefix offsets; [MORI] "NVL / XGMI bandwidth": received rows are
 * token rows).  Every valid pair (t, j) with expert e gets slot
 *     token_slot[t,j] = expert_offset[e] + #{valid (t',j') before (t,j) in
 *                       row-major order with expert e}
 * (a stable counting sort: expert segments in expert order, ascending t
 * inside a segment), and recv_x[slot] is a bitwise copy of row t.  Capacity
 * is T*k rows, so no receive count has to reach the host first.
 * RANK_MAJOR (rank_capacity M > 0): the same order inside each rank, but rank
 * r's rows start at r*M instead of expert_offset[r*E/R]; a pair whose place
 * inside its rank is >= M is dropped (token_slot -1) and raises
 * EP_ERRFLAG_RANK_OVERFLOW.  expert_offset keeps the compacted segment
 * starts, so expert e's rows in rank r's block start at
 * r*M + expert_offset[e] - expert_offset[r*E/R].
 *   x             [T, H] bf16 (x_format BF16) or [T, H] e4m3 (FP8_S128)
 *   x_scales      [T, H/128] fp32 for FP8_S128, else NULL
 *   topk_idx      [T, k] int64
 *   topk_w        [T, k] fp32 (copied bitwise into recv_topk_w)
 *   recv_x        [rows, H] same element type as x (16-byte aligned); rows no
 *                 pair lands in are left untouched
 *   recv_x_scales [rows, H/128] fp32 for FP8_S128, else NULL
 *   recv_src_idx  [rows] int32: source token of each slot
 *   recv_topk_w   [rows] fp32: weight of each slot's pair
 *   token_slot    [T, k] int32: slot of each pair, -1 if masked (handle)
 *   expert_offset [E+1] int32: segment starts, expert_offset[E] = valid
 *                 pairs (handle); rank r's region is
 *                 [expert_offset[r*E/R], expert_offset[(r+1)*E/R]).
 * Deterministic: no order-dependent atomics.  ep_dispatch plans by itself
 * (a small batch, as in ep_dispatch_with_layout, in one launch); the plan it
 * may leave in the workspace is not one ep_dispatch_from_layout may reuse.
 */
int ep_dispatch(const ep_shape *shape, const void *x, const float *x_scales,
                const int64_t *topk_idx, const float *topk_w,
                void *recv_x, float *recv_x_scales, int32_t *recv_src_idx, float *recv_topk_w,
                int32_t *token_slot, int32_t *expert_offset,
                void *ws, size_t ws_bytes, void *stream);

/*
 * Layout and dispatch in one call: the outputs of ep_dispatch_layout and of
 * ep_dispatch together ([PR860] Scope: get_dispatch_layout followed by
 * dispatch).  A small batch -- T * k <= 2048 pairs, compacted layout
 * (rank_capacity 0), rank_rows 0 -- runs as ONE kernel launch: one block
 * computes the layout counts and the segment starts while every other wave
 * finds its token's slots by counting the pairs that sort before them (the
 * stable counting sort's position); results are identical to the two calls.
 * Other batches of 2 to 256 plan tiles (up to T * k = 262144 pairs; either
 * layout) run two launches: the count kernel, which also writes per (expert,
 * tile) the tile's pairs of smaller experts and of the expert, and the copy,
 * whose waves rebuild each slot's position from those sums (and, for
 * RANK_MAJOR, the start of the slot's rank from those of the rank's first
 * expert) and whose first block writes the layout totals.  One tile, or
 * more than 256: the layout launches, then the copy.  Afterwards the
 * workspace holds no plan that ep_dispatch_from_layout may reuse.
 * Arguments: as ep_dispatch_layout and ep_dispatch.
 */
int ep_dispatch_with_layout(const ep_shape *shape, const void *x, const float *x_scales,
                            const int64_t *topk_idx, const float *topk_w, int32_t *num_tokens_per_rank,
                            int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank,
                            int32_t *num_tokens_per_node, int64_t *rdma_algo_token_count, void *recv_x,
                            float *recv_x_scales, int32_t *recv_src_idx, float *recv_topk_w,
                            int32_t *token_slot, int32_t *expert_offset, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments and results as ep_dispatch_with_layout, minus the workspace.
 * The plan lives in a static device array of EP_STATIC_SCRATCH_BYTES per
 * GPU, part of the library's code object (each GPU the library runs on holds
 * its copy until the process ends); nothing is allocated and nothing
 * allocating is called.
 *   - Shapes whose workspace (ep_workspace_bytes) exceeds
 *     EP_STATIC_SCRATCH_BYTES return EP_EWORKSPACE before any device work
 *     (about 4 M (token, slot) pairs at E = 256).
 *   - The first call on a device (the current device) looks the array up and
 *     clears its error word with a fill kernel on `stream`; make that first
 *     call outside stream capture.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's plan: calls that overlap on one GPU (other streams, other host
 *     threads) race and must be ordered by the caller.
 *   - Invalid expert ids are treated as masked and RANK_MAJOR overflows are
 *     dropped, as everywhere; their flags collect in the array's error word,
 *     which ep_check(NULL, 0, stream, &flags) reads and clears.
 */
#define EP_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
int ep_dispatch_with_layout_static(const ep_shape *shape, const void *x, const float *x_scales,
                                   const int64_t *topk_idx, const float *topk_w, int32_t *num_tokens_per_rank,
                                   int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank,
                                   int32_t *num_tokens_per_node, int64_t *rdma_algo_token_count, void *recv_x,
                                   float *recv_x_scales, int32_t *recv_src_idx, float *recv_topk_w,
                                   int32_t *token_slot, int32_t *expert_offset, void *stream);

/*
 * Dispatch that reuses the plan the preceding ep_dispatch_layout call on the
 * SAME workspace and the SAME topk_idx left there (stream-ordered before
 * this call): same arguments and results as ep_dispatch, minus the planning
 * launches.  The pages' cached dispatch ([PR860] cached_notify /
 * previous_handle) reuses a layout the same way.  Calling it without that
 * preceding layout call, or with a different topk_idx, gives unspecified
 * slots (the kernel still never writes outside [0, T*k) rows).  The plan
 * keeps each pair's expert, and the copy checks it against topk_idx: a pair
 * whose expert (or validity) differs from the planned one gets slot -1 and
 * no row, and the call raises EP_ERRFLAG_STALE_PLAN (ep_check).
 */
int ep_dispatch_from_layout(const ep_shape *shape, const void *x, const float *x_scales,
                            const int64_t *topk_idx, const float *topk_w,
                            void *recv_x, float *recv_x_scales, int32_t *recv_src_idx,
                            float *recv_topk_w, int32_t *token_slot, int32_t *expert_offset,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * Cached dispatch ([PR860] Scope: cached_notify; the dispatch that takes a
 * previous_handle): the rows of a previous dispatch's handle, for another
 * tensor of the same tokens -- recv_x[token_slot[t,j]] = x[t] (and the scale
 * rows for FP8_S128) -- with no layout work, no workspace and no metadata
 * writes.  token_slot is the [T, k] handle of ep_dispatch /
 * ep_dispatch_from_layout / ep_dispatch_with_layout for the same shape
 * (compacted or RANK_MAJOR); a slot outside [0, rows) is skipped.  x,
 * x_scales, recv_x, recv_x_scales: as for ep_dispatch.
 */
int ep_dispatch_cached(const ep_shape *shape, const void *x, const float *x_scales,
                       const int32_t *token_slot, void *recv_x, float *recv_x_scales, void *stream);

/*
 * Combine: the top-k weighted gather-reduce back into token order ([MORI]
 * "Combine": reverse of dispatch; [PR860] one copy per dispatched token per
 * expert, combine consumes the receiver-side layout from dispatch):
 *     acc = -0.0f; for j = 0..k-1 with s = token_slot[t,j] >= 0:
 *         acc = fmaf(topk_w[t,j], value(expert_out[s, h]), acc)
 *     y[t,h] = bf16_rne(acc)   (+0.0 if token t has no valid slot)
 * fp32 accumulation in top-k slot order, one rounding to bf16.
 * Combine does not depend on the receive layout: RANK_MAJOR and compacted
 * slots give bit-identical y ([PR860] RANK_MAJOR commit: the combine path is
 * layout-agnostic).
 *   expert_out        [rows, H] bf16 (y_format BF16), [rows, H] e4m3 (MXFP8) or
 *                     [rows, H/2] packed e2m1 (NVFP4); 16-byte aligned
 *   expert_out_scales [rows, H/32] e8m0 bytes for MXFP8 (value = e4m3 *
 *                     2^(e8m0 - 127)); [rows, H/16] bf16 bit patterns for NVFP4
 *                     (value = e2m1 * bf16, 4-byte aligned); NULL for BF16
 *   token_slot, topk_w: from the dispatch handle / the caller ([T, k]); a
 *                     slot outside [0, rows) is treated as masked
 *   y                 [T, H] bf16, 16-byte aligned
 */
int ep_combine(const ep_shape *shape, const void *expert_out, const uint8_t *expert_out_scales,
               const int32_t *token_slot, const float *topk_w, void *y, void *stream);

/* ---- the (token, rank) receive layout ----------------------------------- */

/*
 * Dispatch into (token, rank) rows, the high-throughput layout ([PR860]:
 * DeepEP's expanded receive layout, one row per (token, source rank) pair;
 * [MORI] "NVL / XGMI bandwidth": one received row per token and destination
 * rank, the rows num_tokens_per_rank counts).  A token reaches rank r when
 * one of its valid experts lives there; it then gets exactly one row in r's
 * region.  Regions lie back to back in rank order (rank_offset = exclusive
 * scan of num_tokens_per_rank), tokens ascending inside a region.
 * Requires shape->rank_rows == 1 and the plan that the preceding
 * ep_dispatch_layout call with the same shape, workspace and topk_idx left
 * in the workspace (stream-ordered before this call); without it the rows
 * are unspecified (the kernel still never writes outside the T*min(k,R)
 * receive rows).  The copy checks each token's planned rank set against
 * the one topk_idx gives: a token whose set differs gets no rows (its
 * token_rank_slot entries are -1), and the call raises
 * EP_ERRFLAG_STALE_PLAN (ep_check).
 *   x, x_scales, topk_idx, topk_w: as for ep_dispatch
 *   recv_x         [T*min(k,R), row] bf16 or e4m3 rows, 16-byte aligned; row
 *                  s < rank_offset[R] is a bitwise copy of x[recv_src_idx[s]]
 *   recv_x_scales  [T*min(k,R), H/128] fp32 (FP8_S128), else NULL
 *   recv_src_idx   [T*min(k,R)] source token of each row
 *   recv_topk_idx  [T*min(k,R), k] the token's top-k list as the row's rank r
 *                  sees it: e - r*(E/R) for slots whose expert lives on r, -1
 *                  for every other slot
 *   recv_topk_w    [T*min(k,R), k] the slot's weight there, 0 elsewhere
 *   token_rank_slot[T, R] handle: row of (t, r), -1 if t does not reach r
 *   rank_offset    [R + 1] handle: region starts; rank_offset[R] = rows used
 */
int ep_dispatch_ranks(const ep_shape *shape, const void *x, const float *x_scales,
                      const int64_t *topk_idx, const float *topk_w, void *recv_x,
                      float *recv_x_scales, int32_t *recv_src_idx, int32_t *recv_topk_idx,
                      float *recv_topk_w, int32_t *token_rank_slot, int32_t *rank_offset,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * Layout and (token, rank) dispatch in one call: the outputs of
 * ep_dispatch_layout and of ep_dispatch_ranks together (rank_rows 1).  A
 * small batch -- T * k <= 2048 pairs -- runs as ONE kernel launch: one block
 * computes the layout counts and the region starts while every other block
 * (one token) finds the token's rows by counting the tokens and ranks that
 * come before them; results are identical to the two calls.  Larger batches
 * of up to 256 plan tiles run two launches (the count kernel, which also
 * writes per (rank, tile) the tile's tokens of smaller ranks and of the
 * rank, then the copy, which sums them); beyond that, the two layout
 * launches, then the copy.  Afterwards the workspace holds no plan that
 * ep_dispatch_ranks may reuse.  Arguments: as ep_dispatch_layout
 * and ep_dispatch_ranks.
 */
int ep_dispatch_ranks_with_layout(const ep_shape *shape, const void *x, const float *x_scales,
                                  const int64_t *topk_idx, const float *topk_w, int32_t *num_tokens_per_rank,
                                  int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank,
                                  int32_t *num_tokens_per_node, int64_t *rdma_algo_token_count, void *recv_x,
                                  float *recv_x_scales, int32_t *recv_src_idx, int32_t *recv_topk_idx,
                                  float *recv_topk_w, int32_t *token_rank_slot, int32_t *rank_offset,
                                  void *ws, size_t ws_bytes, void *stream);

/*
 * Cached (token, rank) dispatch: recv_x[token_rank_slot[t,r]] = x[t] for the
 * [T, R] handle of a previous ep_dispatch_ranks of the same shape (rank_rows
 * 1), with the scale rows for FP8_S128; no workspace, no metadata writes; a
 * row outside [0, T*min(k,R)) is skipped.
 */
int ep_dispatch_ranks_cached(const ep_shape *shape, const void *x, const float *x_scales,
                             const int32_t *token_rank_slot, void *recv_x, float *recv_x_scales,
                             void *stream);

/*
 * Expert stage of the (token, rank) layout (outside dispatch and combine: the
 * destination applies its own experts' weights and returns one partial row
 * per received row).  For rows s < rank_offset[R], r the row's rank:
 *     acc = -0.0f; for j = 0..k-1 with l = recv_topk_idx[s,j] >= 0:
 *         o = bf16_rne(v(s,h) * factor[r*(E/R) + l])   (bf16_rne(v) if factor NULL)
 *         acc = fmaf(recv_topk_w[s,j], o, acc)
 *     partial[s,h] = bf16_rne(acc)
 * v is the received bf16 element, or e4m3(q) times its row's fp32 scale for
 * FP8_S128 rows.  Requires rank_rows == 1 and y_format BF16.
 *   recv_x, recv_x_scales, rank_offset, recv_topk_idx, recv_topk_w: from
 *                  ep_dispatch_ranks;  factor [E] fp32 or NULL
 *   partial        [T*min(k,R), H] bf16, 16-byte aligned; rows past
 *                  rank_offset[R] are left untouched
 */
int ep_expert_reduce_ranks(const ep_shape *shape, const void *recv_x, const float *recv_x_scales,
                           const int32_t *rank_offset, const int32_t *recv_topk_idx,
                           const float *recv_topk_w, const float *factor, uint16_t *partial,
                           void *stream);

/*
 * Combine of the (token, rank) layout ([PR860]: combine runs dispatch in
 * reverse over the receiver-side layout; the partials arrive weighted):
 *     acc = -0.0f; for r = 0..R-1 with s = token_rank_slot[t,r] >= 0:
 *         acc = acc + f32(partial[s, h])
 *     y[t,h] = bf16_rne(acc)   (+0.0 if token t reaches no rank)
 * fp32 adds in rank order, one rounding to bf16.  Requires rank_rows == 1
 * and y_format BF16.  A slot outside [0, T*min(k,R)) counts as not reached.
 *   partial [T*min(k,R), H] bf16; token_rank_slot [T, R]; y [T, H] bf16
 *   (16-byte aligned rows)
 */
int ep_combine_ranks(const ep_shape *shape, const uint16_t *partial,
                     const int32_t *token_rank_slot, void *y, void *stream);

/* Synchronize `stream`, read and clear the workspace error word; returns
 * EP_EDEVICE if any kernel flagged bad input (e.g. an expert id >= E), and
 * writes the flags to *flags (host) when flags is not NULL.  ws = NULL
 * (ws_bytes ignored) reads and clears the error word of the current
 * device's static scratch, the one ep_dispatch_with_layout_static uses
 * (flags 0 and EP_OK if no such call has run on that device). */
int ep_check(void *ws, size_t ws_bytes, void *stream, uint32_t *flags);

/* ---- payload conversion and the workloads' expert stage ------------------ */

/* fp8 rows for dispatch ([MORI] script's fp8 factor: one byte per element and
 * one fp32 scale per 128).  Per (row, 128-group): amax = max |x|, scale =
 * amax / 448 (IEEE division; 1 for an all-zero group), q = e4m3_rne_sat(x /
 * scale).  x [rows, H] bf16; q [rows, H] bytes; scales [rows, H/128] fp32.
 * Requires H % 128 == 0. */
int ep_quant_fp8_s128(int64_t rows, int32_t hidden, const uint16_t *x, uint8_t *q,
                      float *scales, void *stream);

/* Expert stage of the workloads (outside dispatch and combine), compacted
 * layout only (rank_capacity 0, else EP_EINVAL).  Rows [0, expert_offset[E])
 * of a receive buffer with capacity T*k; row s belongs to the expert whose
 * segment holds s.
 *   scale_bf16: out[s] = bf16_rne(f32(recv[s]) * factor[e(s)]).
 *   requant_mxfp8: v = e4m3(q[s]) * scales128[s] (times factor[e(s)] when
 *     factor != NULL); per 32-group X = clamp(floor(log2 amax) - 8, -127,
 *     127) (-127 for an all-zero group, OCP Microscaling shared exponent),
 *     out_q = e4m3_rne_sat(v * 2^-X), out_e8m0 = X + 127 ([MEB]). */
/* nvfp4 re-encode of bf16 receive rows (the expert stage for an NVFP4
 * combine payload): v = f32(recv[s]) (times factor[e(s)] when factor !=
 * NULL); per 16-group s = bf16_rne(amax / 6), 1.0 when that is zero;
 * element e2m1_rne_sat(v / s).  out_q [rows, H/2], out_scales [rows, H/16]
 * bf16 bits.  Compacted layout only; requires H % 128 == 0. */
int ep_expert_requant_nvfp4(const ep_shape *shape, const int32_t *expert_offset,
                            const float *factor, const uint16_t *recv, uint8_t *out_q,
                            uint16_t *out_scales, void *stream);
int ep_expert_scale_bf16(const ep_shape *shape, const int32_t *expert_offset,
                         const float *factor, const uint16_t *recv, uint16_t *out, void *stream);
int ep_expert_requant_mxfp8(const ep_shape *shape, const int32_t *expert_offset,
                            const float *factor, const uint8_t *recv_q, const float *recv_scales,
                            uint8_t *out_q, uint8_t *out_e8m0, void *stream);

/* ---- accounting (host arithmetic on host copies of the layout counts) ---- */

/* [MORI] "Bandwidth Computation": RDMA algo tokens are the layout's (token,
 * node) pairs, local node included; physical = algo * (N-1)/N; the exact
 * per-source physical count drops the pairs whose node is own_node; NVL rows
 * of one source are its (token, rank) pairs; bytes = rows x bytes of one row
 * (bf16: 2 per element; fp8: 1 per element + one fp32 scale per 128, whose
 * ratio to bf16 is the pages' fp8 factor); the combine returns the same rows.
 * hbm_* are the minimum HBM bytes of one call on this shape -- every row it
 * moves and every index / weight element it reads or writes, once -- split
 * into bytes read (_read_) and written (_write_), given the valid pair
 * count; hbm_*_ranks the same for the (token, rank) layout, whose rows are
 * nvl_tokens. */
typedef struct ep_accounting_t {
    int64_t rdma_algo_tokens;
    double rdma_physical_tokens;
    int64_t rdma_physical_tokens_exact;
    int64_t nvl_tokens;
    double dispatch_rdma_bytes_bf16;
    double dispatch_nvl_bytes_bf16;
    double combine_rdma_bytes_bf16;
    double combine_nvl_bytes_bf16;
    double fp8_factor;
    double dispatch_rdma_bytes_fp8;
    double dispatch_nvl_bytes_fp8;
    double hbm_layout_bytes;
    double hbm_dispatch_bytes;
    double hbm_combine_bytes;
    double hbm_dispatch_ranks_bytes;
    double hbm_combine_ranks_bytes;
    double hbm_layout_read_bytes, hbm_layout_write_bytes;
    double hbm_dispatch_read_bytes, hbm_dispatch_write_bytes;
    double hbm_combine_read_bytes, hbm_combine_write_bytes;
    double hbm_dispatch_ranks_read_bytes, hbm_dispatch_ranks_write_bytes;
    double hbm_combine_ranks_read_bytes, hbm_combine_ranks_write_bytes;
} ep_accounting_t;

int ep_accounting(const ep_shape *shape, int32_t own_node, const int32_t *num_tokens_per_rank,
                  const int32_t *num_tokens_per_node, int64_t rdma_algo_token_count,
                  int64_t valid_pairs, ep_accounting_t *out);

/* ---- plan introspection (host only) --------------------------------------- */

/* What the library will use for a shape, computed by the same functions its
 * launchers use: the workspace regions (offset and bytes each needs; in this
 * order: error word, tile counts, pair ranks inside their tiles, segment
 * starts, (token, rank) masks, (token, rank) region starts, per-expert tile
 * pairs, per-rank tile pairs -- a region a shape does not use has 0 bytes),
 * the plan tiling, and the dynamic LDS bytes per workgroup of the launches
 * that take it (0 where the shape does not use that launch): the count
 * kernel, the single-launch layout + dispatch form (with its threads per
 * workgroup) and the copy that scans the tile counts.  EP_EINVAL for a shape
 * outside the supported range. */
#define EP_PLAN_REGIONS 8
typedef struct ep_plan_info_t {
    size_t workspace_bytes;
    size_t region_offset[EP_PLAN_REGIONS];
    size_t region_bytes[EP_PLAN_REGIONS];
    int32_t tiles, tile_tokens, tile_waves, count_threads;
    size_t count_lds_bytes;
    size_t single_launch_lds_bytes;
    int32_t single_launch_threads;
    size_t scan_copy_lds_bytes;
} ep_plan_info_t;
int ep_plan_info(const ep_shape *shape, ep_plan_info_t *info);

/* ---- measurement helper --------------------------------------------------- */

/* Plain device copy of `bytes` bytes (16-byte aligned pointers, bytes % 16
 * == 0): a known-size reference for scaling hardware byte counters. */
int ep_calib_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Streaming kernels for measurement: the box's read, write and copy
 * ceilings, and a clean flush of the 256 MB memory-side cache (a plain
 * read of more than it holds evicts every line, writing back the dirty
 * ones, and leaves it clean).  `bytes` are walked in whole chunks of
 * `chunk_bytes` (a multiple of 1024, at most 1 MiB, dividing `bytes`);
 * wave w of `waves` (a multiple of 4, 4 <= waves <= 2^20) takes chunks w,
 * w + waves, ...; each wave instruction moves 1 KiB of one chunk.
 *   EP_STREAM_READ*  : reads src; dst is a 16-byte aligned sink of 16 bytes,
 *                      written only if the XOR of all data read equals a
 *                      fixed 128-bit value (it keeps the loads alive)
 *   EP_STREAM_WRITE* : writes a fixed pattern to dst; src must be NULL
 *   EP_STREAM_COPY*  : dst = src (buffers must not overlap)
 * The _NT kinds use non-temporal loads / stores.  16-byte aligned pointers.
 * Returns EP_EINVAL / EP_EALIGN on bad arguments, else the launch status. */
enum ep_stream_kind {
    EP_STREAM_READ = 0, EP_STREAM_READ_NT = 1,
    EP_STREAM_WRITE = 2, EP_STREAM_WRITE_NT = 3,
    EP_STREAM_COPY = 4, EP_STREAM_COPY_NT = 5
};
int ep_stream(int32_t kind, const void *src, void *dst, size_t bytes, size_t chunk_bytes,
              int32_t waves, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* EP_HIP_H */
