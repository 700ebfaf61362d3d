// ep_abi.hip -- the C ABI of libep_hip (declared in include/ep.h): argument
// validation on the host, workspace carving, kernel launches on the caller's
// stream.  Nothing here allocates device memory or synchronizes, except
// ep_check.
#include "ep.h"
#include "ep_internal.h"

#include <hip/hip_runtime.h>

#include <mutex>

#ifndef EP_PLAN_WAVES
#define EP_PLAN_WAVES 16   // waves (64 pairs each) per plan tile, at most
#endif

namespace {

using ep::Shape;
using ep::WsLayout;

// The current device's static scratch (ep_dispatch_with_layout_static), or
// null if no call has used it on that device yet; defined with the array.
int static_scratch_if_used(void **out);

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(const ep_shape *sh, Shape *out) {
    if (!sh) return EP_EINVAL;
    const int64_t T = sh->num_tokens;
    const int H = sh->hidden, E = sh->num_experts, R = sh->num_ranks, N = sh->num_nodes,
              k = sh->num_topk;
    if (T < 0 || k < 1 || k > 32) return EP_EINVAL;
    if (T * (int64_t)k >= (int64_t(1) << 31)) return EP_EINVAL;
    if (E < 1 || E > 4096 || R < 1 || R > 64 || N < 1 || N > R) return EP_EINVAL;
    if (E % R != 0 || R % N != 0) return EP_EINVAL;
    if (H < 8 || H % 8 != 0) return EP_EINVAL;
    if (sh->x_format != EP_FMT_BF16 && sh->x_format != EP_FMT_FP8_S128) return EP_EINVAL;
    if (sh->y_format != EP_FMT_BF16 && sh->y_format != EP_FMT_MXFP8 && sh->y_format != EP_FMT_NVFP4)
        return EP_EINVAL;
    if ((sh->x_format != EP_FMT_BF16 || sh->y_format != EP_FMT_BF16) && H % 128 != 0)
        return EP_EINVAL;
    if (sh->rank_capacity < 0 || (int64_t)R * sh->rank_capacity >= (int64_t(1) << 31)) return EP_EINVAL;
    if (sh->rank_rows != 0 && sh->rank_rows != 1) return EP_EINVAL;
    if (sh->rank_rows && T * (int64_t)R >= (int64_t(1) << 31)) return EP_EINVAL;
    if (out) {
        out->T = T;
        out->H = H;
        out->E = E;
        out->R = R;
        out->N = N;
        out->k = k;
        out->x_fmt = sh->x_format;
        out->y_fmt = sh->y_format;
        out->M = sh->rank_capacity;
        out->rank_rows = sh->rank_rows;
    }
    return EP_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? EP_OK : EP_EHIP; }

// Bytes of one token row of `H` elements in a payload format: the elements
// plus that row's share of scales (fp8: one fp32 per 128, as the MORI-EP
// Benchmark's fp8 factor counts them; mxfp8: one e8m0 byte per 32; nvfp4:
// one bf16 per 16).
double row_bytes(int fmt, int H) {
    const double h = (double)H;
    switch (fmt) {
        case EP_FMT_FP8_S128: return h * 1.0 + (h / 128.0) * sizeof(float);
        case EP_FMT_MXFP8: return h * 1.0 + (h / 32.0) * 1.0;
        case EP_FMT_NVFP4: return h * 0.5 + (h / 16.0) * sizeof(uint16_t);
        default: return h * sizeof(uint16_t);
    }
}

}  // namespace

namespace ep {

constexpr int kRegionCount = kWsRegions;

WsLayout ws_layout(const Shape &s) {
    WsLayout L;
    // pair masks of one tile (tile_waves * E * 8 bytes) stay within 48 KiB
    int wmax = EP_PLAN_WAVES;
    while (wmax > 1 && (size_t)wmax * (size_t)s.E * 8 > 48 * 1024) wmax >>= 1;
    L.tile_tokens = (wmax * 64) / s.k;
    if (L.tile_tokens < 1) L.tile_tokens = 1;
    L.tile_waves = (L.tile_tokens * s.k + 63) / 64;
    L.count_threads = L.tile_waves * 64;   // >= tile_tokens: one token per thread in the count kernel
    L.tiles = (int)((s.T + L.tile_tokens - 1) / L.tile_tokens);
    if (L.tiles < 1) L.tiles = 1;
    const int64_t TK = s.T * s.k;
    L.tile_token_waves = (L.tile_tokens + 63) / 64;
    // the per-tile pairs serve the copies that scan the tile counts (2 ...
    // kScanCopyMaxTiles tiles); other batches never touch them
    const bool pairs = L.tiles > 1 && L.tiles <= kScanCopyMaxTiles;
    const size_t need[kRegionCount] = {
        kCtrlWords * sizeof(uint32_t),                                               // ctrl
        sizeof(int32_t) * (size_t)L.tiles * (size_t)(s.E + s.R + s.N),               // tile_count
        sizeof(int32_t) * (size_t)(TK > 0 ? TK : 1),                                 // local_rank
        sizeof(int32_t) * (size_t)(s.E + 1),                                         // plan_offset
        s.rank_rows ? sizeof(uint64_t) * (size_t)L.tiles * (size_t)s.R * L.tile_token_waves : 0,   // rank_mask
        sizeof(int32_t) * (size_t)(s.R + 1),                                         // plan_rank_offset
        (pairs && !s.rank_rows) ? 2 * sizeof(int32_t) * (size_t)L.tiles * (size_t)s.E : 0,   // tile_pairs
        (pairs && s.rank_rows) ? 2 * sizeof(int32_t) * (size_t)L.tiles * (size_t)s.R : 0,    // rank_pairs
    };
    size_t *const field[kRegionCount] = {&L.ctrl, &L.tile_count, &L.local_rank, &L.plan_offset, &L.rank_mask,
                                         &L.plan_rank_offset, &L.tile_pairs, &L.rank_pairs};
    size_t off = 0;
    for (int i = 0; i < kRegionCount; ++i) {
        *field[i] = off;
        L.region_bytes[i] = need[i];
        off = align256(off + need[i]);
    }
    L.total = off;
    return L;
}

}  // namespace ep

extern "C" {

int ep_abi_version(void) { return EP_ABI_VERSION; }

const char *ep_strerror(int status) {
    switch (status) {
        case EP_OK: return "ok";
        case EP_EINVAL: return "invalid argument or unsupported shape";
        case EP_EALIGN: return "row buffer not 16-byte aligned";
        case EP_EWORKSPACE: return "workspace missing or too small";
        case EP_EHIP: return "HIP runtime error";
        case EP_EDEVICE: return "a kernel flagged invalid input (expert id >= num_experts)";
        default: return "unknown status";
    }
}

int ep_validate_shape(const ep_shape *shape) { return check_shape(shape, nullptr); }

int ep_workspace_bytes(const ep_shape *shape, size_t *bytes) {
    Shape s;
    const int rc = check_shape(shape, &s);
    if (rc != EP_OK) return rc;
    if (!bytes) return EP_EINVAL;
    *bytes = ep::ws_layout(s).total;
    return EP_OK;
}

int ep_workspace_init(void *ws, size_t ws_bytes, void *stream) {
    if (!ws || ws_bytes < 256 || (ws_bytes & 3) != 0) return EP_EINVAL;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return EP_EALIGN;
    return hip_status(ep::launch_ws_init(static_cast<uint32_t *>(ws), ws_bytes / 4,
                                         static_cast<hipStream_t>(stream)));
}

int ep_dispatch_layout(const ep_shape *shape, const int64_t *topk_idx, int32_t *num_tokens_per_rank,
                       int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank,
                       int32_t *num_tokens_per_node, int64_t *rdma_algo_token_count, void *ws,
                       size_t ws_bytes, void *stream) {
    Shape s;
    int rc = check_shape(shape, &s);
    if (rc != EP_OK) return rc;
    if (!num_tokens_per_rank || !num_tokens_per_expert || !num_tokens_per_node ||
        !rdma_algo_token_count)
        return EP_EINVAL;
    if (s.T > 0 && (!topk_idx || !is_token_in_rank)) return EP_EINVAL;
    if (!aligned16(is_token_in_rank) && (s.R % 4 == 0)) return EP_EALIGN;
    const WsLayout L = ep::ws_layout(s);
    if (!ws || ws_bytes < L.total) return EP_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return EP_EALIGN;
    return hip_status(ep::launch_plan(s, L, topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                                      is_token_in_rank, num_tokens_per_node, rdma_algo_token_count,
                                      static_cast<char *>(ws), static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

int check_dispatch_inputs(const ep_shape *shape, Shape *s, const void *x, const float *x_scales,
                          const int64_t *topk_idx, const float *topk_w, const void *recv_x,
                          const float *recv_x_scales, const int32_t *recv_src_idx,
                          const float *recv_topk_w, const int32_t *token_slot,
                          const int32_t *expert_offset) {
    int rc = check_shape(shape, s);
    if (rc != EP_OK) return rc;
    if (!expert_offset) return EP_EINVAL;
    if (s->T > 0 && (!x || !topk_idx || !topk_w || !recv_x || !recv_src_idx || !recv_topk_w ||
                     !token_slot))
        return EP_EINVAL;
    const bool fp8 = s->x_fmt == EP_FMT_FP8_S128;
    if (fp8 && s->T > 0 && (!x_scales || !recv_x_scales)) return EP_EINVAL;
    if (!fp8 && (x_scales || recv_x_scales)) return EP_EINVAL;
    if (s->T > 0 && (!aligned16(x) || !aligned16(recv_x))) return EP_EALIGN;
    return EP_OK;
}

int check_workspace(const Shape &s, const void *ws, size_t ws_bytes, WsLayout *L) {
    *L = ep::ws_layout(s);
    if (!ws || ws_bytes < L->total) return EP_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return EP_EALIGN;
    return EP_OK;
}

int check_dispatch_args(const ep_shape *shape, Shape *s, const void *x, const float *x_scales,
                        const int64_t *topk_idx, const float *topk_w, const void *recv_x,
                        const float *recv_x_scales, const int32_t *recv_src_idx,
                        const float *recv_topk_w, const int32_t *token_slot,
                        const int32_t *expert_offset, const void *ws, size_t ws_bytes,
                        WsLayout *L) {
    int rc = check_dispatch_inputs(shape, s, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales,
                                   recv_src_idx, recv_topk_w, token_slot, expert_offset);
    if (rc != EP_OK) return rc;
    return check_workspace(*s, ws, ws_bytes, L);
}

int check_layout_outputs(const Shape &s, const int32_t *per_rank, const int32_t *per_expert,
                         const uint8_t *in_rank, const int32_t *per_node, const int64_t *algo) {
    if (!per_rank || !per_expert || !per_node || !algo) return EP_EINVAL;
    if (s.T > 0 && !in_rank) return EP_EINVAL;
    if (!aligned16(in_rank) && (s.R % 4 == 0)) return EP_EALIGN;
    return EP_OK;
}

// Layout + dispatch on a checked shape, with the workspace at w (plan regions
// as in L): a small batch in one launch, else the plan launches and the copy.
int dispatch_with_layout_impl(const Shape &s, const WsLayout &L, const void *x, const float *x_scales,
                              const int64_t *topk_idx, const float *topk_w, int32_t *per_rank,
                              int32_t *per_expert, uint8_t *in_rank, int32_t *per_node, int64_t *algo,
                              void *recv_x, float *recv_x_scales, int32_t *recv_src_idx, float *recv_topk_w,
                              int32_t *token_slot, int32_t *expert_offset, char *w, hipStream_t st) {
    if (ep::fused_dispatch_fits(s))
        return hip_status(ep::launch_dispatch_fused(s, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales,
                                                    recv_src_idx, recv_topk_w, token_slot, expert_offset,
                                                    per_rank, per_expert, in_rank, per_node, algo,
                                                    reinterpret_cast<uint32_t *>(w + L.ctrl), st));
    if (ep::scan_in_copy_fits(s, L)) {   // two launches: counts, then the copy that scans them
        hipError_t e = ep::launch_plan(s, L, topk_idx, per_rank, per_expert, in_rank, per_node, algo, w, st,
                                       /*count_only=*/true);
        if (e != hipSuccess) return EP_EHIP;
        return hip_status(ep::launch_dispatch_scan_copy(s, L, x, x_scales, topk_idx, topk_w, recv_x,
                                                        recv_x_scales, recv_src_idx, recv_topk_w, token_slot,
                                                        expert_offset, per_rank, per_expert, per_node, algo, w,
                                                        st));
    }
    hipError_t e = ep::launch_plan(s, L, topk_idx, per_rank, per_expert, in_rank, per_node, algo, w, st);
    if (e != hipSuccess) return EP_EHIP;
    e = ep::launch_dispatch_copy(s, L, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales,
                                 recv_src_idx, recv_topk_w, token_slot, expert_offset, w, st);
    return hip_status(e);
}

}  // namespace

extern "C" {

int ep_dispatch(const ep_shape *shape, const void *x, const float *x_scales,
                const int64_t *topk_idx, const float *topk_w, void *recv_x, float *recv_x_scales,
                int32_t *recv_src_idx, float *recv_topk_w, int32_t *token_slot,
                int32_t *expert_offset, void *ws, size_t ws_bytes, void *stream) {
    Shape s;
    WsLayout L;
    int rc = check_dispatch_args(shape, &s, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales,
                                 recv_src_idx, recv_topk_w, token_slot, expert_offset, ws, ws_bytes, &L);
    if (rc != EP_OK) return rc;
    // the plan itself (no layout outputs): one launch for a small batch, the
    // count and copy launches for up to kScanCopyMaxTiles tiles, else three
    return dispatch_with_layout_impl(s, L, x, x_scales, topk_idx, topk_w, nullptr, nullptr, nullptr, nullptr,
                                     nullptr, recv_x, recv_x_scales, recv_src_idx, recv_topk_w, token_slot,
                                     expert_offset, static_cast<char *>(ws), static_cast<hipStream_t>(stream));
}

int ep_dispatch_with_layout(const ep_shape *shape, const void *x, const float *x_scales,
                            const int64_t *topk_idx, const float *topk_w, int32_t *num_tokens_per_rank,
                            int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank,
                            int32_t *num_tokens_per_node, int64_t *rdma_algo_token_count, void *recv_x,
                            float *recv_x_scales, int32_t *recv_src_idx, float *recv_topk_w,
                            int32_t *token_slot, int32_t *expert_offset, void *ws, size_t ws_bytes,
                            void *stream) {
    Shape s;
    WsLayout L;
    int rc = check_dispatch_args(shape, &s, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales,
                                 recv_src_idx, recv_topk_w, token_slot, expert_offset, ws, ws_bytes, &L);
    if (rc != EP_OK) return rc;
    rc = check_layout_outputs(s, num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank,
                              num_tokens_per_node, rdma_algo_token_count);
    if (rc != EP_OK) return rc;
    return dispatch_with_layout_impl(s, L, x, x_scales, topk_idx, topk_w, num_tokens_per_rank,
                                     num_tokens_per_expert, is_token_in_rank, num_tokens_per_node,
                                     rdma_algo_token_count, recv_x, recv_x_scales, recv_src_idx, recv_topk_w,
                                     token_slot, expert_offset, static_cast<char *>(ws),
                                     static_cast<hipStream_t>(stream));
}

int ep_dispatch_from_layout(const ep_shape *shape, const void *x, const float *x_scales,
                            const int64_t *topk_idx, const float *topk_w, void *recv_x,
                            float *recv_x_scales, int32_t *recv_src_idx, float *recv_topk_w,
                            int32_t *token_slot, int32_t *expert_offset, void *ws, size_t ws_bytes,
                            void *stream) {
    Shape s;
    WsLayout L;
    int rc = check_dispatch_args(shape, &s, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales,
                                 recv_src_idx, recv_topk_w, token_slot, expert_offset, ws, ws_bytes, &L);
    if (rc != EP_OK) return rc;
    return hip_status(ep::launch_dispatch_copy(s, L, x, x_scales, topk_idx, topk_w, recv_x,
                                               recv_x_scales, recv_src_idx, recv_topk_w, token_slot,
                                               expert_offset, static_cast<char *>(ws),
                                               static_cast<hipStream_t>(stream)));
}

int ep_combine(const ep_shape *shape, const void *expert_out, const uint8_t *expert_out_scales,
               const int32_t *token_slot, const float *topk_w, void *y, void *stream) {
    Shape s;
    int rc = check_shape(shape, &s);
    if (rc != EP_OK) return rc;
    if (s.T == 0) return EP_OK;
    if (!expert_out || !token_slot || !topk_w || !y) return EP_EINVAL;
    const bool scaled = s.y_fmt != EP_FMT_BF16;
    if (scaled && !expert_out_scales) return EP_EINVAL;
    if (!scaled && expert_out_scales) return EP_EINVAL;
    if (!aligned16(expert_out) || !aligned16(y)) return EP_EALIGN;
    if (s.y_fmt == EP_FMT_NVFP4 && (reinterpret_cast<uintptr_t>(expert_out_scales) & 3u) != 0)
        return EP_EALIGN;
    return hip_status(ep::launch_combine(s, expert_out, expert_out_scales, token_slot, topk_w, y,
                                         static_cast<hipStream_t>(stream)));
}

int ep_dispatch_ranks(const ep_shape *shape, const void *x, const float *x_scales,
                      const int64_t *topk_idx, const float *topk_w, void *recv_x,
                      float *recv_x_scales, int32_t *recv_src_idx, int32_t *recv_topk_idx,
                      float *recv_topk_w, int32_t *token_rank_slot, int32_t *rank_offset,
                      void *ws, size_t ws_bytes, void *stream) {
    Shape s;
    int rc = check_shape(shape, &s);
    if (rc != EP_OK) return rc;
    if (!s.rank_rows || !rank_offset) return EP_EINVAL;
    if (s.T > 0 && (!x || !topk_idx || !topk_w || !recv_x || !recv_src_idx || !recv_topk_idx ||
                    !recv_topk_w || !token_rank_slot))
        return EP_EINVAL;
    const bool fp8 = s.x_fmt == EP_FMT_FP8_S128;
    if (fp8 && s.T > 0 && (!x_scales || !recv_x_scales)) return EP_EINVAL;
    if (!fp8 && (x_scales || recv_x_scales)) return EP_EINVAL;
    if (s.T > 0 && (!aligned16(x) || !aligned16(recv_x))) return EP_EALIGN;
    const WsLayout L = ep::ws_layout(s);
    if (!ws || ws_bytes < L.total) return EP_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return EP_EALIGN;
    return hip_status(ep::launch_dispatch_ranks(s, L, x, x_scales, topk_idx, topk_w, recv_x,
                                                recv_x_scales, recv_src_idx, recv_topk_idx,
                                                recv_topk_w, token_rank_slot, rank_offset,
                                                static_cast<char *>(ws),
                                                static_cast<hipStream_t>(stream)));
}

int ep_dispatch_ranks_with_layout(const ep_shape *shape, const void *x, const float *x_scales,
                                  const int64_t *topk_idx, const float *topk_w, int32_t *num_tokens_per_rank,
                                  int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank,
                                  int32_t *num_tokens_per_node, int64_t *rdma_algo_token_count, void *recv_x,
                                  float *recv_x_scales, int32_t *recv_src_idx, int32_t *recv_topk_idx,
                                  float *recv_topk_w, int32_t *token_rank_slot, int32_t *rank_offset,
                                  void *ws, size_t ws_bytes, void *stream) {
    Shape s;
    int rc = check_shape(shape, &s);
    if (rc != EP_OK) return rc;
    if (!s.rank_rows || !rank_offset) return EP_EINVAL;
    if (!num_tokens_per_rank || !num_tokens_per_expert || !num_tokens_per_node || !rdma_algo_token_count)
        return EP_EINVAL;
    if (s.T > 0 && (!x || !topk_idx || !topk_w || !recv_x || !recv_src_idx || !recv_topk_idx ||
                    !recv_topk_w || !token_rank_slot || !is_token_in_rank))
        return EP_EINVAL;
    const bool fp8 = s.x_fmt == EP_FMT_FP8_S128;
    if (fp8 && s.T > 0 && (!x_scales || !recv_x_scales)) return EP_EINVAL;
    if (!fp8 && (x_scales || recv_x_scales)) return EP_EINVAL;
    if (s.T > 0 && (!aligned16(x) || !aligned16(recv_x))) return EP_EALIGN;
    if (!aligned16(is_token_in_rank) && (s.R % 4 == 0)) return EP_EALIGN;
    const WsLayout L = ep::ws_layout(s);
    if (!ws || ws_bytes < L.total) return EP_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return EP_EALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(ws);
    if (ep::fused_ranks_fits(s))   // small batch: one launch, no plan in the workspace
        return hip_status(ep::launch_dispatch_ranks_fused(
            s, x, x_scales, topk_idx, topk_w, num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank,
            num_tokens_per_node, rdma_algo_token_count, recv_x, recv_x_scales, recv_src_idx, recv_topk_idx,
            recv_topk_w, token_rank_slot, rank_offset, reinterpret_cast<uint32_t *>(w + L.ctrl), st));
    if (ep::ranks_scan_fits(s, L)) {   // two launches: counts, then the copy that scans them
        hipError_t e = ep::launch_plan(s, L, topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                                       is_token_in_rank, num_tokens_per_node, rdma_algo_token_count, w, st,
                                       /*count_only=*/true);
        if (e != hipSuccess) return EP_EHIP;
        return hip_status(ep::launch_dispatch_ranks_scan(
            s, L, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales, recv_src_idx, recv_topk_idx, recv_topk_w,
            token_rank_slot, rank_offset, num_tokens_per_rank, num_tokens_per_expert, num_tokens_per_node,
            rdma_algo_token_count, w, st));
    }
    hipError_t e = ep::launch_plan(s, L, topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                                   is_token_in_rank, num_tokens_per_node, rdma_algo_token_count, w, st);
    if (e != hipSuccess) return EP_EHIP;
    return hip_status(ep::launch_dispatch_ranks(s, L, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales,
                                                recv_src_idx, recv_topk_idx, recv_topk_w, token_rank_slot,
                                                rank_offset, w, st));
}

int ep_expert_reduce_ranks(const ep_shape *shape, const void *recv_x, const float *recv_x_scales,
                           const int32_t *rank_offset, const int32_t *recv_topk_idx,
                           const float *recv_topk_w, const float *factor, uint16_t *partial,
                           void *stream) {
    Shape s;
    int rc = check_shape(shape, &s);
    if (rc != EP_OK) return rc;
    if (!s.rank_rows || s.y_fmt != EP_FMT_BF16) return EP_EINVAL;
    if (s.T == 0) return EP_OK;
    if (!recv_x || !rank_offset || !recv_topk_idx || !recv_topk_w || !partial) return EP_EINVAL;
    const bool fp8 = s.x_fmt == EP_FMT_FP8_S128;
    if (fp8 != (recv_x_scales != nullptr)) return EP_EINVAL;
    if (!aligned16(recv_x) || !aligned16(partial)) return EP_EALIGN;
    return hip_status(ep::launch_expert_reduce_ranks(s, recv_x, recv_x_scales, rank_offset,
                                                     recv_topk_idx, recv_topk_w, factor, partial,
                                                     static_cast<hipStream_t>(stream)));
}

int ep_combine_ranks(const ep_shape *shape, const uint16_t *partial,
                     const int32_t *token_rank_slot, void *y, void *stream) {
    Shape s;
    int rc = check_shape(shape, &s);
    if (rc != EP_OK) return rc;
    if (!s.rank_rows || s.y_fmt != EP_FMT_BF16) return EP_EINVAL;
    if (s.T == 0) return EP_OK;
    if (!partial || !token_rank_slot || !y) return EP_EINVAL;
    if (!aligned16(partial) || !aligned16(y)) return EP_EALIGN;
    return hip_status(ep::launch_combine_ranks(s, partial, token_rank_slot, y,
                                               static_cast<hipStream_t>(stream)));
}

int ep_dispatch_cached(const ep_shape *shape, const void *x, const float *x_scales,
                       const int32_t *token_slot, void *recv_x, float *recv_x_scales, void *stream) {
    Shape s;
    int rc = check_shape(shape, &s);
    if (rc != EP_OK) return rc;
    if (s.T == 0) return EP_OK;
    if (!x || !token_slot || !recv_x) return EP_EINVAL;
    const bool fp8 = s.x_fmt == EP_FMT_FP8_S128;
    if (fp8 != (x_scales != nullptr) || fp8 != (recv_x_scales != nullptr)) return EP_EINVAL;
    if (!aligned16(x) || !aligned16(recv_x)) return EP_EALIGN;
    return hip_status(ep::launch_dispatch_cached(s, x, x_scales, token_slot, recv_x, recv_x_scales,
                                                 static_cast<hipStream_t>(stream)));
}

int ep_dispatch_ranks_cached(const ep_shape *shape, const void *x, const float *x_scales,
                             const int32_t *token_rank_slot, void *recv_x, float *recv_x_scales,
                             void *stream) {
    Shape s;
    int rc = check_shape(shape, &s);
    if (rc != EP_OK) return rc;
    if (!s.rank_rows) return EP_EINVAL;
    if (s.T == 0) return EP_OK;
    if (!x || !token_rank_slot || !recv_x) return EP_EINVAL;
    const bool fp8 = s.x_fmt == EP_FMT_FP8_S128;
    if (fp8 != (x_scales != nullptr) || fp8 != (recv_x_scales != nullptr)) return EP_EINVAL;
    if (!aligned16(x) || !aligned16(recv_x)) return EP_EALIGN;
    return hip_status(ep::launch_dispatch_ranks_cached(s, x, x_scales, token_rank_slot, recv_x, recv_x_scales,
                                                       static_cast<hipStream_t>(stream)));
}

int ep_check(void *ws, size_t ws_bytes, void *stream, uint32_t *flags) {
    if (!ws) {   // the error word of ep_dispatch_with_layout_static's scratch on the current device
        const int rc = static_scratch_if_used(&ws);
        if (rc != EP_OK) return rc;
        if (!ws) {   // no allocation-free call on this device yet: nothing flagged
            if (flags) *flags = 0;
            return EP_OK;
        }
        ws_bytes = 256;
    }
    if (ws_bytes < 256) return EP_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(st) != hipSuccess) return EP_EHIP;
    uint32_t word = 0;
    if (hipMemcpy(&word, ws, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return EP_EHIP;
    if (word != 0) {
        const uint32_t zero = 0;
        if (hipMemcpy(ws, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return EP_EHIP;
    }
    if (flags) *flags = word;
    return word ? EP_EDEVICE : EP_OK;
}

int ep_quant_fp8_s128(int64_t rows, int32_t hidden, const uint16_t *x, uint8_t *q, float *scales,
                      void *stream) {
    if (rows < 0 || hidden < 128 || hidden % 128 != 0) return EP_EINVAL;
    if (rows == 0) return EP_OK;
    if (!x || !q || !scales) return EP_EINVAL;
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(q) & 7u) != 0) return EP_EALIGN;
    return hip_status(ep::launch_quant_fp8(rows, hidden, x, q, scales, static_cast<hipStream_t>(stream)));
}

int ep_expert_scale_bf16(const ep_shape *shape, const int32_t *expert_offset, const float *factor,
                         const uint16_t *recv, uint16_t *out, void *stream) {
    Shape s;
    int rc = check_shape(shape, &s);
    if (rc != EP_OK) return rc;
    if (s.M != 0) return EP_EINVAL;
    if (s.T == 0) return EP_OK;
    if (!expert_offset || !factor || !recv || !out) return EP_EINVAL;
    if (!aligned16(recv) || !aligned16(out)) return EP_EALIGN;
    return hip_status(ep::launch_expert_scale_bf16(s, expert_offset, factor, recv, out,
                                                   static_cast<hipStream_t>(stream)));
}

int ep_expert_requant_mxfp8(const ep_shape *shape, const int32_t *expert_offset, const float *factor,
                            const uint8_t *recv_q, const float *recv_scales, uint8_t *out_q,
                            uint8_t *out_e8m0, void *stream) {
    Shape s;
    int rc = check_shape(shape, &s);
    if (rc != EP_OK) return rc;
    if (s.H % 128 != 0 || s.M != 0) return EP_EINVAL;
    if (s.T == 0) return EP_OK;
    if (!expert_offset || !recv_q || !recv_scales || !out_q || !out_e8m0) return EP_EINVAL;
    if (!aligned16(recv_q) || !aligned16(out_q)) return EP_EALIGN;
    return hip_status(ep::launch_expert_requant_mxfp8(s, expert_offset, factor, recv_q, recv_scales,
                                                      out_q, out_e8m0,
                                                      static_cast<hipStream_t>(stream)));
}

int ep_expert_requant_nvfp4(const ep_shape *shape, const int32_t *expert_offset, const float *factor,
                            const uint16_t *recv, uint8_t *out_q, uint16_t *out_scales,
                            void *stream) {
    Shape s;
    int rc = check_shape(shape, &s);
    if (rc != EP_OK) return rc;
    if (s.H % 128 != 0 || s.M != 0) return EP_EINVAL;
    if (s.T == 0) return EP_OK;
    if (!expert_offset || !recv || !out_q || !out_scales) return EP_EINVAL;
    if (!aligned16(recv) || (reinterpret_cast<uintptr_t>(out_q) & 7u) != 0) return EP_EALIGN;
    return hip_status(ep::launch_expert_requant_nvfp4(s, expert_offset, factor, recv, out_q, out_scales,
                                                      static_cast<hipStream_t>(stream)));
}

int ep_accounting(const ep_shape *shape, int32_t own_node, const int32_t *num_tokens_per_rank,
                  const int32_t *num_tokens_per_node, int64_t rdma_algo_token_count,
                  int64_t valid_pairs, ep_accounting_t *out) {
    Shape s;
    int rc = check_shape(shape, &s);
    if (rc != EP_OK) return rc;
    if (!num_tokens_per_rank || !num_tokens_per_node || !out) return EP_EINVAL;
    if (own_node < 0 || own_node >= s.N || valid_pairs < 0 || valid_pairs > s.T * s.k)
        return EP_EINVAL;
    // The pages' token counts (MORI-EP Benchmark, "Algo BW vs Physical BW",
    // "NVL / XGMI bandwidth"): every (token, node) pair of the layout crosses
    // RDMA once, the local node included; a fraction (N-1)/N of them leaves
    // the node; every (token, rank) pair is one NVL row.
    int64_t nvl = 0;
    for (int r = 0; r < s.R; ++r) nvl += num_tokens_per_rank[r];
    const int64_t algo = rdma_algo_token_count;
    out->rdma_algo_tokens = algo;
    out->rdma_physical_tokens = (double)algo * (double)(s.N - 1) / (double)s.N;
    out->rdma_physical_tokens_exact = algo - num_tokens_per_node[own_node];
    out->nvl_tokens = nvl;
    // Bytes = rows x bytes of one row in the payload format; the combine
    // sends the same rows back.
    const double bf16_row = row_bytes(EP_FMT_BF16, s.H), fp8_row = row_bytes(EP_FMT_FP8_S128, s.H);
    out->dispatch_rdma_bytes_bf16 = (double)algo * bf16_row;
    out->dispatch_nvl_bytes_bf16 = (double)nvl * bf16_row;
    out->combine_rdma_bytes_bf16 = (double)algo * bf16_row;
    out->combine_nvl_bytes_bf16 = (double)nvl * bf16_row;
    out->fp8_factor = fp8_row / bf16_row;
    out->dispatch_rdma_bytes_fp8 = (double)algo * fp8_row;
    out->dispatch_nvl_bytes_fp8 = (double)nvl * fp8_row;

    // Minimum HBM traffic of one call each on this GPU: every row it moves
    // and every index / weight element it reads or writes, exactly once.
    const double T = (double)s.T, TK = (double)s.T * s.k, V = (double)valid_pairs, NR = (double)nvl;
    const double R = s.R, E = s.E, N = s.N, k = s.k;
    const double xrow = row_bytes(s.x_fmt, s.H), yrow = row_bytes(s.y_fmt, s.H), out_row = bf16_row;
    // layout: topk_idx in; token-in-rank map, the three count vectors and the algo count out
    out->hbm_layout_read_bytes = TK * sizeof(int64_t);
    out->hbm_layout_write_bytes = T * R * sizeof(uint8_t) + (R + N + E) * sizeof(int32_t) + sizeof(int64_t);
    // dispatch: x rows, topk_idx, topk_w in; one row per valid pair, token_slot,
    // recv_src_idx, recv_topk_w and expert_offset out
    out->hbm_dispatch_read_bytes = T * xrow + TK * (sizeof(int64_t) + sizeof(float));
    out->hbm_dispatch_write_bytes = V * xrow + TK * sizeof(int32_t) + V * (sizeof(int32_t) + sizeof(float)) +
                                    (E + 1) * sizeof(int32_t);
    // combine: one row per valid pair, token_slot, topk_w in; y out
    out->hbm_combine_read_bytes = V * yrow + TK * (sizeof(int32_t) + sizeof(float));
    out->hbm_combine_write_bytes = T * out_row;
    // (token, rank) rows: one per (t, r) pair, i.e. nvl_tokens rows; the
    // metadata per row is its source index and its k-wide local top-k list
    out->hbm_dispatch_ranks_read_bytes = T * xrow + TK * (sizeof(int64_t) + sizeof(float));
    out->hbm_dispatch_ranks_write_bytes = NR * xrow + T * R * sizeof(int32_t) +
                                          NR * (sizeof(int32_t) + k * (sizeof(int32_t) + sizeof(float))) +
                                          (R + 1) * sizeof(int32_t);
    out->hbm_combine_ranks_read_bytes = NR * out_row + T * R * sizeof(int32_t);
    out->hbm_combine_ranks_write_bytes = T * out_row;
    out->hbm_layout_bytes = out->hbm_layout_read_bytes + out->hbm_layout_write_bytes;
    out->hbm_dispatch_bytes = out->hbm_dispatch_read_bytes + out->hbm_dispatch_write_bytes;
    out->hbm_combine_bytes = out->hbm_combine_read_bytes + out->hbm_combine_write_bytes;
    out->hbm_dispatch_ranks_bytes = out->hbm_dispatch_ranks_read_bytes + out->hbm_dispatch_ranks_write_bytes;
    out->hbm_combine_ranks_bytes = out->hbm_combine_ranks_read_bytes + out->hbm_combine_ranks_write_bytes;
    return EP_OK;
}

int ep_plan_info(const ep_shape *shape, ep_plan_info_t *info) {
    Shape s;
    const int rc = check_shape(shape, &s);
    if (rc != EP_OK) return rc;
    if (!info) return EP_EINVAL;
    const WsLayout L = ep::ws_layout(s);
    *info = ep_plan_info_t{};
    info->workspace_bytes = L.total;
    const size_t offs[ep::kWsRegions] = {L.ctrl, L.tile_count, L.local_rank, L.plan_offset, L.rank_mask,
                                         L.plan_rank_offset, L.tile_pairs, L.rank_pairs};
    static_assert(ep::kWsRegions == EP_PLAN_REGIONS, "region count and header disagree");
    for (int i = 0; i < ep::kWsRegions; ++i) {
        info->region_offset[i] = offs[i];
        info->region_bytes[i] = L.region_bytes[i];
    }
    info->tiles = L.tiles;
    info->tile_tokens = L.tile_tokens;
    info->tile_waves = L.tile_waves;
    info->count_threads = L.count_threads;
    info->count_lds_bytes = s.T > 0 ? ep::plan_count_lds(s, L) : 0;
    int threads = 0;
    if (ep::fused_dispatch_fits(s)) {
        info->single_launch_lds_bytes = ep::fused_dispatch_lds(s, &threads);
        info->single_launch_threads = threads;
    } else if (ep::fused_ranks_fits(s)) {
        info->single_launch_lds_bytes = ep::fused_ranks_lds(s, &threads);
        info->single_launch_threads = threads;
    }
    const bool scan = s.rank_rows ? ep::ranks_scan_fits(s, L) : ep::scan_in_copy_fits(s, L);
    info->scan_copy_lds_bytes = scan ? ep::scan_copy_lds(s) : 0;
    return EP_OK;
}

int ep_calib_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (!src || !dst || bytes % 16 != 0) return EP_EINVAL;
    if (!aligned16(src) || !aligned16(dst)) return EP_EALIGN;
    return hip_status(ep::launch_calib_copy(src, dst, bytes, static_cast<hipStream_t>(stream)));
}

int ep_stream(int32_t kind, const void *src, void *dst, size_t bytes, size_t chunk_bytes, int32_t waves,
              void *stream) {
    if (kind < EP_STREAM_READ || kind > EP_STREAM_COPY_NT) return EP_EINVAL;
    if (chunk_bytes < 1024 || chunk_bytes % 1024 != 0 || chunk_bytes > (size_t(1) << 20)) return EP_EINVAL;
    if (bytes % chunk_bytes != 0 || waves < 4 || waves % 4 != 0 || waves > (1 << 20)) return EP_EINVAL;
    const int k = kind / 2;   // 0 read, 1 write, 2 copy
    if (!dst || (k == 1) != (src == nullptr)) return EP_EINVAL;
    if (!aligned16(dst) || (src && !aligned16(src))) return EP_EALIGN;
    if (k == 2) {   // overlapping copies are not supported
        const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
        if (bytes && s0 < d0 + bytes && d0 < s0 + bytes) return EP_EINVAL;
    }
    return hip_status(ep::launch_stream(k, (kind & 1) != 0, src, dst, bytes, chunk_bytes, waves,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- allocation-free layout + dispatch ---------------------------------

namespace {

constexpr size_t kStaticScratchBytes = size_t(16) << 20;   // EP_STATIC_SCRATCH_BYTES in ep.h
static_assert(kStaticScratchBytes == EP_STATIC_SCRATCH_BYTES, "scratch size and header disagree");
constexpr int kMaxDevices = 64;

// The workspace of ep_dispatch_with_layout_static: one copy per GPU, held
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not the device array: kernels get the address from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch; looked up (and its error
// word cleared by a fill kernel on `st`) at the first call on that device.
int static_scratch(void **out, hipStream_t st) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return EP_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return EP_EHIP;
        if ((reinterpret_cast<uintptr_t>(p) & 255u) != 0) return EP_EHIP;
        if (ep::launch_ws_init(static_cast<uint32_t *>(p), ep::kCtrlWords, st) != hipSuccess) return EP_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return EP_OK;
}

int static_scratch_if_used(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return EP_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    *out = g_scratch_ptr[dev];
    return EP_OK;
}

}  // namespace

extern "C" int ep_dispatch_with_layout_static(const ep_shape *shape, const void *x, const float *x_scales,
                                              const int64_t *topk_idx, const float *topk_w,
                                              int32_t *num_tokens_per_rank, int32_t *num_tokens_per_expert,
                                              uint8_t *is_token_in_rank, int32_t *num_tokens_per_node,
                                              int64_t *rdma_algo_token_count, void *recv_x, float *recv_x_scales,
                                              int32_t *recv_src_idx, float *recv_topk_w, int32_t *token_slot,
                                              int32_t *expert_offset, void *stream) {
    Shape s;
    int rc = check_dispatch_inputs(shape, &s, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales,
                                   recv_src_idx, recv_topk_w, token_slot, expert_offset);
    if (rc != EP_OK) return rc;
    rc = check_layout_outputs(s, num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank,
                              num_tokens_per_node, rdma_algo_token_count);
    if (rc != EP_OK) return rc;
    const WsLayout L = ep::ws_layout(s);
    if (L.total > kStaticScratchBytes) return EP_EWORKSPACE;   // before any device work
    hipStream_t st = static_cast<hipStream_t>(stream);
    void *w = nullptr;
    rc = static_scratch(&w, st);
    if (rc != EP_OK) return rc;
    return dispatch_with_layout_impl(s, L, x, x_scales, topk_idx, topk_w, num_tokens_per_rank,
                                     num_tokens_per_expert, is_token_in_rank, num_tokens_per_node,
                                     rdma_algo_token_count, recv_x, recv_x_scales, recv_src_idx, recv_topk_w,
                                     token_slot, expert_offset, static_cast<char *>(w), st);
}
