// ep_abi.hip -- the C ABI of libep_hip (declared in include/ep.h): argument
// validation on the host, workspace carving, kernel launches on the caller's
// stream.  Nothing here allocates device memory or synchronizes, except
// ep_check.
#include "ep.h"
#include "ep_internal.h"

#include <hip/hip_runtime.h>

#ifndef EP_PLAN_WAVES
#define EP_PLAN_WAVES 16   // waves (64 pairs each) per plan tile, at most
#endif

namespace {

using ep::Shape;
using ep::WsLayout;

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

}  // namespace

namespace ep {

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
    size_t off = 0;
    L.ctrl = off;
    off = align256(off + kCtrlWords * sizeof(uint32_t));
    L.tile_count = off;
    off = align256(off + sizeof(int32_t) * (size_t)L.tiles * (size_t)(s.E + s.R + s.N));
    L.local_rank = off;
    off = align256(off + sizeof(int32_t) * (size_t)(TK > 0 ? TK : 1));
    L.plan_offset = off;
    off = align256(off + sizeof(int32_t) * (size_t)(s.E + 1));
    L.tile_token_waves = (L.tile_tokens + 63) / 64;
    L.rank_mask = off;
    off = align256(off + (s.rank_rows ? sizeof(uint64_t) * (size_t)L.tiles * (size_t)s.R * L.tile_token_waves : 0));
    L.plan_rank_offset = off;
    off = align256(off + sizeof(int32_t) * (size_t)(s.R + 1));
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

int check_dispatch_args(const ep_shape *shape, Shape *s, const void *x, const float *x_scales,
                        const int64_t *topk_idx, const float *topk_w, const void *recv_x,
                        const float *recv_x_scales, const int32_t *recv_src_idx,
                        const float *recv_topk_w, const int32_t *token_slot,
                        const int32_t *expert_offset, const void *ws, size_t ws_bytes,
                        WsLayout *L) {
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
    *L = ep::ws_layout(*s);
    if (!ws || ws_bytes < L->total) return EP_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return EP_EALIGN;
    return EP_OK;
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
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(ws);
    if (ep::fused_dispatch_fits(s))   // small batch: one launch, no plan in the workspace
        return hip_status(ep::launch_dispatch_fused(s, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales,
                                                    recv_src_idx, recv_topk_w, token_slot, expert_offset,
                                                    nullptr, nullptr, nullptr, nullptr, nullptr,
                                                    reinterpret_cast<uint32_t *>(w + L.ctrl), st));
    hipError_t e = ep::launch_plan(s, L, topk_idx, nullptr, nullptr, nullptr, nullptr, nullptr, w, st);
    if (e != hipSuccess) return EP_EHIP;
    e = ep::launch_dispatch_copy(s, L, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales,
                                 recv_src_idx, recv_topk_w, token_slot, expert_offset, w, st);
    return hip_status(e);
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
    if (!num_tokens_per_rank || !num_tokens_per_expert || !num_tokens_per_node || !rdma_algo_token_count)
        return EP_EINVAL;
    if (s.T > 0 && !is_token_in_rank) return EP_EINVAL;
    if (!aligned16(is_token_in_rank) && (s.R % 4 == 0)) return EP_EALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(ws);
    if (ep::fused_dispatch_fits(s))
        return hip_status(ep::launch_dispatch_fused(s, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales,
                                                    recv_src_idx, recv_topk_w, token_slot, expert_offset,
                                                    num_tokens_per_rank, num_tokens_per_expert,
                                                    is_token_in_rank, num_tokens_per_node,
                                                    rdma_algo_token_count,
                                                    reinterpret_cast<uint32_t *>(w + L.ctrl), st));
    hipError_t e = ep::launch_plan(s, L, topk_idx, num_tokens_per_rank, num_tokens_per_expert,
                                   is_token_in_rank, num_tokens_per_node, rdma_algo_token_count, w, st);
    if (e != hipSuccess) return EP_EHIP;
    e = ep::launch_dispatch_copy(s, L, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales,
                                 recv_src_idx, recv_topk_w, token_slot, expert_offset, w, st);
    return hip_status(e);
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
    if (!ws || ws_bytes < 256) return EP_EINVAL;
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
    int64_t nvl = 0;
    for (int r = 0; r < s.R; ++r) nvl += num_tokens_per_rank[r];
    const double H = (double)s.H;
    out->rdma_algo_tokens = rdma_algo_token_count;
    out->rdma_physical_tokens = (double)rdma_algo_token_count * (double)(s.N - 1) / (double)s.N;
    out->rdma_physical_tokens_exact = rdma_algo_token_count - num_tokens_per_node[own_node];
    out->nvl_tokens = nvl;
    out->dispatch_rdma_bytes_bf16 = (double)rdma_algo_token_count * H * 2.0;
    out->dispatch_nvl_bytes_bf16 = (double)nvl * H * 2.0;
    out->combine_rdma_bytes_bf16 = out->dispatch_rdma_bytes_bf16;
    out->combine_nvl_bytes_bf16 = out->dispatch_nvl_bytes_bf16;
    out->fp8_factor = (1.0 + 4.0 / 128.0) / 2.0;
    out->dispatch_rdma_bytes_fp8 = out->dispatch_rdma_bytes_bf16 * out->fp8_factor;
    out->dispatch_nvl_bytes_fp8 = out->dispatch_nvl_bytes_bf16 * out->fp8_factor;
    // minimum HBM traffic of one call each (payload rows + index/weight metadata)
    const double T = (double)s.T, TK = (double)s.T * s.k, V = (double)valid_pairs;
    const double xrow = (s.x_fmt == EP_FMT_FP8_S128) ? H + 4.0 * H / 128.0 : 2.0 * H;
    const double yrow = (s.y_fmt == EP_FMT_MXFP8) ? H + H / 32.0
                        : (s.y_fmt == EP_FMT_NVFP4) ? H / 2.0 + 2.0 * H / 16.0 : 2.0 * H;
    out->hbm_layout_bytes = TK * 8.0 + T * s.R + 4.0 * (s.R + s.N + s.E) + 8.0;
    out->hbm_dispatch_bytes = T * xrow + V * xrow             // rows: read once, written per pair
                              + TK * (8.0 + 4.0 + 4.0)        // topk_idx, topk_w read; token_slot written
                              + V * (4.0 + 4.0)               // recv_src_idx, recv_topk_w written
                              + 4.0 * (s.E + 1);              // expert_offset
    out->hbm_combine_bytes = V * yrow + T * 2.0 * H          // rows gathered, y written
                             + TK * (4.0 + 4.0);             // token_slot, topk_w read
    // (token, rank) rows: one per (t, r) pair, i.e. nvl_tokens rows
    const double NR = (double)nvl;
    out->hbm_dispatch_ranks_bytes = T * xrow + NR * xrow       // rows: read once, written per rank
                                    + TK * (8.0 + 4.0)         // topk_idx, topk_w read
                                    + T * s.R * 4.0            // token_rank_slot written
                                    + NR * (4.0 + 8.0 * s.k)   // recv_src_idx, recv_topk_idx / _w
                                    + 4.0 * (s.R + 1);         // rank_offset
    out->hbm_combine_ranks_bytes = NR * 2.0 * H + T * 2.0 * H  // partials gathered, y written
                                   + T * s.R * 4.0;            // token_rank_slot read
    return EP_OK;
}

int ep_calib_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (!src || !dst || bytes % 16 != 0) return EP_EINVAL;
    if (!aligned16(src) || !aligned16(dst)) return EP_EALIGN;
    return hip_status(ep::launch_calib_copy(src, dst, bytes, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
