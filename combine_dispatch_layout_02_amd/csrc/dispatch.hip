// dispatch.hip -- the row permutation on gfx950.
//
// What it computes (MSCCL++ PR 860, RANK_MAJOR commit: the default layout
// puts each dispatched token at a compacted prefix offset; MORI-EP Benchmark,
// "NVL / XGMI bandwidth": the receive tensor holds token rows): every valid
// pair (t, j) with expert e gets the slot
//     expert_offset[e] + (pairs of e in earlier tiles) + (rank inside its tile)
// from the plan (plan.hip), and the slot's receive row is a bitwise copy of
// token row t (bf16 row, or e4m3 row plus its fp32 scales).
//
// How: one wave per (token, row part).  Lanes 0..k-1 form the token's k slots
// and readlane broadcasts them to scalar registers, so the k destinations are
// wave-uniform.  Every lane loads its 16-byte vectors of row t once and
// stores them k times.  Stores are plain (write-back): part of the receive
// rows is then still in the memory-side cache when the combine reads them,
// which measured faster for the dispatch -> combine sequence than
// non-temporal stores.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

#ifndef EP_DISPATCH_NT_STORE
#define EP_DISPATCH_NT_STORE 0   // non-temporal stores for the receive rows
#endif
#ifndef EP_DISPATCH_WAVES
#define EP_DISPATCH_WAVES 4096   // waves the copy aims for (4 per CU)
#endif

struct CopyArgs {
    const char *x;            // [T][row_bytes]
    const float *x_scales;    // [T][G] or null
    const int64_t *topk_idx;
    const float *topk_w;
    char *recv_x;             // [T*k][row_bytes]
    float *recv_scales;       // [T*k][G] or null
    int32_t *recv_src_idx;
    float *recv_topk_w;
    int32_t *token_slot;
    const int32_t *plan_offset;   // [E + 1] segment starts (workspace)
    int32_t *expert_offset;       // [E + 1] handle copy of plan_offset
    const int32_t *tile_prefix;   // [ntiles][E + R + N] (expert columns first)
    const int32_t *local_rank;    // [T*k]
    uint32_t *ctrl;               // error word
    int64_t T;
    int k, E, TT;             // TT: tokens per plan tile
    int M;                    // rank_capacity (0: compacted layout)
    int epr, epr_shift;       // experts per rank, its log2 (or -1)
    int64_t rows;             // receive rows
    int cols;                 // columns of the tile matrix: E + R + N
    int64_t row_bytes;        // payload bytes per row (multiple of 16)
    int nvec;                 // row_bytes / 16
    int G;                    // fp32 scales per row (0 for bf16 rows)
    int S;                    // waves per token
};

// VPL: 16-byte vectors each lane holds per pass.
template <int VPL>
__global__ __launch_bounds__(256) void ep_dispatch_copy_kernel(CopyArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int64_t t = gw / a.S;
    const int sub = (int)(gw - t * a.S);
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g <= a.E) a.expert_offset[g] = a.plan_offset[g];   // handle copy of the segment starts
    if (t >= a.T) return;   // wave-uniform

    // the first pass of row t does not depend on the slots: issue its loads
    // before the slot lookups so the two latencies overlap
    const char *src = a.x + t * a.row_bytes;
    const int stride = kWave * a.S;            // vectors between a lane's consecutive vectors
    const int v_first = lane + kWave * sub;
    vec16 buf[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int v = v_first + i * stride;
        if (v < a.nvec) buf[i] = ld16(src + (int64_t)v * 16);
    }
    // fp32 scales of an fp8 row (one per 128 elements): this wave's share,
    // loaded with the row (G <= 64 * S, one value per lane, in every shape the
    // ABI accepts with hidden <= 8192 * S; larger rows loop below)
    const int g_first = lane + kWave * sub;
    float sc0 = 0.0f;
    if (g_first < a.G) sc0 = a.x_scales[t * a.G + g_first];

    // lanes 0..k-1: the token's slots
    int32_t slot = -1;
    if (lane < a.k) {
        const int64_t p = t * a.k + lane;
        const int32_t lr = a.local_rank[p];
        if (lr >= 0) {
            const int e = (int)a.topk_idx[p];
            slot = a.plan_offset[e] + a.tile_prefix[(t / a.TT) * a.cols + e] + lr;
            if (a.M > 0) {   // RANK_MAJOR: the same place inside the rank, at the rank's fixed block
                const int r = a.epr_shift >= 0 ? e >> a.epr_shift : e / a.epr;
                const int32_t in_rank = slot - a.plan_offset[r * a.epr];
                if (in_rank < a.M) {
                    slot = r * a.M + in_rank;
                } else {
                    atomicOr(&a.ctrl[0], kErrRankOverflow);
                    slot = -1;
                }
            }
            if (slot >= 0 && (uint64_t)slot >= (uint64_t)a.rows) {   // cannot happen; never write outside
                atomicOr(&a.ctrl[0], kErrBadSlot);
                slot = -1;
            }
        }
        if (sub == 0) {
            a.token_slot[p] = slot;
            if (slot >= 0) {
                a.recv_src_idx[slot] = (int32_t)t;
                a.recv_topk_w[slot] = a.topk_w[p];
            }
        }
    }
    if (__ballot(slot >= 0) == 0) return;   // no valid slot: nothing to store

    // fp32 scale rows (fp8 payload): lanes spread over the waves of the token
    if (a.G > 0) {
        for (int gi = g_first; gi < a.G; gi += kWave * a.S) {
            const float sc = (gi == g_first) ? sc0 : a.x_scales[t * a.G + gi];
            for (int j = 0; j < a.k; ++j) {
                const int32_t s = readlane(slot, j);
                if (s >= 0) a.recv_scales[(int64_t)s * a.G + gi] = sc;
            }
        }
    }

    for (int v0 = v_first; v0 < a.nvec; v0 += stride * VPL) {
        if (v0 != v_first) {
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int v = v0 + i * stride;
                if (v < a.nvec) buf[i] = ld16(src + (int64_t)v * 16);
            }
        }
        for (int j = 0; j < a.k; ++j) {
            const int32_t s = readlane(slot, j);
            if (s < 0) continue;
            char *dst = a.recv_x + (int64_t)s * a.row_bytes;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int v = v0 + i * stride;
                if (v < a.nvec) {
                    if (EP_DISPATCH_NT_STORE) st16_nt(dst + (int64_t)v * 16, buf[i]);
                    else st16(dst + (int64_t)v * 16, buf[i]);
                }
            }
        }
    }
}

}  // namespace

int waves_per_token(int64_t T, int64_t row_vectors, int64_t target) {
    // aim for `target` waves, keep >= 64 row vectors per wave
    int S = 1;
    while (T * S < target && (row_vectors / (2 * S)) >= kWave && S < 64) S *= 2;
    return S;
}

hipError_t launch_dispatch_copy(const Shape &s, const WsLayout &L, const void *x,
                                const float *x_scales, const int64_t *topk_idx,
                                const float *topk_w, void *recv_x, float *recv_x_scales,
                                int32_t *recv_src_idx, float *recv_topk_w, int32_t *token_slot,
                                int32_t *expert_offset, char *ws, hipStream_t stream) {
    CopyArgs a;
    a.x = static_cast<const char *>(x);
    a.x_scales = x_scales;
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    a.recv_x = static_cast<char *>(recv_x);
    a.recv_scales = recv_x_scales;
    a.recv_src_idx = recv_src_idx;
    a.recv_topk_w = recv_topk_w;
    a.token_slot = token_slot;
    a.plan_offset = reinterpret_cast<const int32_t *>(ws + L.plan_offset);
    a.expert_offset = expert_offset;
    a.tile_prefix = reinterpret_cast<const int32_t *>(ws + L.tile_count);
    a.local_rank = reinterpret_cast<const int32_t *>(ws + L.local_rank);
    a.ctrl = reinterpret_cast<uint32_t *>(ws + L.ctrl);
    a.T = s.T;
    a.k = s.k;
    a.E = s.E;
    a.TT = L.tile_tokens;
    a.cols = s.E + s.R + s.N;
    a.M = s.M;
    a.epr = s.E / s.R;
    a.epr_shift = (a.epr & (a.epr - 1)) == 0 ? __builtin_ctz((unsigned)a.epr) : -1;
    a.rows = s.rows();
    const bool fp8 = (s.x_fmt == 1);
    a.row_bytes = fp8 ? (int64_t)s.H : 2 * (int64_t)s.H;
    a.nvec = (int)(a.row_bytes / 16);
    a.G = fp8 ? s.H / 128 : 0;
    a.S = waves_per_token(s.T, a.nvec, EP_DISPATCH_WAVES);
    const int per_lane = (a.nvec + kWave * a.S - 1) / (kWave * a.S);
    const int64_t waves = s.T * a.S;
    int64_t blocks = (waves + 3) / 4;
    if (blocks * 256 < s.E + 1) blocks = (s.E + 1 + 255) / 256;   // threads to copy expert_offset
    const dim3 grid((unsigned)blocks), block(256);
    if (per_lane <= 2) {
        hipLaunchKernelGGL(ep_dispatch_copy_kernel<2>, grid, block, 0, stream, a);
    } else if (per_lane <= 4) {
        hipLaunchKernelGGL(ep_dispatch_copy_kernel<4>, grid, block, 0, stream, a);
    } else if (per_lane <= 8) {
        hipLaunchKernelGGL(ep_dispatch_copy_kernel<8>, grid, block, 0, stream, a);
    } else {
        hipLaunchKernelGGL(ep_dispatch_copy_kernel<16>, grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace ep
