// small_layout.h -- the layout of a small batch by one block, for the
// single-launch dispatch kernels (token-major and (token, rank) rows).
//
// What it computes (MORI-EP Benchmark, "Why DeepEP and Mori RDMA token
// counts are equivalent", Steps 1-3): per-expert pair counts and their
// exclusive scan (the expert segment starts), and, when requested, per token
// the set of ranks and of nodes its valid experts live on with the per-rank /
// per-node token counts, the token-in-rank map, the RDMA algo count and the
// exclusive scan of the per-rank counts (the (token, rank) region starts).
// Ids >= E count as masked and raise the bad-expert flag.
//
// How: the batch's ids staged in LDS once; per-expert counts are LDS integer
// adds (order-independent), and so are the per-rank / per-node counts (one
// add per rank / node a token reaches, from its rank / node mask); scans are
// the block and wave scans of ep_device.h.  LDS: 4 * (T*k + E + R + N + blockDim/64 + 1)
// bytes (dynamic).
#pragma once

#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

struct SmallLayout {
    const int64_t *topk_idx;   // [T][k]
    int64_t T;
    int k, E, R, N, epr, epr_shift, epn, epn_shift;
    uint32_t *ctrl;            // error word
    int32_t *per_expert;       // [E] or null
    int32_t *expert_offset;    // [E + 1] segment starts, or null
    int32_t *per_rank;         // [R] or null (then per_node, in_rank, algo are too)
    int32_t *per_node;         // [N]
    uint8_t *in_rank;          // [T][R]
    int64_t *algo;
    int32_t *rank_offset;      // [R + 1] region starts, or null (needs the rank counts)
};

// Called by every thread of one block (block-uniform control flow).
__device__ inline void small_layout_block(const SmallLayout &a) {
    extern __shared__ int32_t sm[];
    const int TK = (int)(a.T * a.k);
    int32_t *ids = sm;                    // [TK]
    int32_t *hist = ids + TK;             // [E]
    int32_t *rn = hist + a.E;             // [R + N]
    int32_t *tmp = rn + a.R + a.N;        // [blockDim / 64 + 1]
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & (kWave - 1);
    for (int i = tid; i < a.E; i += nt) hist[i] = 0;
    for (int i = tid; i < a.R + a.N; i += nt) rn[i] = 0;
    __syncthreads();
    bool bad = false;
    for (int q = tid; q < TK; q += nt) {
        const int64_t v = a.topk_idx[q];
        bad |= (v >= a.E);
        const int32_t id = (v >= 0 && v < a.E) ? (int32_t)v : -1;
        ids[q] = id;
        if (id >= 0) atomicAdd(&hist[id], 1);
    }
    if (__ballot(bad) && lane == 0) atomicOr(&a.ctrl[0], kErrBadExpert);
    __syncthreads();
    if (a.per_expert)
        for (int e = tid; e < a.E; e += nt) a.per_expert[e] = hist[e];
    if (a.expert_offset) block_exclusive_scan(hist, a.expert_offset, a.E, tmp);
    const bool ranks_wanted = a.per_rank || a.rank_offset;
    if (!ranks_wanted) return;   // block-uniform
    for (int tb = 0; tb < a.T; tb += nt) {
        const int64_t t = tb + tid;
        uint64_t rmask = 0, nmask = 0;
        if (t < a.T) {
            for (int j = 0; j < a.k; ++j) {
                const int e = ids[t * a.k + j];
                if (e < 0) continue;
                rmask |= 1ull << (a.epr_shift >= 0 ? e >> a.epr_shift : e / a.epr);
                nmask |= 1ull << (a.epn_shift >= 0 ? e >> a.epn_shift : e / a.epn);
            }
            if (a.in_rank) {
                uint8_t *out = a.in_rank + t * a.R;
                if ((a.R & 3) == 0) {   // 4 flags per 32-bit store (rows of R bytes, R % 4 == 0)
                    for (int r0 = 0; r0 < a.R; r0 += 4) {
                        uint32_t wd = 0;
                        for (int b = 0; b < 4; ++b) wd |= (uint32_t)((rmask >> (r0 + b)) & 1u) << (8 * b);
                        *reinterpret_cast<uint32_t *>(out + r0) = wd;
                    }
                } else {
                    for (int r = 0; r < a.R; ++r) out[r] = (uint8_t)((rmask >> r) & 1u);
                }
            }
        }
        for (uint64_t m = rmask; m; m &= m - 1) atomicAdd(&rn[__builtin_ctzll(m)], 1);
        for (uint64_t m = nmask; m; m &= m - 1) atomicAdd(&rn[a.R + __builtin_ctzll(m)], 1);
    }
    __syncthreads();
    if (a.per_rank) {
        for (int i = tid; i < a.R + a.N; i += nt) {
            if (i < a.R) a.per_rank[i] = rn[i]; else a.per_node[i - a.R] = rn[i];
        }
        if (tid == 0) {
            int64_t al = 0;
            for (int n = 0; n < a.N; ++n) al += rn[a.R + n];
            *a.algo = al;
        }
    }
    if (a.rank_offset && tid < kWave) wave_exclusive_scan(tid < a.R ? rn[tid] : 0, a.R, a.rank_offset);
}

}  // namespace ep
