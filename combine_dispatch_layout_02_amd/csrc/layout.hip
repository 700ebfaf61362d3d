// layout.hip -- the layout pass on gfx950.
//
// What it computes (MORI-EP Benchmark, "Why DeepEP and Mori RDMA token counts
// are equivalent", Steps 1-3; the reference script's per-rank counts): for
// every token the set of virtual ranks and the set of virtual nodes its valid
// experts live on (rank = e / (E/R), node = e / (E/N)), with repeats
// collapsed; per-rank and per-node token counts, per-expert pair counts, the
// token-in-rank map and the RDMA algo count (deduplicated (token, node)
// pairs, local node included).
//
// How: one lane per token.  The deduplication happens in registers: the
// token's ranks and nodes are OR-ed into two 64-bit masks, so a repeated rank
// or node is a no-op.  Per-rank / per-node counts are wavefront ballots of one
// mask bit followed by a popcount (one scalar add per wave and bit); expert
// counts go through an LDS histogram with integer atomics.  Blocks publish
// their counts to the workspace and the last block to finish (a ticket
// counter) sums them in block order, so the outputs are written in full in one
// launch, with no pre-zeroed output and no order-dependent result.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

struct LayoutArgs {
    const int64_t *topk_idx;
    int64_t T;
    int k, E, R, N, epr, epn;
    int32_t *per_rank, *per_expert, *per_node;
    uint8_t *in_rank;
    int64_t *algo;
    int32_t *partial;
    uint32_t *ctrl;
    int nblocks;
};

__global__ __launch_bounds__(kLayoutTokens) void ep_layout_kernel(LayoutArgs a) {
    extern __shared__ int32_t hist[];   // [R + N + E]: ranks, nodes, experts
    __shared__ uint32_t last_block;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int ncnt = a.R + a.N + a.E;
    for (int i = tid; i < ncnt; i += blockDim.x) hist[i] = 0;
    __syncthreads();

    const int64_t t = (int64_t)blockIdx.x * kLayoutTokens + tid;
    uint64_t rmask = 0, nmask = 0;
    bool bad = false;
    if (t < a.T) {
        const int64_t *row = a.topk_idx + t * a.k;
        for (int j = 0; j < a.k; ++j) {
            const int64_t e = row[j];
            if (e < 0) continue;                       // masked slot
            if (e >= a.E) { bad = true; continue; }    // invalid id: treated as masked
            const int ei = (int)e;
            rmask |= 1ull << (ei / a.epr);
            nmask |= 1ull << (ei / a.epn);
            atomicAdd(&hist[a.R + a.N + ei], 1);
        }
        // token-in-rank row: R bytes, widest aligned stores the row allows
        uint8_t *out = a.in_rank + t * a.R;
        if ((a.R & 15) == 0) {
            for (int r0 = 0; r0 < a.R; r0 += 16) {
                vec16 v;
                for (int q = 0; q < 4; ++q) {
                    uint32_t w = 0;
                    for (int b = 0; b < 4; ++b) w |= (uint32_t)((rmask >> (r0 + 4 * q + b)) & 1u) << (8 * b);
                    v[q] = w;
                }
                st16(out + r0, v);
            }
        } else if ((a.R & 3) == 0) {
            for (int r0 = 0; r0 < a.R; r0 += 4) {
                uint32_t w = 0;
                for (int b = 0; b < 4; ++b) w |= (uint32_t)((rmask >> (r0 + b)) & 1u) << (8 * b);
                *reinterpret_cast<uint32_t *>(out + r0) = w;
            }
        } else {
            for (int r = 0; r < a.R; ++r) out[r] = (uint8_t)((rmask >> r) & 1u);
        }
    }

    // per-rank / per-node token counts: ballot of one bit, popcount, one add per wave
    for (int r = 0; r < a.R; ++r) {
        const uint64_t b = __ballot((rmask >> r) & 1u);
        if (lane == 0 && b) atomicAdd(&hist[r], (int)__popcll(b));
    }
    for (int n = 0; n < a.N; ++n) {
        const uint64_t b = __ballot((nmask >> n) & 1u);
        if (lane == 0 && b) atomicAdd(&hist[a.R + n], (int)__popcll(b));
    }
    if (__ballot(bad) && lane == 0) atomicOr(&a.ctrl[0], kErrBadExpert);
    __syncthreads();

    int32_t *mine = a.partial + (size_t)blockIdx.x * ncnt;
    for (int i = tid; i < ncnt; i += blockDim.x) mine[i] = hist[i];
    __threadfence();   // publish this block's counts before taking a ticket
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&a.ctrl[1], 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        last_block = (prev == (uint32_t)(a.nblocks - 1));
    }
    __syncthreads();
    if (!last_block) return;
    __threadfence();

    // last block: sum the partial counts in block order
    for (int i = tid; i < ncnt; i += blockDim.x) {
        int32_t s = 0;
        for (int b = 0; b < a.nblocks; ++b)
            s += __hip_atomic_load(a.partial + (size_t)b * ncnt + i, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        if (i < a.R) a.per_rank[i] = s;
        else if (i < a.R + a.N) a.per_node[i - a.R] = s;
        else a.per_expert[i - a.R - a.N] = s;
        hist[i] = s;
    }
    __syncthreads();
    if (tid == 0) {
        int64_t algo = 0;
        for (int n = 0; n < a.N; ++n) algo += hist[a.R + n];
        *a.algo = algo;
        __hip_atomic_store(&a.ctrl[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace

hipError_t launch_layout(const Shape &s, const WsLayout &L, const int64_t *topk_idx,
                         int32_t *per_rank, int32_t *per_expert, uint8_t *in_rank,
                         int32_t *per_node, int64_t *algo, char *ws, hipStream_t stream) {
    LayoutArgs a;
    a.topk_idx = topk_idx;
    a.T = s.T;
    a.k = s.k;
    a.E = s.E;
    a.R = s.R;
    a.N = s.N;
    a.epr = s.E / s.R;
    a.epn = s.E / s.N;
    a.per_rank = per_rank;
    a.per_expert = per_expert;
    a.per_node = per_node;
    a.in_rank = in_rank;
    a.algo = algo;
    a.partial = reinterpret_cast<int32_t *>(ws + L.partial);
    a.ctrl = reinterpret_cast<uint32_t *>(ws + L.ctrl);
    a.nblocks = L.layout_blocks;
    const size_t lds = sizeof(int32_t) * (size_t)(s.R + s.N + s.E);
    hipLaunchKernelGGL(ep_layout_kernel, dim3(L.layout_blocks), dim3(kLayoutTokens), lds, stream, a);
    return hipGetLastError();
}

}  // namespace ep
