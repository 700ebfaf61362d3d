// dispatch.hip -- slot assignment and the row permutation on gfx950.
//
// What it computes (MSCCL++ PR 860, RANK_MAJOR commit: the default layout
// puts each dispatched token at a compacted prefix offset; MORI-EP Benchmark,
// "NVL / XGMI bandwidth": the receive tensor holds token rows): a stable
// counting sort of the valid (t, j) pairs by expert.  Expert segments lie
// back to back in expert order (expert_offset = exclusive scan of per-expert
// counts) and inside a segment the pairs keep row-major (t, j) order.  Each
// pair's slot receives a bitwise copy of token row t.
//
// Two launches:
//   ep_slot_count  one block per tile of W*64 consecutive pairs.  Each wave
//                  sets bit `lane` of an LDS 64-bit mask per (wave, expert)
//                  with an atomic OR (order-independent); a pair's rank
//                  inside its tile is the popcount of its expert's masks of
//                  earlier waves plus the popcount of its own wave's mask
//                  below its lane.  Tile counts go to the workspace; the last
//                  block (ticket) scans them: for each expert the exclusive
//                  prefix over tiles, then the exclusive scan over experts
//                  (expert_offset).  No order-dependent atomics, so slots are
//                  deterministic.
//   ep_dispatch_copy  one wave per (token, row part): lanes 0..k-1 form the
//                  token's k slots and broadcast them to scalar registers
//                  with readlane; every lane loads its 16-byte vectors of
//                  row t once and stores them k times.  Stores are plain
//                  (write-back) so the receive rows can stay in the
//                  memory-side cache for the combine that follows.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {
namespace {

// Exclusive scan of n ints (in / out may be LDS or global; out has n + 1
// entries, out[n] = total).  All threads of the block must call it.
__device__ void block_exclusive_scan(const int32_t *in, int32_t *out, int n, int32_t *tmp) {
    const int nt = blockDim.x, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wid = tid / kWave, nw = (nt + kWave - 1) / kWave;
    const int chunk = (n + nt - 1) / nt;
    const int b = min(tid * chunk, n), e = min(b + chunk, n);
    int32_t s = 0;
    for (int i = b; i < e; ++i) s += in[i];
    int32_t v = s;
    for (int off = 1; off < kWave; off <<= 1) {
        const int32_t u = __shfl_up(v, off);
        if (lane >= off) v += u;
    }
    if (lane == kWave - 1) tmp[wid] = v;
    __syncthreads();
    if (tid == 0) {
        int32_t run = 0;
        for (int w = 0; w < nw; ++w) {
            const int32_t x = tmp[w];
            tmp[w] = run;
            run += x;
        }
        tmp[nw] = run;
    }
    __syncthreads();
    int32_t excl = tmp[wid] + v - s;
    for (int i = b; i < e; ++i) {
        const int32_t x = in[i];
        out[i] = excl;
        excl += x;
    }
    if (tid == 0) out[n] = tmp[nw];
    __syncthreads();
}

struct SlotArgs {
    const int64_t *topk_idx;
    int64_t TK;          // T * k pairs
    int E, tile, ntiles;
    int32_t *tile_count;  // [ntiles][E]
    int32_t *local_rank;  // [TK]
    int32_t *expert_offset;
    uint32_t *ctrl;
};

constexpr int kScanMax = 4096;   // largest supported E

__global__ __launch_bounds__(1024) void ep_slot_count_kernel(SlotArgs a) {
    extern __shared__ uint64_t masks[];        // [W][E]
    __shared__ int32_t part[kScanMax + 1];     // last block: per-(q, e) sums, then totals
    __shared__ int32_t tmp[1024 / kWave + 1];
    __shared__ uint32_t last_block;
    const int tid = threadIdx.x, nt = blockDim.x;
    const int lane = tid & (kWave - 1), w = tid / kWave, W = nt / kWave;
    const int E = a.E;
    for (int i = tid; i < W * E; i += nt) masks[i] = 0ull;
    __syncthreads();

    const int64_t p = (int64_t)blockIdx.x * a.tile + tid;
    int e = -1;
    bool bad = false;
    if (p < a.TK) {
        const int64_t v = a.topk_idx[p];
        if (v >= 0 && v < E) {
            e = (int)v;
            atomicOr((unsigned long long *)&masks[w * E + e], 1ull << lane);
        } else if (v >= E) {
            bad = true;
        }
    }
    __syncthreads();
    if (p < a.TK) {
        int32_t r = -1;
        if (e >= 0) {
            r = (int32_t)__popcll(masks[w * E + e] & lanemask_lt());
            for (int w2 = 0; w2 < w; ++w2) r += (int32_t)__popcll(masks[w2 * E + e]);
        }
        a.local_rank[p] = r;
    }
    int32_t *mine = a.tile_count + (size_t)blockIdx.x * E;
    for (int e2 = tid; e2 < E; e2 += nt) {
        int32_t c = 0;
        for (int w2 = 0; w2 < W; ++w2) c += (int32_t)__popcll(masks[w2 * E + e2]);
        mine[e2] = c;
    }
    if (__ballot(bad) && lane == 0) atomicOr(&a.ctrl[0], kErrBadExpert);
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&a.ctrl[2], 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        last_block = (prev == (uint32_t)(a.ntiles - 1));
    }
    __syncthreads();
    if (!last_block) return;
    __threadfence();

    // ---- last block: prefix over tiles per expert, then scan over experts.
    // Q threads share one expert's tiles when E < blockDim.
    const int Q = (nt >= E) ? nt / E : 1;
    const int chunk = (a.ntiles + Q - 1) / Q;
    for (int idx = tid; idx < E * Q; idx += nt) {
        const int ee = idx % E, q = idx / E;
        const int t0 = min(q * chunk, a.ntiles), t1 = min(t0 + chunk, a.ntiles);
        int32_t s = 0;
        for (int t = t0; t < t1; ++t)
            s += __hip_atomic_load(a.tile_count + (size_t)t * E + ee, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        part[idx] = s;   // idx = q * E + ee
    }
    __syncthreads();
    for (int idx = tid; idx < E * Q; idx += nt) {
        const int ee = idx % E, q = idx / E;
        int32_t run = 0;
        for (int q2 = 0; q2 < q; ++q2) run += part[q2 * E + ee];
        const int t0 = min(q * chunk, a.ntiles), t1 = min(t0 + chunk, a.ntiles);
        for (int t = t0; t < t1; ++t) {
            int32_t *cell = a.tile_count + (size_t)t * E + ee;
            const int32_t c = __hip_atomic_load(cell, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *cell = run;
            run += c;
        }
    }
    __syncthreads();
    // totals per expert into part[0..E) (q = 0 row), summing the Q partials
    for (int ee = tid; ee < E; ee += nt) {
        int32_t s = 0;
        for (int q = 0; q < Q; ++q) s += part[q * E + ee];
        part[ee] = s;   // only this thread reads/writes column ee
    }
    __syncthreads();
    block_exclusive_scan(part, a.expert_offset, E, tmp);
    if (tid == 0) __hip_atomic_store(&a.ctrl[2], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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
    const int32_t *expert_offset;
    const int32_t *tile_prefix;   // [ntiles][E]
    const int32_t *local_rank;    // [T*k]
    uint32_t *ctrl;               // error word
    int64_t T;
    int k, E, tile;
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
    if (t >= a.T) return;   // wave-uniform

    // lanes 0..k-1: the token's slots
    int32_t slot = -1;
    if (lane < a.k) {
        const int64_t p = t * a.k + lane;
        const int32_t lr = a.local_rank[p];
        if (lr >= 0) {
            const int e = (int)a.topk_idx[p];
            slot = a.expert_offset[e] + a.tile_prefix[(p / a.tile) * a.E + e] + lr;
            if ((uint64_t)slot >= (uint64_t)(a.T * a.k)) {   // cannot happen; never write outside
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
    if (__ballot(slot >= 0) == 0) return;   // no valid slot: the row is not read

    // fp32 scale rows (fp8 payload): lanes spread over the waves of the token
    if (a.G > 0) {
        for (int g = lane + kWave * sub; g < a.G; g += kWave * a.S) {
            const float sc = a.x_scales[t * a.G + g];
            for (int j = 0; j < a.k; ++j) {
                const int32_t s = readlane(slot, j);
                if (s >= 0) a.recv_scales[(int64_t)s * a.G + g] = sc;
            }
        }
    }

    const char *src = a.x + t * a.row_bytes;
    const int stride = kWave * a.S;            // vectors between a lane's consecutive vectors
    for (int v0 = lane + kWave * sub; v0 < a.nvec; v0 += stride * VPL) {
        vec16 buf[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int v = v0 + i * stride;
            if (v < a.nvec) buf[i] = ld16(src + (int64_t)v * 16);
        }
        for (int j = 0; j < a.k; ++j) {
            const int32_t s = readlane(slot, j);
            if (s < 0) continue;
            char *dst = a.recv_x + (int64_t)s * a.row_bytes;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int v = v0 + i * stride;
                if (v < a.nvec) st16(dst + (int64_t)v * 16, buf[i]);
            }
        }
    }
}

}  // namespace

hipError_t launch_slot_count(const Shape &s, const WsLayout &L, const int64_t *topk_idx,
                             int32_t *expert_offset, char *ws, hipStream_t stream) {
    SlotArgs a;
    a.topk_idx = topk_idx;
    a.TK = s.T * s.k;
    a.E = s.E;
    a.tile = L.slot_tile;
    a.ntiles = L.slot_tiles;
    a.tile_count = reinterpret_cast<int32_t *>(ws + L.tile_count);
    a.local_rank = reinterpret_cast<int32_t *>(ws + L.local_rank);
    a.expert_offset = expert_offset;
    a.ctrl = reinterpret_cast<uint32_t *>(ws + L.ctrl);
    const size_t lds = sizeof(uint64_t) * (size_t)L.slot_waves * (size_t)s.E;
    hipLaunchKernelGGL(ep_slot_count_kernel, dim3(L.slot_tiles), dim3(L.slot_tile), lds, stream, a);
    return hipGetLastError();
}

int waves_per_token(int64_t T, int64_t row_vectors) {
    int S = 1;
    while (T * S < 2048 && (row_vectors / (2 * S)) >= kWave && S < 64) S *= 2;
    return S;
}

hipError_t launch_dispatch_copy(const Shape &s, const WsLayout &L, const void *x,
                                const float *x_scales, const int64_t *topk_idx,
                                const float *topk_w, void *recv_x, float *recv_x_scales,
                                int32_t *recv_src_idx, float *recv_topk_w, int32_t *token_slot,
                                const int32_t *expert_offset, char *ws, hipStream_t stream) {
    if (s.T == 0) return hipSuccess;
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
    a.expert_offset = expert_offset;
    a.tile_prefix = reinterpret_cast<const int32_t *>(ws + L.tile_count);
    a.local_rank = reinterpret_cast<const int32_t *>(ws + L.local_rank);
    a.ctrl = reinterpret_cast<uint32_t *>(ws + L.ctrl);
    a.T = s.T;
    a.k = s.k;
    a.E = s.E;
    a.tile = L.slot_tile;
    const bool fp8 = (s.x_fmt == 1);
    a.row_bytes = fp8 ? (int64_t)s.H : 2 * (int64_t)s.H;
    a.nvec = (int)(a.row_bytes / 16);
    a.G = fp8 ? s.H / 128 : 0;
    a.S = waves_per_token(s.T, a.nvec);
    const int per_lane = (a.nvec + kWave * a.S - 1) / (kWave * a.S);
    const int64_t waves = s.T * a.S;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (per_lane <= 4) {
        hipLaunchKernelGGL(ep_dispatch_copy_kernel<4>, grid, block, 0, stream, a);
    } else if (per_lane <= 8) {
        hipLaunchKernelGGL(ep_dispatch_copy_kernel<8>, grid, block, 0, stream, a);
    } else {
        hipLaunchKernelGGL(ep_dispatch_copy_kernel<16>, grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace ep
