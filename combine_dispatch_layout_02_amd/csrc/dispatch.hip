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
// stores them k times.  When the combine may read the receive rows as they
// are (bf16 rows, bf16 combine payload), the rows of the first tokens, up to
// EP_DISPATCH_PLAIN_MIB, are stored plain (write-back) and stay in the 256 MB
// memory-side cache until the combine reads them; the later tokens' rows are
// stored non-temporal so they do not evict the first ones.  The waves take
// the two kinds of token interleaved (position g of P cached tokens among T
// goes to a cached token when floor((g+1)P/T) > floor(gP/T)), so writes into
// the cache and writes to HBM run side by side instead of one phase after
// the other (T = 4096, hidden 7168, top-8: 83 -> 78 us; T = 8192 skewed:
// 174 -> 158 us).  The combine reads the tokens last to first (the rows that
// come from HBM first) and stores y non-temporal.  Other format pairs store
// every row non-temporal.
//
// The cached form (ep_dispatch_cached) takes the slots from a previous
// dispatch's handle instead of a plan: the same rows, for another tensor of
// the same tokens, with no layout work and no metadata writes.
//
// Batches of at most kFusedPairs (2048) pairs (compacted layout) can run as ONE
// launch that also does the layout: block 0 computes the counts, the
// token-in-rank map and the segment starts (the handle) while every other
// wave finds its token's slots by counting, over all pairs of the batch,
// the pairs that sort before each of them -- the stable counting sort's
// position written out -- so no wave waits for a plan.
#include "ep_device.h"
#include "ep_internal.h"
#include "small_layout.h"

namespace ep {
namespace {

#ifndef EP_DISPATCH_NT_STORE
#define EP_DISPATCH_NT_STORE 0   // 1: non-temporal stores for every receive row
#endif
#ifndef EP_DISPATCH_WAVES
#define EP_DISPATCH_WAVES 4096   // waves the copy aims for (4 per CU)
#endif
#ifndef EP_DISPATCH_ORDER
#define EP_DISPATCH_ORDER 1      // 1: tokens stored plain interleaved with the non-temporal ones
#endif
#ifndef EP_DISPATCH_PLAIN_MIB
#define EP_DISPATCH_PLAIN_MIB 192   // receive bytes (MiB) stored plain when the combine reads them
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
    const int32_t *slots_in;      // [T*k] a previous dispatch's token_slot (cached form), else null
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
    int nt_store;             // non-temporal row stores for every token (see copy_args)
    int64_t plain_tokens;     // otherwise: tokens t < plain_tokens store plain, the rest non-temporal
    // single-launch form only: layout outputs (null when not wanted)
    int R, N, epn, epn_shift;
    int32_t *per_rank, *per_expert, *per_node;
    uint8_t *in_rank;
    int64_t *algo;
    // copy that rebuilds the plan (layout + dispatch in two launches): the
    // raw tile counts (in tile_prefix) and, per expert e and tile u, {pairs
    // of u with an expert below e, pairs of u with e} ([E][ntiles])
    const int2 *tile_pairs;
    int ntiles;
};

constexpr int kFusedPairs = 2048;   // pairs a single-launch batch may hold (32 ids per lane)

// Slot of pair (t, j) held by lane j < k, by counting: the valid pairs whose
// expert sorts before e_j, plus the pairs of e_j earlier in row-major (t, j)
// order.  The block stages the batch's pair ids in LDS once (masked and
// invalid ids as INT_MAX, which sorts after every expert); each lane then
// holds KEYS of them in registers (KEYS * 64 >= T * k) and the counts are
// ballots.  The token's S waves share the work (wave `sub` counts slots j =
// sub, sub + S, ...) and exchange the results through LDS: one token per
// block, every thread of the block calls this.
template <int KEYS>
__device__ __forceinline__ int32_t counted_slot(const CopyArgs &a, int64_t t, int lane, int sub) {
    extern __shared__ int32_t ids_sm[];   // [T * k]
    __shared__ int32_t slot_sm[32];
    const int TK = (int)(a.T * a.k);
    for (int q = threadIdx.x; q < TK; q += blockDim.x) {
        const int64_t id = a.topk_idx[q];
        ids_sm[q] = (id >= 0 && id < a.E) ? (int32_t)id : 0x7FFFFFFF;
    }
    __syncthreads();
    int32_t key[KEYS];
#pragma unroll
    for (int i = 0; i < KEYS; ++i) {
        const int q = lane + kWave * i;
        key[i] = q < TK ? ids_sm[q] : 0x7FFFFFFF;
    }
    const int32_t mine = lane < a.k ? ids_sm[t * a.k + lane] : 0x7FFFFFFF;   // lane j < k: slot j's id
    for (int j = sub; j < a.k; j += a.S) {
        const int32_t e = readlane(mine, j);
        int32_t c = -1;                  // masked slot
        if (e != 0x7FFFFFFF) {           // uniform
            const int p = (int)(t * a.k + j);
            c = 0;
#pragma unroll
            for (int i = 0; i < KEYS; ++i) {
                const int q = lane + kWave * i;
                c += (int32_t)__popcll(__ballot(key[i] < e || (key[i] == e && q < p)));
            }
        }
        if (lane == 0) slot_sm[j] = c;
    }
    __syncthreads();
    return lane < a.k ? slot_sm[lane] : -1;
}

// Segment start of each of the token's valid slots plus the pairs of the same
// expert in earlier tiles, rebuilt from the tile counts: for slot j with
// expert e, the sum over tiles u of the pairs of u with smaller experts, plus,
// for u before the token's tile, the pairs of u with e.  One tile per lane
// (one 8-byte load of e's contiguous per-tile pairs) and one wave sum per
// slot, eight slots at a time; lane j < k returns slot j's value.  em: lane
// j's expert, -1 when masked.
__device__ __forceinline__ int32_t slot_bases(const CopyArgs &a, int em, int tile, int lane) {
    int32_t base = 0;
    for (int j0 = 0; j0 < a.k; j0 += 8) {
        int32_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)   // lanes >= k hold -1 (j0 + q < 64)
            v[q] = tile_pair_sum_lane(a.tile_pairs, a.ntiles, readlane(em, j0 + q), tile, lane);
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = wave_sum(v[q]);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (lane == j0 + q) base = v[q];
    }
    return base;
}

// Row t's vectors of this wave into the token's valid slots, VPL vectors per
// lane per pass (the first pass is already in buf); NT: non-temporal stores.
template <int VPL, bool NT>
__device__ __forceinline__ void store_rows(const CopyArgs &a, const char *src, int32_t slot, vec16 (&buf)[VPL],
                                           int v_first, int stride) {
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
                    if (NT) st16_nt(dst + (int64_t)v * 16, buf[i]);
                    else st16(dst + (int64_t)v * 16, buf[i]);
                }
            }
        }
    }
}

// VPL: 16-byte vectors each lane holds per pass.  KEYS > 0: the single-launch
// form (block 0 does the layout, the other blocks count their slots over
// KEYS pair ids per lane); KEYS == 0: slots from the plan.
// The single-launch form runs one token per block (S waves of 64).  NT:
// non-temporal row stores (a compile-time choice: a run-time test between
// the two store kinds is merged by the compiler into plain stores).
// SCAN: the copy of layout + dispatch in two launches -- block 0 writes the
// layout totals and the handle's segment starts (plan_totals_block), and
// every wave rebuilds its slots' segment starts from the tile counts
// (slot_bases) instead of reading a scanned plan.
template <int VPL, int KEYS, bool NT, bool SCAN = false>
__global__ __launch_bounds__(KEYS ? 1024 : 256) void ep_dispatch_copy_kernel(CopyArgs a) {
    constexpr bool FUSED = KEYS > 0;
    if (SCAN && blockIdx.x == 0) {
        extern __shared__ int32_t tot_sm[];
        plan_totals_block(a.tile_prefix, a.ntiles, a.E, a.R, a.N, a.per_expert, a.per_rank, a.per_node, a.algo,
                          a.expert_offset, nullptr, tot_sm);
        return;
    }
    if (FUSED && blockIdx.x == 0) {
        SmallLayout L{};
        L.topk_idx = a.topk_idx;
        L.T = a.T;
        L.k = a.k;
        L.E = a.E;
        L.R = a.R;
        L.N = a.N;
        L.epr = a.epr;
        L.epr_shift = a.epr_shift;
        L.epn = a.epn;
        L.epn_shift = a.epn_shift;
        L.ctrl = a.ctrl;
        L.per_expert = a.per_expert;
        L.expert_offset = a.expert_offset;
        L.per_rank = a.per_rank;
        L.per_node = a.per_node;
        L.in_rank = a.in_rank;
        L.algo = a.algo;
        small_layout_block(L);
        return;
    }
    const int lane = threadIdx.x & (kWave - 1);
    int64_t t;
    int sub;
    if (FUSED) {
        t = (int64_t)blockIdx.x - 1;   // < T: the grid has 1 + T blocks
        sub = threadIdx.x / kWave;
    } else {
        const int64_t gw = ((int64_t)blockIdx.x - (SCAN ? 1 : 0)) * (blockDim.x / kWave) + threadIdx.x / kWave;
        const int64_t pos = gw / a.S;
        sub = (int)(gw - pos * a.S);
        t = (EP_DISPATCH_ORDER && pos < a.T) ? interleaved_token(pos, a.T, a.plain_tokens) : pos;
        const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
        if (!SCAN && !a.slots_in && g <= a.E) a.expert_offset[g] = a.plan_offset[g];   // handle copy of the segment starts
    }
    if (t >= a.T) return;   // wave-uniform (never taken in the single-launch form)

    // A wave's vector loads return in issue order.  The inputs of the
    // token's slots are loaded first (lanes 0..k-1), then the first pass of
    // row t, which does not depend on them; the plan lookups that need the
    // inputs are issued as soon as those arrive, while the row is still in
    // flight, instead of queueing behind the whole row.
    int32_t pw = -1, slot_in = -1;
    int64_t eid = -1;
    float wv = 0.0f;
    if (lane < a.k) {
        const int64_t p = t * a.k + lane;
        if (!FUSED && a.slots_in) {
            slot_in = a.slots_in[p];
        } else {
            wv = a.topk_w[p];
            if (!FUSED) {
                pw = a.local_rank[p];   // the plan word: expert and local rank, or -1
                eid = a.topk_idx[p];
            }
        }
    }
    // fp32 scales of an fp8 row (one per 128 elements): this wave's share
    // (G <= 64 * S, one value per lane, in every shape the ABI accepts with
    // hidden <= 8192 * S; larger rows loop below)
    const int g_first = lane + kWave * sub;
    float sc0 = 0.0f;
    if (g_first < a.G) sc0 = a.x_scales[t * a.G + g_first];
    const char *src = a.x + t * a.row_bytes;
    const int stride = kWave * a.S;            // vectors between a lane's consecutive vectors
    const int v_first = lane + kWave * sub;
    // Unconditional loads (a vector past the row re-reads its last vector and
    // is not stored), so the compiler knows how many row loads are younger
    // than the slot inputs and waits for those inputs alone.
    vec16 buf[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int v = min(v_first + i * stride, a.nvec - 1);
        buf[i] = ld16(src + (int64_t)v * 16);
    }

    // The plan was made for the pair's expert: a pair whose expert in
    // topk_idx is not the planned one (a plan reused with other ids) gets no
    // slot, and the call raises kErrStalePlan.
    int32_t lr = -1;
    if (!FUSED && lane < a.k && !a.slots_in) {
        const bool now_valid = eid >= 0 && eid < a.E;
        if (pw >= 0 && now_valid && (pw >> kPlanLrBits) == (int32_t)eid) {
            lr = pw & ((1 << kPlanLrBits) - 1);
        } else if (pw >= 0 || now_valid) {   // planned but not valid now, valid but not planned, or moved
            atomicOr(&a.ctrl[0], kErrStalePlan);
        }
    }

    // lanes 0..k-1: the token's slots
    int32_t slot = FUSED ? counted_slot<(KEYS > 0 ? KEYS : 1)>(a, t, lane, sub) : -1;
    const int32_t base = SCAN ? slot_bases(a, (lane < a.k && lr >= 0) ? (int)eid : -1, (int)(t / a.TT), lane) : 0;
    // RANK_MAJOR in the scanning copy: the compacted start of the slot's
    // rank, i.e. the segment start of the rank's first expert (the sum of
    // that expert's pairs below it over all tiles: tile 0 adds no earlier
    // tiles)
    int32_t rank_start = 0;
    if (SCAN && a.M > 0) {   // uniform
        const int r0 = (lane < a.k && lr >= 0)
                           ? (a.epr_shift >= 0 ? (int)eid >> a.epr_shift : (int)eid / a.epr) * a.epr : -1;
        rank_start = slot_bases(a, r0, 0, lane);
    }
    if (lane < a.k) {
        const int64_t p = t * a.k + lane;
        if (!FUSED && a.slots_in) {   // cached: the slots of a previous dispatch's handle
            slot = slot_in;
            if ((uint64_t)slot >= (uint64_t)a.rows) slot = -1;   // masked, or not a receive row
        }
        if (lr >= 0) {   // a valid pair (the plan's local rank is -1 for masked ones)
            const int e = (int)eid;
            slot = SCAN ? base + lr : a.plan_offset[e] + a.tile_prefix[(t / a.TT) * a.cols + e] + lr;
            if (a.M > 0) {   // RANK_MAJOR: the same place inside the rank, at the rank's fixed block
                const int r = a.epr_shift >= 0 ? e >> a.epr_shift : e / a.epr;
                const int32_t in_rank = slot - (SCAN ? rank_start : a.plan_offset[r * a.epr]);
                if (in_rank < a.M) {
                    slot = r * a.M + in_rank;
                } else {
                    atomicOr(&a.ctrl[0], kErrRankOverflow);
                    slot = -1;
                }
            }
        }
        if (slot >= 0 && (uint64_t)slot >= (uint64_t)a.rows) {   // cannot happen; never write outside
            atomicOr(&a.ctrl[0], kErrBadSlot);
            slot = -1;
        }
        if (sub == 0 && !a.slots_in) {
            a.token_slot[p] = slot;
            if (slot >= 0) {
                a.recv_src_idx[slot] = (int32_t)t;
                a.recv_topk_w[slot] = wv;
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

    // wave-uniform choice between two copies of the store loop (one store
    // kind each, so the compiler keeps both)
    if (EP_DISPATCH_NT_STORE || NT || t >= a.plain_tokens)
        store_rows<VPL, true>(a, src, slot, buf, v_first, stride);
    else
        store_rows<VPL, false>(a, src, slot, buf, v_first, stride);
}

}  // namespace

// Tokens whose receive rows are stored plain when the combine reads the
// receive rows as they are: the first ones, up to EP_DISPATCH_PLAIN_MIB of
// rows (under the 256 MB memory-side cache, leaving room for x); the later
// tokens' rows are stored non-temporal, so they do not evict the first ones.
// Measured per dispatch -> combine step against plain stores for every row:
// T = 2048, 4096 and 8192 (skewed) at hidden 7168, top-8: 105 -> 94,
// 193 -> 181 and 413 -> 376 us.  The combine derives the same count from the
// shape.
int64_t cached_tokens(const Shape &s) {
    if (!(s.x_fmt == 0 && s.y_fmt == 0)) return 0;   // the combine reads re-encoded rows
    const int64_t bytes_per_token = (int64_t)s.k * 2 * s.H;
    const int64_t n = ((int64_t)EP_DISPATCH_PLAIN_MIB << 20) / bytes_per_token;
    return n < s.T ? n : s.T;
}

int waves_per_token(int64_t T, int64_t row_vectors, int64_t target) {
    // aim for `target` waves, keep >= 64 row vectors per wave
    int S = 1;
    while (T * S < target && (row_vectors / (2 * S)) >= kWave && S < 64) S *= 2;
    return S;
}

namespace {

CopyArgs copy_args(const Shape &s, const void *x, const float *x_scales, const int64_t *topk_idx,
                   const float *topk_w, void *recv_x, float *recv_x_scales, int32_t *recv_src_idx,
                   float *recv_topk_w, int32_t *token_slot, int32_t *expert_offset) {
    CopyArgs a{};
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
    a.T = s.T;
    a.k = s.k;
    a.E = s.E;
    a.R = s.R;
    a.N = s.N;
    a.cols = s.E + s.R + s.N;
    a.M = s.M;
    a.epr = s.E / s.R;
    a.epr_shift = (a.epr & (a.epr - 1)) == 0 ? __builtin_ctz((unsigned)a.epr) : -1;
    a.epn = s.E / s.N;
    a.epn_shift = (a.epn & (a.epn - 1)) == 0 ? __builtin_ctz((unsigned)a.epn) : -1;
    a.rows = s.rows();
    const bool fp8 = (s.x_fmt == 1);
    a.row_bytes = fp8 ? (int64_t)s.H : 2 * (int64_t)s.H;
    a.nvec = (int)(a.row_bytes / 16);
    a.G = fp8 ? s.H / 128 : 0;
    a.S = waves_per_token(s.T, a.nvec, EP_DISPATCH_WAVES);
    // When the combine payload has another format than the dispatched rows
    // (fp8 rows -> mxfp8, bf16 rows -> nvfp4), the combine never reads the
    // receive rows: the expert stage re-encodes them.  Their stores then
    // bypass the memory-side cache instead of filling it with lines the
    // combine will not read (quant: 128 -> 118 us per step, nvfp4: 165 ->
    // 158 us).  When the formats match, the combine may read them as they
    // are, and the first plain_tokens tokens' rows stay in that cache.
    a.nt_store = !(s.x_fmt == 0 && s.y_fmt == 0);
    a.plain_tokens = cached_tokens(s);
    return a;
}

template <int KEYS, bool NT, bool SCAN>
void launch_copy_nt(const CopyArgs &a, const dim3 &grid, const dim3 &block, size_t lds, hipStream_t stream) {
    const int per_lane = (a.nvec + kWave * a.S - 1) / (kWave * a.S);
    if constexpr (KEYS == 0) {
        // hidden 7168 at one wave per token: exactly 14 (bf16) or 7 (e4m3)
        // vectors per lane, so no lane loads a vector past the row
        if (a.nvec == 14 * kWave * a.S) {
            hipLaunchKernelGGL((ep_dispatch_copy_kernel<14, KEYS, NT, SCAN>), grid, block, lds, stream, a);
            return;
        }
        if (a.nvec == 7 * kWave * a.S) {
            hipLaunchKernelGGL((ep_dispatch_copy_kernel<7, KEYS, NT, SCAN>), grid, block, lds, stream, a);
            return;
        }
    }
    if (per_lane <= 2) {
        hipLaunchKernelGGL((ep_dispatch_copy_kernel<2, KEYS, NT, SCAN>), grid, block, lds, stream, a);
    } else if (per_lane <= 4) {
        hipLaunchKernelGGL((ep_dispatch_copy_kernel<4, KEYS, NT, SCAN>), grid, block, lds, stream, a);
    } else if (per_lane <= 8 || KEYS) {   // the single-launch form has at most 8 (fused_dispatch_fits)
        hipLaunchKernelGGL((ep_dispatch_copy_kernel<8, KEYS, NT, SCAN>), grid, block, lds, stream, a);
    } else {
        hipLaunchKernelGGL((ep_dispatch_copy_kernel<16, KEYS, NT, SCAN>), grid, block, lds, stream, a);
    }
}

template <int KEYS, bool SCAN = false>
void launch_copy(const CopyArgs &a, int64_t blocks, int threads, size_t lds, hipStream_t stream) {
    const dim3 grid((unsigned)blocks), block(threads);
    if (a.nt_store) launch_copy_nt<KEYS, true, SCAN>(a, grid, block, lds, stream);
    else launch_copy_nt<KEYS, false, SCAN>(a, grid, block, lds, stream);
}

}  // namespace

hipError_t launch_dispatch_copy(const Shape &s, const WsLayout &L, const void *x,
                                const float *x_scales, const int64_t *topk_idx,
                                const float *topk_w, void *recv_x, float *recv_x_scales,
                                int32_t *recv_src_idx, float *recv_topk_w, int32_t *token_slot,
                                int32_t *expert_offset, char *ws, hipStream_t stream) {
    CopyArgs a = copy_args(s, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales, recv_src_idx,
                           recv_topk_w, token_slot, expert_offset);
    a.plan_offset = reinterpret_cast<const int32_t *>(ws + L.plan_offset);
    a.tile_prefix = reinterpret_cast<const int32_t *>(ws + L.tile_count);
    a.local_rank = reinterpret_cast<const int32_t *>(ws + L.local_rank);
    a.ctrl = reinterpret_cast<uint32_t *>(ws + L.ctrl);
    a.TT = L.tile_tokens;
    int64_t blocks = (s.T * a.S + 3) / 4;
    if (blocks * 256 < s.E + 1) blocks = (s.E + 1 + 255) / 256;   // threads to copy expert_offset
    launch_copy<0>(a, blocks, 256, 0, stream);
    return hipGetLastError();
}

bool scan_in_copy_fits(const Shape &s, const WsLayout &L) {
    return s.T > 0 && !s.rank_rows && L.tiles > 1 && L.tiles <= kScanCopyMaxTiles;
}

hipError_t launch_dispatch_scan_copy(const Shape &s, const WsLayout &L, const void *x,
                                     const float *x_scales, const int64_t *topk_idx,
                                     const float *topk_w, void *recv_x, float *recv_x_scales,
                                     int32_t *recv_src_idx, float *recv_topk_w, int32_t *token_slot,
                                     int32_t *expert_offset, int32_t *per_rank, int32_t *per_expert,
                                     int32_t *per_node, int64_t *algo, char *ws, hipStream_t stream) {
    CopyArgs a = copy_args(s, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales, recv_src_idx,
                           recv_topk_w, token_slot, expert_offset);
    a.tile_prefix = reinterpret_cast<const int32_t *>(ws + L.tile_count);   // raw tile counts
    a.tile_pairs = reinterpret_cast<const int2 *>(ws + L.tile_pairs);
    a.local_rank = reinterpret_cast<const int32_t *>(ws + L.local_rank);
    a.ctrl = reinterpret_cast<uint32_t *>(ws + L.ctrl);
    a.TT = L.tile_tokens;
    a.ntiles = L.tiles;
    a.per_rank = per_rank;
    a.per_expert = per_expert;
    a.per_node = per_node;
    a.algo = algo;
    // block 0: the totals; then the copy blocks (4 waves each)
    const int64_t blocks = 1 + (s.T * a.S + 3) / 4;
    launch_copy<0, true>(a, blocks, 256, scan_copy_lds(s), stream);
    return hipGetLastError();
}

#ifndef EP_FUSED_NT_MIB
#define EP_FUSED_NT_MIB 4        // single-launch form: receive bytes (MiB) from which every row is stored non-temporal
#endif

// Waves per token of the single-launch form: enough for the row copy, and at
// least one per slot (up to 16) so each wave counts few slots.
#ifndef EP_FUSED_MIN_WAVES
#define EP_FUSED_MIN_WAVES 1     // waves per token of the single-launch form, at least
#endif

int fused_waves(const Shape &s, int nvec) {
    int S = waves_per_token(s.T, nvec, EP_DISPATCH_WAVES);
    int want = s.k < 16 ? s.k : 16;
    if (want < EP_FUSED_MIN_WAVES) want = EP_FUSED_MIN_WAVES;
    while (S < want) S *= 2;
    return S > 16 ? 16 : S;
}

hipError_t launch_dispatch_cached(const Shape &s, const void *x, const float *x_scales,
                                  const int32_t *token_slot, void *recv_x, float *recv_x_scales,
                                  hipStream_t stream) {
    CopyArgs a = copy_args(s, x, x_scales, nullptr, nullptr, recv_x, recv_x_scales, nullptr, nullptr,
                           nullptr, nullptr);
    a.slots_in = token_slot;
    const int64_t blocks = (s.T * a.S + 3) / 4;
    if (blocks > 0) launch_copy<0>(a, blocks, 256, 0, stream);
    return hipGetLastError();
}

bool fused_dispatch_fits(const Shape &s) {
    if (!(s.T > 0 && s.T * s.k <= kFusedPairs && s.M == 0 && !s.rank_rows)) return false;
    const int nvec = (int)((s.x_fmt == 1 ? (int64_t)s.H : 2 * (int64_t)s.H) / 16);
    const int S = fused_waves(s, nvec);
    return (nvec + kWave * S - 1) / (kWave * S) <= 8;   // registers for 1024-thread blocks
}

hipError_t launch_dispatch_fused(const Shape &s, const void *x, const float *x_scales,
                                 const int64_t *topk_idx, const float *topk_w, void *recv_x,
                                 float *recv_x_scales, int32_t *recv_src_idx, float *recv_topk_w,
                                 int32_t *token_slot, int32_t *expert_offset, int32_t *per_rank,
                                 int32_t *per_expert, uint8_t *in_rank, int32_t *per_node,
                                 int64_t *algo, uint32_t *ctrl, hipStream_t stream) {
    CopyArgs a = copy_args(s, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales, recv_src_idx,
                           recv_topk_w, token_slot, expert_offset);
    a.ctrl = ctrl;
    a.per_rank = per_rank;
    a.per_expert = per_expert;
    a.in_rank = in_rank;
    a.per_node = per_node;
    a.algo = algo;
    // block 0: the layout; then one block of S waves per token (LDS: the
    // layout's staging, which is larger than the other blocks' pair ids)
    a.S = fused_waves(s, a.nvec);
    // A single-launch batch is over in a few microseconds; from a few MiB of
    // receive rows on, non-temporal stores make the whole dispatch -> combine
    // step faster (T = 128 at hidden 7168, top-8, 14.7 MB: 11.3 -> 10.7 us;
    // T = 256: 24.4 -> 22.6 us), below it plain ones (T = 1 .. 32: 0.3 -
    // 0.5 us faster).  A likely reason: plain-stored rows are still dirty in
    // the L2s when so short a kernel ends, and the kernel boundary writes
    // them back.
    if ((int64_t)s.T * s.k * a.row_bytes >= ((int64_t)EP_FUSED_NT_MIB << 20)) {
        a.nt_store = 1;
        a.plain_tokens = 0;
    }
    int threads = 0;
    const size_t lds = fused_dispatch_lds(s, &threads);
    if (s.T * s.k <= 16 * kWave) launch_copy<16>(a, 1 + s.T, threads, lds, stream);
    else launch_copy<32>(a, 1 + s.T, threads, lds, stream);
    return hipGetLastError();
}

size_t fused_dispatch_lds(const Shape &s, int *threads) {
    const int nvec = (int)((s.x_fmt == 1 ? (int64_t)s.H : 2 * (int64_t)s.H) / 16);
    const int t = kWave * fused_waves(s, nvec);
    if (threads) *threads = t;
    // the layout block's staging (pair ids, counts, scan scratch), larger than
    // the other blocks' pair ids
    return sizeof(int32_t) * ((size_t)s.T * s.k + s.E + s.R + s.N + t / kWave + 1);
}

size_t scan_copy_lds(const Shape &s) {   // the totals block of a copy that scans the tile counts
    return sizeof(int32_t) * ((size_t)s.E + s.R + s.N + 1 + 256 / kWave + 1);
}

}  // namespace ep
