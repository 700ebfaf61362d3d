// ranks.hip -- the (token, rank) receive layout on gfx950.
//
// What it computes (MSCCL++ PR 860: DeepEP's high-throughput path receives
// one row per (token, source rank) pair, its "expanded" receive layout;
// MORI-EP Benchmark, "NVL / XGMI bandwidth": one received row per token and
// destination rank, which is what num_tokens_per_rank counts): a token that
// reaches rank r (one of its valid experts lives on r) gets exactly one row
// in r's region.  Regions lie back to back in rank order, tokens ascending
// inside a region, so row = rank_offset[r] + (tokens of r in earlier plan
// tiles) + (rank of t among its tile's tokens of r), all from the plan.
// The destination applies its own experts' top-k weights and returns one
// partial row per received row; combine sums a token's partials.
//
//   ep_dispatch_ranks_kernel   row t read once, stored once per rank it
//       reaches; writes the handle (token_rank_slot, rank_offset), the source
//       index and the token's top-k list as each rank sees it.
//   ep_expert_reduce_ranks_kernel   the stand-in expert stage: per received
//       row, the fp32 fma chain over the row's local top-k slots (ascending
//       j) of w * bf16(v * factor[e]), one bf16 rounding.
//   ep_combine_ranks_kernel    y[t] = bf16_rne(fp32 sum over the token's
//       ranks, ascending, of its partials), from -0.0; +0.0 when it reaches
//       no rank.
//
// The cached form (ep_dispatch_ranks_cached) takes the rows from a previous
// dispatch's token_rank_slot: the same rows for another tensor of the same
// tokens, no plan and no metadata writes.
//
// How: one wave per (token or row, row part), as in the token-major kernels.
// Lanes 0..R-1 of a token's wave hold its row on each rank; a ballot gives
// the uniform mask of ranks reached, walked in ascending order with readlane,
// so every store and every add happens in a fixed order.
#include "ep_device.h"
#include "ep_internal.h"
#include "small_layout.h"

namespace ep {
namespace {

#ifndef EP_RANKS_WAVES
#define EP_RANKS_WAVES 4096      // waves the dispatch copy aims for
#endif
#ifndef EP_RANKS_COMBINE_WAVES
#define EP_RANKS_COMBINE_WAVES 16384
#endif
#ifndef EP_RANKS_INPUTS_FIRST
#define EP_RANKS_INPUTS_FIRST 1      // 1: the plan inputs are loaded ahead of the row (0: after it)
#endif
#ifndef EP_RANKS_NT_STORE
#define EP_RANKS_NT_STORE 1          // non-temporal stores for the received rows
#endif
#ifndef EP_RANKS_Y_NT
#define EP_RANKS_Y_NT 1              // non-temporal stores for y (whole lines per instruction)
#endif
#ifndef EP_RANKS_COMBINE_SMALL_WAVES
#define EP_RANKS_COMBINE_SMALL_WAVES 4096   // fewer combine waves than this -> one vector per lane
#endif
#ifndef EP_RANKS_COMBINE_ONE_PASS
#define EP_RANKS_COMBINE_ONE_PASS 1   // waves per token so that one pass covers a wave's part of the row
#endif
#ifndef EP_RANKS_COMBINE_VECS
#define EP_RANKS_COMBINE_VECS 4      // 16-byte vectors per lane per pass in combine
#endif

struct RankCopyArgs {
    const char *x;                  // [T][row_bytes]
    const float *x_scales;          // [T][G] or null
    const int64_t *topk_idx;        // [T][k]
    const float *topk_w;            // [T][k]
    char *recv_x;                   // [cap][row_bytes]
    float *recv_scales;             // [cap][G] or null
    int32_t *recv_src_idx;          // [cap]
    int32_t *recv_topk_idx;         // [cap][k]
    float *recv_topk_w;             // [cap][k]
    int32_t *token_rank_slot;       // [T][R] handle
    int32_t *rank_offset;           // [R + 1] handle copy
    const int32_t *plan_rank_offset;   // [R + 1] (workspace)
    const int32_t *tile_prefix;     // [ntiles][E + R + N]; rank columns: prefix over tiles
    const uint64_t *rank_mask;      // [ntiles][R][TW] tokens of each 64-token wave of a tile reaching each rank
    const int32_t *slots_in;        // [T][R] a previous dispatch's token_rank_slot (cached form), else null
    uint32_t *ctrl;
    int64_t T;
    int k, E, R, TT, TW, cols;
    int epr, epr_shift;
    int64_t cap;                    // receive rows: T * min(k, R)
    int64_t row_bytes;
    int nvec, G, S;
    // copy that rebuilds the plan (layout + dispatch in two launches): the raw
    // tile counts (in tile_prefix), per rank and tile {tokens reaching lower
    // ranks, tokens reaching the rank} ([R][ntiles]), the layout outputs
    const int2 *rank_pairs;
    int ntiles, N;
    int32_t *per_rank, *per_expert, *per_node;
    int64_t *algo;
};

// Start of each reached rank's region plus the tile's earlier-tile tokens of
// it, rebuilt from rank_pairs: one sum over tiles per rank (eight ranks at a
// time); lane r returns rank r's value.  reach: the uniform mask of ranks
// the token reaches.
__device__ __forceinline__ int32_t rank_bases(const RankCopyArgs &a, uint64_t reach, int tile, int lane) {
    int32_t base = 0;
    while (reach) {   // uniform: at most min(k, R) ranks
        int rr[8];
        int32_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            rr[q] = reach ? (int)__builtin_ctzll(reach) : -1;
            reach &= reach - 1;   // stays 0 once empty
            v[q] = tile_pair_sum_lane(a.rank_pairs, a.ntiles, rr[q], tile, lane);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = wave_sum(v[q]);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (lane == rr[q]) base = v[q];
    }
    return base;
}

constexpr int kRankFusedPairs = 2048;   // pairs a single-launch batch may hold

// Row of (t, r) for every rank r the token reaches, by counting (single-launch
// form, one token per block, every thread of the block calls this): the
// block ORs each pair's rank bit into an LDS mask per token (order-
// independent), then, for each rank r of token t (spread over the S waves),
//   row = #{(t', r') : t' reaches r', r' < r}      (the region start of r)
//       + #{t' < t : t' reaches r}                 (t's place in the region)
// over the masks of all tokens (TOK per lane): the first term a wave sum of
// popcounts, the second ballots.  Returns lane r's row (-1 when t does not
// reach r).
template <int TOK>
__device__ __forceinline__ int32_t counted_rank_slot(const RankCopyArgs &a, int64_t t, int lane, int sub) {
    extern __shared__ uint64_t tok_mask[];   // [T]
    __shared__ int32_t row_sm[64];
    const int TK = (int)(a.T * a.k);
    const int nt = blockDim.x;
    for (int i = threadIdx.x; i < a.T; i += nt) tok_mask[i] = 0ull;
    __syncthreads();
    for (int q0 = threadIdx.x; q0 < TK; q0 += 4 * nt) {   // four loads in flight per thread
        int64_t e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) e[u] = a.topk_idx[min(q0 + u * nt, TK - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q = q0 + u * nt;
            if (q < TK && e[u] >= 0 && e[u] < a.E) {
                const int r = a.epr_shift >= 0 ? (int)e[u] >> a.epr_shift : (int)e[u] / a.epr;
                atomicOr((unsigned long long *)&tok_mask[q / a.k], 1ull << r);
            }
        }
    }
    __syncthreads();
    const uint64_t mine = tok_mask[t];
    int idx = 0;
    for (uint64_t m = mine; m; m &= m - 1, ++idx) {
        if (idx % a.S != sub) continue;   // this rank belongs to another wave (uniform)
        const int r = __builtin_ctzll(m);
        const uint64_t below = (1ull << r) - 1;
        int32_t before = 0, lower = 0;
#pragma unroll
        for (int i = 0; i < TOK; ++i) {
            const int tt = lane + kWave * i;
            const uint64_t mk = tt < a.T ? tok_mask[tt] : 0ull;
            before += (int32_t)__popcll(__ballot(tt < t && ((mk >> r) & 1u)));
            lower += (int32_t)__popcll(mk & below);
        }
        for (int off = kWave / 2; off > 0; off >>= 1) lower += __shfl_xor(lower, off);
        if (lane == 0) row_sm[r] = lower + before;
    }
    __syncthreads();
    return (lane < a.R && ((mine >> lane) & 1u)) ? row_sm[lane] : -1;
}

// TOK > 0: the single-launch form (block 0 does the layout, every other block
// holds one token in S waves and counts its rows); TOK == 0: rows from the
// plan, or from a previous handle (cached form).  SCAN: the copy of layout +
// dispatch in two launches -- block 0 writes the layout totals and the
// handle's region starts, every wave rebuilds its region starts from the
// tile counts (rank_bases).
template <int VPL, int TOK, bool SCAN = false>
__global__ __launch_bounds__(TOK ? 1024 : 256) void ep_dispatch_ranks_kernel(RankCopyArgs a, SmallLayout L) {
    constexpr bool FUSED = TOK > 0;
    if (FUSED && blockIdx.x == 0) {
        small_layout_block(L);
        return;
    }
    if (SCAN && blockIdx.x == 0) {
        extern __shared__ int32_t tot_sm[];
        plan_totals_block(a.tile_prefix, a.ntiles, a.E, a.R, a.N, a.per_expert, a.per_rank, a.per_node, a.algo,
                          nullptr, a.rank_offset, tot_sm);
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
        t = gw / a.S;
        sub = (int)(gw - t * a.S);
        const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
        if (!SCAN && !a.slots_in && g <= a.R) a.rank_offset[g] = a.plan_rank_offset[g];   // handle copy of the region starts
    }
    if (t >= a.T) return;   // wave-uniform (never taken in the single-launch form)

    const char *src = a.x + t * a.row_bytes;
    const int stride = kWave * a.S;
    const int v_first = lane + kWave * sub;
    // With EP_RANKS_INPUTS_FIRST the plan path's inputs (t's ids and, per
    // rank, the mask word of t's 64-token wave) are loaded ahead of the row,
    // whose loads are then unconditional (a vector past the row re-reads the
    // last one and is not stored), so the waits for the inputs do not cover
    // the row.
    const bool plan_path = !FUSED && !a.slots_in;
    const int64_t tile = plan_path ? t / a.TT : 0;
    const int pos = (int)(t - tile * a.TT);
    const int wt = pos >> 6, bit = pos & 63;
    int64_t eid_in = -1;
    uint64_t mw_in = 0;
    if (EP_RANKS_INPUTS_FIRST && plan_path) {
        if (lane < a.k) eid_in = a.topk_idx[t * a.k + lane];
        if (lane < a.R) mw_in = a.rank_mask[((size_t)tile * a.R + lane) * a.TW + wt];
    }
    vec16 buf[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int v = v_first + i * stride;
        if (EP_RANKS_INPUTS_FIRST) buf[i] = ld16(src + (int64_t)min(v, a.nvec - 1) * 16);
        else if (v < a.nvec) buf[i] = ld16(src + (int64_t)v * 16);
    }

    // lanes 0..R-1: the token's row on each rank (-1: not reached)
    int32_t slot = -1;
    if (FUSED) {
        slot = counted_rank_slot<(TOK > 0 ? TOK : 1)>(a, t, lane, sub);
        if (lane < a.R) {
            if ((uint64_t)slot >= (uint64_t)a.cap && slot != -1) {   // cannot happen; never write outside
                atomicOr(&a.ctrl[0], kErrBadSlot);
                slot = -1;
            }
            if (sub == 0) a.token_rank_slot[t * a.R + lane] = slot;
        }
    } else if (lane < a.R && a.slots_in) {   // cached: the rows of a previous dispatch's handle
        slot = a.slots_in[t * a.R + lane];
        if ((uint64_t)slot >= (uint64_t)a.cap) slot = -1;
    } else if (!a.slots_in) {
        // t's place among its tile's tokens reaching rank `lane`: the set
        // bits before t's bit in the tile's mask of that rank
        int32_t start = 0, lr = 0;
        bool reached = false;
        int re = -1;   // rank of slot `lane`'s expert by topk_idx (lanes < k)
        if (lane < a.k) {
            const int64_t e = EP_RANKS_INPUTS_FIRST ? eid_in : a.topk_idx[t * a.k + lane];
            if (e >= 0 && e < a.E) re = a.epr_shift >= 0 ? (int)(e >> a.epr_shift) : (int)(e / a.epr);
        }
        if (lane < a.R) {
            const uint64_t *m = a.rank_mask + ((size_t)tile * a.R + lane) * a.TW;
            // every lookup is independent of the others: one memory round trip
            const uint64_t mw = EP_RANKS_INPUTS_FIRST ? mw_in : m[wt];
            if (!SCAN) start = a.plan_rank_offset[lane] + a.tile_prefix[tile * a.cols + a.E + lane];
            lr = (int32_t)__popcll(mw & ((1ull << bit) - 1ull));
            for (int i = 0; i < wt; ++i) lr += (int32_t)__popcll(m[i]);
            reached = (mw >> bit) & 1u;
        }
        // The plan's rank set for t must be the one topk_idx gives now; a
        // plan reused with other ids gets no rows for t, and the call raises
        // kErrStalePlan.
        uint64_t planned = __ballot(reached), now = 0;
        for (int j = 0; j < a.k; ++j) {
            const int rj = readlane(re, j);
            if (rj >= 0) now |= 1ull << rj;
        }
        if (now != planned) {   // wave-uniform
            if (lane == 0) atomicOr(&a.ctrl[0], kErrStalePlan);
            reached = false;
            planned = 0;
        }
        if (SCAN) start = rank_bases(a, planned, (int)tile, lane);
        if (lane < a.R) {
            if (reached) {
                slot = start + lr;
                if ((uint64_t)slot >= (uint64_t)a.cap) {   // cannot happen; never write outside
                    atomicOr(&a.ctrl[0], kErrBadSlot);
                    slot = -1;
                }
            }
            if (sub == 0) a.token_rank_slot[t * a.R + lane] = slot;
        }
    }
    const uint64_t live = __ballot(slot >= 0);
    if (live == 0) return;

    if (sub == 0 && !a.slots_in) {   // source index and the token's top-k list as each rank sees it
        int e = -1;
        float w = 0.0f;
        if (lane < a.k) {
            const int64_t v = a.topk_idx[t * a.k + lane];
            e = (v >= 0 && v < a.E) ? (int)v : -1;
            w = a.topk_w[t * a.k + lane];
        }
        const int re = e < 0 ? -1 : (a.epr_shift >= 0 ? e >> a.epr_shift : e / a.epr);
        for (uint64_t m = live; m; m &= m - 1) {
            const int r = __builtin_ctzll(m);
            const int64_t s = readlane(slot, r);
            if (lane == 0) a.recv_src_idx[s] = (int32_t)t;
            if (lane < a.k) {
                const bool on = (re == r);
                a.recv_topk_idx[s * a.k + lane] = on ? e - r * a.epr : -1;
                a.recv_topk_w[s * a.k + lane] = on ? w : 0.0f;
            }
        }
    }

    if (a.G > 0) {   // fp32 scale rows of an fp8 payload
        for (int gi = v_first; gi < a.G; gi += stride) {
            const float sc = a.x_scales[t * a.G + gi];
            for (uint64_t m = live; m; m &= m - 1) {
                const int64_t s = readlane(slot, __builtin_ctzll(m));
                a.recv_scales[s * a.G + gi] = sc;
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
        for (uint64_t m = live; m; m &= m - 1) {
            const int64_t s = readlane(slot, __builtin_ctzll(m));
            char *dst = a.recv_x + s * a.row_bytes;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int v = v0 + i * stride;
                if (v < a.nvec) {
                    if (EP_RANKS_NT_STORE) st16_nt(dst + (int64_t)v * 16, buf[i]);
                    else st16(dst + (int64_t)v * 16, buf[i]);
                }
            }
        }
    }
}

struct ReduceArgs {
    const char *recv;               // [cap][row_bytes]: bf16, or e4m3
    const float *recv_scales;       // [cap][H/128] (e4m3 rows) or null
    const int32_t *rank_offset;     // [R + 1]
    const int32_t *recv_topk_idx;   // [cap][k] local expert ids, -1 elsewhere
    const float *recv_topk_w;       // [cap][k]
    const float *factor;            // [E] or null (identity expert)
    uint16_t *partial;              // [cap][H] bf16
    int64_t cap;
    int k, R, H, epr;
    int fp8;
    int nvec;                       // 16-byte vectors per received row
    int S;
};

// value of one received element after the expert: bf16_rne(v * factor)
__device__ __forceinline__ float expert_value(float v, float f, bool scaled) {
    if (scaled) v = v * f;
    return u2f(f32_to_bf16(v) << 16);
}

__global__ __launch_bounds__(256) void ep_expert_reduce_ranks_kernel(ReduceArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int64_t s = gw / a.S;
    const int sub = (int)(gw - s * a.S);
    if (s >= a.cap) return;
    if (s >= a.rank_offset[a.R]) return;   // past the last region (uniform)
    // the row's rank: the last r with rank_offset[r] <= s (empty regions
    // before it share its start, those after it start past s)
    const int32_t ro = lane < a.R ? a.rank_offset[lane] : 0x7FFFFFFF;
    const int r = (int)__popcll(__ballot(lane < a.R && ro <= s)) - 1;
    if (r < 0) return;   // rank_offset[0] > s: not a plan's offsets (uniform)

    int le_id = -1;
    float wt = 0.0f, fac = 1.0f;
    if (lane < a.k) {
        le_id = a.recv_topk_idx[s * a.k + lane];
        if (le_id >= a.epr) le_id = -1;   // not a local expert id: skipped
        wt = a.recv_topk_w[s * a.k + lane];
        if (le_id >= 0 && a.factor) fac = a.factor[r * a.epr + le_id];
    }
    const bool scaled = a.factor != nullptr;
    const uint64_t on = __ballot(lane < a.k && le_id >= 0);
    const char *row = a.recv + s * (int64_t)a.nvec * 16;
    uint16_t *out = a.partial + s * (int64_t)a.H;
    for (int v = lane + kWave * sub; v < a.nvec; v += kWave * a.S) {
        const vec16 in = ld16(row + (int64_t)v * 16);
        if (!a.fp8) {   // 8 bf16 elements
            float x[8], acc[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x[2 * q] = bf16_lo(in[q]);
                x[2 * q + 1] = bf16_hi(in[q]);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = -0.0f;
            for (uint64_t m = on; m; m &= m - 1) {
                const int j = __builtin_ctzll(m);
                const float w = readlane(wt, j), f = readlane(fac, j);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(w, expert_value(x[i], f, scaled), acc[i]);
            }
            vec16 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
            st16(out + (int64_t)v * 8, o);
        } else {        // 16 e4m3 elements, one fp32 scale per 128
            const float sc = a.recv_scales[s * (a.H / 128) + v / 8];
            float x[16], acc[16];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int b = 0; b < 4; ++b) x[4 * q + b] = e4m3_to_f32((in[q] >> (8 * b)) & 0xFFu) * sc;
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = -0.0f;
            for (uint64_t m = on; m; m &= m - 1) {
                const int j = __builtin_ctzll(m);
                const float w = readlane(wt, j), f = readlane(fac, j);
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] = __builtin_fmaf(w, expert_value(x[i], f, scaled), acc[i]);
            }
            vec16 o0, o1;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                o0[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
                o1[q] = pack_bf16x2(acc[8 + 2 * q], acc[8 + 2 * q + 1]);
            }
            st16(out + (int64_t)v * 16, o0);
            st16(out + (int64_t)v * 16 + 8, o1);
        }
    }
}

struct RankCombineArgs {
    const char *partial;            // [cap][2H]
    const int32_t *token_rank_slot; // [T][R]
    char *y;                        // [T][2H]
    int64_t T, cap;
    int R, nvec, S;
};

constexpr int kRankBatch = 8;   // partial rows whose loads are issued together

template <int C>
__global__ __launch_bounds__(256) void ep_combine_ranks_kernel(RankCombineArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int64_t t = gw / a.S;
    const int sub = (int)(gw - t * a.S);
    if (t >= a.T) return;
    int32_t slot = -1;
    if (lane < a.R) {
        slot = a.token_rank_slot[t * a.R + lane];
        if ((uint64_t)slot >= (uint64_t)a.cap) slot = -1;   // outside the receive rows: not reached
    }
    const uint64_t live = __ballot(slot >= 0);
    char *yrow = a.y + t * (int64_t)a.nvec * 16;
    const int stride = kWave * a.S;

    for (int v0 = lane + kWave * sub; v0 < a.nvec; v0 += stride * C) {
        float acc[C][8];
#pragma unroll
        for (int i = 0; i < C; ++i)
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[i][q] = -0.0f;
        for (uint64_t m = live; m;) {
            // the next (up to) kRankBatch ranks, ascending
            int64_t rows[kRankBatch];
            int nb = 0;
#pragma unroll
            for (int jj = 0; jj < kRankBatch; ++jj) {
                rows[jj] = 0;
                if (m) {
                    rows[jj] = readlane(slot, __builtin_ctzll(m));
                    m &= m - 1;
                    nb = jj + 1;
                }
            }
            vec16 buf[kRankBatch][C];
#pragma unroll
            for (int jj = 0; jj < kRankBatch; ++jj) {
                if (jj >= nb) break;   // uniform
                const char *row = a.partial + rows[jj] * (int64_t)a.nvec * 16;
#pragma unroll
                for (int i = 0; i < C; ++i) {
                    const int v = v0 + i * stride;
                    if (v < a.nvec) buf[jj][i] = ld16_nt(row + (int64_t)v * 16);
                }
            }
#pragma unroll
            for (int jj = 0; jj < kRankBatch; ++jj) {
                if (jj >= nb) break;
#pragma unroll
                for (int i = 0; i < C; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[i][2 * q] = acc[i][2 * q] + bf16_lo(buf[jj][i][q]);
                        acc[i][2 * q + 1] = acc[i][2 * q + 1] + bf16_hi(buf[jj][i][q]);
                    }
            }
        }
        float flat[8 * C];
#pragma unroll
        for (int i = 0; i < C; ++i)
#pragma unroll
            for (int q = 0; q < 8; ++q) flat[8 * i + q] = acc[i][q];
        uint32_t packed[4 * C];
        pack_bf16(flat, packed);
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int v = v0 + i * stride;
            if (v >= a.nvec) continue;
            vec16 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = live ? packed[4 * i + q] : 0u;
            if (EP_RANKS_Y_NT) st16_nt(yrow + (int64_t)v * 16, o);
            else st16(yrow + (int64_t)v * 16, o);
        }
    }
}

template <int TOK, bool SCAN = false>
void launch_ranks_copy(const RankCopyArgs &a, const SmallLayout &L, const dim3 &grid, const dim3 &block,
                       size_t lds, hipStream_t stream) {
    const int per_lane = (a.nvec + kWave * a.S - 1) / (kWave * a.S);
    if (per_lane <= 2) {
        hipLaunchKernelGGL((ep_dispatch_ranks_kernel<2, TOK, SCAN>), grid, block, lds, stream, a, L);
    } else if (per_lane <= 4) {
        hipLaunchKernelGGL((ep_dispatch_ranks_kernel<4, TOK, SCAN>), grid, block, lds, stream, a, L);
    } else if (per_lane <= 8 || TOK) {   // the single-launch form has at most 8 (fused_ranks_fits)
        hipLaunchKernelGGL((ep_dispatch_ranks_kernel<8, TOK, SCAN>), grid, block, lds, stream, a, L);
    } else {
        hipLaunchKernelGGL((ep_dispatch_ranks_kernel<16, TOK, SCAN>), grid, block, lds, stream, a, L);
    }
}

// Waves per token of the single-launch form: enough for the row copy and at
// least one per rank the token can reach (up to 16).
int fused_rank_waves(const Shape &s, int nvec) {
    int S = waves_per_token(s.T, nvec, EP_RANKS_WAVES);
    const int kr = s.k < s.R ? s.k : s.R;
    const int want = kr < 16 ? kr : 16;
    while (S < want) S *= 2;
    return S > 16 ? 16 : S;
}

}  // namespace

bool fused_ranks_fits(const Shape &s) {
    if (!(s.T > 0 && s.T * s.k <= kRankFusedPairs && s.rank_rows && s.M == 0)) return false;
    const int nvec = (int)((s.x_fmt == 1 ? (int64_t)s.H : 2 * (int64_t)s.H) / 16);
    const int S = fused_rank_waves(s, nvec);
    return (nvec + kWave * S - 1) / (kWave * S) <= 8;   // registers for 1024-thread blocks
}

hipError_t launch_dispatch_ranks_fused(const Shape &s, const void *x, const float *x_scales,
                                       const int64_t *topk_idx, const float *topk_w, int32_t *per_rank,
                                       int32_t *per_expert, uint8_t *in_rank, int32_t *per_node,
                                       int64_t *algo, void *recv_x, float *recv_x_scales,
                                       int32_t *recv_src_idx, int32_t *recv_topk_idx, float *recv_topk_w,
                                       int32_t *token_rank_slot, int32_t *rank_offset, uint32_t *ctrl,
                                       hipStream_t stream) {
    RankCopyArgs a{};
    a.x = static_cast<const char *>(x);
    a.x_scales = x_scales;
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    a.recv_x = static_cast<char *>(recv_x);
    a.recv_scales = recv_x_scales;
    a.recv_src_idx = recv_src_idx;
    a.recv_topk_idx = recv_topk_idx;
    a.recv_topk_w = recv_topk_w;
    a.token_rank_slot = token_rank_slot;
    a.ctrl = ctrl;
    a.T = s.T;
    a.k = s.k;
    a.E = s.E;
    a.R = s.R;
    a.epr = s.E / s.R;
    a.epr_shift = (a.epr & (a.epr - 1)) == 0 ? __builtin_ctz((unsigned)a.epr) : -1;
    a.cap = s.rank_rows_cap();
    const bool fp8 = (s.x_fmt == 1);
    a.row_bytes = fp8 ? (int64_t)s.H : 2 * (int64_t)s.H;
    a.nvec = (int)(a.row_bytes / 16);
    a.G = fp8 ? s.H / 128 : 0;
    a.S = fused_rank_waves(s, a.nvec);
    SmallLayout L{};
    L.topk_idx = topk_idx;
    L.T = s.T;
    L.k = s.k;
    L.E = s.E;
    L.R = s.R;
    L.N = s.N;
    L.epr = a.epr;
    L.epr_shift = a.epr_shift;
    L.epn = s.E / s.N;
    L.epn_shift = (L.epn & (L.epn - 1)) == 0 ? __builtin_ctz((unsigned)L.epn) : -1;
    L.ctrl = ctrl;
    L.per_expert = per_expert;
    L.per_rank = per_rank;
    L.per_node = per_node;
    L.in_rank = in_rank;
    L.algo = algo;
    L.rank_offset = rank_offset;
    int threads = 0;
    const size_t lds = fused_ranks_lds(s, &threads);
    const dim3 grid((unsigned)(1 + s.T)), block(threads);
    if (s.T <= 8 * kWave) launch_ranks_copy<8>(a, L, grid, block, lds, stream);
    else launch_ranks_copy<32>(a, L, grid, block, lds, stream);
    return hipGetLastError();
}

size_t fused_ranks_lds(const Shape &s, int *threads) {
    const int nvec = (int)((s.x_fmt == 1 ? (int64_t)s.H : 2 * (int64_t)s.H) / 16);
    const int t = kWave * fused_rank_waves(s, nvec);
    if (threads) *threads = t;
    // block 0: the layout's staging; the other blocks: one rank mask per token
    const size_t lds_layout = sizeof(int32_t) * ((size_t)s.T * s.k + s.E + s.R + s.N + t / kWave + 1);
    const size_t lds_masks = sizeof(uint64_t) * (size_t)s.T;
    return lds_layout > lds_masks ? lds_layout : lds_masks;
}

namespace {

RankCopyArgs plan_copy_args(const Shape &s, const WsLayout &L, const void *x, const float *x_scales,
                            const int64_t *topk_idx, const float *topk_w, void *recv_x, float *recv_x_scales,
                            int32_t *recv_src_idx, int32_t *recv_topk_idx, float *recv_topk_w,
                            int32_t *token_rank_slot, int32_t *rank_offset, const char *ws) {
    RankCopyArgs a{};
    a.x = static_cast<const char *>(x);
    a.x_scales = x_scales;
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    a.recv_x = static_cast<char *>(recv_x);
    a.recv_scales = recv_x_scales;
    a.recv_src_idx = recv_src_idx;
    a.recv_topk_idx = recv_topk_idx;
    a.recv_topk_w = recv_topk_w;
    a.token_rank_slot = token_rank_slot;
    a.rank_offset = rank_offset;
    a.plan_rank_offset = reinterpret_cast<const int32_t *>(ws + L.plan_rank_offset);
    a.tile_prefix = reinterpret_cast<const int32_t *>(ws + L.tile_count);
    a.rank_mask = reinterpret_cast<const uint64_t *>(ws + L.rank_mask);
    a.TW = L.tile_token_waves;
    a.ctrl = reinterpret_cast<uint32_t *>(const_cast<char *>(ws) + L.ctrl);
    a.T = s.T;
    a.k = s.k;
    a.E = s.E;
    a.R = s.R;
    a.N = s.N;
    a.TT = L.tile_tokens;
    a.cols = s.E + s.R + s.N;
    a.epr = s.E / s.R;
    a.epr_shift = (a.epr & (a.epr - 1)) == 0 ? __builtin_ctz((unsigned)a.epr) : -1;
    a.cap = s.rank_rows_cap();
    const bool fp8 = (s.x_fmt == 1);
    a.row_bytes = fp8 ? (int64_t)s.H : 2 * (int64_t)s.H;
    a.nvec = (int)(a.row_bytes / 16);
    a.G = fp8 ? s.H / 128 : 0;
    a.S = waves_per_token(s.T, a.nvec, EP_RANKS_WAVES);
    return a;
}

}  // namespace

hipError_t launch_dispatch_ranks(const Shape &s, const WsLayout &L, const void *x,
                                 const float *x_scales, const int64_t *topk_idx,
                                 const float *topk_w, void *recv_x, float *recv_x_scales,
                                 int32_t *recv_src_idx, int32_t *recv_topk_idx, float *recv_topk_w,
                                 int32_t *token_rank_slot, int32_t *rank_offset, const char *ws,
                                 hipStream_t stream) {
    const RankCopyArgs a = plan_copy_args(s, L, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales, recv_src_idx,
                                          recv_topk_idx, recv_topk_w, token_rank_slot, rank_offset, ws);
    int64_t blocks = (s.T * a.S + 3) / 4;
    if (blocks * 256 < s.R + 1) blocks = 1;   // threads to copy rank_offset (R <= 64)
    const dim3 grid((unsigned)blocks), block(256);
    launch_ranks_copy<0>(a, SmallLayout{}, grid, block, 0, stream);
    return hipGetLastError();
}

bool ranks_scan_fits(const Shape &s, const WsLayout &L) {
    return s.T > 0 && s.rank_rows && L.tiles > 1 && L.tiles <= kScanCopyMaxTiles;
}

hipError_t launch_dispatch_ranks_scan(const Shape &s, const WsLayout &L, const void *x,
                                      const float *x_scales, const int64_t *topk_idx, const float *topk_w,
                                      void *recv_x, float *recv_x_scales, int32_t *recv_src_idx,
                                      int32_t *recv_topk_idx, float *recv_topk_w, int32_t *token_rank_slot,
                                      int32_t *rank_offset, int32_t *per_rank, int32_t *per_expert,
                                      int32_t *per_node, int64_t *algo, char *ws, hipStream_t stream) {
    RankCopyArgs a = plan_copy_args(s, L, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales, recv_src_idx,
                                    recv_topk_idx, recv_topk_w, token_rank_slot, rank_offset, ws);
    a.rank_pairs = reinterpret_cast<const int2 *>(ws + L.rank_pairs);
    a.ntiles = L.tiles;
    a.per_rank = per_rank;
    a.per_expert = per_expert;
    a.per_node = per_node;
    a.algo = algo;
    // block 0: the totals; then the copy blocks (4 waves each)
    const int64_t blocks = 1 + (s.T * a.S + 3) / 4;
    launch_ranks_copy<0, true>(a, SmallLayout{}, dim3((unsigned)blocks), dim3(256), scan_copy_lds(s), stream);
    return hipGetLastError();
}

hipError_t launch_dispatch_ranks_cached(const Shape &s, const void *x, const float *x_scales,
                                        const int32_t *token_rank_slot, void *recv_x,
                                        float *recv_x_scales, hipStream_t stream) {
    RankCopyArgs a{};
    a.x = static_cast<const char *>(x);
    a.x_scales = x_scales;
    a.recv_x = static_cast<char *>(recv_x);
    a.recv_scales = recv_x_scales;
    a.slots_in = token_rank_slot;
    a.T = s.T;
    a.k = s.k;
    a.E = s.E;
    a.R = s.R;
    a.cap = s.rank_rows_cap();
    const bool fp8 = (s.x_fmt == 1);
    a.row_bytes = fp8 ? (int64_t)s.H : 2 * (int64_t)s.H;
    a.nvec = (int)(a.row_bytes / 16);
    a.G = fp8 ? s.H / 128 : 0;
    a.S = waves_per_token(s.T, a.nvec, EP_RANKS_WAVES);
    const int64_t blocks = (s.T * a.S + 3) / 4;
    if (blocks == 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), block(256);
    launch_ranks_copy<0>(a, SmallLayout{}, grid, block, 0, stream);
    return hipGetLastError();
}

hipError_t launch_expert_reduce_ranks(const Shape &s, const void *recv_x, const float *recv_scales,
                                      const int32_t *rank_offset, const int32_t *recv_topk_idx,
                                      const float *recv_topk_w, const float *factor,
                                      uint16_t *partial, hipStream_t stream) {
    ReduceArgs a{};
    a.recv = static_cast<const char *>(recv_x);
    a.recv_scales = recv_scales;
    a.rank_offset = rank_offset;
    a.recv_topk_idx = recv_topk_idx;
    a.recv_topk_w = recv_topk_w;
    a.factor = factor;
    a.partial = partial;
    a.cap = s.rank_rows_cap();
    a.k = s.k;
    a.R = s.R;
    a.H = s.H;
    a.epr = s.E / s.R;
    a.fp8 = (s.x_fmt == 1);
    a.nvec = a.fp8 ? s.H / 16 : s.H / 8;
    a.S = waves_per_token(a.cap, a.nvec, EP_RANKS_COMBINE_WAVES);
    const int64_t waves = a.cap * a.S;
    hipLaunchKernelGGL(ep_expert_reduce_ranks_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

hipError_t launch_combine_ranks(const Shape &s, const uint16_t *partial,
                                const int32_t *token_rank_slot, void *y, hipStream_t stream) {
    RankCombineArgs a{};
    a.partial = reinterpret_cast<const char *>(partial);
    a.token_rank_slot = token_rank_slot;
    a.y = static_cast<char *>(y);
    a.T = s.T;
    a.cap = s.rank_rows_cap();
    a.R = s.R;
    a.nvec = s.H / 8;
    a.S = waves_per_token(s.T, a.nvec, EP_RANKS_COMBINE_WAVES);
    if (EP_RANKS_COMBINE_ONE_PASS) {   // the smallest power of two with one pass per wave
        a.S = 1;
        while ((int64_t)kWave * EP_RANKS_COMBINE_VECS * a.S < a.nvec && a.S < 64) a.S *= 2;
    }
    const int64_t waves = s.T * a.S;
    if (waves < EP_RANKS_COMBINE_SMALL_WAVES) {
        // a small batch: one wave per 64 vectors of a row, one vector per lane
        a.S = (a.nvec + kWave - 1) / kWave;
        hipLaunchKernelGGL(ep_combine_ranks_kernel<1>, dim3((unsigned)((s.T * a.S + 3) / 4)), dim3(256), 0, stream, a);
    } else {
        hipLaunchKernelGGL(ep_combine_ranks_kernel<EP_RANKS_COMBINE_VECS>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                           stream, a);
    }
    return hipGetLastError();
}

}  // namespace ep
