// plan.hip -- the layout pass and the dispatch plan on gfx950.
//
// What it computes:
//  * layout (MORI-EP Benchmark, "Why DeepEP and Mori RDMA token counts are
//    equivalent", Steps 1-3; the reference script's per-rank counts): per
//    token the set of virtual ranks and of virtual nodes its valid experts
//    live on (rank = e / (E/R), node = e / (E/N)), repeats collapsed; per-rank
//    and per-node token counts, per-expert pair counts, the token-in-rank map
//    and the RDMA algo count (deduplicated (token, node) pairs, local node
//    included);
//  * the dispatch plan (MSCCL++ PR 860, RANK_MAJOR commit: the default layout
//    places tokens at compacted prefix offsets): a stable counting sort of
//    the valid (t, j) pairs by expert -- expert segments back to back in
//    expert order, pairs in row-major (t, j) order inside a segment.
//
// How (two launches; the kernel boundary publishes the first one's results,
// so no cross-block fence or ticket is needed):
//  ep_plan_count_kernel  one block per tile of TT whole tokens.  The tile's
//      topk_idx is staged in LDS once.
//      - pairs (lane = pair): bit `lane` of an LDS 64-bit mask per (wave,
//        expert) is set with an atomic OR (order-independent); a pair's rank
//        among the tile's earlier pairs of the same expert is the popcount of
//        that expert's masks of earlier waves plus its own wave's mask below
//        the lane.  Per-tile expert counts are popcounts of the masks.
//      - tokens (lane = token): the token's ranks and nodes are OR-ed into two
//        64-bit masks in registers (a repeated rank / node is a no-op), the
//        token-in-rank row is written from the rank mask, and per-rank /
//        per-node counts are LDS integer adds, one per rank / node a token
//        reaches (order-independent; a wavefront ballot per rank cost
//        2.4 us more at 16 ranks).
//      - (token, rank) rows, when planned: per (rank, 64-token wave) the
//        ballot of the wave's tokens reaching the rank, written as one 64-bit
//        word; the dispatch takes a token's place among the tile's tokens of
//        a rank as the popcount of the bits before it.
//  ep_plan_scan_kernel   one block: per expert (and per rank, when (token,
//      rank) rows are planned) the exclusive prefix of the tile counts over
//      tiles (in place) and the total; the exclusive scan of the expert totals
//      (segment starts) and of the rank totals (region starts); per rank /
//      node the sum over tiles.  Integer sums only: the plan and the counts
//      are deterministic.
//  A batch that fits one tile (T * k <= 1024 pairs at E <= 384) is planned by
//  the count kernel alone: its block holds every count and scans them in LDS.
//  For layout + dispatch in one call (count_only), the scan launch is left
//  out: each count block also writes, per expert, its tile's count and the
//  tile's pairs of smaller experts, and the dispatch rebuilds every segment
//  start and prefix over tiles it needs from those (one sum over tiles per
//  slot; dispatch.hip).
#include "ep_device.h"
#include "ep_internal.h"

#ifndef EP_PLAN_ROTATE
#define EP_PLAN_ROTATE 1   // 1: the count kernel's expert pass starts on the upper half of the block
#endif

namespace ep {
namespace {

struct CountArgs {
    const int64_t *topk_idx;
    int64_t T;
    int k, E, R, N, epr, epn;
    int epr_shift, epn_shift; // log2 of epr / epn when powers of two, else -1
    int TT;                   // tokens per tile
    int W;                    // waves whose masks exist (pairs per tile / 64, rounded up)
    uint8_t *in_rank;         // [T][R] or null
    int32_t *tile_count;      // [ntiles][E + R + N]: experts, ranks, nodes
    int32_t *local_rank;      // [T * k]
    uint32_t *ctrl;
    uint64_t *rank_mask;      // [ntiles][R][TW]: bit i of word w = token w * 64 + i of the tile
                              // reaches rank r; null unless (token, rank) rows are planned
    int TW;                   // 64-token waves per tile: ceil(TT / 64)
    // single-tile batches (one block) finish the plan in the same launch:
    int32_t *plan_offset;     // [E + 1]
    int32_t *plan_rank_offset;   // [R + 1] (token, rank) region starts
    int32_t *per_expert, *per_rank, *per_node;   // layout outputs or null
    int64_t *algo;
    // multi-tile batches, for a dispatch that rebuilds segment starts itself
    // (or null): per expert e and tile u, {pairs of u whose expert is below
    // e, pairs of u with expert e} ([E][ntiles], the tiles of one expert
    // side by side)
    int2 *tile_pairs;
    // the same for (token, rank) rows: per rank r and tile u, {tokens of u
    // reaching ranks below r (counted once per rank), tokens of u reaching r}
    // ([R][ntiles]); or null
    int2 *rank_pairs;
};

__global__ __launch_bounds__(1024) void ep_plan_count_kernel(CountArgs a) {
    extern __shared__ uint64_t lds[];
    uint64_t *masks = lds;                                            // [W][E]
    int32_t *ids = reinterpret_cast<int32_t *>(masks + (size_t)a.W * a.E);   // [TT * k]
    int32_t *rn = ids + a.TT * a.k;                                   // [R + N]
    const int tid = threadIdx.x, nt = blockDim.x;
    const int lane = tid & (kWave - 1), w = tid / kWave;
    const int E = a.E, k = a.k;
    const int64_t t0 = (int64_t)blockIdx.x * a.TT;
    const int ntok = (int)min<int64_t>(a.TT, a.T - t0);
    const int npairs = ntok * k;

    // Each wave clears its own mask row and sets its own pairs' bits in it,
    // so only the barrier after the bits are set is needed (a wave's LDS
    // operations are waited for before its atomics).  One pair per thread:
    // the host sizes a tile to at most blockDim pairs.
    int64_t v = -1;
    if (tid < npairs) v = a.topk_idx[t0 * k + tid];   // in flight while the LDS is cleared
    for (int i = lane; i < E; i += kWave) masks[w * E + i] = 0ull;
    for (int i = tid; i < a.R + a.N; i += nt) rn[i] = 0;
    const bool bad = v >= E;
    const int e = (v >= 0 && v < E) ? (int32_t)v : -1;   // invalid ids become masked
    if (tid < npairs) ids[tid] = e;
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's row is cleared
    // ---- pairs: ranks inside the tile
    if (e >= 0) atomicOr((unsigned long long *)&masks[w * E + e], 1ull << lane);
    __syncthreads();
    if (tid < npairs) {
        int32_t r = -1;
        if (e >= 0) {
            r = (int32_t)__popcll(masks[w * E + e] & lanemask_lt());
            // earlier waves' masks, four loads in flight at a time (the
            // index is clamped so every load of a batch is issued)
            for (int w0 = 0; w0 < w; w0 += 4) {
                uint64_t m[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) m[q] = masks[min(w0 + q, w - 1) * E + e];
#pragma unroll
                for (int q = 0; q < 4; ++q) r += (w0 + q < w) ? (int32_t)__popcll(m[q]) : 0;
            }
        }
        a.local_rank[t0 * k + tid] = r >= 0 ? (e << kPlanLrBits) | r : -1;   // the plan word
    }
    int32_t *tc = a.tile_count + (size_t)blockIdx.x * (E + a.R + a.N);
    const bool single = gridDim.x == 1;   // the whole batch is this tile
    int32_t *cnt = rn + a.R + a.N;        // [E] tile counts (single-tile finish)
    // experts from the upper half of the block first: the token pass below
    // runs on the lowest waves, so the two proceed side by side
    const int rot = EP_PLAN_ROTATE * (nt / kWave / 2) * kWave;   // whole waves: a wave's experts stay consecutive
    // Tile pairs without a block scan when E <= blockDim: a thread then holds
    // at most one expert and a wave 64 consecutive ones, so a wave prefix
    // sum in registers plus the totals of the waves before it give each
    // expert's pairs below it.
    const bool wave_pairs = a.tile_pairs && !single && E <= nt;
    const int e_wave = (w * kWave + rot) % nt;   // expert of lane 0 of this wave in the pass below
    int32_t my_c = 0;
    for (int e2 = (tid + rot) % nt; e2 < E; e2 += nt) {
        int32_t c = 0;
        for (int w0 = 0; w0 < a.W; w0 += 4) {
            uint64_t m[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) m[q] = masks[min(w0 + q, a.W - 1) * E + e2];
#pragma unroll
            for (int q = 0; q < 4; ++q) c += (w0 + q < a.W) ? (int32_t)__popcll(m[q]) : 0;
        }
        tc[e2] = single ? 0 : c;          // single tile: no earlier tiles, prefix 0
        if (single || (a.tile_pairs && !wave_pairs)) cnt[e2] = c;
        if (single && a.per_expert) a.per_expert[e2] = c;
        my_c = c;
    }
    int32_t my_below = 0;                 // this expert's pairs below it within the wave
    int32_t *wave_tot = cnt + E + 1;      // [blockDim / 64] pair totals of the expert waves
    if (wave_pairs && e_wave < E) {       // wave-uniform
        int32_t incl = my_c;              // 0 on lanes past E
        for (int off = 1; off < kWave; off <<= 1) {
            const int32_t u = __shfl_up(incl, off);
            if (lane >= off) incl += u;
        }
        my_below = incl - my_c;
        if (lane == kWave - 1) wave_tot[e_wave / kWave] = incl;
    }

    // ---- tokens: rank / node sets in registers, one token per thread (the
    // host sizes a tile to at most blockDim tokens)
    const bool has_tok = tid < ntok;
    uint64_t rmask = 0, nmask = 0;
    if (has_tok) {
        // the token's ids, four LDS loads in flight at a time (clamped index)
        for (int j0 = 0; j0 < k; j0 += 4) {
            int ej[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) ej[q] = ids[tid * k + min(j0 + q, k - 1)];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (j0 + q >= k || ej[q] < 0) continue;
                const int r = a.epr_shift >= 0 ? ej[q] >> a.epr_shift : ej[q] / a.epr;
                const int n = a.epn_shift >= 0 ? ej[q] >> a.epn_shift : ej[q] / a.epn;
                rmask |= 1ull << r;
                nmask |= 1ull << n;
            }
        }
        if (a.in_rank) {
            uint8_t *out = a.in_rank + (t0 + tid) * a.R;
            if ((a.R & 15) == 0) {
                for (int r0 = 0; r0 < a.R; r0 += 16) {
                    vec16 v;
                    for (int q = 0; q < 4; ++q) {
                        uint32_t wd = 0;
                        for (int b = 0; b < 4; ++b)
                            wd |= (uint32_t)((rmask >> (r0 + 4 * q + b)) & 1u) << (8 * b);
                        v[q] = wd;
                    }
                    st16(out + r0, v);
                }
            } else if ((a.R & 3) == 0) {
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
    const bool tok_wave = w * kWave < ntok;   // the wave holds a token (wave-uniform)
    if (a.rank_mask && tok_wave) {
        // (token, rank) rows: per rank, the wave's tokens reaching it as one
        // ballot; lane r keeps rank r's and writes it (R <= 64)
        uint64_t mine = 0;
        for (int r = 0; r < a.R; ++r) {
            const uint64_t b = __ballot((rmask >> r) & 1u);
            if (lane == r) mine = b;
        }
        if (lane < a.R) a.rank_mask[((size_t)blockIdx.x * a.R + lane) * a.TW + w] = mine;
    }
    // one LDS add per rank / node the token reaches (integer adds: the counts
    // do not depend on their order)
    for (uint64_t m = rmask; m; m &= m - 1) atomicAdd(&rn[__builtin_ctzll(m)], 1);
    for (uint64_t m = nmask; m; m &= m - 1) atomicAdd(&rn[a.R + __builtin_ctzll(m)], 1);
    if (__ballot(bad) && lane == 0) atomicOr(&a.ctrl[0], kErrBadExpert);
    __syncthreads();
    // single tile: the rank columns hold the prefix over earlier tiles (0)
    // when (token, rank) rows are planned, else the counts
    for (int i = tid; i < a.R + a.N; i += nt) tc[E + i] = (single && a.rank_mask && i < a.R) ? 0 : rn[i];
    if (!single) {   // block-uniform
        if (a.rank_pairs && tid < kWave) {   // wave 0: the tile's tokens per rank, prefixed over the ranks
            const int32_t c = tid < a.R ? rn[tid] : 0;
            int32_t incl = c;
            for (int off = 1; off < kWave; off <<= 1) {
                const int32_t u = __shfl_up(incl, off);
                if (lane >= off) incl += u;
            }
            if (tid < a.R) a.rank_pairs[(size_t)tid * gridDim.x + blockIdx.x] = make_int2(incl - c, c);
        }
        if (wave_pairs) {   // the wave totals were written before the barrier above
            const int e2 = (tid + rot) % nt;
            if (e2 < E) {
                int32_t below = my_below;
                for (int j = 0; j < e2 / kWave; ++j) below += wave_tot[j];
                a.tile_pairs[(size_t)e2 * gridDim.x + blockIdx.x] = make_int2(below, my_c);
            }
        } else if (a.tile_pairs) {   // this tile's counts, prefixed over the experts (in place)
            block_exclusive_scan(cnt, cnt, E, reinterpret_cast<int32_t *>(cnt + E + 1));
            for (int e2 = tid; e2 < E; e2 += nt)
                a.tile_pairs[(size_t)e2 * gridDim.x + blockIdx.x] = make_int2(cnt[e2], cnt[e2 + 1] - cnt[e2]);
        }
        return;
    }

    // ---- single-tile batch: segment starts and layout outputs right here
    block_exclusive_scan(cnt, a.plan_offset, E, reinterpret_cast<int32_t *>(cnt + E));
    if (a.rank_mask && tid < kWave) wave_exclusive_scan(tid < a.R ? rn[tid] : 0, a.R, a.plan_rank_offset);
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
}

struct ScanArgs {
    int E, R, N, ntiles;
    int32_t *tile_count;      // [ntiles][E + R + N]; expert columns -> exclusive prefix over tiles
    int32_t *plan_offset;     // [E + 1] segment starts (workspace copy)
    int32_t *plan_rank_offset;   // [R + 1] (token, rank) region starts, or null
    int32_t *per_expert;      // [E] or null
    int32_t *per_rank;        // [R] or null
    int32_t *per_node;        // [N] or null
    int64_t *algo;            // [1] or null
};

constexpr int kScanMaxCols = 4096 + 128;
constexpr int kScanRegs = 32;   // tiles a thread keeps in registers

__global__ __launch_bounds__(1024) void ep_plan_scan_kernel(ScanArgs a) {
    __shared__ int32_t part[kScanMaxCols + 1];
    __shared__ int32_t tmp[1024 / kWave + 1];
    const int tid = threadIdx.x, nt = blockDim.x, E = a.E;
    const int cols = E + a.R + a.N;
    // Q threads share one column's tiles (columns < blockDim); each owns `chunk` tiles
    const int Q = (nt >= cols) ? nt / cols : 1;
    const int chunk = (a.ntiles + Q - 1) / Q;
    // block-uniform choice: every thread owns at most one (column, part) and
    // at most kScanRegs tiles -> one batch of loads kept in registers
    const bool in_regs = (cols * Q <= nt) && (chunk <= kScanRegs);
    // columns that need prefixes over tiles: experts, and ranks when (token,
    // rank) rows are planned
    const int pcols = E + (a.plan_rank_offset ? a.R : 0);
    if (in_regs) {
        const bool live = tid < cols * Q;
        const int c = tid % cols, q = tid / cols;
        const int ta = min(q * chunk, a.ntiles), tb = min(ta + chunk, a.ntiles);
        int32_t *col = a.tile_count + c;
        int32_t v[kScanRegs];
        int32_t s = 0;
        // Batches of 8 loads, each load unconditional (the tile index is
        // clamped to the thread's last tile, or tile 0 for an empty range;
        // the value is dropped outside the range), so a batch is in flight
        // together.  In this form tiles * cols <= kScanRegs * blockDim.x, so
        // 32-bit byte offsets from the kernel argument address the counts.
        const int lastt = max(tb - 1, 0);
        const char *base = reinterpret_cast<const char *>(a.tile_count);
#pragma unroll
        for (int u0 = 0; u0 < kScanRegs; u0 += 8) {
            if (ta + u0 < tb) {
#pragma unroll
                for (int u = u0; u < u0 + 8; ++u) {
                    const uint32_t off = ((uint32_t)min(ta + u, lastt) * (uint32_t)cols + (uint32_t)c) * 4u;
                    v[u] = *reinterpret_cast<const int32_t *>(base + off);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kScanRegs; ++u) {
            v[u] = (live && ta + u < tb) ? v[u] : 0;
            s += v[u];
        }
        if (live) part[tid] = s;   // tid = q * cols + c
        __syncthreads();
        if (live && c < pcols) {
            int32_t run = 0;
            for (int q2 = 0; q2 < q; ++q2) run += part[q2 * cols + c];
#pragma unroll
            for (int u = 0; u < kScanRegs; ++u) {
                if (ta + u < tb) col[(size_t)(ta + u) * cols] = run;
                run += v[u];
            }
        }
    } else {
        // the same sums in batches of kScanRegs tiles; every load of a batch
        // is unconditional (clamped index, value dropped past the range) so
        // the batch is in flight together
        for (int idx = tid; idx < cols * Q; idx += nt) {
            const int c = idx % cols, q = idx / cols;
            const int ta = min(q * chunk, a.ntiles), tb = min(ta + chunk, a.ntiles);
            const int32_t *col = a.tile_count + c;
            int32_t s = 0;
            for (int t0 = ta; t0 < tb; t0 += kScanRegs) {
                int32_t v[kScanRegs];
#pragma unroll
                for (int u = 0; u < kScanRegs; ++u) v[u] = col[(size_t)min(t0 + u, tb - 1) * cols];
#pragma unroll
                for (int u = 0; u < kScanRegs; ++u) s += (t0 + u < tb) ? v[u] : 0;
            }
            part[idx] = s;
        }
        __syncthreads();
        for (int idx = tid; idx < cols * Q; idx += nt) {
            const int c = idx % cols, q = idx / cols;
            if (c >= pcols) continue;
            const int ta = min(q * chunk, a.ntiles), tb = min(ta + chunk, a.ntiles);
            int32_t *col = a.tile_count + c;
            int32_t run = 0;
            for (int q2 = 0; q2 < q; ++q2) run += part[q2 * cols + c];
            for (int t0 = ta; t0 < tb; t0 += kScanRegs) {
                int32_t v[kScanRegs];
#pragma unroll
                for (int u = 0; u < kScanRegs; ++u) v[u] = col[(size_t)min(t0 + u, tb - 1) * cols];
#pragma unroll
                for (int u = 0; u < kScanRegs; ++u) {
                    if (t0 + u < tb) {
                        col[(size_t)(t0 + u) * cols] = run;
                        run += v[u];
                    }
                }
            }
        }
    }
    __syncthreads();
    // column totals into part[0..cols) (row q = 0), summing the Q partials
    for (int c = tid; c < cols; c += nt) {
        int32_t s = 0;
        for (int q = 0; q < Q; ++q) s += part[q * cols + c];
        part[c] = s;   // column c is read and written by this thread only
        if (c < E) {
            if (a.per_expert) a.per_expert[c] = s;
        } else if (a.per_rank) {
            if (c < E + a.R) a.per_rank[c - E] = s; else a.per_node[c - E - a.R] = s;
        }
    }
    __syncthreads();
    if (a.algo && tid == 0) {
        int64_t al = 0;
        for (int n = 0; n < a.N; ++n) al += part[E + a.R + n];
        *a.algo = al;
    }
    if (a.plan_rank_offset && tid < kWave) wave_exclusive_scan(tid < a.R ? part[E + tid] : 0, a.R, a.plan_rank_offset);
    block_exclusive_scan(part, a.plan_offset, E, tmp);
}

}  // namespace

size_t plan_count_lds(const Shape &s, const WsLayout &L) {
    // pair masks [waves][E], staged ids, rank / node counts, expert counts
    // and block-scan scratch (one slot more than the scan's 1024 / 64 + 1)
    return sizeof(uint64_t) * (size_t)L.tile_waves * s.E +
           sizeof(int32_t) * ((size_t)L.tile_tokens * s.k + s.R + s.N + s.E + 1 + 1024 / kWave + 2);
}

hipError_t launch_plan(const Shape &s, const WsLayout &L, const int64_t *topk_idx,
                       int32_t *per_rank, int32_t *per_expert, uint8_t *in_rank,
                       int32_t *per_node, int64_t *algo, char *ws, hipStream_t stream, bool count_only) {
    CountArgs c{};
    c.topk_idx = topk_idx;
    c.T = s.T;
    c.k = s.k;
    c.E = s.E;
    c.R = s.R;
    c.N = s.N;
    c.epr = s.E / s.R;
    c.epn = s.E / s.N;
    c.epr_shift = (c.epr & (c.epr - 1)) == 0 ? __builtin_ctz((unsigned)c.epr) : -1;
    c.epn_shift = (c.epn & (c.epn - 1)) == 0 ? __builtin_ctz((unsigned)c.epn) : -1;
    c.TT = L.tile_tokens;
    c.W = L.tile_waves;
    c.in_rank = in_rank;
    c.tile_count = reinterpret_cast<int32_t *>(ws + L.tile_count);
    c.local_rank = reinterpret_cast<int32_t *>(ws + L.local_rank);
    c.ctrl = reinterpret_cast<uint32_t *>(ws + L.ctrl);
    c.plan_offset = reinterpret_cast<int32_t *>(ws + L.plan_offset);
    c.rank_mask = s.rank_rows ? reinterpret_cast<uint64_t *>(ws + L.rank_mask) : nullptr;
    c.TW = L.tile_token_waves;
    c.plan_rank_offset = reinterpret_cast<int32_t *>(ws + L.plan_rank_offset);
    c.per_expert = per_expert;
    c.per_rank = per_rank;
    c.per_node = per_node;
    c.algo = algo;
    c.tile_pairs = (count_only && !s.rank_rows) ? reinterpret_cast<int2 *>(ws + L.tile_pairs) : nullptr;
    c.rank_pairs = (count_only && s.rank_rows) ? reinterpret_cast<int2 *>(ws + L.rank_pairs) : nullptr;
    if (s.T > 0) {
        hipLaunchKernelGGL(ep_plan_count_kernel, dim3(L.tiles), dim3(L.count_threads), plan_count_lds(s, L), stream,
                           c);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess || L.tiles == 1 || count_only) return e;   // one tile: the plan is complete
    }
    ScanArgs a{};
    a.E = s.E;
    a.R = s.R;
    a.N = s.N;
    a.ntiles = s.T > 0 ? L.tiles : 0;
    a.tile_count = c.tile_count;
    a.plan_offset = reinterpret_cast<int32_t *>(ws + L.plan_offset);
    a.plan_rank_offset = s.rank_rows ? reinterpret_cast<int32_t *>(ws + L.plan_rank_offset) : nullptr;
    a.per_expert = per_expert;
    a.per_rank = per_rank;
    a.per_node = per_node;
    a.algo = algo;
    hipLaunchKernelGGL(ep_plan_scan_kernel, dim3(1), dim3(1024), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ep
