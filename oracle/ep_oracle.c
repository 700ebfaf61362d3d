/*
 * ep_oracle.c -- plain CPU oracle for MoE expert-parallel dispatch / combine.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load this library.  It shares no
 * code with the HIP library.  Every function is a direct, unblocked statement
 * of what the pages define (see ep_oracle.h for the page list); where the
 * pages leave a step open, the reading taken is named in the comment.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no -ffast-math), so every
 * float operation below is one IEEE-754 binary32 operation in program order
 * and fmaf() is the correctly rounded fused multiply-add of the C library.
 */
#include "ep_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ======================================================================== */
/* Layout                                                                    */
/* ======================================================================== */

/*
 * Expert -> rank is integer division by experts-per-rank ([MORI] Reference
 * script, rank-layout block); expert -> node is integer division by
 * experts-per-node ([MORI] "Why ... equivalent", Step 1).  Each token's rank
 * set and node set are plain sets, so repeated ranks / nodes collapse
 * (Step 2); the RDMA algo count is the number of (token, node) pairs, local
 * node included ([MORI] "RDMA bandwidth", "Algo BW vs Physical BW", Step 3).
 * num_tokens_per_rank[r] counts tokens whose rank set holds r (the script's
 * per-rank count after deduplication).
 */
int64_t oracle_layout(int64_t T, int32_t k, int32_t E, int32_t R, int32_t N,
                      const int64_t *topk_idx, int32_t *num_tokens_per_rank,
                      int32_t *num_tokens_per_expert, uint8_t *is_token_in_rank,
                      int32_t *num_tokens_per_node, int64_t *rdma_algo_token_count)
{
    const int32_t experts_per_rank = E / R;
    const int32_t experts_per_node = E / N;
    int64_t invalid = 0;
    uint8_t *rank_hit = (uint8_t *)calloc((size_t)R, 1);
    uint8_t *node_hit = (uint8_t *)calloc((size_t)N, 1);

    for (int32_t r = 0; r < R; ++r) num_tokens_per_rank[r] = 0;
    for (int32_t n = 0; n < N; ++n) num_tokens_per_node[n] = 0;
    for (int32_t e = 0; e < E; ++e) num_tokens_per_expert[e] = 0;

    for (int64_t t = 0; t < T; ++t) {
        memset(rank_hit, 0, (size_t)R);
        memset(node_hit, 0, (size_t)N);
        for (int32_t j = 0; j < k; ++j) {
            int64_t e = topk_idx[t * k + j];
            if (e < 0) continue;                 /* masked slot */
            if (e >= E) { ++invalid; continue; } /* invalid id: treated as masked */
            num_tokens_per_expert[e] += 1;
            rank_hit[e / experts_per_rank] = 1;
            node_hit[e / experts_per_node] = 1;
        }
        for (int32_t r = 0; r < R; ++r) {
            is_token_in_rank[t * R + r] = rank_hit[r];
            num_tokens_per_rank[r] += rank_hit[r];
        }
        for (int32_t n = 0; n < N; ++n) num_tokens_per_node[n] += node_hit[n];
    }

    int64_t algo = 0;
    for (int32_t n = 0; n < N; ++n) algo += num_tokens_per_node[n];
    *rdma_algo_token_count = algo;
    free(rank_hit);
    free(node_hit);
    return invalid;
}

/*
 * The DeepEP-side deduplication ([MORI] Step 2 and the script's unique
 * helper): per row, count how often each id in [0, num_slots) occurs
 * (negative entries go to an overflow bin that is dropped), keep the ids
 * whose count is non-zero in descending id order, write the first
 * min(num_slots, cols) of them and fill the rest of the row with -1.
 */
void oracle_unique_rows(int64_t rows, int32_t cols, int32_t num_slots, int64_t *ids)
{
    int64_t *count = (int64_t *)malloc(sizeof(int64_t) * (size_t)(num_slots + 1));
    int64_t *kept = (int64_t *)malloc(sizeof(int64_t) * (size_t)(num_slots + 1));
    const int32_t valid_len = num_slots < cols ? num_slots : cols;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t *row = ids + r * cols;
        for (int32_t b = 0; b <= num_slots; ++b) count[b] = 0;
        for (int32_t c = 0; c < cols; ++c) {
            int64_t v = row[c] < 0 ? num_slots : row[c];
            count[v] += 1;
        }
        int32_t nkept = 0;
        for (int32_t b = num_slots - 1; b >= 0; --b)
            if (count[b] > 0) kept[nkept++] = b;
        for (int32_t c = 0; c < cols; ++c) row[c] = -1;
        for (int32_t c = 0; c < valid_len && c < nkept; ++c) row[c] = kept[c];
    }
    free(count);
    free(kept);
}

/* [MORI] DeepEP column of the RDMA token-count table: node id per slot by
 * division by experts-per-node, masked slots stay -1, per-row unique, then
 * count the entries that are not -1. */
int64_t oracle_algo_by_unique(int64_t T, int32_t k, int32_t E, int32_t N,
                              const int64_t *topk_idx, int64_t *node_rows)
{
    const int32_t experts_per_node = E / N;
    int64_t *rows = node_rows ? node_rows
                              : (int64_t *)malloc(sizeof(int64_t) * (size_t)(T * k));
    for (int64_t i = 0; i < T * k; ++i) {
        int64_t e = topk_idx[i];
        rows[i] = (e < 0 || e >= E) ? -1 : e / experts_per_node;
    }
    oracle_unique_rows(T, k, N, rows);
    int64_t algo = 0;
    for (int64_t i = 0; i < T * k; ++i) algo += (rows[i] != -1);
    if (!node_rows) free(rows);
    return algo;
}

/* [MORI] Mori column: mark presence[t, node] for every slot (marking twice is
 * a no-op), then count the marks. */
int64_t oracle_algo_by_presence(int64_t T, int32_t k, int32_t E, int32_t N,
                                const int64_t *topk_idx, uint8_t *presence)
{
    const int32_t experts_per_node = E / N;
    uint8_t *p = presence ? presence : (uint8_t *)malloc((size_t)(T * N));
    memset(p, 0, (size_t)(T * N));
    for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
            int64_t e = topk_idx[t * k + j];
            if (e < 0 || e >= E) continue;
            p[t * N + e / experts_per_node] = 1;
        }
    int64_t algo = 0;
    for (int64_t i = 0; i < T * N; ++i) algo += p[i];
    if (!presence) free(p);
    return algo;
}

/* ======================================================================== */
/* Accounting                                                                */
/* ======================================================================== */

/*
 * [MORI] "Algo BW vs Physical BW": physical = algo * (nodes - 1) / nodes;
 * the script's exact physical count drops the pairs whose node is the
 * sender's own node.  "NVL / XGMI bandwidth": tokens times token size;
 * one sender's share of the NVL rows is its (token, rank) pair count.
 * "Combine": same byte counts as dispatch, reversed.  The script's fp8
 * factor is (1 + 4/128) / 2 (one byte per element plus one fp32 scale per
 * 128 elements, relative to two bytes per bf16 element).
 */
void oracle_accounting(int32_t H, int32_t R, int32_t N, int32_t own_node,
                       const int32_t *num_tokens_per_rank, const int32_t *num_tokens_per_node,
                       int64_t rdma_algo_token_count, oracle_accounting_t *out)
{
    int64_t nvl = 0;
    for (int32_t r = 0; r < R; ++r) nvl += num_tokens_per_rank[r];
    out->rdma_algo_tokens = rdma_algo_token_count;
    out->rdma_physical_tokens = (double)rdma_algo_token_count * (double)(N - 1) / (double)N;
    out->rdma_physical_tokens_exact = rdma_algo_token_count - num_tokens_per_node[own_node];
    out->nvl_tokens = nvl;
    out->dispatch_rdma_bytes_bf16 = (double)rdma_algo_token_count * (double)H * 2.0;
    out->dispatch_nvl_bytes_bf16 = (double)nvl * (double)H * 2.0;
    out->combine_rdma_bytes_bf16 = out->dispatch_rdma_bytes_bf16;
    out->combine_nvl_bytes_bf16 = out->dispatch_nvl_bytes_bf16;
    out->fp8_factor = (1.0 + 4.0 / 128.0) / 2.0;
    out->dispatch_rdma_bytes_fp8 = out->dispatch_rdma_bytes_bf16 * out->fp8_factor;
    out->dispatch_nvl_bytes_fp8 = out->dispatch_nvl_bytes_bf16 * out->fp8_factor;
}

/* ======================================================================== */
/* Slots and dispatch                                                        */
/* ======================================================================== */

/*
 * Token-major compacted slots ([PR860] "compacted DeepEP prefix offset"):
 * expert segments are laid out back to back in expert order, a segment's
 * start is the exclusive prefix sum of the per-expert counts, and inside a
 * segment the pairs keep their (t, j) order (a stable counting sort).  A
 * virtual rank's receive region is the union of its experts' segments.
 */
void oracle_slots(int64_t T, int32_t k, int32_t E, const int64_t *topk_idx,
                  const float *topk_w, int32_t *token_slot, int32_t *expert_offset,
                  int32_t *recv_src_idx, float *recv_topk_w)
{
    int32_t *count = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int64_t i = 0; i < T * k; ++i) {
        int64_t e = topk_idx[i];
        if (e >= 0 && e < E) count[e] += 1;
    }
    expert_offset[0] = 0;
    for (int32_t e = 0; e < E; ++e) expert_offset[e + 1] = expert_offset[e] + count[e];
    for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
            int64_t e = topk_idx[t * k + j];
            if (e < 0 || e >= E) { token_slot[t * k + j] = -1; continue; }
            int32_t s = expert_offset[e] + fill[e];
            fill[e] += 1;
            token_slot[t * k + j] = s;
            recv_src_idx[s] = (int32_t)t;
            recv_topk_w[s] = topk_w[t * k + j];
        }
    free(count);
    free(fill);
}

/* RANK_MAJOR: rows grouped by destination rank at fixed offsets r * M; the
 * order inside a rank's block is expert, then (t, j).  Written as a direct
 * walk over each rank's experts and the pairs routed to them. */
int64_t oracle_slots_rank_major(int64_t T, int32_t k, int32_t E, int32_t R, int32_t M,
                                const int64_t *topk_idx, const float *topk_w,
                                int32_t *token_slot, int32_t *recv_src_idx, float *recv_topk_w)
{
    const int32_t experts_per_rank = E / R;
    int64_t dropped = 0;
    for (int64_t i = 0; i < T * k; ++i) token_slot[i] = -1;
    for (int32_t r = 0; r < R; ++r) {
        int64_t filled = 0;
        for (int32_t e = r * experts_per_rank; e < (r + 1) * experts_per_rank; ++e)
            for (int64_t t = 0; t < T; ++t)
                for (int32_t j = 0; j < k; ++j) {
                    if (topk_idx[t * k + j] != e) continue;
                    if (filled >= M) { ++dropped; continue; }
                    const int64_t s = (int64_t)r * M + filled;
                    filled += 1;
                    token_slot[t * k + j] = (int32_t)s;
                    recv_src_idx[s] = (int32_t)t;
                    recv_topk_w[s] = topk_w[t * k + j];
                }
    }
    return dropped;
}

/* (token, rank) rows: a token reaches rank r when any of its valid experts
 * lives there; rank regions in rank order, ascending t inside. */
void oracle_slots_ranks(int64_t T, int32_t k, int32_t E, int32_t R, const int64_t *topk_idx,
                        const float *topk_w, int32_t *token_rank_slot, int32_t *rank_offset,
                        int32_t *recv_src_idx, int32_t *recv_topk_idx, float *recv_topk_w)
{
    const int32_t experts_per_rank = E / R;
    uint8_t *hit = (uint8_t *)calloc((size_t)(T * R > 0 ? T * R : 1), 1);
    for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
            int64_t e = topk_idx[t * k + j];
            if (e < 0 || e >= E) continue;
            hit[t * R + e / experts_per_rank] = 1;
        }
    rank_offset[0] = 0;
    for (int32_t r = 0; r < R; ++r) {
        int32_t n = 0;
        for (int64_t t = 0; t < T; ++t) n += hit[t * R + r];
        rank_offset[r + 1] = rank_offset[r] + n;
    }
    for (int32_t r = 0; r < R; ++r) {
        int32_t fill = 0;
        for (int64_t t = 0; t < T; ++t) {
            if (!hit[t * R + r]) { token_rank_slot[t * R + r] = -1; continue; }
            const int32_t s = rank_offset[r] + fill++;
            token_rank_slot[t * R + r] = s;
            recv_src_idx[s] = (int32_t)t;
            /* the token's top-k list as rank r sees it: local expert ids of
             * the slots on r, -1 (weight 0) for every other slot */
            for (int32_t j = 0; j < k; ++j) {
                int64_t e = topk_idx[t * k + j];
                const int on_r = (e >= 0 && e < E && e / experts_per_rank == r);
                recv_topk_idx[(int64_t)s * k + j] = on_r ? (int32_t)(e - (int64_t)r * experts_per_rank) : -1;
                recv_topk_w[(int64_t)s * k + j] = on_r ? topk_w[t * k + j] : 0.0f;
            }
        }
    }
    free(hit);
}

void oracle_expert_reduce_ranks(int64_t T, int32_t k, int32_t E, int32_t R, int32_t H,
                                const int64_t *topk_idx, const float *topk_w, const float *factor,
                                const int32_t *rank_offset, const int32_t *recv_src_idx,
                                const uint16_t *recv, const uint8_t *recv_q, const float *recv_scales,
                                uint16_t *partial)
{
    (void)T;
    const int32_t experts_per_rank = E / R;
    float *acc = (float *)malloc(sizeof(float) * (size_t)H);
    for (int32_t r = 0; r < R; ++r)
        for (int64_t s = rank_offset[r]; s < rank_offset[r + 1]; ++s) {
            const int64_t t = recv_src_idx[s];
            for (int32_t h = 0; h < H; ++h) acc[h] = -0.0f;
            for (int32_t j = 0; j < k; ++j) {
                int64_t e = topk_idx[t * k + j];
                if (e < 0 || e >= E || e / experts_per_rank != r) continue;
                const float w = topk_w[t * k + j];
                for (int32_t h = 0; h < H; ++h) {
                    /* the expert's output element: the received value (bf16,
                     * or e4m3 times its group's scale), times the expert's
                     * factor, as a bf16 */
                    float v = recv_q ? oracle_e4m3_to_f32(recv_q[s * H + h]) * recv_scales[s * (H / 128) + h / 128]
                                     : oracle_bf16_to_f32(recv[s * H + h]);
                    if (factor) v = v * factor[e];
                    v = oracle_bf16_to_f32(oracle_f32_to_bf16(v));
                    acc[h] = fmaf(w, v, acc[h]);
                }
            }
            for (int32_t h = 0; h < H; ++h) partial[s * H + h] = oracle_f32_to_bf16(acc[h]);
        }
    free(acc);
}

void oracle_combine_ranks(int64_t T, int32_t R, int32_t H, const uint16_t *partial,
                          const int32_t *token_rank_slot, uint16_t *y)
{
    float *acc = (float *)malloc(sizeof(float) * (size_t)H);
    for (int64_t t = 0; t < T; ++t) {
        int32_t nvalid = 0;
        for (int32_t h = 0; h < H; ++h) acc[h] = -0.0f;
        for (int32_t r = 0; r < R; ++r) {
            const int32_t s = token_rank_slot[t * R + r];
            if (s < 0) continue;
            ++nvalid;
            for (int32_t h = 0; h < H; ++h) acc[h] = acc[h] + oracle_bf16_to_f32(partial[(int64_t)s * H + h]);
        }
        for (int32_t h = 0; h < H; ++h)
            y[t * H + h] = nvalid ? oracle_f32_to_bf16(acc[h]) : (uint16_t)0;
    }
    free(acc);
}

/* Dispatch moves bytes only: each valid (t, j) pair receives a copy of row t
 * ([MORI] "NVL / XGMI bandwidth": the received tensor holds token rows). */
void oracle_dispatch_rows(int64_t T, int32_t k, int64_t row_bytes, const void *src,
                          const int32_t *token_slot, void *recv)
{
    const uint8_t *s = (const uint8_t *)src;
    uint8_t *d = (uint8_t *)recv;
    for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
            int32_t slot = token_slot[t * k + j];
            if (slot < 0) continue;
            memcpy(d + (int64_t)slot * row_bytes, s + t * row_bytes, (size_t)row_bytes);
        }
}

/* ======================================================================== */
/* Number formats                                                            */
/* ======================================================================== */

/* bfloat16 is the top half of a binary32; widening is exact. */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* binary32 -> bfloat16, round to nearest, ties to even (adding 0x7FFF plus
 * the lowest kept bit carries exactly when the dropped half is above the
 * midpoint, or at the midpoint with an odd kept part).  NaN -> 0x7FC0. */
uint16_t oracle_f32_to_bf16(float f)
{
    if (isnan(f)) return 0x7FC0;
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/*
 * OCP 8-bit floating point, E4M3 ("fn" variant): 1 sign, 4 exponent bits
 * with bias 7, 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9;
 * S.1111.111 is NaN; there is no infinity; largest finite value 448.
 * Encoding rounds to nearest, ties to even, and saturates finite overflow
 * (and infinities) to +-448.  The value is handled in double, where scaling
 * by powers of two is exact and nearbyint() rounds ties to even.
 */
uint8_t oracle_f32_to_e4m3(float f)
{
    const uint8_t sign = signbit(f) ? 0x80 : 0x00;
    if (isnan(f)) return sign | 0x7F;
    double a = fabs((double)f);
    if (isinf(a)) return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal spacing 2^-9; a result of 8 is the smallest normal 0x08 */
        double m = nearbyint(a * 512.0);
        return sign | (uint8_t)m;
    }
    int e = ilogb(a);                        /* floor(log2 a) */
    double m = nearbyint(ldexp(a, 3 - e));   /* significand * 8, in [8, 16] */
    if (m == 16.0) { m = 8.0; e += 1; }
    int biased = e + 7;
    if (biased > 15 || (biased == 15 && (int)m - 8 == 7)) return sign | 0x7E;
    return sign | (uint8_t)((biased << 3) | ((int)m - 8));
}

float oracle_e4m3_to_f32(uint8_t q)
{
    const int s = q >> 7, ex = (q >> 3) & 0xF, m = q & 7;
    if (ex == 15 && m == 7) return s ? -NAN : NAN;
    double v = (ex == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), ex - 10);
    return (float)(s ? -v : v);
}

/* OCP Microscaling E8M0 scale: 2^(e - 127); 0xFF is NaN. */
float oracle_e8m0_to_f32(uint8_t e)
{
    if (e == 0xFF) return NAN;
    return ldexpf(1.0f, (int)e - 127);
}

/*
 * OCP 4-bit floating point, E2M1: 1 sign, 2 exponent bits with bias 1, 1
 * mantissa bit; exponent field 0 holds the subnormal 0.5 * m; no NaN, no
 * infinity; magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  Encoding rounds to
 * nearest, ties to the even code, and saturates to +-6.
 */
uint8_t oracle_f32_to_e2m1(float f)
{
    const uint8_t sign = signbit(f) ? 0x8 : 0x0;
    if (isnan(f)) return sign | 0x7;   /* no NaN code: saturate */
    double a = fabs((double)f);
    if (a >= 6.0) return sign | 0x7;
    if (a < 1.0) {
        double m = nearbyint(a * 2.0);   /* steps of 0.5; 2 means 1.0 = code 2 */
        return sign | (uint8_t)m;
    }
    int e = ilogb(a);                    /* 0, 1 or 2 */
    double m = nearbyint(ldexp(a, 1 - e));   /* significand * 2, in [2, 4] */
    if (m == 4.0) { m = 2.0; e += 1; }
    if (e + 1 > 3) return sign | 0x7;
    return sign | (uint8_t)(((e + 1) << 1) | ((int)m - 2));
}

float oracle_e2m1_to_f32(uint8_t q)
{
    const int s = (q >> 3) & 1, ex = (q >> 1) & 3, m = q & 1;
    double v = (ex == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, ex - 1);
    return (float)(s ? -v : v);
}

/*
 * fp8 dispatch rows: one e4m3 byte per element and one fp32 scale per 128
 * channels ([MORI] Reference script's fp8 factor).  The pages fix only the
 * format; the rule taken: amax of the group, scale = amax / 448 (IEEE
 * division), 1 for an all-zero group, element = e4m3(x / scale).
 */
void oracle_quant_fp8_s128(int64_t rows, int32_t H, const uint16_t *x_bf16, uint8_t *q,
                           float *scales)
{
    const int32_t groups = H / 128;
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t g = 0; g < groups; ++g) {
            const uint16_t *xs = x_bf16 + r * H + g * 128;
            float amax = 0.0f;
            for (int32_t i = 0; i < 128; ++i) {
                float a = fabsf(oracle_bf16_to_f32(xs[i]));
                if (a > amax) amax = a;
            }
            float scale = (amax == 0.0f) ? 1.0f : amax / 448.0f;
            scales[r * groups + g] = scale;
            for (int32_t i = 0; i < 128; ++i)
                q[r * H + g * 128 + i] = oracle_f32_to_e4m3(oracle_bf16_to_f32(xs[i]) / scale);
        }
}

/*
 * mxfp8 ([MEB] MEGA_COMBINE_DTYPE: 32 e4m3 elements share one e8m0 scale).
 * The shared exponent follows the OCP Microscaling v1.0 conversion: the
 * largest power of two not above amax, minus the largest exponent of e4m3
 * (8), clamped to the e8m0 range; an all-zero group takes the smallest
 * scale.  Elements are e4m3(v * 2^-X) with saturation.
 */
void oracle_quant_mxfp8(int64_t rows, int32_t H, const float *v, uint8_t *q, uint8_t *e8m0)
{
    const int32_t groups = H / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t g = 0; g < groups; ++g) {
            const float *vs = v + r * H + g * 32;
            float amax = 0.0f;
            for (int32_t i = 0; i < 32; ++i) {
                float a = fabsf(vs[i]);
                if (a > amax) amax = a;
            }
            int X;
            if (amax == 0.0f) {
                X = -127;
            } else {
                int ex;
                frexpf(amax, &ex);   /* amax = f * 2^ex, f in [0.5, 1) */
                X = (ex - 1) - 8;
                if (X < -127) X = -127;
                if (X > 127) X = 127;
            }
            float p = ldexpf(1.0f, -X);  /* exact for X in [-127, 127] */
            e8m0[r * groups + g] = (uint8_t)(X + 127);
            for (int32_t i = 0; i < 32; ++i)
                q[r * H + g * 32 + i] = oracle_f32_to_e4m3(vs[i] * p);
        }
}

/*
 * nvfp4 ([MEB] MEGA_COMBINE_DTYPE: "16e2m1xbf16").  The pages fix the shape
 * only; the rule taken: s = bf16_rne(amax / 6) (6 = largest e2m1), 1.0 when
 * that is zero, element e2m1(v / s) with saturation.
 */
void oracle_quant_nvfp4(int64_t rows, int32_t H, const float *v, uint8_t *q, uint16_t *scales)
{
    const int32_t groups = H / 16;
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t g = 0; g < groups; ++g) {
            const float *vs = v + r * H + g * 16;
            float amax = 0.0f;
            for (int32_t i = 0; i < 16; ++i) {
                float a = fabsf(vs[i]);
                if (a > amax) amax = a;
            }
            uint16_t sb = oracle_f32_to_bf16(amax / 6.0f);
            if (oracle_bf16_to_f32(sb) == 0.0f) sb = 0x3F80;
            const float s = oracle_bf16_to_f32(sb);
            scales[r * groups + g] = sb;
            for (int32_t i = 0; i < 16; i += 2) {
                uint8_t lo = oracle_f32_to_e2m1(vs[i] / s);
                uint8_t hi = oracle_f32_to_e2m1(vs[i + 1] / s);
                q[r * (H / 2) + (g * 16 + i) / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
}

void oracle_expert_requant_nvfp4(int32_t E, int32_t H, const int32_t *expert_offset,
                                 const float *factor, const uint16_t *recv, uint8_t *out_q,
                                 uint16_t *out_scales)
{
    float *v = (float *)malloc(sizeof(float) * (size_t)H);
    for (int32_t e = 0; e < E; ++e)
        for (int64_t s = expert_offset[e]; s < expert_offset[e + 1]; ++s) {
            for (int32_t h = 0; h < H; ++h) {
                v[h] = oracle_bf16_to_f32(recv[s * H + h]);
                if (factor) v[h] = v[h] * factor[e];
            }
            oracle_quant_nvfp4(1, H, v, out_q + s * (H / 2), out_scales + s * (H / 16));
        }
    free(v);
}

/* ======================================================================== */
/* Combine                                                                   */
/* ======================================================================== */

/*
 * [MORI] "Combine": the reverse of dispatch; [PR860] LL combine commit: each
 * expert returns one row per dispatched (token, expert) pair.  The reduce is
 * the top-k weighted sum with fp32 accumulation in slot order: from -0.0f
 * (the additive identity of IEEE addition, so the chain equals "first
 * product, then fused adds" and keeps the sign of a zero), acc =
 * fmaf(w[t,j], value, acc) for j = 0..k-1 (masked slots skipped), one round
 * to bf16 at the end.  A token with no valid slot gets +0.0.  The loop runs
 * over j outside h; each element's own sequence of operations is exactly the
 * one above.
 */
void oracle_combine_bf16(int64_t T, int32_t k, int32_t H, const uint16_t *expert_out,
                         const int32_t *token_slot, const float *topk_w, uint16_t *y)
{
    float *acc = (float *)malloc(sizeof(float) * (size_t)H);
    for (int64_t t = 0; t < T; ++t) {
        int32_t nvalid = 0;
        for (int32_t h = 0; h < H; ++h) acc[h] = -0.0f;
        for (int32_t j = 0; j < k; ++j) {
            int32_t s = token_slot[t * k + j];
            if (s < 0) continue;
            ++nvalid;
            const float w = topk_w[t * k + j];
            const uint16_t *row = expert_out + (int64_t)s * H;
            for (int32_t h = 0; h < H; ++h) acc[h] = fmaf(w, oracle_bf16_to_f32(row[h]), acc[h]);
        }
        for (int32_t h = 0; h < H; ++h)
            y[t * H + h] = nvalid ? oracle_f32_to_bf16(acc[h]) : (uint16_t)0;
    }
    free(acc);
}

/* mxfp8 payload: element value = e4m3(q) * 2^(e8m0 - 127), which is exact in
 * binary32 (a 4-bit significand times a power of two). */
void oracle_combine_mxfp8(int64_t T, int32_t k, int32_t H, const uint8_t *expert_q,
                          const uint8_t *expert_e8m0, const int32_t *token_slot,
                          const float *topk_w, uint16_t *y)
{
    const int32_t groups = H / 32;
    float *acc = (float *)malloc(sizeof(float) * (size_t)H);
    for (int64_t t = 0; t < T; ++t) {
        int32_t nvalid = 0;
        for (int32_t h = 0; h < H; ++h) acc[h] = -0.0f;
        for (int32_t j = 0; j < k; ++j) {
            int32_t s = token_slot[t * k + j];
            if (s < 0) continue;
            ++nvalid;
            const float w = topk_w[t * k + j];
            const uint8_t *row = expert_q + (int64_t)s * H;
            const uint8_t *sc = expert_e8m0 + (int64_t)s * groups;
            for (int32_t h = 0; h < H; ++h) {
                float v = oracle_e4m3_to_f32(row[h]) * oracle_e8m0_to_f32(sc[h / 32]);
                acc[h] = fmaf(w, v, acc[h]);
            }
        }
        for (int32_t h = 0; h < H; ++h)
            y[t * H + h] = nvalid ? oracle_f32_to_bf16(acc[h]) : (uint16_t)0;
    }
    free(acc);
}

/* nvfp4 payload: element value = e2m1 * f32(bf16 scale), exact in binary32
 * (a 2-bit significand times an 8-bit one). */
void oracle_combine_nvfp4(int64_t T, int32_t k, int32_t H, const uint8_t *expert_q,
                          const uint16_t *expert_scales, const int32_t *token_slot,
                          const float *topk_w, uint16_t *y)
{
    float *acc = (float *)malloc(sizeof(float) * (size_t)H);
    for (int64_t t = 0; t < T; ++t) {
        int32_t nvalid = 0;
        for (int32_t h = 0; h < H; ++h) acc[h] = -0.0f;
        for (int32_t j = 0; j < k; ++j) {
            int32_t s = token_slot[t * k + j];
            if (s < 0) continue;
            ++nvalid;
            const float w = topk_w[t * k + j];
            const uint8_t *row = expert_q + (int64_t)s * (H / 2);
            const uint16_t *sc = expert_scales + (int64_t)s * (H / 16);
            for (int32_t h = 0; h < H; ++h) {
                uint8_t code = (uint8_t)((row[h / 2] >> (4 * (h & 1))) & 0xF);
                float v = oracle_e2m1_to_f32(code) * oracle_bf16_to_f32(sc[h / 16]);
                acc[h] = fmaf(w, v, acc[h]);
            }
        }
        for (int32_t h = 0; h < H; ++h)
            y[t * H + h] = nvalid ? oracle_f32_to_bf16(acc[h]) : (uint16_t)0;
    }
    free(acc);
}

void oracle_combine_bf16_f64(int64_t T, int32_t k, int32_t H, const uint16_t *expert_out,
                             const int32_t *token_slot, const float *topk_w, double *y)
{
    for (int64_t t = 0; t < T; ++t)
        for (int32_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                int32_t s = token_slot[t * k + j];
                if (s < 0) continue;
                acc += (double)topk_w[t * k + j] *
                       (double)oracle_bf16_to_f32(expert_out[(int64_t)s * H + h]);
            }
            y[t * H + h] = acc;
        }
}

/* ======================================================================== */
/* Expert stage used by the workloads                                        */
/* ======================================================================== */

void oracle_expert_scale_bf16(int32_t E, int32_t H, const int32_t *expert_offset,
                              const float *factor, const uint16_t *recv, uint16_t *out)
{
    for (int32_t e = 0; e < E; ++e)
        for (int64_t s = expert_offset[e]; s < expert_offset[e + 1]; ++s)
            for (int32_t h = 0; h < H; ++h)
                out[s * H + h] = oracle_f32_to_bf16(oracle_bf16_to_f32(recv[s * H + h]) * factor[e]);
}

void oracle_expert_requant_mxfp8(int32_t E, int32_t H, const int32_t *expert_offset,
                                 const float *factor, const uint8_t *recv_q,
                                 const float *recv_scales, uint8_t *out_q, uint8_t *out_e8m0)
{
    const int32_t g128 = H / 128;
    float *v = (float *)malloc(sizeof(float) * (size_t)H);
    for (int32_t e = 0; e < E; ++e)
        for (int64_t s = expert_offset[e]; s < expert_offset[e + 1]; ++s) {
            for (int32_t h = 0; h < H; ++h) {
                v[h] = oracle_e4m3_to_f32(recv_q[s * H + h]) * recv_scales[s * g128 + h / 128];
                if (factor) v[h] = v[h] * factor[e];
            }
            oracle_quant_mxfp8(1, H, v, out_q + s * H, out_e8m0 + s * (H / 32));
        }
    free(v);
}
