/*
 * ep_oracle.h -- plain, slow, single-threaded CPU oracle for MoE expert-parallel
 * dispatch and combine (layout, slot permutation, top-k weighted gather-reduce).
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load this library.  It shares no
 * code, header, table or helper with the HIP library; the two meet only through
 * the seeded input generators.
 *
 * Sources (web pages):
 *   [MORI]  "MORI-EP Benchmark" (rocm.github.io/mori), sections "Bandwidth
 *           Computation" (RDMA bandwidth; Algo BW vs Physical BW; NVL / XGMI
 *           bandwidth), "Why DeepEP and Mori RDMA token counts are equivalent"
 *           (Steps 1-3), "Combine", and "Reference: print_bw_values.py".
 *   [MEB]   "MoE-EP Benchmark" README (moe_ep_benchmark), "Environment
 *           reference" table (MEGA_COMBINE_DTYPE, MEGA_ACC rows).
 *   [PR860] "ep(bench): add mscclpp high-throughput (rank-major) backend ..."
 *           (microsoft/mscclpp pull request 860): the RANK_MAJOR / TOKEN_MAJOR
 *           layout commit ("compacted DeepEP prefix offset"), the LL combine
 *           byte-count commit (one copy per dispatched token per expert).
 *
 * Conventions shared by every function:
 *   - topk_idx is [T, k] int64, row-major; any negative id means "no expert"
 *     (masked) and is skipped everywhere; an id >= E is invalid, is treated
 *     as masked and is counted in the return value of the layout function.
 *   - bf16 values travel as their uint16 bit patterns, e4m3 and e8m0 as bytes.
 *   - All pointers are host pointers owned by the caller.
 */
#ifndef EP_ORACLE_H
#define EP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- layout ----------------------------------------------------------- */

/* Set-based layout.  Returns the number of invalid (>= E) ids seen. */
int64_t oracle_layout(int64_t T, int32_t k, int32_t E, int32_t R, int32_t N,
                      const int64_t *topk_idx,
                      int32_t *num_tokens_per_rank,   /* [R] */
                      int32_t *num_tokens_per_expert, /* [E] */
                      uint8_t *is_token_in_rank,      /* [T, R] (0/1) */
                      int32_t *num_tokens_per_node,   /* [N] */
                      int64_t *rdma_algo_token_count);

/* Per-row "unique ids, sorted descending, padded with -1" rewrite of a
 * [rows, cols] id matrix with ids in [0, num_slots) or negative. */
void oracle_unique_rows(int64_t rows, int32_t cols, int32_t num_slots, int64_t *ids);

/* Node deduplication by the per-row unique rewrite; returns the count of
 * non-(-1) entries.  node_rows [T, k] receives the rewritten rows (may be NULL). */
int64_t oracle_algo_by_unique(int64_t T, int32_t k, int32_t E, int32_t N,
                              const int64_t *topk_idx, int64_t *node_rows);

/* Node deduplication by a [T, N] presence matrix; returns the count of set
 * entries.  presence may be NULL. */
int64_t oracle_algo_by_presence(int64_t T, int32_t k, int32_t E, int32_t N,
                                const int64_t *topk_idx, uint8_t *presence);

/* ---- accounting (host arithmetic on counts) ---------------------------- */

typedef struct {
    int64_t rdma_algo_tokens;          /* deduped (token, node) pairs, local node included */
    double  rdma_physical_tokens;      /* algo * (N - 1) / N */
    int64_t rdma_physical_tokens_exact;/* (token, node) pairs with node != own_node */
    int64_t nvl_tokens;                /* sum over ranks of num_tokens_per_rank */
    double  dispatch_rdma_bytes_bf16;  /* algo * H * 2 */
    double  dispatch_nvl_bytes_bf16;   /* nvl_tokens * H * 2 */
    double  combine_rdma_bytes_bf16;   /* equal to dispatch rdma bytes */
    double  combine_nvl_bytes_bf16;    /* equal to dispatch nvl bytes */
    double  fp8_factor;                /* (1 + 4/128) / 2 */
    double  dispatch_rdma_bytes_fp8;
    double  dispatch_nvl_bytes_fp8;
} oracle_accounting_t;

void oracle_accounting(int32_t H, int32_t R, int32_t N, int32_t own_node,
                       const int32_t *num_tokens_per_rank, const int32_t *num_tokens_per_node,
                       int64_t rdma_algo_token_count, oracle_accounting_t *out);

/* ---- slot assignment and dispatch ------------------------------------- */

/* Stable counting sort of the valid (t, j) pairs by expert.  token_slot[t,j]
 * is -1 for masked/invalid pairs.  recv_src_idx / recv_topk_w have capacity
 * T*k; entries at or beyond expert_offset[E] are left untouched. */
void oracle_slots(int64_t T, int32_t k, int32_t E, const int64_t *topk_idx,
                  const float *topk_w,
                  int32_t *token_slot,    /* [T, k] */
                  int32_t *expert_offset, /* [E + 1] */
                  int32_t *recv_src_idx,  /* [T*k] */
                  float *recv_topk_w);    /* [T*k] */

/* RANK_MAJOR fixed-slot layout ([PR860] RANK_MAJOR commit: each dispatched
 * token at a fixed [num_ranks, max_tokens_per_rank, hidden] slot instead of a
 * compacted prefix offset).  For one source: virtual rank r owns receive rows
 * [r*M, (r+1)*M); inside, the rank's expert segments in expert order, pairs
 * in row-major (t, j) order.  Pairs past a rank's capacity M get slot -1 and
 * are counted in the return value.  recv_src_idx / recv_topk_w have R*M
 * entries; rows a rank does not fill are left untouched. */
int64_t oracle_slots_rank_major(int64_t T, int32_t k, int32_t E, int32_t R, int32_t M,
                                const int64_t *topk_idx, const float *topk_w,
                                int32_t *token_slot, int32_t *recv_src_idx, float *recv_topk_w);

/* (token, rank) receive rows, the high-throughput layout ([PR860]: DeepEP's
 * expanded receive layout, one row per (token, source rank) pair; [MORI]
 * "NVL / XGMI bandwidth": one received row per token and rank).  For one
 * source: a token reaches rank r when one of its valid experts lives on r;
 * it then gets exactly one row in r's region.  Regions back to back in rank
 * order (rank_offset = exclusive scan of num_tokens_per_rank), ascending t
 * inside a region.  token_rank_slot [T, R] (-1 when t does not reach r),
 * rank_offset [R+1], recv_src_idx [T*min(k,R)].  Per row s, the token's
 * top-k list as its rank sees it: recv_topk_idx [rows, k] = e - r*EPR for
 * the slots whose expert lives on r, else -1; recv_topk_w [rows, k] = the
 * slot's weight there, else 0. */
void oracle_slots_ranks(int64_t T, int32_t k, int32_t E, int32_t R, const int64_t *topk_idx,
                        const float *topk_w, int32_t *token_rank_slot, int32_t *rank_offset,
                        int32_t *recv_src_idx, int32_t *recv_topk_idx, float *recv_topk_w);

/* Expert stage of the (token, rank) layout (the weights are applied on the
 * destination, which returns one partial row per received row):
 * partial[s] = bf16_rne( fp32 fma chain over the token's slots j (ascending)
 * whose expert e lives on row s's rank, from -0.0f:
 * acc = fmaf(w[t,j], o_e, acc) ), where the expert's output element is
 * o_e = bf16_rne(v * factor[e]) (factor NULL: bf16_rne(v)) and v is the
 * received bf16 element (recv_q NULL) or e4m3(recv_q) * its group's fp32
 * scale (recv_scales [rows, H/128]). */
void oracle_expert_reduce_ranks(int64_t T, int32_t k, int32_t E, int32_t R, int32_t H,
                                const int64_t *topk_idx, const float *topk_w, const float *factor,
                                const int32_t *rank_offset, const int32_t *recv_src_idx,
                                const uint16_t *recv, const uint8_t *recv_q, const float *recv_scales,
                                uint16_t *partial);

/* Combine of the (token, rank) layout: y[t] = bf16_rne(sum over the token's
 * ranks, ascending, of f32(partial[token_rank_slot[t,r]])), fp32 adds from
 * -0.0f; +0.0 for a token that reaches no rank. */
void oracle_combine_ranks(int64_t T, int32_t R, int32_t H, const uint16_t *partial,
                          const int32_t *token_rank_slot, uint16_t *y);

/* recv[token_slot[t,j]] = src[t] for every valid pair: a bitwise copy of
 * row_bytes bytes per row (works for bf16 rows, e4m3 rows and scale rows). */
void oracle_dispatch_rows(int64_t T, int32_t k, int64_t row_bytes, const void *src,
                          const int32_t *token_slot, void *recv);

/* ---- combine ----------------------------------------------------------- */

/* y[t,h] = bf16_rne( fma chain over valid j in ascending order, from -0.0f,
 *                    acc = fmaf(topk_w[t,j], value(token_slot[t,j], h), acc) );
 * a token with no valid slot gets +0.0. */
void oracle_combine_bf16(int64_t T, int32_t k, int32_t H, const uint16_t *expert_out,
                         const int32_t *token_slot, const float *topk_w, uint16_t *y);

/* Same with mxfp8 rows: value = e4m3(q) * 2^(e8m0 - 127), one e8m0 per 32. */
void oracle_combine_mxfp8(int64_t T, int32_t k, int32_t H, const uint8_t *expert_q,
                          const uint8_t *expert_e8m0, const int32_t *token_slot,
                          const float *topk_w, uint16_t *y);

/* fp64 evaluation of the same weighted sum, without rounding to bf16 (for
 * error-bound checks of the fp32 chain). */
void oracle_combine_bf16_f64(int64_t T, int32_t k, int32_t H, const uint16_t *expert_out,
                             const int32_t *token_slot, const float *topk_w, double *y);

/* ---- number formats and quantization ----------------------------------- */

uint16_t oracle_f32_to_bf16(float f);
float    oracle_bf16_to_f32(uint16_t b);
uint8_t  oracle_f32_to_e4m3(float f);        /* RNE, saturate to +-448, NaN -> 0x7F|s */
float    oracle_e4m3_to_f32(uint8_t q);
float    oracle_e8m0_to_f32(uint8_t e);      /* 2^(e-127); 255 -> NaN */

uint8_t  oracle_f32_to_e2m1(float f);        /* 4-bit code: RNE, saturate to +-6 */
float    oracle_e2m1_to_f32(uint8_t q);      /* low 4 bits */

/* fp8 rows: per (row, 128-channel group) amax, scale = amax/448 (1 if 0),
 * q = e4m3(x / scale). */
void oracle_quant_fp8_s128(int64_t rows, int32_t H, const uint16_t *x_bf16,
                           uint8_t *q, float *scales /* [rows, H/128] */);

/* mxfp8 encode of fp32 rows: per 32-group X = clamp(floor(log2 amax) - 8,
 * -127, 127) (-127 for an all-zero group), q = e4m3(v * 2^-X), byte X + 127. */
void oracle_quant_mxfp8(int64_t rows, int32_t H, const float *v, uint8_t *q, uint8_t *e8m0);

/* nvfp4 ([MEB] MEGA_COMBINE_DTYPE: 16 e2m1 elements share one bf16 scale).
 * Per 16-group: s = bf16_rne(amax / 6) (1.0 when that is zero), element
 * e2m1_rne_sat(v / s); two elements per byte, the even element in the low
 * nibble.  q is [rows, H/2] bytes, scales [rows, H/16] bf16 bits. */
void oracle_quant_nvfp4(int64_t rows, int32_t H, const float *v, uint8_t *q, uint16_t *scales);

/* Combine over nvfp4 rows: value = e2m1 * f32(scale bf16). */
void oracle_combine_nvfp4(int64_t T, int32_t k, int32_t H, const uint8_t *expert_q,
                          const uint16_t *expert_scales, const int32_t *token_slot,
                          const float *topk_w, uint16_t *y);

/* Expert stage for the nvfp4 payload: out = nvfp4(f32(recv[s]) * factor[e(s)])
 * (factor may be NULL: identity). */
void oracle_expert_requant_nvfp4(int32_t E, int32_t H, const int32_t *expert_offset,
                                 const float *factor, const uint16_t *recv, uint8_t *out_q,
                                 uint16_t *out_scales);

/* Expert stage used by the workloads (not part of dispatch or combine):
 *  scale_bf16:  out[s] = bf16( f32(recv[s]) * factor[e(s)] )
 *  requant:     v = e4m3(q[s]) * scale128[s]  (times factor[e(s)] if factor),
 *               then mxfp8-encode v.
 * e(s) is the expert whose segment [expert_offset[e], expert_offset[e+1])
 * holds row s. */
void oracle_expert_scale_bf16(int32_t E, int32_t H, const int32_t *expert_offset,
                              const float *factor, const uint16_t *recv, uint16_t *out);
void oracle_expert_requant_mxfp8(int32_t E, int32_t H, const int32_t *expert_offset,
                                 const float *factor, const uint8_t *recv_q,
                                 const float *recv_scales, uint8_t *out_q, uint8_t *out_e8m0);

#ifdef __cplusplus
}
#endif
#endif /* EP_ORACLE_H */
