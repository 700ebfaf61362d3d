/*
 * The C ABI of libep_hip used from plain C (no torch, no C++): device memory
 * from the HIP runtime, one stream, the layout -> dispatch -> combine calls,
 * and the single-call layout + dispatch, each result compared with the CPU
 * oracle (oracle/ep_oracle.h, test infrastructure) on the same inputs.
 *
 * Inputs are drawn here with a 64-bit xorshift generator: finite bf16 rows
 * (random sign, exponents 2^-7 .. 2^7, random mantissas), k distinct experts
 * per token with about one slot in ten masked, fp32 weights in [0, 1).
 *
 * Exit status 0 when every output matches (integer outputs and rows bitwise,
 * y bitwise -- both sides run the same fp32 chain), 1 on a mismatch, 2 on an
 * API or runtime error.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep.h"
#include "ep_oracle.h"

#define T_ 300
#define H_ 512
#define E_ 32
#define R_ 8
#define N_ 2
#define K_ 4

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
    uint64_t x = rng_state;
    x ^= x << 13;
    x ^= x >> 7;
    x ^= x << 17;
    return rng_state = x;
}

#define HIP_OK(call)                                                         \
    do {                                                                     \
        hipError_t e_ = (call);                                              \
        if (e_ != hipSuccess) {                                              \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_)); \
            exit(2);                                                         \
        }                                                                    \
    } while (0)
#define EP_OK_(call)                                                         \
    do {                                                                     \
        int rc_ = (call);                                                    \
        if (rc_ != EP_OK) {                                                  \
            fprintf(stderr, "%s failed: %s\n", #call, ep_strerror(rc_));     \
            exit(2);                                                         \
        }                                                                    \
    } while (0)

static int same(const char *what, const void *a, const void *b, size_t bytes) {
    if (memcmp(a, b, bytes) == 0) return 1;
    fprintf(stderr, "mismatch: %s\n", what);
    return 0;
}

static void *dev_copy(const void *src, size_t bytes) {
    void *d = NULL;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 16));
    if (bytes) HIP_OK(hipMemcpy(d, src, bytes, hipMemcpyHostToDevice));
    return d;
}

int main(void) {
    const int64_t T = T_, TK = (int64_t)T_ * K_;
    static uint16_t x[T_ * H_];
    static int64_t idx[T_ * K_];
    static float w[T_ * K_];
    for (int64_t i = 0; i < T * H_; ++i) {
        const uint64_t r = next_u64();
        const uint16_t sign = (uint16_t)((r & 1u) << 15);
        const uint16_t expo = (uint16_t)(120 + (r >> 1) % 15);   /* 2^-7 .. 2^7 */
        x[i] = (uint16_t)(sign | (expo << 7) | ((r >> 8) & 0x7F));
    }
    for (int64_t t = 0; t < T; ++t) {
        int perm[E_];
        for (int e = 0; e < E_; ++e) perm[e] = e;
        for (int j = 0; j < K_; ++j) {   /* partial Fisher-Yates: k distinct experts */
            const int p = j + (int)(next_u64() % (uint64_t)(E_ - j));
            const int tmp = perm[j];
            perm[j] = perm[p];
            perm[p] = tmp;
            idx[t * K_ + j] = (next_u64() % 10 == 0) ? -1 : perm[j];
            w[t * K_ + j] = (float)(next_u64() >> 40) / (float)(1 << 24);
        }
    }

    ep_shape sh;
    memset(&sh, 0, sizeof sh);
    sh.num_tokens = T;
    sh.hidden = H_;
    sh.num_experts = E_;
    sh.num_ranks = R_;
    sh.num_nodes = N_;
    sh.num_topk = K_;
    sh.x_format = EP_FMT_BF16;
    sh.y_format = EP_FMT_BF16;
    if (ep_abi_version() != EP_ABI_VERSION) {
        fprintf(stderr, "ABI version %d, header %d\n", ep_abi_version(), EP_ABI_VERSION);
        return 2;
    }
    EP_OK_(ep_validate_shape(&sh));
    size_t wsb = 0;
    EP_OK_(ep_workspace_bytes(&sh, &wsb));
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    void *ws = NULL;
    HIP_OK(hipMalloc(&ws, wsb));
    EP_OK_(ep_workspace_init(ws, wsb, st));

    void *d_x = dev_copy(x, sizeof x), *d_idx = dev_copy(idx, sizeof idx), *d_w = dev_copy(w, sizeof w);
    void *d_per_rank, *d_per_expert, *d_in_rank, *d_per_node, *d_algo, *d_recv, *d_src, *d_rw, *d_slot, *d_off, *d_y;
    HIP_OK(hipMalloc(&d_per_rank, 4 * R_));
    HIP_OK(hipMalloc(&d_per_expert, 4 * E_));
    HIP_OK(hipMalloc(&d_in_rank, (size_t)T * R_));
    HIP_OK(hipMalloc(&d_per_node, 4 * N_));
    HIP_OK(hipMalloc(&d_algo, 8));
    HIP_OK(hipMalloc(&d_recv, (size_t)TK * H_ * 2));
    HIP_OK(hipMalloc(&d_src, 4 * (size_t)TK));
    HIP_OK(hipMalloc(&d_rw, 4 * (size_t)TK));
    HIP_OK(hipMalloc(&d_slot, 4 * (size_t)TK));
    HIP_OK(hipMalloc(&d_off, 4 * (E_ + 1)));
    HIP_OK(hipMalloc(&d_y, (size_t)T * H_ * 2));

    /* the oracle */
    static int32_t o_per_rank[R_], o_per_expert[E_], o_per_node[N_], o_slot[T_ * K_], o_off[E_ + 1], o_src[T_ * K_];
    static uint8_t o_in_rank[T_ * R_];
    static float o_rw[T_ * K_];
    static uint16_t o_recv[T_ * K_ * H_], o_y[T_ * H_];
    int64_t o_algo = 0;
    oracle_layout(T, K_, E_, R_, N_, idx, o_per_rank, o_per_expert, o_in_rank, o_per_node, &o_algo);
    oracle_slots(T, K_, E_, idx, w, o_slot, o_off, o_src, o_rw);
    oracle_dispatch_rows(T, K_, 2 * H_, x, o_slot, o_recv);
    oracle_combine_bf16(T, K_, H_, o_recv, o_slot, w, o_y);
    const int32_t V = o_off[E_];

    int ok = 1;
    for (int pass = 0; pass < 2; ++pass) {
        if (pass == 0) {   /* layout, then the dispatch that reuses its plan */
            EP_OK_(ep_dispatch_layout(&sh, d_idx, d_per_rank, d_per_expert, d_in_rank, d_per_node, d_algo, ws,
                                      wsb, st));
            EP_OK_(ep_dispatch_from_layout(&sh, d_x, NULL, d_idx, d_w, d_recv, NULL, d_src, d_rw, d_slot, d_off,
                                           ws, wsb, st));
        } else {           /* one call (a single launch at this size) */
            HIP_OK(hipMemsetAsync(d_recv, 0, (size_t)TK * H_ * 2, st));
            EP_OK_(ep_dispatch_with_layout(&sh, d_x, NULL, d_idx, d_w, d_per_rank, d_per_expert, d_in_rank,
                                           d_per_node, d_algo, d_recv, NULL, d_src, d_rw, d_slot, d_off, ws, wsb,
                                           st));
        }
        EP_OK_(ep_combine(&sh, d_recv, NULL, d_slot, d_w, d_y, st));
        uint32_t flags = 0;
        EP_OK_(ep_check(ws, wsb, st, &flags));

        static int32_t g_per_rank[R_], g_per_expert[E_], g_per_node[N_], g_slot[T_ * K_], g_off[E_ + 1],
            g_src[T_ * K_];
        static uint8_t g_in_rank[T_ * R_];
        static float g_rw[T_ * K_];
        static uint16_t g_recv[T_ * K_ * H_], g_y[T_ * H_];
        int64_t g_algo = 0;
        HIP_OK(hipMemcpy(g_per_rank, d_per_rank, sizeof g_per_rank, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_per_expert, d_per_expert, sizeof g_per_expert, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_per_node, d_per_node, sizeof g_per_node, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_in_rank, d_in_rank, sizeof g_in_rank, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(&g_algo, d_algo, 8, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_slot, d_slot, sizeof g_slot, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_off, d_off, sizeof g_off, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_src, d_src, sizeof g_src, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_rw, d_rw, sizeof g_rw, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_recv, d_recv, sizeof g_recv, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(g_y, d_y, sizeof g_y, hipMemcpyDeviceToHost));

        ok &= same("num_tokens_per_rank", g_per_rank, o_per_rank, sizeof o_per_rank);
        ok &= same("num_tokens_per_expert", g_per_expert, o_per_expert, sizeof o_per_expert);
        ok &= same("num_tokens_per_node", g_per_node, o_per_node, sizeof o_per_node);
        ok &= same("is_token_in_rank", g_in_rank, o_in_rank, sizeof o_in_rank);
        ok &= same("rdma_algo_token_count", &g_algo, &o_algo, 8);
        ok &= same("token_slot", g_slot, o_slot, sizeof o_slot);
        ok &= same("expert_offset", g_off, o_off, sizeof o_off);
        ok &= same("recv_src_idx", g_src, o_src, 4 * (size_t)V);
        ok &= same("recv_topk_w", g_rw, o_rw, 4 * (size_t)V);
        ok &= same("recv_x", g_recv, o_recv, (size_t)V * H_ * 2);
        ok &= same("y", g_y, o_y, sizeof o_y);
        printf("pass %d (%s): %s, %d valid pairs, algo %lld\n", pass,
               pass == 0 ? "layout + dispatch_from_layout" : "dispatch_with_layout", ok ? "match" : "MISMATCH",
               (int)V, (long long)g_algo);
    }
    return ok ? 0 : 1;
}
