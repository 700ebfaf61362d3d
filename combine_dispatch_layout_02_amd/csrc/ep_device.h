// ep_device.h -- device-side helpers shared by the gfx950 kernels of libep_hip.
//
// Number formats (bit-exact definitions, written for the hardware's integer
// and IEEE float units; no fast-math, no flush-to-zero):
//   bf16   : top 16 bits of a binary32; narrowing rounds to nearest even,
//            NaN becomes 0x7FC0.
//   e4m3   : OCP 8-bit float "E4M3" (fn variant): bias 7, 3 mantissa bits,
//            S.1111.111 = NaN, no infinities, largest finite 448.  Encoding
//            rounds to nearest even and saturates finite overflow and
//            infinities to +-448.
//   e8m0   : OCP Microscaling scale, 2^(e - 127); 0xFF = NaN.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bit casts

__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return u2f(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return u2f(pair & 0xFFFF0000u); }

// binary32 -> bf16 bits, round to nearest even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = f2u(f);
    uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC0u : r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// The same two narrowings by gfx950's v_cvt_pk_bf16_f32 (one instruction):
// round to nearest even, bit for bit f32_to_bf16 on every non-NaN binary32
// (checked over all 2^32 patterns on MI355X); a NaN keeps its payload
// (quieted) instead of becoming 0x7FC0, so it is used only where no input is
// NaN (pack_bf16).
__device__ __forceinline__ uint32_t pack_bf16x2_cvt(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// M binary32 values of a lane (M even) -> M / 2 bf16 pairs, the even value in
// the low half.  When no lane of the wave holds a NaN, by the packing
// instruction; else by f32_to_bf16 (NaN -> 0x7FC0).  The test: the fp32 sum
// of a lane's values is NaN when one of them is (and when +inf meets -inf,
// which only sends the wave down the exact path).  Called by the whole wave:
// the choice is wave-uniform.
template <int M>
__device__ __forceinline__ void pack_bf16(const float (&v)[M], uint32_t (&out)[M / 2]) {
    float s = v[0];
#pragma unroll
    for (int i = 1; i < M; ++i) s += v[i];
    if (__ballot(s != s) == 0) {
#pragma unroll
        for (int i = 0; i < M / 2; ++i) out[i] = pack_bf16x2_cvt(v[2 * i], v[2 * i + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < M / 2; ++i) out[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    }
}

// ---------------------------------------------------------------- e4m3

// binary32 -> e4m3 byte (RNE, saturating).
//   |f| >= 448 (or inf)       -> 0x7E with sign
//   normal e4m3 range (>=2^-6): drop 20 mantissa bits with RNE on the integer
//                               pattern (a carry moves into the exponent),
//                               rebias 127 -> 7 (subtract 120 << 3)
//   below 2^-6                 -> subnormal steps of 2^-9: rint(|f| * 512)
//                               (the scaling is exact; 8 is the smallest
//                               normal code 0x08)
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
    const uint32_t u = f2u(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a > 0x7F800000u) {
        code = 0x7Fu;
    } else if (a >= 0x43E00000u) {        // 448.0f
        code = 0x7Eu;
    } else if (a >= 0x3C800000u) {        // 2^-6
        uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
        code = (r >> 20) - (120u << 3);
    } else {
        code = (uint32_t)__builtin_rintf(u2f(a) * 512.0f);
    }
    return sign | code;
}

// e4m3 byte -> binary32 (exact).  The byte's exponent+mantissa bits placed at
// binary32 bits 20..26 read as a float equal to value * 2^-120 for normals and
// subnormals alike; multiplying by 2^120 is exact.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t mag = b & 0x7Fu;
    float v = u2f(mag << 20) * 0x1p120f;
    v = (mag == 0x7Fu) ? __builtin_nanf("") : v;
    return (b & 0x80u) ? -v : v;
}

// ---------------------------------------------------------------- e2m1

// binary32 -> e2m1 code (OCP 4-bit E2M1: bias 1, one mantissa bit,
// magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), RNE, saturating to +-6.
//   |f| >= 6 (or inf / NaN) -> 0x7 with sign
//   [1, 6): keep one of 23 mantissa bits with RNE on the integer pattern,
//           rebias 127 -> 1 (a carry moves into the exponent)
//   below 1: steps of 0.5: rint(|f| * 2) (2 is the code of 1.0)
__device__ __forceinline__ uint32_t f32_to_e2m1(float f) {
    const uint32_t u = f2u(f);
    const uint32_t sign = (u >> 28) & 0x8u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a >= 0x40C00000u) {            // 6.0f, inf, NaN
        code = 0x7u;
    } else if (a >= 0x3F800000u) {     // 1.0f
        const uint32_t r = a + 0x1FFFFFu + ((a >> 22) & 1u);
        code = (r >> 22) - (126u << 1);
    } else {
        code = (uint32_t)__builtin_rintf(u2f(a) * 2.0f);
    }
    return sign | code;
}

// ---------------------------------------------------------------- e8m0

// 2^(e - 127) as a binary32 (exact; e = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    float v = (e == 0u) ? u2f(0x00400000u) : u2f(e << 23);
    return (e == 0xFFu) ? __builtin_nanf("") : v;
}

// Shared exponent X of an mxfp8 32-group with largest magnitude amax:
// clamp(floor(log2 amax) - 8, -127, 127); -127 for amax == 0 or a binary32
// subnormal amax (whose floor(log2) is below -126).
__device__ __forceinline__ int mx_shared_exp(float amax) {
    const uint32_t a = f2u(amax) & 0x7FFFFFFFu;
    if (a < 0x00800000u) return -127;
    const int x = (int)(a >> 23) - 127 - 8;
    return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// 2^-X as a binary32 for X in [-127, 127] (exact).
__device__ __forceinline__ float pow2_neg(int X) {
    const int e = 127 - X;   // biased exponent of 2^-X
    return (e <= 0) ? u2f(0x00400000u) : u2f((uint32_t)e << 23);
}

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return (l == 0) ? 0ull : (~0ull >> (64 - l));
}

template <typename T>
__device__ __forceinline__ T readlane(T v, int lane);

template <>
__device__ __forceinline__ int readlane<int>(int v, int lane) {
    return __builtin_amdgcn_readlane(v, lane);
}
template <>
__device__ __forceinline__ float readlane<float>(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

typedef f32x2_t f32x2;

// 16-byte vector type used for every row copy (one global_load/store_dwordx4).
typedef uint32_t vec16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ vec16 ld16(const void *p) {
    return *reinterpret_cast<const vec16 *>(p);
}
__device__ __forceinline__ void st16(void *p, vec16 v) {
    *reinterpret_cast<vec16 *>(p) = v;
}
// Non-temporal variants: streamed data that is not re-read by this kernel.
__device__ __forceinline__ vec16 ld16_nt(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const vec16 *>(p));
}
__device__ __forceinline__ void st16_nt(void *p, vec16 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<vec16 *>(p));
}

// ---------------------------------------------------------------- token orders

// Execution position g in [0, T) -> token, spreading the tokens [0, P) evenly
// among the tokens [P, T): position g takes the next token of [0, P) when
// floor((g + 1) P / T) > floor(g P / T), else the next token of [P, T).  A
// bijection of [0, T) (the first kind occurs exactly P times).
__device__ __forceinline__ int64_t interleaved_token(int64_t g, int64_t T, int64_t P) {
    if (P <= 0 || P >= T) return g;
    const int64_t c0 = (g * P) / T, c1 = ((g + 1) * P) / T;
    return c1 > c0 ? c0 : P + (g - c0);
}

// ---------------------------------------------------------------- scans

// Exclusive scan of n ints held in LDS (`in`), written to `out` (n + 1
// entries, out[n] = total).  Called by every thread of the block.
__device__ __forceinline__ void block_exclusive_scan(const int32_t *in, int32_t *out, int n, int32_t *tmp) {
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
    if (wid == 0) {   // the wave totals (nw <= 16), scanned by the first wave
        const int32_t x = lane < nw ? tmp[lane] : 0;
        int32_t incl = x;
        for (int off = 1; off < kWave; off <<= 1) {
            const int32_t u = __shfl_up(incl, off);
            if (lane >= off) incl += u;
        }
        if (lane < nw) tmp[lane] = incl - x;
        if (lane == kWave - 1) tmp[nw] = incl;
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

// Exclusive scan of n <= 64 values held one per lane by the first wave
// (lanes >= n hold 0): out[i] for i < n, and out[n] = total.
__device__ __forceinline__ void wave_exclusive_scan(int32_t v, int n, int32_t *out) {
    const int lane = threadIdx.x & (kWave - 1);
    int32_t incl = v;
    for (int off = 1; off < kWave; off <<= 1) {
        const int32_t u = __shfl_up(incl, off);
        if (lane >= off) incl += u;
    }
    if (lane < n) out[lane] = incl - v;
    if (lane == kWave - 1) out[n] = incl;
}

// Sum over the 64 lanes (every lane active), returned wave-uniform: an
// inclusive scan inside each 16-lane row by DPP row shifts, the rows' totals
// carried on by row broadcasts, lane 63's value read back.
__device__ __forceinline__ int32_t wave_sum(int32_t v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
    return __builtin_amdgcn_readlane(v, kWave - 1);
}

// ---------------------------------------------------------------- plan totals

// Layout totals of a multi-tile batch from the tile count matrix [ntiles][E +
// R + N] (raw counts: experts, ranks, nodes), by one block of a copy launch
// while its other blocks copy: per column the sum over tiles -> the layout
// outputs (each may be null), the RDMA algo count (sum of the node totals),
// and the exclusive scan of the expert totals into expert_offset [E + 1] and
// / or of the rank totals into rank_offset [R + 1] (either may be null).
// Integer sums only.  tot: LDS of E + R + N + 1 + blockDim / 64 + 1 ints.
// Called by every thread of the block (blockDim <= 1024, a multiple of 64).
__device__ inline void plan_totals_block(const int32_t *tile_count, int ntiles, int E, int R, int N,
                                         int32_t *per_expert, int32_t *per_rank, int32_t *per_node,
                                         int64_t *algo, int32_t *expert_offset, int32_t *rank_offset,
                                         int32_t *tot) {
    const int tid = threadIdx.x, nt = blockDim.x, cols = E + R + N;
    for (int c = tid; c < cols; c += nt) {
        int32_t sum = 0;
        for (int t0 = 0; t0 < ntiles; t0 += 8) {   // 8 loads in flight (clamped index)
            int32_t v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = tile_count[(size_t)min(t0 + q, ntiles - 1) * cols + c];
#pragma unroll
            for (int q = 0; q < 8; ++q) sum += (t0 + q < ntiles) ? v[q] : 0;
        }
        tot[c] = sum;
        if (c < E) {
            if (per_expert) per_expert[c] = sum;
        } else if (c < E + R) {
            if (per_rank) per_rank[c - E] = sum;
        } else if (per_node) {
            per_node[c - E - R] = sum;
        }
    }
    __syncthreads();
    if (algo && tid == 0) {
        int64_t al = 0;
        for (int n = 0; n < N; ++n) al += tot[E + R + n];
        *algo = al;
    }
    if (rank_offset && tid < kWave) wave_exclusive_scan(tid < R ? tot[E + tid] : 0, R, rank_offset);
    if (expert_offset) block_exclusive_scan(tot, expert_offset, E, tot + cols + 1);
}

// Start of a region plus the earlier tiles' members of it, rebuilt from
// per-tile pairs {members of tile u in earlier regions, members of tile u in
// this region} stored region-major (pairs[region][ntiles], one region's tiles
// side by side): the sum over tiles u of the first plus, for u before `tile`,
// the second.  One tile per lane (an 8-byte load) and a wave sum; returns the
// value for `region` (>= 0) to every lane, 0 for region < 0.  Called by the
// whole wave.
__device__ __forceinline__ int32_t tile_pair_sum_lane(const int2 *pairs, int ntiles, int region, int tile,
                                                      int lane) {
    const int rs = region < 0 ? 0 : region;
    int32_t acc = 0;
    for (int u0 = 0; u0 < ntiles; u0 += kWave) {   // one pass up to 64 tiles
        const int u = u0 + lane;
        const int2 p = pairs[(size_t)rs * ntiles + min(u, ntiles - 1)];   // clamped: always issued
        acc += (u < ntiles) ? p.x + (u < tile ? p.y : 0) : 0;
    }
    return region < 0 ? 0 : acc;
}

}  // namespace ep
